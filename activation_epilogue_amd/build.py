"""Build libfused_linear.so for gfx950 with hipcc, in-tree.

Ten translation units compiled in parallel: the host/ABI unit (with the
elementwise kernels), one unit of fused GEMM kernels per dtype, one of
quantized-output kernels per 16-bit dtype, one of FP8-input kernels per
16-bit output dtype and one of backward-epilogue kernels per 16-bit dtype.
Every device compile carries -Xclang -target-feature -Xclang -packed-fp32-ops so
that no packed fp32 instructions are generated.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfused_linear.so")
BUILD_DIR = os.path.join(PKG, "_build")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall", "-Wno-unused-command-line-argument"]

UNITS = [
    ("fused_linear.hip", []),
    ("fl_fused_inst.hip", ["-DFL_INST_DTYPE=0"]),
    ("fl_fused_inst.hip", ["-DFL_INST_DTYPE=1"]),
    ("fl_fused_inst.hip", ["-DFL_INST_DTYPE=2"]),
    ("fl_quant_inst.hip", ["-DFL_INST_DTYPE=1"]),
    ("fl_quant_inst.hip", ["-DFL_INST_DTYPE=2"]),
    ("fl_fp8_inst.hip", ["-DFL_INST_DTYPE=1"]),
    ("fl_fp8_inst.hip", ["-DFL_INST_DTYPE=2"]),
    ("fl_bwd_inst.hip", ["-DFL_INST_DTYPE=1"]),
    ("fl_bwd_inst.hip", ["-DFL_INST_DTYPE=2"]),
]


def _compile(unit, extra, obj, save_temps):
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, unit), "-o", obj]
    if save_temps:
        cmd.insert(1, "-save-temps=obj")
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {unit} {extra}:\n{err}")
    return err


def build(verbose: bool = False, save_temps: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = [os.path.join(BUILD_DIR, f"u{i}.o") for i in range(len(UNITS))]
    with ThreadPoolExecutor(max_workers=len(UNITS)) as ex:
        futs = [ex.submit(_compile, u, e, o, save_temps) for (u, e), o in zip(UNITS, objs)]
        for f in futs:
            msg = f.result()
            if verbose and msg.strip():
                print(msg, file=sys.stderr)
    tmp = LIB + f".tmp{os.getpid()}"
    subprocess.run([HIPCC, "-shared", f"--offload-arch={ARCH}", *objs, "-o", tmp], check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True, save_temps="--save-temps" in sys.argv))
