"""The benchmark's byte accounting against the figures the pages print
(tests/golden/traffic_counts.txt, each with its source) and the closed forms
of the algorithmic bytes.  CPU only: bench.py's accounting functions are
pure and import nothing from the GPU path."""
import os

import pytest

import bench
from activation_epilogue_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "traffic_counts.txt")


def _golden():
    vals = {}
    for line in open(GOLDEN):
        line = line.strip()
        if line and not line.startswith("#"):
            k, _, v = line.partition("=")
            vals[k.strip()] = int(v)
    return vals


@pytest.mark.parametrize("M,N", [(4096, 4096), (127, 129), (1, 1)])
def test_fp32_activation_traffic_is_20MN_against_4MN(M, N):
    """"Triton: Fused Matmul + Bias + ReLU (Epilogue Fusion)", "The HBM
    traffic": fp32, the unfused GEMM, bias and ReLU passes move 20*M*N bytes
    of activations, the fused kernel 4*M*N (5x less)."""
    g = _golden()
    t = bench.activation_traffic_bytes(M, N, 4, "relu")
    assert t["unfused"] == g["fp32_unfused_bytes_per_element"] * M * N
    assert t["fused"] == g["fp32_fused_bytes_per_element"] * M * N
    assert t["unfused"] == 5 * t["fused"]


def test_gate_traffic_matches_the_glu_block_figures():
    """"Optimizing GEMM + Activation on CDNA4 with TLX", "The GLU Block": X at
    M=1024, N=21568 in fp16 is 44,171,264 bytes; the two-kernel path (a
    library GEMM with the bias folded in, then the gate pass) moves about
    4 X-sized tensors (~176 MB), and fusion saves about 88 MB (one write and
    one read of X)."""
    g = _golden()
    M, N = g["glu_M"], g["glu_N"]
    x_bytes = M * N * 2
    assert x_bytes == g["glu_X_bytes"]
    t2 = bench.activation_traffic_bytes(M, N, 2, "glu", kernels=2)
    assert t2["unfused"] == 4 * x_bytes
    assert int(t2["unfused"] / 1e6) == g["glu_unfused_MB_approx"]  # 176.7 MB: "about 176"
    saved = t2["unfused"] - t2["fused"]
    assert saved == 2 * x_bytes
    assert int(saved / 1e6) == g["glu_saved_MB_approx"]
    # this library's three-kernel chain adds the bias pass (one more read and write of X)
    t3 = bench.activation_traffic_bytes(M, N, 2, "glu")
    assert t3["unfused"] - t2["unfused"] == 2 * x_bytes
    assert t3["fused"] == t2["fused"] == 2 * x_bytes  # Y read, out written


def test_unknown_chain_length_is_rejected():
    with pytest.raises(ValueError):
        bench.activation_traffic_bytes(4, 4, 2, "relu", kernels=4)


@pytest.mark.parametrize("name,expected", [
    # (M*K + K*N + N + M*N) * 2 bytes: A, B, bias read once, out written once
    ("relu_f16_4096x4096x4096", (3 * 4096 * 4096 + 4096) * 2),
    ("relu_f32_4096x4096x4096", (3 * 4096 * 4096 + 4096) * 4),
    ("relu_bf16_4097x3071x1537", (4097 * 1537 + 1537 * 3071 + 3071 + 4097 * 3071) * 2),
    # the gate also reads Y (M,N)
    ("glu_f16_1024x21568x4096", (1024 * 4096 + 4096 * 21568 + 21568 + 2 * 1024 * 21568) * 2),
    ("gelu_bf16_8192x14336x4096", (8192 * 4096 + 4096 * 14336 + 14336 + 8192 * 14336) * 2),
])
def test_algorithmic_bytes_closed_form(name, expected):
    w = synth.WORKLOADS[name]
    es = bench.ES[w.dtype]
    got = bench.algorithmic_bytes(w.M, w.N, w.K, es, w.act, residual=w.residual, qfmt=w.qfmt, in8=w.in8,
                                  bwd=w.bwd)
    assert got == expected


def test_algorithmic_bytes_variants():
    M, N, K = 300, 200, 100
    base = bench.algorithmic_bytes(M, N, K, 2, "relu")
    assert base == (M * K + K * N + N + M * N) * 2
    # a residual is one more (M,N) read
    assert bench.algorithmic_bytes(M, N, K, 2, "relu", residual=True) == base + M * N * 2
    # a one-byte quantized output instead of the 2-byte one
    assert bench.algorithmic_bytes(M, N, K, 2, "relu", qfmt="fp8_e4m3") == base - M * N
    # FP8 operands: one byte per A and B element
    assert bench.algorithmic_bytes(M, N, K, 2, "relu", in8=True) == base - (M * K + K * N)
    # backward: G, W, X read, dX written, dbias zeroed and added to (fp32)
    assert bench.algorithmic_bytes(M, N, K, 2, "relu", bwd=True) == (M * K + K * N + 2 * M * N) * 2 + 2 * N * 4
    assert bench.algorithmic_bytes(M, N, K, 2, "glu", bwd=True) == (M * K + K * N + 4 * M * N) * 2 + 2 * N * 4


def test_parity_stats_report_errors_and_violations():
    """The bench line's parity statistics: max abs / rel error and the
    violation count of a device output against the oracle's rows."""
    import numpy as np
    import oracle
    w = synth.WORKLOADS["relu_f32_127x129x96"]
    d = synth.draw_workload(w)
    rows = np.array([0, 5, 126])
    ref = bench._oracle_rows(w, d, rows)
    good = bench.parity_stats(w, ref.copy(), ref)
    assert good["ok"] and good["violations"] == 0 and good["max_abs"] == 0.0
    bad = ref.copy()
    bad[1, 3] += np.float32(1.0)
    r = bench.parity_stats(w, bad, ref)
    assert not r["ok"] and r["violations"] == 1 and abs(r["max_abs"] - 1.0) < 1e-6


def test_cpu_model_names_the_host():
    info = bench.cpu_model()
    assert info["logical_cpus"] >= 1


def test_more_than_one_gpu_is_refused():
    """One GPU only: --gpus 2 exits with a message before touching a device."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(os.path.dirname(bench.__file__), "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_committed_traffic_records_match_the_sources():
    """Every profiles/traffic_<workload>.json was taken on the kernel sources
    as they are now (its recorded hash of the listed files, comments and
    whitespace removed, matches), names a known workload and a summary page
    that exists, so the bench line's roofline.traffic is never null for a
    profiled workload and never stale."""
    import glob
    import json
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    recs = sorted(glob.glob(os.path.join(root, "profiles", "traffic_*.json")))
    assert recs, "no traffic records"
    for path in recs:
        rec = json.load(open(path))
        name = os.path.basename(path)[len("traffic_"):-len(".json")]
        assert rec["workload"] == name and name in synth.WORKLOADS, path
        assert rec["source_hash"] == bench.source_hash(rec["sources"]), f"{path} is stale: profile again"
        assert os.path.exists(os.path.join(root, "profiles", rec["summary"])), rec["summary"]
        assert bench.measured_traffic(name) == rec["bytes_per_launch"] > 0
