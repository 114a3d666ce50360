"""FP64 CPU oracle for out = act(A@B + bias) -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the CPU-baseline leg of the benchmark
may import this package.  The product path (the HIP library and its binding)
never imports, links or calls it, and shares no code with it.

The arithmetic lives in ``fused_linear_oracle.c`` (plain C, FP64, OpenMP over
output rows, no blocking or fusion).  This module loads it with ctypes,
building it with gcc first when the shared object is missing or stale, and
adds the tolerance check used to compare a device result with the oracle.

Sources (page title, section):
  * "Triton: Fused Matmul + Bias + ReLU (Epilogue Fusion)": opening formula,
    per-column bias added once after the K loop, then max(0, .).
  * "I3. Fuse a GEMM epilogue and change tile scheduling": FP64 reference
    rounded once at the end ("Why the baseline uses FP32"); grouped program
    map ("Tiles and grouped ownership").
  * "Optimizing GEMM + Activation on CDNA4 with TLX", "The GLU Block": the
    gate X + X*Y.
  * "Triton: Fused Matmul + Bias + ReLU (Epilogue Fusion)", "Variants": a
    same-shape residual added to the accumulator before the activation.
  * GELU(tanh): not printed on the pages; Hendrycks & Gimpel (2016).
  * "Optimizing GEMM + Activation on CDNA4 with TLX", "Future Work": the
    epilogue fusion in the backward pass (``fused_linear_bwd``; derivatives
    by the chain rule from the forward definitions).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "fused_linear_oracle.c")
LIB = os.path.join(HERE, "liborc_fused_linear.so")

DTYPES = {"f32": 0, "f16": 1, "bf16": 2}
ACTS = {"none": 0, "relu": 1, "gelu_tanh": 2, "glu": 3}
# raw numpy storage of each dtype; bf16 travels as its uint16 bit pattern
STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}
# |dev - ref| <= atol + rtol * |ref|, from the stated parity bar
TOLERANCE = {"f32": (1e-4, 1e-4), "f16": (4e-3, 1e-2), "bf16": (4e-3, 1e-2)}

_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain x86-64, -O2, OpenMP)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
               "-D_DEFAULT_SOURCE", SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(LIB)
            p, i64, c_int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
            lib.orc_fused_linear.argtypes = [c_int, c_int, p, p, p, p, p, p, i64, i64, i64, p, i64, c_int, p]
            lib.orc_fused_linear.restype = c_int
            lib.orc_unfused_chain.argtypes = [c_int, c_int, p, p, p, p, p, i64, i64, i64, p, i64, c_int, p]
            lib.orc_unfused_chain.restype = c_int
            lib.orc_fused_linear_quant.argtypes = [c_int, c_int, p, p, p, p, p, i64, i64, i64, c_int,
                                                   ctypes.c_float, p, i64, c_int, p]
            lib.orc_fused_linear_quant.restype = c_int
            lib.orc_fused_linear_fp8.argtypes = [c_int, c_int, p, p, ctypes.c_double, p, p, p, i64, i64, i64, p,
                                                 i64, c_int, p]
            lib.orc_fused_linear_fp8.restype = c_int
            lib.orc_quantize.argtypes = [c_int, p, i64, p]
            lib.orc_dequantize.argtypes = [c_int, p, i64, p]
            lib.orc_element.argtypes = [c_int, c_int, p, p, p, p, p, i64, i64, i64, i64, i64, p]
            lib.orc_element.restype = c_int
            lib.orc_decode.argtypes = [c_int, p, i64, p]
            lib.orc_encode.argtypes = [c_int, p, i64, p]
            lib.orc_tile_of_pid.argtypes = [i64, i64, i64, i64, p, p]
            lib.orc_gelu_tanh.argtypes = [ctypes.c_double]
            lib.orc_gelu_tanh.restype = ctypes.c_double
            lib.orc_gelu_tanh_grad.argtypes = [ctypes.c_double]
            lib.orc_gelu_tanh_grad.restype = ctypes.c_double
            lib.orc_fused_linear_bwd.argtypes = [c_int, c_int, p, p, p, p, p, p, p, i64, i64, i64, p, i64, c_int, p]
            lib.orc_fused_linear_bwd.restype = c_int
            lib.orc_unfused_bwd_chain.argtypes = [c_int, c_int, p, p, p, p, p, p, p, i64, i64, i64, p, i64, c_int, p]
            lib.orc_unfused_bwd_chain.restype = c_int
            lib.orc_max_threads.restype = c_int
            _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _raw(a, dtype):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype != STORAGE[dtype]:
        raise TypeError(f"{dtype} data must be stored as {STORAGE[dtype].__name__}, got {a.dtype}")
    return a


def _call(fname, A, B, bias, Y, act, dtype, rows, threads, want_x, R=None):
    lib = _load()
    A, B, bias, Y, R = (_raw(x, dtype) for x in (A, B, bias, Y, R))
    M, K = A.shape
    K2, N = B.shape
    if K2 != K:
        raise ValueError("A is (M,K) and B is (K,N)")
    if bias is not None and bias.shape != (N,):
        raise ValueError("bias is (N,)")
    if act == "glu" and (Y is None or Y.shape != (M, N)):
        raise ValueError("the gate needs Y of shape (M,N)")
    if R is not None and R.shape != (M, N):
        raise ValueError("the residual R is (M,N)")
    if rows is None:
        nrows, rows_arr = M, None
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        nrows = rows_arr.size
    out = np.empty((nrows, N), dtype=STORAGE[dtype])
    x = np.empty((nrows, N), dtype=np.float64) if want_x else None
    head = (DTYPES[dtype], ACTS[act], _ptr(A), _ptr(B), _ptr(bias))
    tail = (_ptr(Y), _ptr(out), M, N, K, _ptr(rows_arr), nrows, int(threads or 0), _ptr(x))
    if fname == "orc_fused_linear":
        st = lib.orc_fused_linear(*head, _ptr(R), *tail)
    else:
        if R is not None:
            raise ValueError("the unfused chain has no residual stage")
        st = getattr(lib, fname)(*head, *tail)
    if st != 0:
        raise RuntimeError(f"{fname} failed with status {st}")
    return (out, x) if want_x else out


def fused_linear(A, B, bias, Y=None, act="relu", dtype="f32", rows=None, threads=None, want_x=False, R=None):
    """round_once(act(A@B + bias [+ R])) in the storage type of ``dtype``.

    ``R`` is an optional (M,N) residual added before the activation.
    ``rows`` selects output rows (the result then has len(rows) rows).
    ``want_x`` also returns the unrounded FP64 epilogue value."""
    return _call("orc_fused_linear", A, B, bias, Y, act, dtype, rows, threads, want_x, R)


QFORMATS = {"fp8_e4m3": 0, "int8": 1}


def fused_linear_quant(A, B, bias, Y=None, act="relu", dtype="f16", qfmt="fp8_e4m3", scale=1.0, rows=None,
                       threads=None, want_u=False):
    """Quantized output: uint8 codes of Q(fp32(fp32(act(A@B + bias)) * scale)),
    Q = saturating RNE to OCP FP8 E4M3 or RNE + clamp to int8 (int8 codes as
    their two's-complement bytes).  ``want_u`` also returns the binary32
    value Q decides on, as float64."""
    lib = _load()
    A, B, bias, Y = (_raw(x, dtype) for x in (A, B, bias, Y))
    M, K = A.shape
    N = B.shape[1]
    if B.shape[0] != K:
        raise ValueError("A is (M,K) and B is (K,N)")
    if act == "glu" and (Y is None or Y.shape != (M, N)):
        raise ValueError("the gate needs Y of shape (M,N)")
    rows_arr = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    nrows = M if rows_arr is None else rows_arr.size
    out = np.empty((nrows, N), dtype=np.uint8)
    u = np.empty((nrows, N), dtype=np.float64) if want_u else None
    st = lib.orc_fused_linear_quant(DTYPES[dtype], ACTS[act], _ptr(A), _ptr(B), _ptr(bias), _ptr(Y), _ptr(out),
                                    M, N, K, QFORMATS[qfmt], float(scale), _ptr(rows_arr), nrows,
                                    int(threads or 0), _ptr(u))
    if st != 0:
        raise RuntimeError(f"orc_fused_linear_quant failed with status {st}")
    return (out, u) if want_u else out


def fused_linear_fp8(A8, B8, ab_scale, bias, Y=None, act="relu", out_dtype="f16", rows=None, threads=None,
                     want_x=False):
    """round_once(act(ab_scale * (A8@B8) + bias)) in ``out_dtype`` storage: A8
    (M,K) and B8 (K,N) are uint8 arrays of OCP FP8 E4M3 codes; bias (N,) and
    Y (M,N) are ``out_dtype`` storage arrays."""
    lib = _load()
    A8 = np.ascontiguousarray(A8, dtype=np.uint8)
    B8 = np.ascontiguousarray(B8, dtype=np.uint8)
    bias, Y = (_raw(x, out_dtype) for x in (bias, Y))
    M, K = A8.shape
    K2, N = B8.shape
    if K2 != K:
        raise ValueError("A8 is (M,K) and B8 is (K,N)")
    if act == "glu" and (Y is None or Y.shape != (M, N)):
        raise ValueError("the gate needs Y of shape (M,N)")
    rows_arr = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    nrows = M if rows_arr is None else rows_arr.size
    out = np.empty((nrows, N), dtype=STORAGE[out_dtype])
    x = np.empty((nrows, N), dtype=np.float64) if want_x else None
    st = lib.orc_fused_linear_fp8(DTYPES[out_dtype], ACTS[act], _ptr(A8), _ptr(B8), float(ab_scale), _ptr(bias),
                                  _ptr(Y), _ptr(out), M, N, K, _ptr(rows_arr), nrows, int(threads or 0), _ptr(x))
    if st != 0:
        raise RuntimeError(f"orc_fused_linear_fp8 failed with status {st}")
    return (out, x) if want_x else out


def gelu_tanh_grad(x):
    return _load().orc_gelu_tanh_grad(float(x))


def unfused_bwd_chain(G, W, X, Y=None, act="relu", dtype="f16", rows=None, threads=None, want_dx=False):
    """As fused_linear_bwd for the three-pass chain: D stored in dtype before
    the elementwise pass, dbias summed from the stored dX."""
    return fused_linear_bwd(G, W, X, Y, act, dtype, rows, threads, want_dx, _fn="orc_unfused_bwd_chain")


def fused_linear_bwd(G, W, X, Y=None, act="relu", dtype="f16", rows=None, threads=None, want_dx=False,
                     _fn="orc_fused_linear_bwd"):
    """Backward epilogue: D = G @ W^T (G (M,K), W (N,K), FP64), then
    dX = round(D * act'(X)), for the gate also dY = round(D * X), and
    dbias = sum over rows of the unrounded dX (FP64; over the selected rows
    when ``rows`` is given).  X and Y (M,N) are the saved forward values.
    Returns (dX, dY or None, dbias[, unrounded dX])."""
    lib = _load()
    G, W, X, Y = (_raw(a, dtype) for a in (G, W, X, Y))
    M, K = G.shape
    N, K2 = W.shape
    if K2 != K:
        raise ValueError("G is (M,K) and W is (N,K)")
    if X.shape != (M, N):
        raise ValueError("X must be (M,N)")
    if act == "glu" and (Y is None or Y.shape != (M, N)):
        raise ValueError("the gate needs Y of shape (M,N)")
    rows_arr = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    nrows = M if rows_arr is None else rows_arr.size
    dX = np.empty((nrows, N), dtype=STORAGE[dtype])
    dY = np.empty((nrows, N), dtype=STORAGE[dtype]) if act == "glu" else None
    dbias = np.empty(N, dtype=np.float64)
    dx = np.empty((nrows, N), dtype=np.float64) if want_dx else None
    st = getattr(lib, _fn)(DTYPES[dtype], ACTS[act], _ptr(G), _ptr(W), _ptr(X), _ptr(Y), _ptr(dX), _ptr(dY),
                           _ptr(dbias), M, N, K, _ptr(rows_arr), nrows, int(threads or 0), _ptr(dx))
    if st != 0:
        raise RuntimeError(f"{_fn} failed with status {st}")
    return (dX, dY, dbias, dx) if want_dx else (dX, dY, dbias)


def compare_dbias(dev, ref, abs_colsum, M):
    """Bias-gradient parity: |dev - ref| <= (M * 2^-24 + 1e-4) * sum_i |dX[i,j]|
    + 1e-6 per column: the worst-case error of an fp32 sum of M terms
    (M * unit roundoff, relative to the sum of magnitudes) plus 1e-4 for the
    fp32 accumulation and epilogue of each term."""
    dev = np.asarray(dev, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    tol = (M * 2.0 ** -24 + 1e-4) * np.asarray(abs_colsum, dtype=np.float64) + 1e-6
    err = np.abs(dev - ref)
    bad = err > tol
    return {"ok": not bad.any(), "violations": int(bad.sum()), "max_abs_err": float(err.max(initial=0.0)),
            "worst": int(np.argmax(err / tol)) if err.size else -1}


def quantize(u, qfmt):
    """uint8 codes of saturating RNE FP8 E4M3 (or RNE + clamp int8) of float64 values."""
    u = np.ascontiguousarray(u, dtype=np.float64)
    out = np.empty(u.shape, dtype=np.uint8)
    _load().orc_quantize(QFORMATS[qfmt], _ptr(u), u.size, _ptr(out))
    return out


def dequantize(codes, qfmt):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(codes.shape, dtype=np.float64)
    _load().orc_dequantize(QFORMATS[qfmt], _ptr(codes), codes.size, _ptr(out))
    return out


def compare_quant(dev_codes, ref_codes, ref_u, qfmt, rel=1e-4, abs_=1e-6):
    """Quantized parity: codes equal, except where the oracle's binary32
    value u lies within rel*|u| + abs_ of the point where Q changes its
    decision (then the neighbouring code is accepted too: the device's fp32
    sum differs from the FP64 one by rounding).  Returns a dict with ok,
    mismatches, accepted_near_boundary and the worst index."""
    dev = np.asarray(dev_codes, dtype=np.uint8)
    ref = np.asarray(ref_codes, dtype=np.uint8)
    if dev.shape != ref.shape:
        raise ValueError("shape mismatch")
    diff = dev != ref
    band = rel * np.abs(ref_u) + abs_
    lo = quantize(ref_u - band, qfmt)
    hi = quantize(ref_u + band, qfmt)
    ok_alt = diff & ((dev == lo) | (dev == hi))
    bad = diff & ~ok_alt
    worst = None
    if bad.any():
        worst = tuple(int(v) for v in np.argwhere(bad)[0])
    return {"ok": not bad.any(), "mismatches": int(bad.sum()), "accepted_near_boundary": int(ok_alt.sum()),
            "worst": worst}


def unfused_chain(A, B, bias, Y=None, act="relu", dtype="f32", rows=None, threads=None):
    """round(act(round(round(A@B) + bias))): separate stages, each stored in dtype."""
    return _call("orc_unfused_chain", A, B, bias, Y, act, dtype, rows, threads, False)


def element(A, B, bias, Y, act, dtype, i, j, R=None):
    """Unrounded FP64 act(A[i,:]@B[:,j] + bias[j] [+ R[i,j]])."""
    lib = _load()
    A, B, bias, Y, R = (_raw(x, dtype) for x in (A, B, bias, Y, R))
    M, K = A.shape
    N = B.shape[1]
    v = ctypes.c_double()
    st = lib.orc_element(DTYPES[dtype], ACTS[act], _ptr(A), _ptr(B), _ptr(bias), _ptr(R), _ptr(Y),
                         M, N, K, int(i), int(j), ctypes.addressof(v))
    if st != 0:
        raise RuntimeError("orc_element failed")
    return v.value


def decode(raw, dtype):
    raw = _raw(np.asarray(raw), dtype)
    out = np.empty(raw.shape, dtype=np.float64)
    _load().orc_decode(DTYPES[dtype], _ptr(raw), raw.size, _ptr(out))
    return out


def encode(x, dtype):
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=STORAGE[dtype])
    _load().orc_encode(DTYPES[dtype], _ptr(x), x.size, _ptr(out))
    return out


def gelu_tanh(x):
    f = _load().orc_gelu_tanh
    return np.vectorize(lambda v: f(float(v)), otypes=[np.float64])(x)


def tile_of_pid(pid, tiles_m, tiles_n, group):
    m, n = ctypes.c_int64(), ctypes.c_int64()
    st = _load().orc_tile_of_pid(pid, tiles_m, tiles_n, group, ctypes.addressof(m), ctypes.addressof(n))
    if st != 0:
        raise ValueError("pid or tiling out of range")
    return m.value, n.value


def max_threads():
    return _load().orc_max_threads()


def compare(dev_raw, ref_raw, dtype, atol=None, rtol=None):
    """Element-wise |dev - ref| <= atol + rtol*|ref| in FP64.

    Both arguments are raw storage arrays of ``dtype``; ``ref`` is the oracle's
    once-rounded output.  Returns a dict with ok, max_abs, max_rel, violations
    and the index of the worst violation (or None).  NaN anywhere fails."""
    d_atol, d_rtol = TOLERANCE[dtype]
    atol = d_atol if atol is None else atol
    rtol = d_rtol if rtol is None else rtol
    dev = decode(np.asarray(dev_raw), dtype)
    ref = decode(np.asarray(ref_raw), dtype)
    if dev.shape != ref.shape:
        raise ValueError(f"shape mismatch {dev.shape} vs {ref.shape}")
    diff = np.abs(dev - ref)
    bound = atol + rtol * np.abs(ref)
    bad = ~(diff <= bound)  # NaN compares false -> counted as a violation
    nviol = int(bad.sum())
    rel = diff / np.maximum(np.abs(ref), 1e-30)
    worst = None
    if nviol:
        worst = tuple(int(v) for v in np.unravel_index(np.argmax(np.where(bad, diff - bound, -np.inf)), dev.shape))
    return {
        "ok": nviol == 0,
        "max_abs": float(np.nanmax(diff)) if diff.size else 0.0,
        "max_rel": float(np.nanmax(rel)) if rel.size else 0.0,
        "violations": nviol,
        "worst": worst,
    }
