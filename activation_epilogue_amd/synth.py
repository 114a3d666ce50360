"""Seeded synthetic inputs for out = act(A@B + bias).

This module only draws random numbers and stores them in the I/O dtype; it
holds none of the method's arithmetic.  The same bytes feed the device path
and the FP64 oracle.

Recipe: ``numpy.random.default_rng(seed)`` (PCG64), draws in float64 in the
order A, B, bias, Y, R; A and B ~ N(0, 1/K) (1/K is the variance, so the standard
deviation is K**-0.5), bias ~ N(0, bias_var), Y ~ U(-1, 1) (gate only), R ~
N(0, 1) (residual workloads only); each
array is then stored in the dtype with round-to-nearest-even (numpy's cast for
fp32/fp16, torch's fp32->bf16 cast for bf16).  Storage: fp32 as float32, fp16
as float16, bf16 as the uint16 bit pattern.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    dtype: str
    act: str
    bias_var: float = 1.0
    seed: int = 0
    residual: bool = False
    qfmt: str = ""       # quantized output ("fp8_e4m3" or "int8"), else the I/O dtype
    scale: float = 1.0   # quantized output scale
    in8: bool = False    # A and B as FP8 E4M3 codes (dtype is then the output / bias / Y dtype)
    bwd: bool = False    # the backward epilogue: G (M,K), W (N,K), saved X (M,N) [, Y]; see draw_bwd

    @property
    def flops(self) -> int:
        """GEMM flops 2*M*N*K (epilogue flops are not counted)."""
        return 2 * self.M * self.N * self.K


# The synthetic workloads: named by what they compute and their sizes.
WORKLOADS = {w.name: w for w in [
    Workload("relu_f32_127x129x96", 127, 129, 96, "f32", "relu"),
    Workload("relu_f32_4096x4096x4096", 4096, 4096, 4096, "f32", "relu"),
    Workload("relu_f16_4096x4096x4096", 4096, 4096, 4096, "f16", "relu"),
    Workload("relu_bf16_4097x3071x1537", 4097, 3071, 1537, "bf16", "relu"),
    Workload("glu_f16_1024x21568x4096", 1024, 21568, 4096, "f16", "glu"),
    Workload("gelu_bf16_8192x14336x4096", 8192, 14336, 4096, "bf16", "gelu_tanh", bias_var=0.1),
    # the gate at the TLX page's own shape and K sweep (its MI350X table)
    Workload("glu_f16_1024x21568x256", 1024, 21568, 256, "f16", "glu"),
    Workload("glu_f16_1024x21568x512", 1024, 21568, 512, "f16", "glu"),
    Workload("glu_f16_1024x21568x1024", 1024, 21568, 1024, "f16", "glu"),
    # FFN down-projection with the residual added in the epilogue (no activation)
    Workload("residual_bf16_8192x4096x14336", 8192, 4096, 14336, "bf16", "none", residual=True),
    # FFN up-projection whose GELU output is stored as FP8 E4M3 codes for the next layer
    Workload("gelu_fp8out_bf16_8192x14336x4096", 8192, 14336, 4096, "bf16", "gelu_tanh", bias_var=0.1,
             qfmt="fp8_e4m3", scale=64.0),
    # the projection in FP8 (A, B as E4M3 codes, ab_scale 1/sqrt(K)), 16-bit epilogue: the gate at the
    # TLX page's shape, and ReLU at 4096^3
    Workload("glu_fp8in_f16_1024x21568x4096", 1024, 21568, 4096, "f16", "glu", in8=True),
    Workload("relu_fp8in_f16_4096x4096x4096", 4096, 4096, 4096, "f16", "relu", in8=True),
    # the backward of the GELU FFN's up-projection: the gradient reaching its output is
    # dOut2 (8192x4096) @ W_down^T with W_down (14336x4096), then gelu'(X) and the bias gradient
    Workload("gelu_bwd_bf16_8192x14336x4096", 8192, 14336, 4096, "bf16", "gelu_tanh", bwd=True),
    # the same for the gate at the TLX page's shape (dX and dY)
    Workload("glu_bwd_f16_1024x21568x4096", 1024, 21568, 4096, "f16", "glu", bwd=True),
]}


def to_storage(x64: np.ndarray, dtype: str) -> np.ndarray:
    """Store float64 data in the dtype's raw numpy storage, RNE."""
    if dtype == "f32":
        return np.ascontiguousarray(x64, dtype=np.float32)
    if dtype == "f16":
        return np.ascontiguousarray(x64.astype(np.float16))
    if dtype == "bf16":
        import torch
        t = torch.from_numpy(np.ascontiguousarray(x64, dtype=np.float32)).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    raise ValueError(dtype)


def draw(M, N, K, dtype, act, bias_var=1.0, seed=0, with_bias=True, residual=False):
    """Return dict(A, B, bias, Y, R) of raw storage arrays (Y None unless
    gate, R None unless residual)."""
    rng = np.random.default_rng(seed)
    sd = 1.0 / np.sqrt(K) if K > 0 else 1.0
    A = rng.standard_normal((M, K)) * sd
    B = rng.standard_normal((K, N)) * sd
    bias = rng.standard_normal(N) * np.sqrt(bias_var) if with_bias else None
    Y = rng.uniform(-1.0, 1.0, (M, N)) if act == "glu" else None
    R = rng.standard_normal((M, N)) if residual else None
    return {
        "A": to_storage(A, dtype),
        "B": to_storage(B, dtype),
        "bias": None if bias is None else to_storage(bias, dtype),
        "Y": None if Y is None else to_storage(Y, dtype),
        "R": None if R is None else to_storage(R, dtype),
    }


def draw_bwd(M, N, K, dtype, act, seed=0):
    """Backward-epilogue inputs: G ~ N(0, 1) (M,K), W ~ N(0, 1/K) (N,K) (so
    G @ W^T ~ N(0, 1)), the saved pre-activation X ~ N(0, 1) (M,N), and Y ~
    U(-1, 1) (M,N) for the gate.  Draw order G, W, X, Y."""
    rng = np.random.default_rng(seed)
    G = rng.standard_normal((M, K))
    W = rng.standard_normal((N, K)) / np.sqrt(max(K, 1))
    X = rng.standard_normal((M, N))
    Y = rng.uniform(-1.0, 1.0, (M, N)) if act == "glu" else None
    return {"G": to_storage(G, dtype), "W": to_storage(W, dtype), "X": to_storage(X, dtype),
            "Y": None if Y is None else to_storage(Y, dtype)}


def draw_bwd_integer(M, N, K, dtype, act, seed=0):
    """Small integers for the backward epilogue: G, W in {-2..2}, X in
    {-3..3} (exact zeros included), Y in {-2..2}; with K <= 8 every value the
    epilogue forms is exact in the 16-bit dtypes."""
    rng = np.random.default_rng(seed)
    G = rng.integers(-2, 3, (M, K)).astype(np.float64)
    W = rng.integers(-2, 3, (N, K)).astype(np.float64)
    X = rng.integers(-3, 4, (M, N)).astype(np.float64)
    Y = rng.integers(-2, 3, (M, N)).astype(np.float64) if act == "glu" else None
    return {"G": to_storage(G, dtype), "W": to_storage(W, dtype), "X": to_storage(X, dtype),
            "Y": None if Y is None else to_storage(Y, dtype)}


def draw_workload(w: Workload, with_bias=True):
    if w.bwd:
        return draw_bwd(w.M, w.N, w.K, w.dtype, w.act, w.seed)
    if w.in8:
        return draw_fp8(w.M, w.N, w.K, w.dtype, w.act, w.bias_var, w.seed)
    return draw(w.M, w.N, w.K, w.dtype, w.act, w.bias_var, w.seed, with_bias, w.residual)


def to_e4m3(x64: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3 codes (uint8) of float64 data, RNE via torch's float32 ->
    float8_e4m3fn cast (the data drawn here stays far inside +-448)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x64, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


def draw_fp8(M, N, K, out_dtype, act, bias_var=1.0, seed=0):
    """FP8-operand inputs: A, B ~ N(0, 1) stored as E4M3 codes ("A8", "B8"),
    ab_scale = 1/sqrt(K) (so A@B*ab_scale ~ N(0, 1)); bias ~ N(0, bias_var)
    and Y ~ U(-1, 1) in out_dtype.  Draw order A, B, bias, Y."""
    rng = np.random.default_rng(seed)
    A = rng.standard_normal((M, K))
    B = rng.standard_normal((K, N))
    bias = rng.standard_normal(N) * np.sqrt(bias_var)
    Y = rng.uniform(-1.0, 1.0, (M, N)) if act == "glu" else None
    return {"A8": to_e4m3(A), "B8": to_e4m3(B), "ab_scale": float(np.float32(1.0 / np.sqrt(max(K, 1)))),
            "bias": to_storage(bias, out_dtype), "Y": None if Y is None else to_storage(Y, out_dtype), "R": None}


def draw_integer(M, N, K, dtype, act, seed=0, amax=2, bias_max=4):
    """Small-integer inputs: A, B in {-amax..amax}, integer bias, Y in {-1,0,1}.

    With K small enough every partial sum, the bias add and the epilogue are
    exact in fp32 and the result is representable in the out dtype, so any
    summation order gives the same bits."""
    rng = np.random.default_rng(seed)
    A = rng.integers(-amax, amax + 1, (M, K)).astype(np.float64)
    B = rng.integers(-amax, amax + 1, (K, N)).astype(np.float64)
    bias = rng.integers(-bias_max, bias_max + 1, N).astype(np.float64)
    Y = rng.integers(-1, 2, (M, N)).astype(np.float64) if act == "glu" else None
    return {
        "A": to_storage(A, dtype),
        "B": to_storage(B, dtype),
        "bias": to_storage(bias, dtype),
        "Y": None if Y is None else to_storage(Y, dtype),
        "R": None,
    }
