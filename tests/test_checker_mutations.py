"""Checker sensitivity: planted mistakes (CPU-side, numpy) must be flagged.

Each mutant is the plain definition with one of the mistakes the pages warn
about ("Triton: Fused Matmul + Bias + ReLU", "Pitfalls"; "Epilogue concept",
"Why it cannot move earlier" and "Things that break"; "Triton: ReLU", "The 0.0
literal gotcha" and "Pitfalls"), run tile by tile the way a kernel would.  The
comparison used by the parity tests (tolerance check against the oracle, plus
NaN sentinel and guard band) must reject every one of them on the ragged
127x129x96 fp32 workload, and the K=1 / K=3 pair must expose the bias that is
folded into the reduction.
"""
import numpy as np
import pytest

import oracle
from activation_epilogue_amd import synth

BM, BN, BK = 32, 32, 64  # K=96 leaves a ragged last K tile
GUARD = 64


def _inputs(K=96):
    w = synth.WORKLOADS["relu_f32_127x129x96"]
    return synth.draw(w.M, w.N, K, "f32", "relu", seed=0)


def _tiled(A, B, bias, mistake, K):
    """Tile-by-tile fused GEMM+bias+ReLU with one planted mistake.

    Returns (flat output with a guard band, prefilled with NaN)."""
    M, N = A.shape[0], B.shape[1]
    A64, B64, b64 = A.astype(np.float64), B.astype(np.float64), bias.astype(np.float64)
    kpad = -(-K // BK) * BK
    Apad = np.zeros((M, kpad))
    Bpad = np.zeros((kpad, N))
    Apad[:, :K] = A64
    Bpad[:K] = B64
    if mistake == "no_k_mask":
        # the last K tile reads past each row of A / past the end of B
        flatA = np.concatenate([A64.ravel(), np.ones(kpad)])
        for i in range(M):
            Apad[i, K:] = flatA[i * K + K:i * K + kpad]
        Bpad[K:] = 0.5
    bias_pad = np.full(-(-N // BN) * BN, np.nan)
    bias_pad[:N] = b64
    out = np.full(M * N + GUARD, np.nan)
    for m0 in range(0, M, BM):
        for n0 in range(0, N, BN):
            rows = np.arange(m0, min(m0 + BM, M))
            cols = np.arange(n0, n0 + BN)
            colsv = cols[cols < N]
            acc = np.zeros((len(rows), BN))
            Bt = np.zeros((kpad, BN))
            Bt[:, :len(colsv)] = Bpad[:, colsv]
            for k0 in range(0, kpad, BK):
                acc += Apad[rows, k0:k0 + BK] @ Bt[k0:k0 + BK]
                if mistake == "bias_in_loop":
                    acc += b64[colsv].tolist() + [0.0] * (BN - len(colsv))
                if mistake == "relu_partial":
                    acc = np.maximum(acc, 0.0)
            if mistake == "row_bias":
                acc += b64[rows][:, None]
            elif mistake == "relu_before_bias":
                acc = np.maximum(acc, 0.0) + bias_pad[cols][None, :]
            elif mistake != "bias_in_loop":
                bvals = bias_pad[cols] if mistake == "unmasked_store" else np.nan_to_num(bias_pad[cols])
                acc += bvals[None, :]
            if mistake != "relu_before_bias":
                acc = np.maximum(acc, 0.0)
            if mistake == "int_literal":
                acc = np.trunc(acc)
            for r, i in enumerate(rows):
                if mistake == "missing_tail_store" and m0 + BM > M:
                    continue
                if mistake == "unmasked_store":
                    out[i * N + n0:i * N + n0 + BN] = acc[r]
                else:
                    out[i * N + colsv] = acc[r, :len(colsv)]
    return out


def _flagged(out, ref, M, N):
    """The parity check: tolerance against the oracle, sentinel and guard."""
    body = out[:M * N].reshape(M, N).astype(np.float32)
    res = oracle.compare(body, ref, "f32")
    guard_ok = np.isnan(out[M * N:]).all()
    return (not res["ok"]) or (not guard_ok)


def test_correct_tiling_passes():
    d = _inputs()
    ref = oracle.fused_linear(d["A"], d["B"], d["bias"], act="relu", dtype="f32")
    out = _tiled(d["A"], d["B"], d["bias"], None, 96)
    assert not _flagged(out, ref, 127, 129)


@pytest.mark.parametrize("mistake", ["row_bias", "relu_before_bias", "bias_in_loop", "relu_partial",
                                     "int_literal", "missing_tail_store", "unmasked_store", "no_k_mask"])
def test_mutant_is_flagged(mistake):
    d = _inputs()
    ref = oracle.fused_linear(d["A"], d["B"], d["bias"], act="relu", dtype="f32")
    out = _tiled(d["A"], d["B"], d["bias"], mistake, 96)
    assert _flagged(out, ref, 127, 129), mistake


def test_bias_in_reduction_passes_at_k1_fails_at_k3():
    """With BK=1 the folded bias is added once per k: right at K=1, wrong at K=3."""
    global BK
    saved = BK
    BK = 1
    try:
        for K, expect_flag in ((1, False), (3, True)):
            d = _inputs(K)
            chain = oracle.unfused_chain(d["A"], d["B"], d["bias"], act="relu", dtype="f32")
            out = _tiled(d["A"], d["B"], d["bias"], "bias_in_loop", K)
            assert _flagged(out, chain, 127, 129) == expect_flag
    finally:
        BK = saved


@pytest.mark.parametrize("mistake", ["residual_after_relu", "residual_row_broadcast", "residual_transposed"])
def test_residual_mutant_is_flagged(mistake):
    """The residual variant ("Variants": the residual is summed in ahead of
    the activation) with the mistakes a kernel could make; each must fail the
    tolerance check on the ragged workload."""
    w = synth.WORKLOADS["relu_f32_127x129x96"]
    d = synth.draw(w.M, w.N, w.K, "f32", "relu", seed=0)
    R = synth.to_storage(np.random.default_rng(5).standard_normal((w.M, w.N)), "f32")
    ref = oracle.fused_linear(d["A"], d["B"], d["bias"], act="relu", dtype="f32", R=R)
    A, B, b, R64 = (x.astype(np.float64) for x in (d["A"], d["B"], d["bias"], R))
    X = A @ B + b[None, :]
    if mistake == "residual_after_relu":
        out = np.maximum(X, 0.0) + R64
    elif mistake == "residual_row_broadcast":
        out = np.maximum(X + R64[:, :1], 0.0)
    else:
        Rt = R64.ravel()[:w.M * w.N].reshape(w.N, w.M).T  # (N,M) storage read as (M,N)
        out = np.maximum(X + Rt, 0.0)
    assert not oracle.compare(out.astype(np.float32), ref, "f32")["ok"], mistake
    good = np.maximum(X + R64, 0.0)
    assert oracle.compare(good.astype(np.float32), ref, "f32")["ok"]
