"""fl_fused_linear_bwd_noalloc (the backward with a reproducible dbias whose
partial sums live in the library's fixed per-GPU array) against the entry
point it varies, fl_fused_linear_bwd_ws with a torch-allocated workspace:
the same bits for dX, dY and dbias, on two calls in a row (the second with
a smaller problem, so it runs over the array the first one left behind),
and within the oracle's tolerance."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import activation_epilogue_amd as fl
from activation_epilogue_amd import synth
from gpu_util import say, to_dev, to_host, sentinel_out, guard_intact

pytestmark = pytest.mark.gpu


def _noalloc(d, act, dtype):
    """One call of fl_fused_linear_bwd_noalloc through the C ABI."""
    lib = fl.load_library()
    M, K = d["G"].shape
    N = d["W"].shape[0]
    G, W, X, Y = (to_dev(d[k], dtype) for k in ("G", "W", "X", "Y"))
    dX, bufx = sentinel_out(M, N, dtype)
    dY, bufy = sentinel_out(M, N, dtype) if act == "glu" else (None, None)
    dbias = torch.full((N + 64,), float("nan"), dtype=torch.float32, device="cuda")
    ptr = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None
    code = {"f16": 1, "bf16": 2}[dtype]
    st = lib.fl_fused_linear_bwd_noalloc(ptr(G), ptr(W), ptr(X), ptr(Y), ptr(dX), ptr(dY), ptr(dbias), M, N, K,
                                         fl.ACTS[act], code,
                                         ctypes.c_void_p(torch.cuda.current_stream().cuda_stream), None)
    assert st == 0, lib.fl_last_error().decode()
    torch.cuda.synchronize()
    assert guard_intact(bufx, M, N) and (dY is None or guard_intact(bufy, M, N))
    assert bool(torch.isnan(dbias[N:]).all().item()), "write past the end of dbias"
    return (to_host(dX, dtype), None if dY is None else to_host(dY, dtype),
            dbias[:N].cpu().numpy().astype(np.float64))


def _ws(d, act, dtype):
    """The same problem through fl_fused_linear_bwd_ws (workspace from torch)."""
    G, W, X, Y = (to_dev(d[k], dtype) for k in ("G", "W", "X", "Y"))
    dX, dY, db = fl.fused_linear_bwd(G, W, X, Y, act=act, workspace=True)
    torch.cuda.synchronize()
    return to_host(dX, dtype), None if dY is None else to_host(dY, dtype), db.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("dtype,act", [("bf16", "glu"), ("f16", "gelu_tanh")])
def test_noalloc_matches_the_workspace_entry_twice(dtype, act):
    for M, N, K in [(1100, 700, 300), (300, 260, 77)]:
        d = synth.draw_bwd(M, N, K, dtype, act, seed=M + N)
        say("noalloc", dtype, act, M, N, K)
        got = _noalloc(d, act, dtype)
        ref = _ws(d, act, dtype)
        assert np.array_equal(got[0].view(np.uint8), ref[0].view(np.uint8))
        if act == "glu":
            assert np.array_equal(got[1].view(np.uint8), ref[1].view(np.uint8))
        assert np.array_equal(got[2].view(np.uint64), ref[2].view(np.uint64)), np.abs(got[2] - ref[2]).max()
        rX, rY, rdb, rdx = oracle.fused_linear_bwd(d["G"], d["W"], d["X"], d["Y"], act=act, dtype=dtype,
                                                   want_dx=True)
        res = oracle.compare_dbias(got[2], rdb, np.abs(rdx).sum(axis=0), M)
        assert res["ok"], res
