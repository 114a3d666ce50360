"""The library under HIP graph capture (torch.cuda.CUDAGraph).

The entry points only launch kernels on the caller's stream (the backward's
dbias is cleared by a fill kernel, not a memset), so a captured sequence must
replay with the eager results.  Each replay follows eager work of the
program's own (new inputs copied in, outputs overwritten with NaN) and a
synchronisation, and every replay is checked: the forward output and dX bit
for bit against an eager call on the same inputs, dbias (fp32 atomics, whose
order is not fixed) within its tolerance.
"""
import numpy as np
import pytest
import torch

import oracle
import activation_epilogue_amd as fl
from activation_epilogue_amd import synth
from gpu_util import say, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a device"
    fl.load_library()


def _fresh(seed):
    f = synth.draw(300, 520, 200, "f16", "glu", seed=seed)
    b = synth.draw_bwd(300, 520, 136, "bf16", "gelu_tanh", seed=seed + 1)
    return f, b


def _eager(fw, bw):
    out = fl.fused_linear(fw["A"], fw["B"], fw["bias"], fw["Y"], act="glu")
    dX, _, db = fl.fused_linear_bwd(bw["G"], bw["W"], bw["X"], act="gelu_tanh")
    torch.cuda.synchronize()
    return to_host(out, "f16"), to_host(dX, "bf16"), db.cpu().numpy().astype(np.float64)


def test_graph_replays_match_eager():
    f, b = _fresh(61)
    fw = {k: to_dev(f[k], "f16") for k in ("A", "B", "bias", "Y")}
    bw = {k: to_dev(b[k], "bf16") for k in ("G", "W", "X")}
    out = torch.empty(300, 520, dtype=torch.float16, device="cuda")
    dX = torch.empty(300, 520, dtype=torch.bfloat16, device="cuda")
    dbias = torch.empty(520, dtype=torch.float32, device="cuda")

    def work():
        fl.fused_linear(fw["A"], fw["B"], fw["bias"], fw["Y"], act="glu", out=out)
        fl.fused_linear_bwd(bw["G"], bw["W"], bw["X"], act="gelu_tanh", dX=dX, dbias=dbias)

    say("graph: warm-up on a side stream, then capture")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    torch.cuda.synchronize()

    for r in range(3):
        f, b = _fresh(70 + 7 * r)
        for k in fw:
            fw[k].copy_(to_dev(f[k], "f16"))
        for k in bw:
            bw[k].copy_(to_dev(b[k], "bf16"))
        ref_out, ref_dX, ref_db = _eager(fw, bw)
        out.fill_(float("nan"))
        dX.fill_(float("nan"))
        dbias.fill_(float("nan"))
        torch.cuda.synchronize()
        say("graph replay", r)
        g.replay()
        torch.cuda.synchronize()
        got_out, got_dX = to_host(out, "f16"), to_host(dX, "bf16")
        got_db = dbias.cpu().numpy().astype(np.float64)
        assert np.array_equal(got_out.view(np.uint16), ref_out.view(np.uint16)), f"replay {r}: out"
        assert np.array_equal(got_dX.view(np.uint16), ref_dX.view(np.uint16)), f"replay {r}: dX"
        abs_cols = np.abs(oracle.decode(ref_dX, "bf16")).sum(axis=0)
        res = oracle.compare_dbias(got_db, ref_db, abs_cols, 300)
        assert res["ok"], f"replay {r}: dbias {res}"
        # the replay computed the new inputs, not the captured ones
        rX, _, _ = oracle.fused_linear_bwd(b["G"], b["W"], b["X"], None, act="gelu_tanh", dtype="bf16")
        res = oracle.compare(got_dX, rX, "bf16")
        assert res["ok"], f"replay {r}: dX against the oracle {res}"


def test_graph_reproducible_dbias_replays_bit_exact():
    """The reproducible-dbias backward under capture: fl_fused_linear_bwd_ws
    with a workspace allocated before the capture, and
    fl_fused_linear_bwd_noalloc (its partial sums in the library's fixed
    array; its one-time address lookup happens in the warm-up, before the
    capture).  Every replay's dX and dbias equal an eager call's bit for bit."""
    b = synth.draw_bwd(300, 520, 136, "bf16", "glu", seed=81)
    bw = {k: to_dev(b[k], "bf16") for k in ("G", "W", "X", "Y")}
    ws = torch.empty(fl.bwd_workspace_bytes(300, 520, 136, torch.bfloat16), dtype=torch.uint8, device="cuda")
    outs = {name: (torch.empty(300, 520, dtype=torch.bfloat16, device="cuda"),
                   torch.empty(300, 520, dtype=torch.bfloat16, device="cuda"),
                   torch.empty(520, dtype=torch.float32, device="cuda")) for name in ("ws", "noalloc")}

    def work():
        dX, dY, db = outs["ws"]
        fl.fused_linear_bwd(bw["G"], bw["W"], bw["X"], bw["Y"], act="glu", dX=dX, dY=dY, dbias=db, workspace=ws)
        dX, dY, db = outs["noalloc"]
        fl.fused_linear_bwd_noalloc(bw["G"], bw["W"], bw["X"], bw["Y"], act="glu", dX=dX, dY=dY, dbias=db)

    say("graph (reproducible dbias): warm-up on a side stream, then capture")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    torch.cuda.synchronize()

    for r in range(3):
        b = synth.draw_bwd(300, 520, 136, "bf16", "glu", seed=90 + r)
        for k in bw:
            bw[k].copy_(to_dev(b[k], "bf16"))
        rX, rY, rdb = fl.fused_linear_bwd(bw["G"], bw["W"], bw["X"], bw["Y"], act="glu", workspace=True)
        torch.cuda.synchronize()
        ref = (to_host(rX, "bf16"), to_host(rY, "bf16"), rdb.cpu().numpy())
        for t in outs.values():
            for x in t:
                x.fill_(float("nan"))
        torch.cuda.synchronize()
        say("graph replay (reproducible dbias)", r)
        g.replay()
        torch.cuda.synchronize()
        for name, (dX, dY, db) in outs.items():
            assert np.array_equal(to_host(dX, "bf16").view(np.uint16), ref[0].view(np.uint16)), (r, name, "dX")
            assert np.array_equal(to_host(dY, "bf16").view(np.uint16), ref[1].view(np.uint16)), (r, name, "dY")
            assert np.array_equal(db.cpu().numpy().view(np.uint32), ref[2].view(np.uint32)), (r, name, "dbias")
