"""Operands of more than 2 GiB with a ragged reduction (K % 8 != 0).

The kernels address an operand through a descriptor based at the tile's
first row (or column), with 32-bit offsets that stay below 256 rows of it.
In the last K stage the lane whose 16-byte chunk holds the operand's very
last element reloads that element on its own (FP8 codes: up to the last
three, the ones its partial last dword holds); these tests check that this
reload is right when the whole operand spans more than 2^31 bytes.

Small integers make every value exact, so the rows (or columns) that carry
data must equal the oracle bit for bit.  The last element of the operand is
forced to 1 and the row of the other operand it meets to +-1, so a reload
that read zero, or another element, changes every output of that row.  The
operand is zero everywhere else, and those outputs are checked too.
"""
import numpy as np
import pytest
import torch

import oracle
import activation_epilogue_amd as fl
from gpu_util import say, to_dev, to_host, TORCH_DT
from activation_epilogue_amd import synth

pytestmark = pytest.mark.gpu

K = 1023          # K % 8 == 7: the last A chunk of a row straddles K
BIG = 1_050_000   # BIG * K * 2 bytes = 2,148,300,000 > 2^31


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a device"
    fl.load_library()


def _live(n):
    """The rows with data: both ends, the middle, and both sides of the
    boundary between the last two 256-row tiles."""
    last = (n - 1) // 256 * 256
    return np.array(sorted({0, n // 3, last - 1, last, n - 2, n - 1}), dtype=np.int64)


def _ints(rng, shape, lo=-1, hi=1):
    return rng.integers(lo, hi + 1, shape).astype(np.float64)


@pytest.mark.parametrize("tile_cfg", [0, 1, 5])
def test_forward_A_over_2GiB(tile_cfg):
    M, N, dtype = BIG, 64, "f16"
    assert M * K * 2 > 2 ** 31
    rng = np.random.default_rng(40 + tile_cfg)
    live = _live(M)
    a_live = _ints(rng, (live.size, K))
    a_live[-1, K - 1] = 1.0                         # A[M-1][K-1]
    b = _ints(rng, (K, N))
    b[K - 1] = np.where(rng.integers(0, 2, N) == 0, -1.0, 1.0)
    bias = _ints(rng, N, -3, 3)
    a_live_s, b_s, bias_s = (synth.to_storage(x, dtype) for x in (a_live, b, bias))
    say("A over 2 GiB", M, N, K, "tile_cfg", tile_cfg)
    A = torch.zeros((M, K), dtype=TORCH_DT[dtype], device="cuda")
    A[torch.from_numpy(live).to("cuda")] = to_dev(a_live_s, dtype)
    out = fl.fused_linear(A, to_dev(b_s, dtype), to_dev(bias_s, dtype), act="relu", tile_cfg=tile_cfg)
    torch.cuda.synchronize()
    del A
    h = to_host(out, dtype)
    ref_live = oracle.fused_linear(a_live_s, b_s, bias_s, act="relu", dtype=dtype)
    assert np.array_equal(h[live].view(np.uint16), ref_live.view(np.uint16)), \
        oracle.compare(h[live], ref_live, dtype)
    ref_zero = oracle.fused_linear(np.zeros((1, K), dtype=np.float16), b_s, bias_s, act="relu", dtype=dtype)
    dead = np.ones(M, dtype=bool)
    dead[live] = False
    assert (h[dead].view(np.uint16) == ref_zero.view(np.uint16)).all()


E4M3 = {-1: 0xB8, 0: 0x00, 1: 0x38}  # exact small integers as OCP FP8 E4M3 codes


@pytest.mark.parametrize("tile_cfg", [0, 2, 12])
def test_fp8_A_over_2GiB(tile_cfg):
    """FP8 codes: A of M*K bytes > 2^31 with K % 16 != 0, so the last chunk of
    each row straddles K and the buffer's last dword is partial; the last
    three codes of A are nonzero and must be reloaded."""
    Kf = 1021                      # K % 16 == 13
    M, N = 2_104_003, 64          # M*K % 4 == 3: the last dword of A holds three codes
    assert M * Kf > 2 ** 31
    rng = np.random.default_rng(70 + tile_cfg)
    live = _live(M)
    lut = np.array([E4M3[v] for v in (-1, 0, 1)], dtype=np.uint8)
    a_live = lut[rng.integers(0, 3, (live.size, Kf))]
    a_live[-1, Kf - 3:] = E4M3[1]                   # the last three codes of A
    b = lut[rng.integers(0, 3, (Kf, N))]
    b[Kf - 3:] = np.where(rng.integers(0, 2, (3, N)) == 0, E4M3[-1], E4M3[1])
    bias = synth.to_storage(rng.integers(-3, 4, N).astype(np.float64), "f16")
    say("FP8 A over 2 GiB", M, N, Kf, "tile_cfg", tile_cfg)
    A = torch.zeros((M, Kf), dtype=torch.uint8, device="cuda")
    A[torch.from_numpy(live).to("cuda")] = torch.from_numpy(a_live).to("cuda")
    out = fl.fused_linear_fp8(A, torch.from_numpy(b).to("cuda"), 0.5, to_dev(bias, "f16"), None, act="relu",
                              out_dtype=torch.float16, tile_cfg=tile_cfg)
    torch.cuda.synchronize()
    del A
    h = to_host(out, "f16")
    ref_live = oracle.fused_linear_fp8(a_live, b, 0.5, bias, None, act="relu", out_dtype="f16")
    assert np.array_equal(h[live].view(np.uint16), ref_live.view(np.uint16)), \
        oracle.compare(h[live], ref_live, "f16")
    ref_zero = oracle.fused_linear_fp8(np.zeros((1, Kf), dtype=np.uint8), b, 0.5, bias, None, act="relu",
                                       out_dtype="f16")
    dead = np.ones(M, dtype=bool)
    dead[live] = False
    assert (h[dead].view(np.uint16) == ref_zero.view(np.uint16)).all()


@pytest.mark.parametrize("tile_cfg", [0, 2])
def test_backward_W_over_2GiB(tile_cfg):
    M, N, dtype = 64, BIG, "f16"
    assert N * K * 2 > 2 ** 31
    rng = np.random.default_rng(50 + tile_cfg)
    live = _live(N)
    g = _ints(rng, (M, K))
    g[:, K - 1] = np.where(rng.integers(0, 2, M) == 0, -1.0, 1.0)
    w_live = _ints(rng, (live.size, K))
    w_live[-1, K - 1] = 1.0                         # W[N-1][K-1]
    g_s, w_live_s = (synth.to_storage(x, dtype) for x in (g, w_live))
    say("W over 2 GiB", M, N, K, "tile_cfg", tile_cfg)
    W = torch.zeros((N, K), dtype=TORCH_DT[dtype], device="cuda")
    W[torch.from_numpy(live).to("cuda")] = to_dev(w_live_s, dtype)
    X = torch.ones((M, N), dtype=TORCH_DT[dtype], device="cuda")  # relu'(X) = 1: dX = G @ W^T
    dX, _, dbias = fl.fused_linear_bwd(to_dev(g_s, dtype), W, X, act="relu", tile_cfg=tile_cfg)
    torch.cuda.synchronize()
    del W, X
    h, db = to_host(dX, dtype), dbias.cpu().numpy().astype(np.float64)
    x_live = synth.to_storage(np.ones((M, live.size)), dtype)
    rX, _, rdb = oracle.fused_linear_bwd(g_s, w_live_s, x_live, act="relu", dtype=dtype)
    assert np.array_equal(h[:, live].view(np.uint16), rX.view(np.uint16)), oracle.compare(h[:, live], rX, dtype)
    assert np.array_equal(db[live], rdb)             # integer sums, exact in fp32
    dead = np.ones(N, dtype=bool)
    dead[live] = False
    assert (oracle.decode(h[:, dead], dtype) == 0.0).all()
    assert (db[dead] == 0.0).all()
