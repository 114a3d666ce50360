"""C-ABI checks that need no GPU: exports, argument validation, host tile map.

Validation runs before any HIP call, so every rejected call below returns its
status without touching a device.  Fake device pointers are plain aligned
integers that are never dereferenced.
"""
import ctypes
import os
import re

import pytest

import oracle
import activation_epilogue_amd as fl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fused_linear.h")

OK, INVALID, UNSUPPORTED = 0, 1, 2
F32, F16, BF16 = 0, 1, 2
NONE, RELU, GELU, GLU = 0, 1, 2, 3


@pytest.fixture(scope="module")
def lib():
    return fl.load_library()


def test_header_symbols_are_exported(lib):
    text = open(HEADER).read()
    declared = sorted(set(re.findall(r"\b(fl_[a-z0-9_]+)\s*\(", text)))
    assert declared, "no declarations found"
    for name in declared:
        assert hasattr(lib, name), f"{name} declared in the header but not exported"
    assert set(declared) == set(fl.EXPORTS)


def test_version_and_status_strings(lib):
    assert lib.fl_version() == 10100
    assert lib.fl_status_string(0) == b"ok"
    assert lib.fl_status_string(1) == b"invalid argument"
    assert lib.fl_status_string(3) == b"launch failed"


A_P, B_P, BIAS_P, Y_P, OUT_P = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000


def _fused(lib, A=A_P, B=B_P, bias=BIAS_P, Y=None, out=OUT_P, M=64, N=64, K=64, act=RELU, dt=F16, opt=None):
    if opt is None:
        return lib.fl_fused_linear(A, B, bias, Y, out, M, N, K, act, dt, None)
    return lib.fl_fused_linear_ex(A, B, bias, Y, out, M, N, K, act, dt, None, ctypes.byref(opt))


@pytest.mark.parametrize("kwargs,status,msg", [
    (dict(A=None), INVALID, "A is NULL"),
    (dict(B=None), INVALID, "B is NULL"),
    (dict(out=None), INVALID, "out is NULL"),
    (dict(act=GLU), INVALID, "the gate needs Y"),
    (dict(Y=Y_P), INVALID, "Y is only used by the gate"),
    (dict(M=-1), INVALID, "negative size"),
    (dict(K=-5), INVALID, "negative size"),
    (dict(N=2 ** 31), UNSUPPORTED, "above 2^31-1"),
    (dict(K=2 ** 22), UNSUPPORTED, "too large"),
    (dict(K=32768, N=32768), UNSUPPORTED, "B too large"),  # B of 2 GiB: 32-bit offsets
    (dict(act=7), INVALID, "unknown activation"),
    (dict(dt=9), INVALID, "unknown dtype"),
    (dict(A=A_P + 1), INVALID, "not aligned"),
    (dict(out=A_P + 64), INVALID, "out overlaps A"),
    (dict(out=B_P), INVALID, "out overlaps B"),
    (dict(out=BIAS_P - 2), INVALID, "out overlaps bias"),
    (dict(act=GLU, Y=OUT_P + 2), INVALID, "partially overlaps"),
])
def test_fused_rejects_bad_arguments(lib, kwargs, status, msg):
    assert _fused(lib, **kwargs) == status
    assert msg in lib.fl_last_error().decode()


def test_degenerate_shapes_return_ok_without_launch(lib):
    assert _fused(lib, M=0) == OK
    assert _fused(lib, N=0) == OK
    assert _fused(lib, A=None, M=0, K=0, N=5) == OK
    assert lib.fl_last_error() == b""
    assert lib.fl_bias_add(None, None, 0, 7, F16, None) == OK
    assert lib.fl_activation(None, None, None, 3, 0, RELU, F32, None) == OK


def test_bad_options(lib):
    assert _fused(lib, opt=fl.Options(-1, 0, 0, 0, None)) == INVALID
    assert _fused(lib, opt=fl.Options(0, 2, 0, 0, None)) == INVALID
    assert _fused(lib, opt=fl.Options(0, 0, 99, 0, None)) == UNSUPPORTED
    assert "tile_cfg" in lib.fl_last_error().decode()
    assert _fused(lib, opt=fl.Options(0, 0, 0, 0, None, 2)) == INVALID
    assert b"debug_sync" in lib.fl_last_error()


def test_unfused_entry_points_reject_bad_arguments(lib):
    assert lib.fl_gemm(None, B_P, OUT_P, 8, 8, 8, F32, None) == INVALID
    assert lib.fl_gemm(A_P, B_P, OUT_P, 8, 32768, 32768, F16, None) == UNSUPPORTED
    assert "B too large" in lib.fl_last_error().decode()
    assert lib.fl_bias_add(OUT_P, None, 8, 8, F32, None) == INVALID
    assert lib.fl_bias_add(OUT_P, OUT_P + 4, 8, 8, F32, None) == INVALID
    assert lib.fl_activation(OUT_P, None, OUT_P + 2, 8, 8, RELU, F16, None) == INVALID
    assert lib.fl_activation(OUT_P, None, OUT_P, 8, 8, GLU, F16, None) == INVALID
    assert lib.fl_activation(OUT_P, Y_P, OUT_P, 8, 8, RELU, F16, None) == INVALID
    assert lib.fl_activation(OUT_P, None, OUT_P, 8, 8, 4, F16, None) == INVALID


def test_tile_grid(lib):
    # automatic choice: 256-wide tiles unless 128-wide ones need fewer
    # "waves x relative tile time" on 256 compute units
    assert fl.tile_grid(4096, 4096, 4096, F16) == (256, 256, 16, 16)
    assert fl.tile_grid(4097, 3071, 1537, BF16) == (256, 256, 17, 12)
    assert fl.tile_grid(8192, 14336, 4096, BF16) == (256, 256, 32, 56)
    assert fl.tile_grid(1024, 21568, 4096, F16) == (256, 192, 4, 113)
    assert fl.tile_grid(4096, 4608, 4096, F16) == (256, 192, 16, 24)
    assert fl.tile_grid(1024, 21568, 1024, F16) == (256, 128, 4, 169)  # two per CU
    assert fl.tile_grid(1024, 21568, 1280, F16) == (256, 192, 4, 113)
    assert fl.tile_grid(1024, 21568, 3072, F16) == (256, 192, 4, 113)
    assert fl.tile_grid(127, 129, 96, F16) == (256, 128, 1, 2)
    assert fl.tile_grid(127, 129, 96, F32) == (256, 256, 1, 1)
    assert fl.tile_grid(1024, 21568, 4096, F16, tile_cfg=1) == (256, 256, 4, 85)
    assert fl.tile_grid(4096, 4096, 4096, BF16, tile_cfg=2) == (256, 128, 16, 32)
    with pytest.raises(fl.FusedLinearError):
        fl.tile_grid(64, 64, 64, F32, tile_cfg=2)
    assert fl.tile_grid(4096, 4096, 4096, F16, tile_cfg=5) == (256, 256, 16, 16)
    assert fl.tile_grid(4096, 4096, 4096, F16, tile_cfg=6) == (256, 128, 16, 32)
    # short reductions whose 256x128 grid fills two workgroups per CU
    assert fl.tile_grid(1024, 21568, 256, F16) == (256, 128, 4, 169)
    assert fl.tile_grid(8192, 8192, 256, F16) == (256, 128, 32, 64)
    assert fl.tile_grid(8192, 8192, 384, F16) == (256, 256, 32, 32)
    with pytest.raises(fl.FusedLinearError):
        fl.tile_grid(64, 64, 64, F32, tile_cfg=6)
    # 256x192 tiles (192 = 3*64, not a power of two): N = 21568 = 112*192 + 64
    assert fl.tile_grid(1024, 21568, 4096, F16, tile_cfg=7) == (256, 192, 4, 113)
    assert fl.tile_grid(4097, 3071, 1537, BF16, tile_cfg=8) == (256, 192, 17, 16)
    for cfg in (7, 8):
        with pytest.raises(fl.FusedLinearError):
            fl.tile_grid(64, 64, 64, F32, tile_cfg=cfg)
    # 16x16x32 MFMA blocks: 256x256 with 4 or 8 waves, 256x192, 256x128
    assert fl.tile_grid(4096, 4096, 4096, F16, tile_cfg=9) == (256, 256, 16, 16)
    assert fl.tile_grid(4096, 4096, 4096, F16, tile_cfg=10) == (256, 256, 16, 16)
    assert fl.tile_grid(1024, 21568, 4096, F16, tile_cfg=11) == (256, 192, 4, 113)
    assert fl.tile_grid(4097, 3071, 1537, BF16, tile_cfg=12) == (256, 128, 17, 24)
    assert fl.tile_grid(4096, 4096, 4096, F16, tile_cfg=13) == (256, 256, 16, 16)
    assert fl.tile_grid(4096, 4096, 4096, F16, tile_cfg=14) == (256, 256, 16, 16)
    assert fl.tile_grid(1024, 21568, 4096, F16, tile_cfg=15) == (256, 192, 4, 113)
    for cfg in (9, 10, 11, 12, 13, 14, 15):
        with pytest.raises(fl.FusedLinearError):
            fl.tile_grid(64, 64, 64, F32, tile_cfg=cfg)
    with pytest.raises(fl.FusedLinearError):
        fl.tile_grid(64, 64, 64, F16, tile_cfg=16)


def test_host_tile_map_matches_oracle_without_xcd_step(lib):
    # the printed six-program example and a brute-force sweep
    assert [fl.tile_of_program(p, 6, 3, 2, 2, 0) for p in range(6)] == [(0, 0), (1, 0), (0, 1), (1, 1), (2, 0), (2, 1)]
    for tm in range(1, 18, 2):
        for tn in range(1, 14, 3):
            for g in (1, 2, 4, 8, 9):
                for p in range(tm * tn):
                    assert fl.tile_of_program(p, tm * tn, tm, tn, g, 0) == oracle.tile_of_pid(p, tm, tn, g)


@pytest.mark.parametrize("tm,tn,g", [(16, 16, 8), (17, 12, 4), (17, 12, 8), (4, 85, 8), (32, 56, 8), (1, 1, 1),
                                     (3, 5, 2), (33, 24, 8)])
def test_host_tile_map_with_xcd_step_is_a_bijection(lib, tm, tn, g):
    n = tm * tn
    tiles = [fl.tile_of_program(p, n, tm, tn, g, 1) for p in range(n)]
    assert sorted(tiles) == sorted((m, k) for m in range(tm) for k in range(tn))
    # programs on one XCD (p % 8 equal) receive consecutive grouped positions
    pos = {oracle.tile_of_pid(q, tm, tn, g): q for q in range(n)}
    for x in range(min(8, n)):
        qs = [pos[tiles[p]] for p in range(x, n, 8)]
        assert qs == list(range(qs[0], qs[0] + len(qs)))


R_P = 0x60000000


def _res(lib, R=R_P, Y=None, out=OUT_P, act=RELU, M=64, N=64, K=64, dt=F16):
    return lib.fl_fused_linear_residual(A_P, B_P, BIAS_P, R, Y, out, M, N, K, act, dt, None, None)


@pytest.mark.parametrize("kwargs,status,msg", [
    (dict(R=None), INVALID, "R is NULL"),
    (dict(R=R_P + 1), INVALID, "not aligned"),
    (dict(R=OUT_P + 2), INVALID, "R partially overlaps out"),
    (dict(out=R_P, R=R_P + 64), INVALID, "R partially overlaps out"),
    (dict(act=GLU), INVALID, "the gate needs Y"),
    (dict(Y=Y_P), INVALID, "Y is only used by the gate"),
])
def test_residual_rejects_bad_arguments(lib, kwargs, status, msg):
    assert _res(lib, **kwargs) == status
    assert msg in lib.fl_last_error().decode()


def test_residual_degenerate_shapes_return_ok(lib):
    assert _res(lib, R=None, M=0) == OK
    assert _res(lib, R=None, N=0) == OK


def _quant(lib, out=OUT_P, scale=1.0, q=0, dt=F16, act=RELU, Y=None, opt=None, M=64, N=64, K=64):
    return lib.fl_fused_linear_quant(A_P, B_P, BIAS_P, Y, out, scale, M, N, K, act, dt, q, None,
                                     ctypes.byref(opt) if opt is not None else None)


@pytest.mark.parametrize("kwargs,status,msg", [
    (dict(q=5), INVALID, "unknown qformat"),
    (dict(scale=float("nan")), INVALID, "scale must be finite"),
    (dict(scale=float("inf")), INVALID, "scale must be finite"),
    (dict(dt=F32), UNSUPPORTED, "fp16 or bf16"),
    (dict(out=None), INVALID, "out is NULL"),
    (dict(out=A_P + 100), INVALID, "out overlaps A"),
    (dict(act=GLU, Y=Y_P, out=Y_P + 8191), INVALID, "out overlaps Y"),
    (dict(opt=fl.Options(0, 0, 1, 0, None)), UNSUPPORTED, "tile_cfg 0, 2, 5, 6, 7, 10, 11, 12 and 15"),
    (dict(opt=fl.Options(0, 0, 3, 0, None)), UNSUPPORTED, "tile_cfg 0, 2, 5, 6, 7, 10, 11, 12 and 15"),
])
def test_quant_rejects_bad_arguments(lib, kwargs, status, msg):
    assert _quant(lib, **kwargs) == status
    assert msg in lib.fl_last_error().decode()


def test_quant_degenerate_shapes_return_ok(lib):
    assert _quant(lib, out=None, M=0) == OK
    assert _quant(lib, out=None, N=0) == OK


def _fp8(lib, A=A_P, B=B_P, ab=1.0, out=OUT_P, dt=F16, M=64, N=64, K=64, act=RELU, Y=None, opt=None):
    return lib.fl_fused_linear_fp8(A, B, ab, BIAS_P, Y, out, M, N, K, act, dt, None,
                                   ctypes.byref(opt) if opt is not None else None)


@pytest.mark.parametrize("kwargs,status,msg", [
    (dict(ab=float("nan")), INVALID, "ab_scale must be finite"),
    (dict(dt=F32), UNSUPPORTED, "fp16 or bf16"),
    (dict(N=2), UNSUPPORTED, "N >= 3"),
    (dict(N=1), UNSUPPORTED, "N >= 3"),
    (dict(A=A_P + 8), INVALID, "16-byte aligned"),
    (dict(A=None), INVALID, "A is NULL"),
    (dict(out=A_P + 64), INVALID, "out overlaps A"),
    (dict(act=GLU), INVALID, "the gate needs Y"),
    (dict(opt=fl.Options(0, 0, 4, 0, None)), UNSUPPORTED, "tile_cfg 0, 1, 2, 5, 6, 7 and 12"),
    (dict(opt=fl.Options(0, 0, 16, 0, None)), UNSUPPORTED, "tile_cfg 16"),
    (dict(opt=fl.Options(0, 0, 10, 0, None)), UNSUPPORTED, "tile_cfg 0, 1, 2, 5, 6, 7 and 12"),
    (dict(K=65536, N=32768), UNSUPPORTED, "B too large"),
])
def test_fp8_rejects_bad_arguments(lib, kwargs, status, msg):
    assert _fp8(lib, **kwargs) == status
    assert msg in lib.fl_last_error().decode()


# ------------------------------------------------------ backward epilogue

X_P = 0x7000000    # saved pre-activation (M,N)
DY_P = 0x7800000   # second output of the gate
DB_P = 0x7F00000   # bias gradient (N,) fp32


def _bwd(lib, G=A_P, W=B_P, X=X_P, Y=None, dX=OUT_P, dY=None, db=DB_P, dt=F16, M=64, N=64, K=64, act=RELU,
         opt=None):
    return lib.fl_fused_linear_bwd(G, W, X, Y, dX, dY, db, M, N, K, act, dt, None,
                                   ctypes.byref(opt) if opt is not None else None)


@pytest.mark.parametrize("kwargs,status,msg", [
    (dict(dt=F32), UNSUPPORTED, "fp16 and bf16"),
    (dict(X=None), INVALID, "X (the saved pre-activation) is NULL"),
    (dict(act=GLU, Y=Y_P), INVALID, "the gate's backward needs dY"),
    (dict(act=GLU), INVALID, "the gate needs Y"),
    (dict(dY=DY_P), INVALID, "dY is only written for the gate"),
    (dict(X=A_P + 128), INVALID, "X overlaps G or W"),
    (dict(X=OUT_P + 2), INVALID, "R partially overlaps out"),
    (dict(act=GLU, Y=Y_P, dY=X_P + 64), INVALID, "dY overlaps"),
    (dict(act=GLU, Y=Y_P, dY=Y_P + 2), INVALID, "dY partially overlaps Y"),
    (dict(db=X_P + 16), INVALID, "dbias overlaps"),
    (dict(db=DB_P + 2), INVALID, "dbias is not 4-byte aligned"),
    (dict(dX=A_P + 64), INVALID, "out overlaps A"),
    (dict(opt=fl.Options(0, 0, 7, 0, None)), UNSUPPORTED, "tile_cfg 0, 2, 5, 10 and 12"),
    (dict(opt=fl.Options(0, 0, 1, 0, None)), UNSUPPORTED, "tile_cfg 0, 2, 5, 10 and 12"),
    (dict(K=2 ** 22), UNSUPPORTED, "too large"),
])
def test_bwd_rejects_bad_arguments(lib, kwargs, status, msg):
    assert _bwd(lib, **kwargs) == status
    assert msg in lib.fl_last_error().decode()


WS_P = 0x9000000   # backward workspace


def _bwd_ws(lib, ws=WS_P, ws_bytes=1 << 20, **kw):
    G, W, X, Y, dX, dY, db = (kw.pop(k, d) for k, d in (("G", A_P), ("W", B_P), ("X", X_P), ("Y", None),
                                                         ("dX", OUT_P), ("dY", None), ("db", DB_P)))
    M, N, K = kw.pop("M", 64), kw.pop("N", 64), kw.pop("K", 64)
    assert not kw
    return lib.fl_fused_linear_bwd_ws(G, W, X, Y, dX, dY, db, M, N, K, RELU, F16, None, None, ws, ws_bytes)


def _ws_bytes(lib, M, N, K=64, dt=F16):
    n = ctypes.c_size_t(12345)
    st = lib.fl_bwd_workspace_bytes(M, N, K, dt, ctypes.byref(n))
    return st, n.value


def test_bwd_workspace_bytes():
    """Two fp32 rows of partial column sums per 256-row tile row."""
    lib = fl.load_library()
    assert _ws_bytes(lib, 8192, 14336) == (0, 2 * 32 * 14336 * 4)
    assert _ws_bytes(lib, 257, 10) == (0, 2 * 2 * 10 * 4)
    assert _ws_bytes(lib, 1, 1) == (0, 8)
    assert _ws_bytes(lib, 0, 100) == (0, 0) and _ws_bytes(lib, 100, 0) == (0, 0)
    assert _ws_bytes(lib, 64, 64, dt=F32)[0] == UNSUPPORTED
    assert _ws_bytes(lib, -1, 64)[0] == INVALID
    assert lib.fl_bwd_workspace_bytes(64, 64, 64, F16, None) == INVALID


@pytest.mark.parametrize("kwargs,msg", [
    (dict(ws=None), "workspace is NULL (512 bytes needed)"),
    (dict(ws_bytes=511), "workspace of 511 bytes is too small (512 bytes needed)"),
    (dict(ws=WS_P + 2), "workspace is not 4-byte aligned"),
    (dict(ws=DB_P + 128), "workspace overlaps an operand"),
    (dict(ws=X_P + 64), "workspace overlaps an operand"),
    (dict(ws=A_P), "workspace overlaps an operand"),
])
def test_bwd_ws_rejects_bad_workspace(lib, kwargs, msg):
    assert _bwd_ws(lib, **kwargs) == INVALID
    assert msg in lib.fl_last_error().decode()


def test_bwd_ws_checks_the_rest_as_the_plain_entry(lib):
    """The workspace entry validates its other arguments exactly as
    fl_fused_linear_bwd (same status and message, no launch)."""
    assert _bwd_ws(lib, X=None) == INVALID
    assert "X (the saved pre-activation) is NULL" in lib.fl_last_error().decode()
    assert _bwd_ws(lib, db=DB_P + 2) == INVALID
    assert "dbias is not 4-byte aligned" in lib.fl_last_error().decode()


def test_bwd_noalloc_checks_before_any_launch(lib):
    """The no-allocation entry: a dbias whose partial sums exceed the 8 MiB
    static scratch, and the plain entry's argument errors, are reported
    with no HIP call (this host has no GPU)."""
    na = lib.fl_fused_linear_bwd_noalloc
    big = dict(M=65536, N=8192, K=64)     # 2 * 256 * 8192 * 4 = 16 MiB of partial sums
    assert na(A_P, B_P, X_P, None, OUT_P, None, DB_P, big["M"], big["N"], big["K"], RELU, F16, None, None) \
        == UNSUPPORTED
    assert "needs 16777216 bytes of scratch; the static scratch holds 8388608" in lib.fl_last_error().decode()
    assert na(A_P, B_P, None, None, OUT_P, None, DB_P, 64, 64, 64, RELU, F16, None, None) == INVALID
    assert "X (the saved pre-activation) is NULL" in lib.fl_last_error().decode()
    assert na(A_P, B_P, X_P, None, OUT_P, None, DB_P, 64, 64, 64, RELU, F32, None, None) == UNSUPPORTED
    assert na(A_P, B_P, X_P, None, OUT_P, None, DB_P + 2, 64, 64, 64, RELU, F16, None, None) == INVALID
    assert "dbias is not 4-byte aligned" in lib.fl_last_error().decode()
    assert na(A_P, B_P, X_P, None, OUT_P, None, DB_P, -1, 64, 64, RELU, F16, None, None) == INVALID


def test_unfused_bwd_chain_rejects_bad_arguments(lib):
    D_P, X2_P, DX_P = 0x7000000, 0x7800000, OUT_P
    assert lib.fl_gemm_nt(A_P, B_P, OUT_P, 64, 64, 64, F32, None) == UNSUPPORTED
    assert lib.fl_gemm_nt(A_P, B_P, A_P + 64, 64, 64, 64, F16, None) == INVALID
    assert "out overlaps A" in lib.fl_last_error().decode()
    ag = lib.fl_activation_grad
    assert ag(D_P, X2_P, None, DX_P, None, 64, 64, RELU, F32, None) == UNSUPPORTED
    assert ag(D_P, X2_P, None, DX_P, None, 64, 64, GLU, F16, None) == INVALID
    assert "needs Y and dY" in lib.fl_last_error().decode()
    assert ag(D_P, X2_P, Y_P, DX_P, None, 64, 64, RELU, F16, None) == INVALID
    assert ag(D_P, X2_P, None, D_P + 2, None, 64, 64, RELU, F16, None) == INVALID
    assert "partially overlaps D" in lib.fl_last_error().decode()
    assert ag(D_P, X2_P, None, X2_P, None, 64, 64, RELU, F16, None) == INVALID
    assert ag(D_P + 1, X2_P, None, DX_P, None, 64, 64, RELU, F16, None) == INVALID
    assert ag(D_P, X2_P, None, DX_P, None, 64, 64, 7, F16, None) == INVALID
    cs = lib.fl_column_sum
    assert cs(X2_P, None, 64, 64, F16, None) == INVALID
    assert cs(X2_P, X2_P + 64, 64, 64, F16, None) == INVALID
    assert "sums overlaps X" in lib.fl_last_error().decode()
    assert cs(X2_P, DB_P, 64, 64, F32, None) == UNSUPPORTED


def test_error_message_is_per_thread(lib):
    """Each host thread reads the message of its own last failed call
    (validation errors only: nothing is launched)."""
    import threading
    barrier = threading.Barrier(2)
    seen = {}

    def worker(name, kwargs):
        barrier.wait()
        for _ in range(200):
            st = _fused(lib, **kwargs)
            seen[name] = (st, lib.fl_last_error().decode())
            assert seen[name][0] == INVALID

    ta = threading.Thread(target=worker, args=("neg", dict(M=-1)))
    tb = threading.Thread(target=worker, args=("null", dict(A=None)))
    ta.start(); tb.start(); ta.join(); tb.join()
    assert "negative size" in seen["neg"][1] and "A is NULL" not in seen["neg"][1]
    assert "A is NULL" in seen["null"][1] and "negative size" not in seen["null"][1]
    # a successful call clears this thread's message
    assert _fused(lib, M=-1) == INVALID and lib.fl_last_error() != b""
    assert _fused(lib, M=0) == OK and lib.fl_last_error() == b""
