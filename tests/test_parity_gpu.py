"""Parity of the HIP path (through the C ABI) with the FP64 oracle.

Tolerance (|dev - ref| <= atol + rtol*|ref|, ref = the oracle's once-rounded
output): (1e-4, 1e-4) for fp32 outputs and (4e-3, 1e-2) for fp16/bf16.
Bit-exact where the inputs make all arithmetic exact (small integers).
Every output buffer is prefilled with NaN and followed by a NaN guard band:
an element left unwritten fails the comparison and a write past the end
breaks the guard.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import activation_epilogue_amd as fl
from activation_epilogue_amd import synth
from gpu_util import say, to_dev, to_host, sentinel_out, guard_intact, TORCH_DT

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
DTYPES = ["f32", "f16", "bf16"]


def _run_fused(d, act, dtype, **opts):
    M, K = d["A"].shape
    N = d["B"].shape[1]
    A, B, bias, Y = (to_dev(d[k], dtype) for k in ("A", "B", "bias", "Y"))
    R = to_dev(d.get("R"), dtype)
    out, buf = sentinel_out(M, N, dtype)
    fl.fused_linear(A, B, bias, Y, act=act, out=out, R=R, **opts)
    torch.cuda.synchronize()
    assert guard_intact(buf, M, N), "write past the end of out"
    return to_host(out, dtype)


def _run_unfused(d, act, dtype):
    M, K = d["A"].shape
    N = d["B"].shape[1]
    A, B, bias, Y = (to_dev(d[k], dtype) for k in ("A", "B", "bias", "Y"))
    X, buf = sentinel_out(M, N, dtype)
    fl.gemm(A, B, X)
    if bias is not None:
        fl.bias_add(X, bias)
    out = fl.activation(X, Y, out=X, act=act)
    torch.cuda.synchronize()
    assert guard_intact(buf, M, N)
    return to_host(out, dtype)


def _assert_close(dev, ref, dtype, what):
    res = oracle.compare(dev, ref, dtype)
    assert res["ok"], f"{what}: {res}"


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a device"
    fl.load_library()


# ------------------------------------------------------------ worked example

def _golden_inputs(dtype):
    vals = {}
    for line in open(os.path.join(GOLDEN, "worked_example_2x2.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            k, _, rhs = line.partition("=")
            rows = [[float(v) for v in r.split()] for r in rhs.split(";")]
            vals[k.strip()] = np.array(rows if len(rows) > 1 else rows[0])
    return vals


@pytest.mark.parametrize("dtype", DTYPES)
def test_worked_example_bit_exact(dtype):
    g = _golden_inputs(dtype)
    d = {"A": synth.to_storage(g["A"], dtype), "B": synth.to_storage(g["B"], dtype),
         "bias": synth.to_storage(g["bias"], dtype), "Y": None}
    say("worked example", dtype)
    out = _run_fused(d, "relu", dtype)
    assert np.array_equal(oracle.decode(out, dtype), g["relu"])
    out = _run_unfused(d, "relu", dtype)
    assert np.array_equal(oracle.decode(out, dtype), g["relu"])


# ------------------------------------------------------------------- K = 0

@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("act", ["none", "relu", "gelu_tanh", "glu"])
@pytest.mark.parametrize("shape", [(127, 129), (37, 300)])
def test_k0_gives_act_of_bias(dtype, act, shape):
    """K = 0 at the small ragged workload's 127 x 129 (and a wider grid):
    act(bias) on every row."""
    d = synth.draw(*shape, 0, dtype, act, seed=1)
    say("K=0", dtype, act, shape)
    out = _run_fused(d, act, dtype)
    ref = oracle.fused_linear(d["A"], d["B"], d["bias"], d["Y"], act=act, dtype=dtype)
    if act in ("none", "relu"):
        # acc = 0, so X = bias exactly and the store returns the bias bits
        assert np.array_equal(out.view(np.uint8), ref.view(np.uint8))
    _assert_close(out, ref, dtype, f"K=0 {act}")


@pytest.mark.parametrize("seed", range(6))
def test_seeded_random_shapes(seed):
    """Seeded random shapes (ragged M, N and K up to a few hundred, every
    activation and dtype, a residual now and then) through the automatic
    choice and through one random kernel variant of the dtype: the whole
    output against the oracle, and the variant bit-identical to the
    automatic choice wherever both use the same MFMA shape."""
    rng = np.random.default_rng(1000 + seed)
    for case in range(8):
        M, N, K = (int(rng.integers(1, 700)) for _ in range(3))
        dtype = ["f32", "f16", "bf16"][int(rng.integers(0, 3))]
        act = ["none", "relu", "gelu_tanh", "glu"][int(rng.integers(0, 4))]
        residual = bool(rng.integers(0, 4) == 0)
        cfgs = [3] if dtype == "f32" else FAMILY_32 + FAMILY_16
        cfg = cfgs[int(rng.integers(0, len(cfgs)))]
        d = synth.draw(M, N, K, dtype, act, seed=seed * 8 + case, residual=residual)
        say("random shape", seed, case, M, N, K, dtype, act, "residual" if residual else "", "tile_cfg", cfg)
        auto = _run_fused(d, act, dtype)
        var = _run_fused(d, act, dtype, tile_cfg=cfg)
        ref = oracle.fused_linear(d["A"], d["B"], d["bias"], d["Y"], act=act, dtype=dtype, R=d.get("R"))
        _assert_close(auto, ref, dtype, f"random {M}x{N}x{K} {dtype} {act} auto")
        _assert_close(var, ref, dtype, f"random {M}x{N}x{K} {dtype} {act} tile_cfg {cfg}")
        if dtype == "f32" or cfg in FAMILY_16:
            assert np.array_equal(auto.view(np.uint8), var.view(np.uint8)), (M, N, K, dtype, act, cfg)


# --------------------------------------------------- K=1 / K=3 and the chain

@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("K", [1, 3])
def test_k1_k3_fused_matches_unfused_and_oracle(dtype, K):
    d = synth.draw(127, 129, K, dtype, "relu", seed=0)
    say("K1/K3", dtype, K)
    fused = _run_fused(d, "relu", dtype)
    chain = _run_unfused(d, "relu", dtype)
    ref = oracle.fused_linear(d["A"], d["B"], d["bias"], act="relu", dtype=dtype)
    ref_chain = oracle.unfused_chain(d["A"], d["B"], d["bias"], act="relu", dtype=dtype)
    _assert_close(fused, ref, dtype, "fused vs oracle")
    _assert_close(chain, ref_chain, dtype, "unfused chain vs oracle chain")
    _assert_close(fused, chain, dtype, "fused vs unfused chain")


# ------------------------------------------------------- exact integer data

INT_SHAPES = [(1, 1, 1), (3, 5, 7), (2, 9, 0), (64, 64, 64), (67, 65, 70), (65, 8, 8), (31, 136, 64),
              (257, 264, 40), (300, 520, 24), (513, 770, 33), (129, 1024, 16)]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("act", ["none", "relu", "glu"])
@pytest.mark.parametrize("shape", INT_SHAPES)
def test_integer_inputs_bit_exact(dtype, act, shape):
    M, N, K = shape
    d = synth.draw_integer(M, N, K, dtype, act, seed=M + 7 * N + 13 * K, amax=1, bias_max=3)
    say("integer", dtype, act, shape)
    out = _run_fused(d, act, dtype)
    ref = oracle.fused_linear(d["A"], d["B"], d["bias"], d["Y"], act=act, dtype=dtype)
    assert np.array_equal(out.view(np.uint8), ref.view(np.uint8)), oracle.compare(out, ref, dtype)


@pytest.mark.parametrize("dtype", DTYPES)
def test_integer_inputs_no_bias(dtype):
    d = synth.draw_integer(70, 90, 50, dtype, "relu", seed=3)
    d["bias"] = None
    say("integer no bias", dtype)
    out = _run_fused(d, "relu", dtype)
    ref = oracle.fused_linear(d["A"], d["B"], None, act="relu", dtype=dtype)
    assert np.array_equal(out.view(np.uint8), ref.view(np.uint8))


# ----------------------------------------------------- random data, tolerance

@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("act", ["none", "relu", "gelu_tanh", "glu"])
@pytest.mark.parametrize("shape", [(127, 129, 96), (256, 512, 256), (300, 260, 1000), (513, 96, 72)])
def test_random_inputs_within_tolerance(dtype, act, shape):
    M, N, K = shape
    d = synth.draw(M, N, K, dtype, act, bias_var=0.1 if act == "gelu_tanh" else 1.0, seed=5)
    say("random", dtype, act, shape)
    out = _run_fused(d, act, dtype)
    ref = oracle.fused_linear(d["A"], d["B"], d["bias"], d["Y"], act=act, dtype=dtype)
    _assert_close(out, ref, dtype, f"{dtype} {act} {shape}")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("shape,act", [((1, 8200, 1024), "glu"), ((4097, 1, 300), "relu"), ((1, 1, 65536), "relu"),
                                       ((3, 5, 100003), "gelu_tanh"), ((2, 70000, 16), "relu"),
                                       ((70000, 24, 8), "none"), ((33, 7, 4099), "glu")])
def test_extreme_shapes(dtype, shape, act):
    """Degenerate tile grids: one output row or column, a single output,
    reductions of 65536 and of a prime length, and very wide or very tall
    outputs (one tile deep in one direction, hundreds in the other).  The
    whole output is compared and nothing is written past it."""
    M, N, K = shape
    d = synth.draw(M, N, K, dtype, act, bias_var=0.1 if act == "gelu_tanh" else 1.0, seed=31)
    say("extreme shape", dtype, act, shape)
    out = _run_fused(d, act, dtype)
    ref = oracle.fused_linear(d["A"], d["B"], d["bias"], d["Y"], act=act, dtype=dtype)
    _assert_close(out, ref, dtype, f"{dtype} {act} {shape}")


def test_relu_f32_127x129x96_full():
    w = synth.WORKLOADS["relu_f32_127x129x96"]
    d = synth.draw_workload(w)
    say(w.name)
    out = _run_fused(d, w.act, w.dtype)
    ref = oracle.fused_linear(d["A"], d["B"], d["bias"], act=w.act, dtype=w.dtype)
    _assert_close(out, ref, w.dtype, w.name)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("act", ["relu", "gelu_tanh", "glu"])
def test_unfused_chain_matches_oracle_chain(dtype, act):
    d = synth.draw(200, 264, 136, dtype, act, seed=8)
    say("unfused chain", dtype, act)
    chain = _run_unfused(d, act, dtype)
    ref = oracle.unfused_chain(d["A"], d["B"], d["bias"], d["Y"], act=act, dtype=dtype)
    _assert_close(chain, ref, dtype, "unfused chain")


@pytest.mark.parametrize("dtype", DTYPES)
def test_vector_and_element_paths_agree_bitwise(dtype):
    """A misaligned copy of the same data takes the element path."""
    M, N, K = 130, 264, 200
    d = synth.draw(M, N, K, dtype, "relu", seed=12)
    A, B, bias = (to_dev(d[k], dtype) for k in ("A", "B", "bias"))
    say("vector vs element path", dtype)
    out_v = fl.fused_linear(A, B, bias, act="relu")
    A2 = torch.empty(M * K + 1, dtype=A.dtype, device="cuda")[1:].view(M, K)
    A2.copy_(A)
    out_e = fl.fused_linear(A2, B, bias, act="relu")
    torch.cuda.synchronize()
    assert np.array_equal(to_host(out_v, dtype).view(np.uint8), to_host(out_e, dtype).view(np.uint8))


# ----------------------------------------------------------- the full sizes

FULL = ["relu_f32_4096x4096x4096", "relu_f16_4096x4096x4096", "relu_bf16_4097x3071x1537",
        "glu_f16_1024x21568x4096", "gelu_bf16_8192x14336x4096", "glu_f16_1024x21568x256",
        "residual_bf16_8192x4096x14336"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_whole_output(name):
    """Default launch (as timed by the benchmark): no write past the end, and
    every output element equal to the oracle within tolerance ("I3. Fuse a
    GEMM epilogue and change tile scheduling", "Implement in stages")."""
    w = synth.WORKLOADS[name]
    d = synth.draw_workload(w)
    say("full size", name)
    out = _run_fused(d, w.act, w.dtype)
    assert not np.isnan(oracle.decode(out, w.dtype)).any(), "unwritten (NaN sentinel) outputs"
    ref = oracle.fused_linear(d["A"], d["B"], d["bias"], d["Y"], act=w.act, dtype=w.dtype, R=d["R"])
    _assert_close(out, ref, w.dtype, name)


@pytest.mark.parametrize("name", ["relu_bf16_4097x3071x1537", "glu_f16_1024x21568x4096"])
def test_tile_order_does_not_change_bits(name):
    """GROUP in {1,4,8}, XCD step on/off and persistent on/off change which
    workgroup computes a tile, never its arithmetic; each tile is written
    exactly once."""
    w = synth.WORKLOADS[name]
    d = synth.draw_workload(w)
    A, B, bias, Y = (to_dev(d[k], w.dtype) for k in ("A", "B", "bias", "Y"))
    code = {"f32": 0, "f16": 1, "bf16": 2}[w.dtype]
    _, _, tm, tn = fl.tile_grid(w.M, w.N, w.K, code)
    base = None
    for opts in [dict(group_m=8), dict(group_m=1), dict(group_m=4), dict(group_m=8, no_xcd_remap=1),
                 dict(group_m=8, persistent=1), dict(group_m=1, persistent=1, no_xcd_remap=1)]:
        say("tile order", name, opts)
        counts = torch.zeros(tm * tn, dtype=torch.int32, device="cuda")
        out = fl.fused_linear(A, B, bias, Y, act=w.act, debug_tile_count=counts, **opts)
        torch.cuda.synchronize()
        assert bool((counts == 1).all().item()), f"tile written {counts.min().item()}..{counts.max().item()} times"
        h = to_host(out, w.dtype).view(np.uint8)
        if base is None:
            base = h
        else:
            assert np.array_equal(h, base), opts


@pytest.mark.parametrize("cfg,cfg256", [(7, 1), (8, 1), (11, 10), (15, 10)])
def test_npot_tiles_full_gate_shape(cfg, cfg256):
    """256x192 tiles (a width that is not a power of two; "Optimizing GEMM +
    Activation on CDNA4 with TLX", "Future Work") on the gate workload
    M=1024, N=21568, K=4096: 4 x 113 tiles, the last column of tiles 64
    wide.  Each tile is written exactly once, the whole output matches the
    oracle and is bit-identical to the 256x256 kernel's of the same MFMA
    shape (32x32x16: 7, 8; 16x16x32: 11, 15)."""
    w = synth.WORKLOADS["glu_f16_1024x21568x4096"]
    d = synth.draw_workload(w)
    A, B, bias, Y = (to_dev(d[k], w.dtype) for k in ("A", "B", "bias", "Y"))
    _, bn, tm, tn = fl.tile_grid(w.M, w.N, w.K, 1, tile_cfg=cfg)
    assert (bn, tm, tn) == (192, 4, 113)
    say("npot full", cfg)
    counts = torch.zeros(tm * tn, dtype=torch.int32, device="cuda")
    out = fl.fused_linear(A, B, bias, Y, act=w.act, tile_cfg=cfg, debug_tile_count=counts)
    ref256 = fl.fused_linear(A, B, bias, Y, act=w.act, tile_cfg=cfg256)
    torch.cuda.synchronize()
    assert bool((counts == 1).all().item())
    h = to_host(out, w.dtype)
    assert np.array_equal(h.view(np.uint8), to_host(ref256, w.dtype).view(np.uint8))
    ref = oracle.fused_linear(d["A"], d["B"], d["bias"], d["Y"], act=w.act, dtype=w.dtype)
    _assert_close(h, ref, w.dtype, f"{w.name} tile_cfg {cfg}")


@pytest.mark.parametrize("cfg", [0, 2, 3, 5, 6, 7, 9, 10, 11, 12, 14, 15])
@pytest.mark.parametrize("dtype,act,shape", [("f16", "relu", (1024, 2048, 1024)), ("bf16", "glu", (513, 770, 1537)),
                                             ("f32", "relu", (300, 260, 200))])
def test_debug_sync_gives_the_same_bits(cfg, dtype, act, shape):
    """The debugging schedule (an extra full wait for the copies and an extra
    barrier in every K stage) only changes timing: a race between the copies,
    the operand reads and the barriers would show as different bits."""
    if dtype == "f32" and cfg not in (0, 3):
        pytest.skip("fp32 runs the register-staged kernel only")
    M, N, K = shape
    d = synth.draw(M, N, K, dtype, act, seed=61)
    say("debug sync", cfg, dtype, act, shape)
    fast = _run_fused(d, act, dtype, tile_cfg=cfg)
    slow = _run_fused(d, act, dtype, tile_cfg=cfg, debug_sync=1)
    assert np.array_equal(fast.view(np.uint8), slow.view(np.uint8))


@pytest.mark.parametrize("name", ["gelu_bwd_bf16_8192x14336x4096", "glu_bwd_f16_1024x21568x4096"])
def test_debug_sync_gives_the_same_bits_backward(name):
    """The backward epilogue under the debugging schedule: dX and dY keep
    their bits (dbias is summed with atomics, so only its value is checked)."""
    w = synth.WORKLOADS[name]
    d = synth.draw_bwd(1024, 1536, 1024, w.dtype, w.act, seed=62)
    say("debug sync bwd", name)
    fX, fY, fdb = _run_bwd(d, w.act, w.dtype)
    sX, sY, sdb = _run_bwd(d, w.act, w.dtype, debug_sync=1)
    assert np.array_equal(fX.view(np.uint8), sX.view(np.uint8))
    if fY is not None:
        assert np.array_equal(fY.view(np.uint8), sY.view(np.uint8))
    assert np.allclose(fdb, sdb, rtol=1e-5, atol=1e-5)


def test_repeat_runs_are_bitwise_identical():
    w = synth.WORKLOADS["relu_f16_4096x4096x4096"]
    d = synth.draw_workload(w)
    A, B, bias = (to_dev(d[k], w.dtype) for k in ("A", "B", "bias"))
    say("determinism", w.name)
    outs = [to_host(fl.fused_linear(A, B, bias, act="relu"), w.dtype) for _ in range(3)]
    torch.cuda.synchronize()
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


def test_y_may_alias_out():
    M, N, K = 300, 520, 64
    d = synth.draw(M, N, K, "f16", "glu", seed=2)
    A, B, bias, Y = (to_dev(d[k], "f16") for k in ("A", "B", "bias", "Y"))
    say("Y aliases out")
    fl.fused_linear(A, B, bias, Y, act="glu", out=Y)
    torch.cuda.synchronize()
    ref = oracle.fused_linear(d["A"], d["B"], d["bias"], d["Y"], act="glu", dtype="f16")
    _assert_close(to_host(Y, "f16"), ref, "f16", "Y == out")


# ------------------------------------------------------------ kernel variants

# Variants that sum each output in the same order, in 32x32 blocks 16 deep
# (v_mfma_f32_32x32x16) or in 16x16 blocks 32 deep (v_mfma_f32_16x16x32):
# bit-identical within a family.
FAMILY_32 = [1, 2, 3, 4, 5, 6, 7, 8]
FAMILY_16 = [9, 10, 11, 12, 13, 14, 15]


def _same_family_bits(outs):
    """Within each family every variant gives the same bits; the automatic
    choice (cfg 0) gives the bits of one of the families."""
    bases = {}
    for fam in (FAMILY_32, FAMILY_16):
        got = [c for c in fam if c in outs]
        if got:
            bases[got[0]] = outs[got[0]].view(np.uint8)
            for c in got:
                assert np.array_equal(outs[c].view(np.uint8), bases[got[0]]), f"tile_cfg {c} differs from {got[0]}"
    if 0 in outs:
        assert any(np.array_equal(outs[0].view(np.uint8), b) for b in bases.values()), "tile_cfg 0"


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("act", ["relu", "glu"])
@pytest.mark.parametrize("shape", [(127, 129, 96), (300, 520, 1000), (513, 264, 72), (1024, 2048, 1024)])
def test_kernel_variants_bit_identical_and_within_tolerance(dtype, act, shape):
    """Every fp16/bf16 kernel variant (256x256, 256x192 or 256x128 tiles,
    64- or 32-deep K stages, 4 or 8 waves, one or two workgroups per CU,
    direct or register-staged loads) of one MFMA family sums each output in
    the same k order, so results are bit-identical within the family; each
    also passes the oracle check.  The shapes leave ragged last tiles for
    every width (N = 129, 520, 264 and 2048 are not multiples of 192)."""
    M, N, K = shape
    d = synth.draw(M, N, K, dtype, act, seed=21)
    ref = oracle.fused_linear(d["A"], d["B"], d["bias"], d["Y"], act=act, dtype=dtype)
    outs = {}
    for cfg in [0] + FAMILY_32 + FAMILY_16:
        say("variant", cfg, dtype, act, shape)
        outs[cfg] = _run_fused(d, act, dtype, tile_cfg=cfg)
        _assert_close(outs[cfg], ref, dtype, f"tile_cfg {cfg}")
    _same_family_bits(outs)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("act", ["none", "relu", "glu"])
@pytest.mark.parametrize("shape", [(67, 65, 70), (257, 264, 40), (300, 520, 24), (513, 770, 33), (129, 1024, 16)])
def test_integer_inputs_bit_exact_every_variant(dtype, act, shape):
    """Exact small-integer data: every variant, whatever its MFMA shape and
    summation order, must give the oracle's bits on ragged shapes."""
    M, N, K = shape
    d = synth.draw_integer(M, N, K, dtype, act, seed=M + 5 * N + 11 * K, amax=1, bias_max=3)
    ref = oracle.fused_linear(d["A"], d["B"], d["bias"], d["Y"], act=act, dtype=dtype)
    for cfg in FAMILY_32 + FAMILY_16:
        say("integer variant", cfg, dtype, act, shape)
        out = _run_fused(d, act, dtype, tile_cfg=cfg)
        assert np.array_equal(out.view(np.uint8), ref.view(np.uint8)), (cfg, oracle.compare(out, ref, dtype))



# ------------------------------------------------------------ residual add
# out = act(A@B + bias + R) through fl_fused_linear_residual ("Triton: Fused
# Matmul + Bias + ReLU (Epilogue Fusion)", "Variants").

def _with_residual(d, dtype, seed, integer=False):
    M, N = d["A"].shape[0], d["B"].shape[1]
    rng = np.random.default_rng(seed)
    R = rng.integers(-3, 4, (M, N)).astype(np.float64) if integer else rng.standard_normal((M, N))
    d = dict(d)
    d["R"] = synth.to_storage(R, dtype)
    return d


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("act", ["none", "relu", "glu"])
@pytest.mark.parametrize("shape", [(1, 1, 1), (3, 5, 7), (2, 9, 0), (67, 65, 70), (257, 264, 40), (513, 770, 33)])
def test_residual_integer_inputs_bit_exact(dtype, act, shape):
    M, N, K = shape
    d = _with_residual(synth.draw_integer(M, N, K, dtype, act, seed=M + 5 * N + 11 * K, amax=1, bias_max=3),
                       dtype, seed=K, integer=True)
    say("residual integer", dtype, act, shape)
    out = _run_fused(d, act, dtype)
    ref = oracle.fused_linear(d["A"], d["B"], d["bias"], d["Y"], act=act, dtype=dtype, R=d["R"])
    assert np.array_equal(out.view(np.uint8), ref.view(np.uint8)), oracle.compare(out, ref, dtype)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("act", ["none", "relu", "gelu_tanh", "glu"])
@pytest.mark.parametrize("shape", [(127, 129, 96), (300, 260, 1000)])
def test_residual_random_within_tolerance(dtype, act, shape):
    M, N, K = shape
    d = _with_residual(synth.draw(M, N, K, dtype, act, seed=6), dtype, seed=7)
    say("residual random", dtype, act, shape)
    out = _run_fused(d, act, dtype)
    ref = oracle.fused_linear(d["A"], d["B"], d["bias"], d["Y"], act=act, dtype=dtype, R=d["R"])
    _assert_close(out, ref, dtype, f"residual {dtype} {act} {shape}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("act", ["relu", "glu"])
def test_residual_kernel_variants_bit_identical(dtype, act):
    M, N, K = 300, 520, 1000
    d = _with_residual(synth.draw(M, N, K, dtype, act, seed=22), dtype, seed=23)
    ref = oracle.fused_linear(d["A"], d["B"], d["bias"], d["Y"], act=act, dtype=dtype, R=d["R"])
    outs = {}
    for cfg in [0] + FAMILY_32 + FAMILY_16:
        say("residual variant", cfg, dtype, act)
        outs[cfg] = _run_fused(d, act, dtype, tile_cfg=cfg)
        _assert_close(outs[cfg], ref, dtype, f"tile_cfg {cfg}")
    _same_family_bits(outs)


@pytest.mark.parametrize("dtype", DTYPES)
def test_residual_may_alias_out(dtype):
    M, N, K = 300, 520, 64
    d = _with_residual(synth.draw(M, N, K, dtype, "relu", seed=2), dtype, seed=3)
    A, B, bias, R = (to_dev(d[k], dtype) for k in ("A", "B", "bias", "R"))
    say("R aliases out", dtype)
    fl.fused_linear(A, B, bias, act="relu", out=R, R=R)
    torch.cuda.synchronize()
    ref = oracle.fused_linear(d["A"], d["B"], d["bias"], act="relu", dtype=dtype, R=d["R"])
    _assert_close(to_host(R, dtype), ref, dtype, "R == out")


# -------------------------------------------------------- quantized output
# out_q = Q(scale * act(A@B + bias)) through fl_fused_linear_quant ("Triton:
# Fused Matmul + Bias + ReLU (Epilogue Fusion)", "Variants"): codes equal to
# the oracle's, except where the oracle's binary32 value sits within the
# fp32-summation error of a rounding boundary (then the neighbour is valid).

def _run_quant(d, act, dtype, qfmt, scale, **opts):
    M, K = d["A"].shape
    N = d["B"].shape[1]
    A, B, bias, Y = (to_dev(d[k], dtype) for k in ("A", "B", "bias", "Y"))
    buf = torch.full((M * N + GUARD_Q,), 0xA5, dtype=torch.uint8, device="cuda")
    out = buf[:M * N].view(M, N)
    fl.fused_linear_quant(A, B, bias, Y, act=act, scale=scale, qfmt=qfmt, out=out, **opts)
    torch.cuda.synchronize()
    assert bool((buf[M * N:] == 0xA5).all().item()), "write past the end of out"
    return out.cpu().numpy()


GUARD_Q = 1024


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("act", ["none", "relu", "glu"])
@pytest.mark.parametrize("qfmt", ["fp8_e4m3", "int8"])
@pytest.mark.parametrize("shape", [(1, 1, 1), (3, 17, 7), (67, 65, 70), (257, 264, 40), (513, 770, 33)])
def test_quant_integer_inputs_bit_exact(dtype, act, qfmt, shape):
    """Exact integers and a power-of-two scale: every intermediate is exact,
    codes must match bit for bit (this also fixes the fp8 format: OCP E4M3)."""
    M, N, K = shape
    d = synth.draw_integer(M, N, K, dtype, act, seed=M + 3 * N + 5 * K, amax=1, bias_max=3)
    scale = 0.25 if qfmt == "fp8_e4m3" else 8.0
    say("quant integer", dtype, act, qfmt, shape)
    got = _run_quant(d, act, dtype, qfmt, scale)
    ref = oracle.fused_linear_quant(d["A"], d["B"], d["bias"], d["Y"], act=act, dtype=dtype, qfmt=qfmt, scale=scale)
    assert np.array_equal(got, ref), (np.argwhere(got != ref)[:5], got[got != ref][:5], ref[got != ref][:5])


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("act", ["none", "relu", "gelu_tanh", "glu"])
@pytest.mark.parametrize("qfmt,scale", [("fp8_e4m3", 150.0), ("fp8_e4m3", 0.02), ("int8", 40.0)])
def test_quant_random_inputs(dtype, act, qfmt, scale):
    """Scale 150 sends part of the values past 448 (saturation), 0.02 into
    the fp8 subnormal range, 40 past the int8 range."""
    M, N, K = 300, 260, 1000
    d = synth.draw(M, N, K, dtype, act, seed=17)
    say("quant random", dtype, act, qfmt, scale)
    got = _run_quant(d, act, dtype, qfmt, scale)
    ref, u = oracle.fused_linear_quant(d["A"], d["B"], d["bias"], d["Y"], act=act, dtype=dtype, qfmt=qfmt,
                                       scale=scale, want_u=True)
    res = oracle.compare_quant(got, ref, u, qfmt)
    assert res["ok"], res
    assert res["accepted_near_boundary"] <= 0.01 * M * N, res


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("qfmt", ["fp8_e4m3", "int8"])
def test_quant_kernel_variants_identical(dtype, qfmt):
    M, N, K = 513, 770, 600
    d = synth.draw(M, N, K, dtype, "relu", seed=19)
    ref, u = oracle.fused_linear_quant(d["A"], d["B"], d["bias"], None, act="relu", dtype=dtype, qfmt=qfmt,
                                       scale=50.0, want_u=True)
    outs = {}
    for cfg in (0, 2, 5, 6, 7, 10, 11, 12, 15):
        say("quant variant", cfg, dtype, qfmt)
        outs[cfg] = _run_quant(d, "relu", dtype, qfmt, 50.0, tile_cfg=cfg)
        res = oracle.compare_quant(outs[cfg], ref, u, qfmt)
        assert res["ok"], (cfg, res)
    for cfg in (5, 6, 7):  # 32x32 blocks
        assert np.array_equal(outs[cfg], outs[2]), cfg
    for cfg in (11, 12, 15):  # 16x16 blocks
        assert np.array_equal(outs[cfg], outs[10]), cfg
    assert np.array_equal(outs[0], outs[10]) or np.array_equal(outs[0], outs[2])


def test_quant_full_size_whole_output():
    w = synth.WORKLOADS["gelu_fp8out_bf16_8192x14336x4096"]
    d = synth.draw_workload(w)
    say("full size", w.name)
    got = _run_quant(d, w.act, w.dtype, w.qfmt, w.scale)
    ref, u = oracle.fused_linear_quant(d["A"], d["B"], d["bias"], d["Y"], act=w.act, dtype=w.dtype, qfmt=w.qfmt,
                                       scale=w.scale, want_u=True)
    res = oracle.compare_quant(got, ref, u, w.qfmt)
    assert res["ok"], res


# ------------------------------------------------------------ FP8 operands
# out = act(ab_scale * (A8@B8) + bias) through fl_fused_linear_fp8 ("Optimizing
# GEMM + Activation on CDNA4 with TLX", "Future Work": the projection in FP8).

FP8_CODES = {-2: 0xC0, -1: 0xB8, 0: 0x00, 1: 0x38, 2: 0x40}  # exact small integers in OCP E4M3
FP8_CFGS = (0, 1, 2, 5, 6, 7, 12)  # automatic; 32x32x64 blocks (1, 2, 5, 6, 7); 16x16x128 blocks (12)


def _run_fp8(d, act, out_dtype, **opts):
    M, K = d["A8"].shape
    N = d["B8"].shape[1]
    A8, B8 = (torch.from_numpy(np.ascontiguousarray(d[k])).to("cuda") for k in ("A8", "B8"))
    bias, Y = to_dev(d["bias"], out_dtype), to_dev(d["Y"], out_dtype)
    out, buf = sentinel_out(M, N, out_dtype)
    fl.fused_linear_fp8(A8, B8, d["ab_scale"], bias, Y, act=act, out_dtype=TORCH_DT[out_dtype], out=out, **opts)
    torch.cuda.synchronize()
    assert guard_intact(buf, M, N), "write past the end of out"
    return to_host(out, out_dtype)


def _fp8_integer_inputs(M, N, K, out_dtype, act, seed):
    rng = np.random.default_rng(seed)
    lut = np.array([FP8_CODES[v] for v in (-2, -1, 0, 1, 2)], dtype=np.uint8)
    return {"A8": lut[rng.integers(0, 5, (M, K))], "B8": lut[rng.integers(0, 5, (K, N))], "ab_scale": 0.5,
            "bias": synth.to_storage(rng.integers(-4, 5, N).astype(np.float64), out_dtype),
            "Y": synth.to_storage(rng.integers(-1, 2, (M, N)).astype(np.float64), out_dtype) if act == "glu" else None}


@pytest.mark.parametrize("out_dtype", ["f16", "bf16"])
@pytest.mark.parametrize("act", ["none", "relu", "glu"])
@pytest.mark.parametrize("shape", [(1, 16, 16), (67, 48, 64), (257, 272, 128), (513, 784, 160), (300, 528, 1008)])
def test_fp8_integer_inputs_bit_exact(out_dtype, act, shape):
    """Small-integer E4M3 codes, a power-of-two scale: every product and sum is
    exact in fp32, so the output of every FP8 kernel (32x32x64 and 16x16x128
    blocks) must match bit for bit (this also pins the operand k-order and the
    transposed 8-bit reads)."""
    M, N, K = shape
    d = _fp8_integer_inputs(M, N, K, out_dtype, act, seed=M + N + K)
    ref = oracle.fused_linear_fp8(d["A8"], d["B8"], d["ab_scale"], d["bias"], d["Y"], act=act, out_dtype=out_dtype)
    for cfg in FP8_CFGS:
        say("fp8 integer", out_dtype, act, shape, "tile_cfg", cfg)
        out = _run_fp8(d, act, out_dtype, tile_cfg=cfg)
        bad = out.view(np.uint16) != ref.view(np.uint16)
        assert not bad.any(), (cfg, np.argwhere(bad)[:5], oracle.compare(out, ref, out_dtype))


@pytest.mark.parametrize("out_dtype", ["f16", "bf16"])
@pytest.mark.parametrize("act", ["relu", "glu"])
@pytest.mark.parametrize("shape", [(1, 3, 1), (7, 5, 2), (5, 17, 3), (67, 49, 65), (130, 131, 129), (257, 273, 131),
                                   (300, 530, 1009), (513, 259, 127), (769, 21, 255)])
def test_fp8_ragged_K_and_N_bit_exact(out_dtype, act, shape):
    """K and N that are not multiples of 16 (rows of A and B not whole 16-byte
    chunks, chunks that straddle rows, last dwords of A and B that run past
    the buffers' ends): the last three codes of A and of B are forced to
    nonzero values, so a code that the kernel reads as zero, or takes from
    the next row, changes the output."""
    M, N, K = shape
    d = _fp8_integer_inputs(M, N, K, out_dtype, act, seed=7 * M + N + K)
    A8, B8 = d["A8"].reshape(-1), d["B8"].reshape(-1)
    A8[-min(3, A8.size):] = FP8_CODES[1]
    B8[-min(3, B8.size):] = FP8_CODES[-2]
    ref = oracle.fused_linear_fp8(d["A8"], d["B8"], d["ab_scale"], d["bias"], d["Y"], act=act, out_dtype=out_dtype)
    for cfg in FP8_CFGS:
        say("fp8 ragged", out_dtype, act, shape, "tile_cfg", cfg)
        out = _run_fp8(d, act, out_dtype, tile_cfg=cfg)
        bad = out.view(np.uint16) != ref.view(np.uint16)
        assert not bad.any(), (cfg, np.argwhere(bad)[:5], oracle.compare(out, ref, out_dtype))


@pytest.mark.parametrize("K", [300, 1021])
def test_fp8_two_per_cu_automatic_choice(K):
    """Where the 256x128 grid fills two workgroups per CU and K is short, the
    automatic FP8 choice is the two-per-CU kernel (64-deep stages): integer
    codes, a ragged K, bit-exact against the oracle and bit-identical to
    tile_cfg 6 and to the one-per-CU 256x128 kernel."""
    M, N = 1024, 16384 + 37                      # 4 x 129 tiles of 256x128
    d = _fp8_integer_inputs(M, N, K, "f16", "glu", seed=K)
    ref = oracle.fused_linear_fp8(d["A8"], d["B8"], d["ab_scale"], d["bias"], d["Y"], act="glu", out_dtype="f16")
    outs = {}
    for cfg in (0, 6, 2):
        say("fp8 two per CU", K, "tile_cfg", cfg)
        outs[cfg] = _run_fp8(d, "glu", "f16", tile_cfg=cfg)
        bad = outs[cfg].view(np.uint16) != ref.view(np.uint16)
        assert not bad.any(), (cfg, np.argwhere(bad)[:5])


@pytest.mark.parametrize("cfg", [1, 2, 5, 6, 7, 12])
def test_fp8_debug_sync_gives_the_same_bits(cfg):
    """The FP8 kernels under the debugging schedule (an extra full wait for
    the copies and an extra barrier in every K stage), on a ragged shape
    whose last stage is fixed up: the same bits."""
    d = synth.draw_fp8(513, 781, 1001, "f16", "glu", seed=63)
    say("fp8 debug sync", cfg)
    fast = _run_fp8(d, "glu", "f16", tile_cfg=cfg)
    slow = _run_fp8(d, "glu", "f16", tile_cfg=cfg, debug_sync=1)
    assert np.array_equal(fast.view(np.uint16), slow.view(np.uint16))


@pytest.mark.parametrize("out_dtype", ["f16", "bf16"])
@pytest.mark.parametrize("act", ["relu", "gelu_tanh", "glu"])
def test_fp8_k0_and_empty(out_dtype, act):
    """K = 0 at 127 x 129: act(bias) on every row, from every FP8 kernel; M = 0
    or N = 0 launches nothing and writes nothing."""
    d = _fp8_integer_inputs(127, 129, 0, out_dtype, act, seed=3)
    ref = oracle.fused_linear_fp8(d["A8"], d["B8"], d["ab_scale"], d["bias"], d["Y"], act=act, out_dtype=out_dtype)
    for cfg in FP8_CFGS:
        say("fp8 K=0", out_dtype, act, "tile_cfg", cfg)
        out = _run_fp8(d, act, out_dtype, tile_cfg=cfg)
        _assert_close(out, ref, out_dtype, f"fp8 K=0 {act} tile_cfg {cfg}")
        if act == "relu":
            assert np.array_equal(out.view(np.uint16), ref.view(np.uint16)), cfg
    tdt = TORCH_DT[out_dtype]
    for M, N in ((0, 129), (127, 0)):
        A8 = torch.zeros((M, 64), dtype=torch.uint8, device="cuda")
        B8 = torch.zeros((64, N), dtype=torch.uint8, device="cuda")
        bias = torch.zeros((N,), dtype=tdt, device="cuda")
        Y = torch.zeros((M, N), dtype=tdt, device="cuda") if act == "glu" else None
        out = torch.full((M, N), 7.0, dtype=tdt, device="cuda")
        fl.fused_linear_fp8(A8, B8, 1.0, bias, Y, act=act, out_dtype=tdt, out=out)
        torch.cuda.synchronize()
        assert out.numel() == 0


@pytest.mark.parametrize("out_dtype", ["f16", "bf16"])
@pytest.mark.parametrize("act", ["none", "relu", "gelu_tanh", "glu"])
@pytest.mark.parametrize("shape", [(300, 528, 1008), (513, 272, 4096), (257, 1000, 1001)])
def test_fp8_random_inputs_within_tolerance(out_dtype, act, shape):
    M, N, K = shape
    d = synth.draw_fp8(M, N, K, out_dtype, act, seed=23)
    say("fp8 random", out_dtype, act, shape)
    out = _run_fp8(d, act, out_dtype)
    ref = oracle.fused_linear_fp8(d["A8"], d["B8"], d["ab_scale"], d["bias"], d["Y"], act=act, out_dtype=out_dtype)
    _assert_close(out, ref, out_dtype, f"fp8 {out_dtype} {act} {shape}")


@pytest.mark.parametrize("out_dtype", ["f16", "bf16"])
def test_fp8_kernel_variants_bit_identical(out_dtype):
    """Random inputs: the kernels of one MFMA family give the same bits, and
    every one is within tolerance of the oracle."""
    d = synth.draw_fp8(513, 784, 1024, out_dtype, "relu", seed=24)
    ref = oracle.fused_linear_fp8(d["A8"], d["B8"], d["ab_scale"], d["bias"], d["Y"], act="relu", out_dtype=out_dtype)
    outs = {}
    for cfg in FP8_CFGS:
        say("fp8 variant", cfg, out_dtype)
        outs[cfg] = _run_fp8(d, "relu", out_dtype, tile_cfg=cfg)
        _assert_close(outs[cfg], ref, out_dtype, f"fp8 tile_cfg {cfg}")
    _same_family_bits(outs)


@pytest.mark.parametrize("name", ["glu_fp8in_f16_1024x21568x4096", "relu_fp8in_f16_4096x4096x4096"])
def test_fp8_full_size_whole_output(name):
    w = synth.WORKLOADS[name]
    d = synth.draw_workload(w)
    say("full size", name)
    out = _run_fp8(d, w.act, w.dtype)
    assert not np.isnan(oracle.decode(out, w.dtype)).any(), "unwritten (NaN sentinel) outputs"
    ref = oracle.fused_linear_fp8(d["A8"], d["B8"], d["ab_scale"], d["bias"], d["Y"], act=w.act, out_dtype=w.dtype)
    _assert_close(out, ref, w.dtype, name)


# ------------------------------------------------------ backward epilogue
# D = G @ W^T (W (N,K) read as its transpose), dX = D * act'(X), the gate's
# dY = D * X, dbias = column sums of dX ("Optimizing GEMM + Activation on
# CDNA4 with TLX", "Future Work").

BWD_DTYPES = ["f16", "bf16"]


def _run_bwd(d, act, dtype, with_dbias=True, **opts):
    M, K = d["G"].shape
    N = d["W"].shape[0]
    G, W, X, Y = (to_dev(d[k], dtype) for k in ("G", "W", "X", "Y"))
    dX, bufx = sentinel_out(M, N, dtype)
    dY, bufy = sentinel_out(M, N, dtype) if act == "glu" else (None, None)
    dbias = torch.full((N + 64,), float("nan"), dtype=torch.float32, device="cuda") if with_dbias else None
    fl.fused_linear_bwd(G, W, X, Y, act=act, dX=dX, dY=dY, dbias=dbias[:N] if with_dbias else None, **opts)
    torch.cuda.synchronize()
    assert guard_intact(bufx, M, N), "write past the end of dX"
    if dY is not None:
        assert guard_intact(bufy, M, N), "write past the end of dY"
    if with_dbias:
        assert bool(torch.isnan(dbias[N:]).all().item()), "write past the end of dbias"
    return (to_host(dX, dtype), None if dY is None else to_host(dY, dtype),
            dbias[:N].cpu().numpy().astype(np.float64) if with_dbias else None)


@pytest.mark.parametrize("dtype", BWD_DTYPES)
@pytest.mark.parametrize("act", ["none", "relu", "glu"])
@pytest.mark.parametrize("shape", [(1, 1, 1), (3, 17, 7), (67, 65, 8), (257, 264, 5), (513, 770, 3)])
def test_bwd_integer_inputs_bit_exact(dtype, act, shape):
    """Small integers: every value exact, so dX, dY and dbias must equal the
    oracle's bits (dbias: exact integer sums in fp32)."""
    M, N, K = shape
    d = synth.draw_bwd_integer(M, N, K, dtype, act, seed=M + 3 * N + 7 * K)
    say("bwd integer", dtype, act, shape)
    dX, dY, db = _run_bwd(d, act, dtype)
    rX, rY, rdb = oracle.fused_linear_bwd(d["G"], d["W"], d["X"], d["Y"], act=act, dtype=dtype)
    assert np.array_equal(dX.view(np.uint8), rX.view(np.uint8)), oracle.compare(dX, rX, dtype)
    if act == "glu":
        assert np.array_equal(dY.view(np.uint8), rY.view(np.uint8))
    assert np.array_equal(db, rdb)


def test_bwd_integer_longer_k_f16():
    """K = 70 (a ragged last K stage) stays exact in fp16."""
    M, N, K = 130, 200, 70
    for act in ("relu", "glu"):
        d = synth.draw_bwd_integer(M, N, K, "f16", act, seed=41)
        say("bwd integer K=70", act)
        dX, dY, db = _run_bwd(d, act, "f16")
        rX, rY, rdb = oracle.fused_linear_bwd(d["G"], d["W"], d["X"], d["Y"], act=act, dtype="f16")
        assert np.array_equal(dX.view(np.uint8), rX.view(np.uint8))
        assert np.array_equal(db, rdb)
        if act == "glu":
            assert np.array_equal(dY.view(np.uint8), rY.view(np.uint8))


def _check_bwd(dX, dY, db, d, act, dtype, what):
    M = d["G"].shape[0]
    rX, rY, rdb, rdx = oracle.fused_linear_bwd(d["G"], d["W"], d["X"], d["Y"], act=act, dtype=dtype, want_dx=True)
    _assert_close(dX, rX, dtype, what + " dX")
    if act == "glu":
        _assert_close(dY, rY, dtype, what + " dY")
    if db is not None:
        res = oracle.compare_dbias(db, rdb, np.abs(rdx).sum(axis=0), M)
        assert res["ok"], f"{what} dbias: {res}"


@pytest.mark.parametrize("dtype", BWD_DTYPES)
@pytest.mark.parametrize("act", ["none", "relu", "gelu_tanh", "glu"])
@pytest.mark.parametrize("shape", [(127, 129, 96), (300, 260, 1000), (513, 264, 72), (256, 512, 33)])
def test_bwd_random_within_tolerance(dtype, act, shape):
    M, N, K = shape
    d = synth.draw_bwd(M, N, K, dtype, act, seed=13)
    say("bwd random", dtype, act, shape)
    dX, dY, db = _run_bwd(d, act, dtype)
    _check_bwd(dX, dY, db, d, act, dtype, f"bwd {dtype} {act} {shape}")


@pytest.mark.parametrize("dtype", BWD_DTYPES)
@pytest.mark.parametrize("act", ["relu", "glu"])
def test_bwd_variants_and_tile_orders_agree(dtype, act):
    """The 8-wave 256x256 and the 256x128 kernels of one MFMA shape (32x32 or
    16x16 blocks), and the tile orders, give bit-identical dX and dY; dbias
    (fp32 atomics) agrees within tolerance; every variant passes the oracle
    check."""
    M, N, K = 600, 520, 300
    d = synth.draw_bwd(M, N, K, dtype, act, seed=17)
    for fam in ((5, 2), (10, 12)):
        outs = []
        for opts in [dict(tile_cfg=fam[0]), dict(tile_cfg=fam[1]), dict(tile_cfg=fam[0], group_m=1, persistent=1),
                     dict(tile_cfg=fam[1], no_xcd_remap=1)]:
            say("bwd variant", dtype, act, opts)
            outs.append(_run_bwd(d, act, dtype, **opts))
            _check_bwd(*outs[-1], d, act, dtype, f"bwd {opts}")
        for o in outs[1:]:
            assert np.array_equal(o[0].view(np.uint8), outs[0][0].view(np.uint8))
            if act == "glu":
                assert np.array_equal(o[1].view(np.uint8), outs[0][1].view(np.uint8))


def test_bwd_aliases_and_no_dbias():
    """dX may overwrite X and dY may overwrite Y; dbias may be omitted."""
    M, N, K = 300, 520, 64
    d = synth.draw_bwd(M, N, K, "f16", "glu", seed=19)
    G, W, X, Y = (to_dev(d[k], "f16") for k in ("G", "W", "X", "Y"))
    say("bwd aliases")
    dX, dY, db = fl.fused_linear_bwd(G, W, X, Y, act="glu", dX=X, dY=Y, dbias=None)
    torch.cuda.synchronize()
    assert db is None and dX.data_ptr() == X.data_ptr() and dY.data_ptr() == Y.data_ptr()
    _check_bwd(to_host(X, "f16"), to_host(Y, "f16"), None, d, "glu", "f16", "aliased")


@pytest.mark.parametrize("dtype", BWD_DTYPES)
def test_bwd_degenerate_sizes(dtype):
    """K = 0 gives zero gradients; M = 0 leaves a zeroed dbias."""
    d = synth.draw_bwd(70, 90, 0, dtype, "relu", seed=23)
    say("bwd K=0", dtype)
    dX, _, db = _run_bwd(d, "relu", dtype)
    assert not oracle.decode(dX, dtype).any() and not db.any()
    G = torch.empty((0, 16), dtype=TORCH_DT[dtype], device="cuda")
    W = torch.zeros((40, 16), dtype=TORCH_DT[dtype], device="cuda")
    X = torch.empty((0, 40), dtype=TORCH_DT[dtype], device="cuda")
    dbias = torch.full((40,), 7.0, dtype=torch.float32, device="cuda")
    fl.fused_linear_bwd(G, W, X, act="relu", dbias=dbias)
    torch.cuda.synchronize()
    assert not dbias.any().item()


@pytest.mark.parametrize("name", ["gelu_bwd_bf16_8192x14336x4096", "glu_bwd_f16_1024x21568x4096"])
def test_bwd_full_size(name):
    """The benchmarked launch: the whole dX (and dY) against the oracle, and
    dbias of every column against the oracle's exact column sums over all
    rows."""
    w = synth.WORKLOADS[name]
    d = synth.draw_workload(w)
    say("bwd full size", name)
    dX, dY, db = _run_bwd(d, w.act, w.dtype)
    assert not np.isnan(oracle.decode(dX, w.dtype)).any()
    rX, rY, rdb, rdx = oracle.fused_linear_bwd(d["G"], d["W"], d["X"], d["Y"], act=w.act, dtype=w.dtype,
                                               want_dx=True)
    _assert_close(dX, rX, w.dtype, name + " dX")
    if w.act == "glu":
        _assert_close(dY, rY, w.dtype, name + " dY")
    res = oracle.compare_dbias(db, rdb, np.abs(rdx).sum(axis=0), w.M)
    assert res["ok"], res
    say("bwd full size, workspace entry", name)
    wX, wY, wdb = _run_bwd(d, w.act, w.dtype, workspace=True)
    assert np.array_equal(wX.view(np.uint8), dX.view(np.uint8))
    if w.act == "glu":
        assert np.array_equal(wY.view(np.uint8), dY.view(np.uint8))
    res = oracle.compare_dbias(wdb, rdb, np.abs(rdx).sum(axis=0), w.M)
    assert res["ok"], res


@pytest.mark.parametrize("dtype", BWD_DTYPES)
@pytest.mark.parametrize("act", ["none", "relu", "gelu_tanh", "glu"])
def test_bwd_ws_dbias_reproducible_and_order_free(dtype, act):
    """fl_fused_linear_bwd_ws: dbias is the same to the bit over repeated
    calls, tile orders (band height, persistent grid, XCD step) and the two
    widths of one MFMA shape; dX and dY equal the plain entry point's bits;
    dbias passes the oracle check."""
    M, N, K = 1100, 700, 300   # 5 tile rows (the last one short), ragged N
    d = synth.draw_bwd(M, N, K, dtype, act, seed=23)
    for fam in ((10, 12), (5, 2)):
        ref = None
        for opts in [dict(tile_cfg=fam[0]), dict(tile_cfg=fam[0]), dict(tile_cfg=fam[1]),
                     dict(tile_cfg=fam[0], group_m=1, persistent=1), dict(tile_cfg=fam[1], group_m=8, no_xcd_remap=1)]:
            say("bwd workspace", dtype, act, opts)
            got = _run_bwd(d, act, dtype, workspace=True, **opts)
            _check_bwd(*got, d, act, dtype, f"bwd workspace {opts}")
            plain = _run_bwd(d, act, dtype, **opts)
            assert np.array_equal(got[0].view(np.uint8), plain[0].view(np.uint8)), opts
            if act == "glu":
                assert np.array_equal(got[1].view(np.uint8), plain[1].view(np.uint8)), opts
            if ref is None:
                ref = got[2]
            assert np.array_equal(got[2].view(np.uint32), ref.view(np.uint32)), (opts, np.abs(got[2] - ref).max())


@pytest.mark.parametrize("dtype", BWD_DTYPES)
@pytest.mark.parametrize("shape", [(1, 1, 1), (3, 17, 7), (257, 264, 5), (513, 770, 3), (600, 300, 64)])
def test_bwd_ws_integer_inputs_bit_exact(dtype, shape):
    """Integer inputs: dbias from the workspace entry equals the oracle's
    exact column sums; a workspace larger than needed and a second, smaller
    call on the same workspace change nothing."""
    M, N, K = shape
    d = synth.draw_bwd_integer(M, N, K, dtype, "glu", seed=M + N + K)
    rX, rY, rdb = oracle.fused_linear_bwd(d["G"], d["W"], d["X"], d["Y"], act="glu", dtype=dtype)
    ws = torch.full((fl.bwd_workspace_bytes(M, N, K, TORCH_DT[dtype]) + 4096,), 0x7F, dtype=torch.uint8,
                    device="cuda")
    for _ in range(2):
        say("bwd workspace integer", dtype, shape)
        dX, dY, db = _run_bwd(d, "glu", dtype, workspace=ws)
        assert np.array_equal(dX.view(np.uint8), rX.view(np.uint8))
        assert np.array_equal(dY.view(np.uint8), rY.view(np.uint8))
        assert np.array_equal(db, rdb)
    small = synth.draw_bwd_integer(5, 9, 3, dtype, "glu", seed=1)
    sX, sY, sdb = oracle.fused_linear_bwd(small["G"], small["W"], small["X"], small["Y"], act="glu", dtype=dtype)
    dX, dY, db = _run_bwd(small, "glu", dtype, workspace=ws)
    assert np.array_equal(db, sdb) and np.array_equal(dX.view(np.uint8), sX.view(np.uint8))


@pytest.mark.parametrize("dtype", BWD_DTYPES)
@pytest.mark.parametrize("act", ["relu", "gelu_tanh", "glu"])
@pytest.mark.parametrize("shape", [(200, 264, 136), (131, 77, 45)])
def test_bwd_unfused_chain_matches_oracle_chain(dtype, act, shape):
    """fl_gemm_nt, fl_activation_grad and fl_column_sum, each storing its
    result, against the oracle's chain that rounds after every stage."""
    M, N, K = shape
    d = synth.draw_bwd(M, N, K, dtype, act, seed=29)
    G, W, X, Y = (to_dev(d[k], dtype) for k in ("G", "W", "X", "Y"))
    say("bwd unfused chain", dtype, act, shape)
    D = fl.gemm_nt(G, W)
    dX, dY = fl.activation_grad(D, X, Y, act=act)
    db = fl.column_sum(dX)
    torch.cuda.synchronize()
    rX, rY, rdb, rdx = oracle.unfused_bwd_chain(d["G"], d["W"], d["X"], d["Y"], act=act, dtype=dtype, want_dx=True)
    _assert_close(to_host(dX, dtype), rX, dtype, "chain dX")
    if act == "glu":
        _assert_close(to_host(dY, dtype), rY, dtype, "chain dY")
    # the column sums are of the device's own stored dX: compare with the
    # FP64 sums of those values (the reduction alone), and with the oracle
    dev_dx = oracle.decode(to_host(dX, dtype), dtype)
    res = oracle.compare_dbias(db.cpu().numpy(), dev_dx.sum(axis=0), np.abs(dev_dx).sum(axis=0), M)
    assert res["ok"], res
    res = oracle.compare_dbias(db.cpu().numpy(), rdb, np.abs(rdx).sum(axis=0) + np.abs(dev_dx).sum(axis=0), M)
    assert res["ok"], res


@pytest.mark.parametrize("dtype", BWD_DTYPES)
def test_bwd_unfused_chain_integer_equals_fused(dtype):
    """Exact values: the chain and the fused kernel give the same bits, and
    D may be overwritten in place by dX."""
    M, N, K = 257, 264, 5
    d = synth.draw_bwd_integer(M, N, K, dtype, "glu", seed=31)
    G, W, X, Y = (to_dev(d[k], dtype) for k in ("G", "W", "X", "Y"))
    say("bwd unfused integer", dtype)
    D = fl.gemm_nt(G, W)
    dX, dY = fl.activation_grad(D, X, Y, act="glu", dX=D)
    db = fl.column_sum(dX)
    fX, fY, fdb = fl.fused_linear_bwd(G, W, X, Y, act="glu")
    torch.cuda.synchronize()
    assert dX.data_ptr() == D.data_ptr()
    assert np.array_equal(to_host(dX, dtype).view(np.uint8), to_host(fX, dtype).view(np.uint8))
    assert np.array_equal(to_host(dY, dtype).view(np.uint8), to_host(fY, dtype).view(np.uint8))
    assert np.array_equal(db.cpu().numpy(), fdb.cpu().numpy())


# ------------------------------------------- epilogue side input: two paths
# With N a multiple of 8 the epilogue's side input (the gate's Y, else the
# residual or the saved X) is copied into LDS before the epilogue; otherwise
# it is loaded into registers.  One extra column (N = 521 against 520) moves
# the same problem onto the other path without changing the arithmetic of
# the first 520 columns, so those must agree bit for bit.

def _first_cols(d, n, keys_cols, keys_rows=()):
    e = dict(d)
    for k in keys_cols:
        if e.get(k) is not None:
            e[k] = np.ascontiguousarray(e[k][..., :n])
    for k in keys_rows:
        if e.get(k) is not None:
            e[k] = np.ascontiguousarray(e[k][:n])
    return e


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("act,residual", [("glu", False), ("relu", True), ("gelu_tanh", True), ("glu", True)])
@pytest.mark.parametrize("cfg", [0, 5, 6, 7, 10, 11, 13, 14, 15])
def test_side_input_paths_bit_identical(dtype, act, residual, cfg):
    M, K = 300, 200
    d = synth.draw(M, 521, K, dtype, act, seed=43)
    if residual:
        d = _with_residual(d, dtype, seed=44)
    d520 = _first_cols(d, 520, ("B", "bias", "Y", "R"))
    say("side input paths", dtype, act, residual, cfg)
    wide = _run_fused(d, act, dtype, tile_cfg=cfg)
    narrow = _run_fused(d520, act, dtype, tile_cfg=cfg)
    ref = oracle.fused_linear(d520["A"], d520["B"], d520["bias"], d520["Y"], act=act, dtype=dtype, R=d520.get("R"))
    _assert_close(narrow, ref, dtype, "N = 520")
    assert np.array_equal(narrow.view(np.uint8), np.ascontiguousarray(wide[:, :520]).view(np.uint8))


@pytest.mark.parametrize("dtype", BWD_DTYPES)
@pytest.mark.parametrize("act", ["relu", "gelu_tanh", "glu"])
@pytest.mark.parametrize("cfg", [5, 2, 10, 12])
def test_bwd_side_input_paths_bit_identical(dtype, act, cfg):
    M, K = 300, 200
    d = synth.draw_bwd(M, 521, K, dtype, act, seed=47)
    d520 = _first_cols(d, 520, ("X", "Y"), ("W",))
    say("bwd side input paths", dtype, act, cfg)
    wX, wY, wdb = _run_bwd(d, act, dtype, tile_cfg=cfg)
    nX, nY, ndb = _run_bwd(d520, act, dtype, tile_cfg=cfg)
    _check_bwd(nX, nY, ndb, d520, act, dtype, "N = 520")
    assert np.array_equal(nX.view(np.uint8), np.ascontiguousarray(wX[:, :520]).view(np.uint8))
    if act == "glu":
        assert np.array_equal(nY.view(np.uint8), np.ascontiguousarray(wY[:, :520]).view(np.uint8))
    _, _, rdb, rdx = oracle.fused_linear_bwd(d520["G"], d520["W"], d520["X"], d520["Y"], act=act, dtype=dtype,
                                             want_dx=True)
    res = oracle.compare_dbias(wdb[:520], rdb, np.abs(rdx).sum(axis=0), M)
    assert res["ok"], res


# ------------------------------------------ the one rounding, bit for bit
# At K = 1 the accumulator is the exact product a*b (two 16-bit values, 22
# significant bits at most), so x = a*b + bias is one fp32 addition that
# numpy's float32 arithmetic reproduces exactly, and the stored output must
# be the round-to-nearest-even of act(x) in the output type: the paired
# conversions of the direct kernels and the single ones of the
# register-staged kernel alike.  Half the rows and columns are scaled down
# so that fp16 results also fall among the subnormals.

def _rne_bf16_bits(x32):
    u = x32.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("act", ["none", "relu"])
@pytest.mark.parametrize("N", [520, 521])
@pytest.mark.parametrize("cfg", [0, 3, 5, 6, 7, 9, 10, 11, 12, 13, 14, 15])
def test_k1_output_rounding_bit_exact(dtype, act, N, cfg):
    M = 300
    rng = np.random.default_rng(N + 7 * cfg)
    a = rng.standard_normal((M, 1)); a[M // 2:] *= 1e-2
    b = rng.standard_normal((1, N)); b[:, N // 2:] *= 1e-2
    bias = rng.standard_normal(N); bias[N // 2:] *= 1e-5
    d = {"A": synth.to_storage(a, dtype), "B": synth.to_storage(b, dtype), "bias": synth.to_storage(bias, dtype),
         "Y": None}
    say("K=1 rounding", dtype, act, N, cfg)
    out = _run_fused(d, act, dtype, tile_cfg=cfg)

    def f32(raw):
        return raw.astype(np.float32) if dtype == "f16" else (raw.astype(np.uint32) << 16).view(np.float32)
    x = f32(d["A"]) * f32(d["B"]) + f32(d["bias"])[None, :]  # one fp32 multiply (exact) and one fp32 add
    if act == "relu":
        x = np.where(x > 0, x, np.float32(0.0))
    ref = x.astype(np.float16).view(np.uint16) if dtype == "f16" else _rne_bf16_bits(x)
    got = out.view(np.uint16)
    nz = x != 0  # the sign of a zero result is not part of the contract
    assert np.array_equal(got[nz], ref[nz]), f"{np.count_nonzero(got[nz] != ref[nz])} outputs differ"
    if dtype == "f16":
        sub = (np.abs(x) < 6.1e-5) & nz
        assert sub.sum() > 1000, "the case must reach fp16 subnormals"


def _shifted(t):
    """A copy of t at an address one element past a 16-byte boundary."""
    s = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)[1:].view(t.shape)
    s.copy_(t)
    return s


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_side_input_unaligned_bit_identical(dtype):
    """Y, R, the saved X and the outputs one element off 16-byte alignment
    (N = 520: the side input goes through LDS in 16-byte copies at those
    addresses) give the aligned run's bits."""
    M, N, K = 300, 520, 200
    d = _with_residual(synth.draw(M, N, K, dtype, "glu", seed=91), dtype, seed=92)
    A, B, bias, Y, R = (to_dev(d[k], dtype) for k in ("A", "B", "bias", "Y", "R"))
    say("unaligned side inputs, forward", dtype)
    for act, kw in (("glu", {}), ("relu", {"R": R}), ("glu", {"R": R})):
        y = Y if act == "glu" else None
        ref = fl.fused_linear(A, B, bias, y, act=act, **kw)
        kw2 = {"R": _shifted(R)} if "R" in kw else {}
        out2 = _shifted(torch.empty_like(ref))
        got = fl.fused_linear(A, B, bias, _shifted(Y) if y is not None else None, act=act, out=out2, **kw2)
        torch.cuda.synchronize()
        assert np.array_equal(to_host(got, dtype).view(np.uint16), to_host(ref, dtype).view(np.uint16)), act
    b = synth.draw_bwd(M, N, K, dtype, "glu", seed=93)
    G, W, X, Yb = (to_dev(b[k], dtype) for k in ("G", "W", "X", "Y"))
    say("unaligned side inputs, backward", dtype)
    for act in ("relu", "glu"):
        y = Yb if act == "glu" else None
        rX, rY, _ = fl.fused_linear_bwd(G, W, X, y, act=act, dbias=None)
        dX2 = _shifted(torch.empty_like(rX))
        dY2 = _shifted(torch.empty_like(rX)) if act == "glu" else None
        gX, gY, _ = fl.fused_linear_bwd(G, W, _shifted(X), _shifted(y) if y is not None else None, act=act,
                                        dX=dX2, dY=dY2, dbias=None)
        torch.cuda.synchronize()
        assert np.array_equal(to_host(gX, dtype).view(np.uint16), to_host(rX, dtype).view(np.uint16)), act
        if act == "glu":
            assert np.array_equal(to_host(gY, dtype).view(np.uint16), to_host(rY, dtype).view(np.uint16))


# ------------------------------ seeded random shapes, the other entry points

QUANT_CFGS = (0, 2, 5, 6, 7, 10, 11, 12, 15)
BWD_CFGS = (0, 2, 5, 10, 12)


@pytest.mark.parametrize("seed", range(8))
def test_seeded_random_shapes_fp8_quant_bwd(seed):
    """Seeded random ragged shapes (M, K up to 700, N from 3) through the
    FP8-operand, quantized-output and backward entry points, each through
    the automatic choice and one random kernel variant of its own list.
    Small-integer inputs keep every fp32 sum exact, so the whole output (and
    dbias) must equal the oracle's bits whatever the kernel's order of
    summation."""
    rng = np.random.default_rng(3000 + seed)
    for case in range(6):
        M, N, K = int(rng.integers(1, 700)), int(rng.integers(3, 700)), int(rng.integers(1, 700))
        dtype = ["f16", "bf16"][int(rng.integers(0, 2))]
        act = ["none", "relu", "glu"][int(rng.integers(0, 3))]
        s = 100 * seed + case
        kind = ("fp8", "quant", "bwd")[case % 3]
        if kind == "fp8":
            cfg = FP8_CFGS[int(rng.integers(1, len(FP8_CFGS)))]
            d = _fp8_integer_inputs(M, N, K, dtype, act, seed=s)
            ref = oracle.fused_linear_fp8(d["A8"], d["B8"], d["ab_scale"], d["bias"], d["Y"], act=act,
                                          out_dtype=dtype)
            for c in (0, cfg):
                say("random fp8", seed, case, M, N, K, dtype, act, "tile_cfg", c)
                out = _run_fp8(d, act, dtype, tile_cfg=c)
                bad = out.view(np.uint16) != ref.view(np.uint16)
                assert not bad.any(), (M, N, K, dtype, act, c, np.argwhere(bad)[:5])
        elif kind == "quant":
            cfg = QUANT_CFGS[int(rng.integers(1, len(QUANT_CFGS)))]
            qfmt = ["fp8_e4m3", "int8"][int(rng.integers(0, 2))]
            scale = 0.25 if qfmt == "fp8_e4m3" else 8.0
            d = synth.draw_integer(M, N, K, dtype, act, seed=s, amax=1, bias_max=3)
            ref = oracle.fused_linear_quant(d["A"], d["B"], d["bias"], d["Y"], act=act, dtype=dtype, qfmt=qfmt,
                                            scale=scale)
            for c in (0, cfg):
                say("random quant", seed, case, M, N, K, dtype, act, qfmt, "tile_cfg", c)
                got = _run_quant(d, act, dtype, qfmt, scale, tile_cfg=c)
                assert np.array_equal(got, ref), (M, N, K, dtype, act, qfmt, c, np.argwhere(got != ref)[:5])
        else:
            cfg = BWD_CFGS[int(rng.integers(1, len(BWD_CFGS)))]
            d = synth.draw_bwd_integer(M, N, K, dtype, act, seed=s)
            rX, rY, rdb = oracle.fused_linear_bwd(d["G"], d["W"], d["X"], d["Y"], act=act, dtype=dtype)
            for c in (0, cfg):
                say("random bwd", seed, case, M, N, K, dtype, act, "tile_cfg", c)
                dX, dY, db = _run_bwd(d, act, dtype, tile_cfg=c)
                assert np.array_equal(dX.view(np.uint8), rX.view(np.uint8)), (M, N, K, dtype, act, c)
                if act == "glu":
                    assert np.array_equal(dY.view(np.uint8), rY.view(np.uint8)), (M, N, K, dtype, act, c)
                assert np.array_equal(db, rdb), (M, N, K, dtype, act, c)
