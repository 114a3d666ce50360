"""activation_epilogue_amd -- gfx950 fused linear layer, out = act(A@B + bias).

Thin ctypes binding over ``libfused_linear.so`` (C ABI in
``include/fused_linear.h``).  This module only marshals arguments: it checks
tensor shapes, dtypes and devices, takes raw device pointers and the current
HIP stream from PyTorch, and calls the library.  Every step of the computation
runs in the library's HIP kernels; there is no fallback.  If the library has
not been built, importing works but every call raises ``LibraryNotBuilt``.

Entry points (same names as the C ABI, without the ``fl_`` prefix):
  fused_linear(A, B, bias=None, Y=None, act="relu", out=None, R=None, **options)
                                          # R: residual -> fl_fused_linear_residual
  fused_linear_quant(A, B, bias=None, Y=None, act="relu", scale=1.0, qfmt="fp8_e4m3", out=None, **options)
                                          # uint8 codes of Q(scale * act(A@B + bias))
  fused_linear_fp8(A8, B8, ab_scale, bias=None, Y=None, act="relu", out_dtype=torch.float16, out=None, **options)
                                          # FP8 E4M3 operands, 16-bit epilogue and output
  fused_linear_bwd(G, W, X, Y=None, act="relu", dX=None, dY=None, dbias=True, **options)
                                          # backward epilogue: dX = (G @ W^T) * act'(X), gate dY, dbias
  gemm_nt(A, Bt, D=None), activation_grad(D, X, Y=None, act=, dX=None, dY=None), column_sum(X, sums=None)
                                          # the unfused backward chain
  gemm(A, B, X=None)                      # unfused step 1: X = A@B
  bias_add(X, bias)                       # unfused step 2: X += bias (in place)
  activation(X, Y=None, out=None, act=)   # unfused step 3: out = act(X[, Y])
  tile_grid(M, N, K, dtype, **options), tile_of_program(...), version()
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libfused_linear.so")

ACTS = {"none": 0, "relu": 1, "gelu_tanh": 2, "glu": 3}
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "launch failed"}
EXPORTS = ("fl_fused_linear", "fl_fused_linear_ex", "fl_fused_linear_residual", "fl_fused_linear_quant",
           "fl_fused_linear_fp8", "fl_fused_linear_bwd", "fl_fused_linear_bwd_ws", "fl_bwd_workspace_bytes",
           "fl_fused_linear_bwd_noalloc",
           "fl_gemm", "fl_gemm_nt", "fl_activation_grad",
           "fl_column_sum", "fl_bias_add", "fl_activation",
           "fl_tile_grid", "fl_tile_of_program", "fl_status_string", "fl_last_error", "fl_version")


class LibraryNotBuilt(RuntimeError):
    pass


class FusedLinearError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class Options(ctypes.Structure):
    """Mirror of fl_options."""
    _fields_ = [("group_m", ctypes.c_int32), ("persistent", ctypes.c_int32), ("tile_cfg", ctypes.c_int32),
                ("no_xcd_remap", ctypes.c_int32), ("debug_tile_count", ctypes.c_void_p),
                ("debug_sync", ctypes.c_int32)]


_lib = None


def load_library():
    """Load (once) and return the ctypes handle of libfused_linear.so."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise LibraryNotBuilt(f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`"
                              " or `python activation_epilogue_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, c_int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int
    P_i32 = ctypes.POINTER(ctypes.c_int32)
    lib.fl_fused_linear.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, c_int, c_int, vp]
    lib.fl_fused_linear_ex.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, c_int, c_int, vp, ctypes.POINTER(Options)]
    lib.fl_fused_linear_residual.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, c_int, c_int, vp,
                                             ctypes.POINTER(Options)]
    lib.fl_fused_linear_quant.argtypes = [vp, vp, vp, vp, vp, ctypes.c_float, i64, i64, i64, c_int, c_int, c_int, vp,
                                          ctypes.POINTER(Options)]
    lib.fl_fused_linear_fp8.argtypes = [vp, vp, ctypes.c_float, vp, vp, vp, i64, i64, i64, c_int, c_int, vp,
                                        ctypes.POINTER(Options)]
    lib.fl_fused_linear_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, c_int, c_int, vp,
                                        ctypes.POINTER(Options)]
    lib.fl_fused_linear_bwd_ws.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, c_int, c_int, vp,
                                           ctypes.POINTER(Options), vp, ctypes.c_size_t]
    lib.fl_bwd_workspace_bytes.argtypes = [i64, i64, i64, c_int, ctypes.POINTER(ctypes.c_size_t)]
    lib.fl_fused_linear_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, c_int, c_int, vp,
                                                ctypes.POINTER(Options)]
    lib.fl_gemm.argtypes = [vp, vp, vp, i64, i64, i64, c_int, vp]
    lib.fl_gemm_nt.argtypes = [vp, vp, vp, i64, i64, i64, c_int, vp]
    lib.fl_activation_grad.argtypes = [vp, vp, vp, vp, vp, i64, i64, c_int, c_int, vp]
    lib.fl_column_sum.argtypes = [vp, vp, i64, i64, c_int, vp]
    lib.fl_bias_add.argtypes = [vp, vp, i64, i64, c_int, vp]
    lib.fl_activation.argtypes = [vp, vp, vp, i64, i64, c_int, c_int, vp]
    lib.fl_tile_grid.argtypes = [i64, i64, i64, c_int, ctypes.POINTER(Options), P_i32, P_i32, P_i32, P_i32]
    lib.fl_tile_of_program.argtypes = [i32, i32, i32, i32, i32, i32, P_i32, P_i32]
    for f in ("fl_fused_linear", "fl_fused_linear_ex", "fl_fused_linear_residual", "fl_fused_linear_quant",
              "fl_fused_linear_fp8", "fl_gemm", "fl_bias_add", "fl_activation", "fl_tile_grid", "fl_tile_of_program"):
        getattr(lib, f).restype = c_int
    lib.fl_status_string.argtypes = [c_int]
    lib.fl_status_string.restype = ctypes.c_char_p
    lib.fl_last_error.restype = ctypes.c_char_p
    lib.fl_version.restype = c_int
    _lib = lib
    return lib


def _check(status):
    if status != 0:
        raise FusedLinearError(status, load_library().fl_last_error().decode())


def _dtype_code(dtype):
    import torch
    codes = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
    if dtype not in codes:
        raise TypeError(f"unsupported dtype {dtype}; use float32, float16 or bfloat16")
    return codes[dtype]


def _dev_ptr(t, name, dtype=None, shape=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (row-major)")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr() or None


def _stream(t, stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(s.cuda_stream)


def _options(group_m=0, persistent=0, tile_cfg=0, no_xcd_remap=0, debug_tile_count=None, debug_sync=0):
    ptr = None
    if debug_tile_count is not None:
        import torch
        if debug_tile_count.dtype != torch.int32 or not debug_tile_count.is_cuda:
            raise TypeError("debug_tile_count must be an int32 device tensor")
        ptr = debug_tile_count.data_ptr()
    return Options(int(group_m), int(persistent), int(tile_cfg), int(no_xcd_remap), ptr, int(debug_sync))


def fused_linear(A, B, bias=None, Y=None, act="relu", out=None, *, R=None, stream=None, **options):
    """out = act(A@B + bias [+ R]) in one kernel.  A (M,K), B (K,N), bias (N,),
    Y (M,N) for act="glu" (out = X + X*Y), R (M,N) an optional residual added
    before the activation (fl_fused_linear_residual).  Returns out (allocated
    with torch if not given).  Keyword options map to fl_options (group_m,
    persistent, tile_cfg, no_xcd_remap, debug_tile_count, debug_sync)."""
    import torch
    lib = load_library()
    if A.dim() != 2 or B.dim() != 2 or A.shape[1] != B.shape[0]:
        raise ValueError("A must be (M,K) and B (K,N)")
    M, K = A.shape
    N = B.shape[1]
    dt = A.dtype
    code = _dtype_code(dt)
    if out is None:
        out = torch.empty((M, N), dtype=dt, device=A.device)
    if R is not None:
        opt = _options(**options)
        _check(lib.fl_fused_linear_residual(
            _dev_ptr(A, "A", dt), _dev_ptr(B, "B", dt, (K, N)), _dev_ptr(bias, "bias", dt, (N,)),
            _dev_ptr(R, "R", dt, (M, N)), _dev_ptr(Y, "Y", dt, (M, N)), _dev_ptr(out, "out", dt, (M, N)),
            M, N, K, ACTS[act], code, _stream(A, stream), ctypes.byref(opt)))
        return out
    args = (_dev_ptr(A, "A", dt), _dev_ptr(B, "B", dt, (K, N)), _dev_ptr(bias, "bias", dt, (N,)),
            _dev_ptr(Y, "Y", dt, (M, N)), _dev_ptr(out, "out", dt, (M, N)), M, N, K, ACTS[act], code,
            _stream(A, stream))
    if options:
        opt = _options(**options)
        _check(lib.fl_fused_linear_ex(*args, ctypes.byref(opt)))
    else:
        _check(lib.fl_fused_linear(*args))
    return out


QFORMATS = {"fp8_e4m3": 0, "int8": 1}


def fused_linear_quant(A, B, bias=None, Y=None, act="relu", scale=1.0, qfmt="fp8_e4m3", out=None, *, stream=None,
                       **options):
    """One-byte codes of Q(scale * act(A@B + bias)) in one kernel
    (fl_fused_linear_quant): Q is saturating round-to-nearest-even to OCP FP8
    E4M3 (qfmt="fp8_e4m3") or to int8 (qfmt="int8").  A, B, bias, Y are
    fp16 or bf16; returns out, a (M,N) uint8 tensor (the codes' bytes)."""
    import torch
    lib = load_library()
    if A.dim() != 2 or B.dim() != 2 or A.shape[1] != B.shape[0]:
        raise ValueError("A must be (M,K) and B (K,N)")
    M, K = A.shape
    N = B.shape[1]
    dt = A.dtype
    if out is None:
        out = torch.empty((M, N), dtype=torch.uint8, device=A.device)
    opt = _options(**options)
    _check(lib.fl_fused_linear_quant(
        _dev_ptr(A, "A", dt), _dev_ptr(B, "B", dt, (K, N)), _dev_ptr(bias, "bias", dt, (N,)),
        _dev_ptr(Y, "Y", dt, (M, N)), _dev_ptr(out, "out", torch.uint8, (M, N)), float(scale), M, N, K, ACTS[act],
        _dtype_code(dt), QFORMATS[qfmt], _stream(A, stream), ctypes.byref(opt)))
    return out


def fused_linear_fp8(A8, B8, ab_scale, bias=None, Y=None, act="relu", out_dtype=None, out=None, *, stream=None,
                     **options):
    """out = act(ab_scale * (A8@B8) + bias) (fl_fused_linear_fp8): A8 (M,K) and
    B8 (K,N) hold OCP FP8 E4M3 codes (torch.uint8 or torch.float8_e4m3fn);
    bias (N,), Y (M,N) and out are fp16 or bf16 (out_dtype, default fp16 or
    bias's dtype)."""
    import torch
    lib = load_library()
    if A8.dim() != 2 or B8.dim() != 2 or A8.shape[1] != B8.shape[0]:
        raise ValueError("A8 must be (M,K) and B8 (K,N)")
    M, K = A8.shape
    N = B8.shape[1]
    if out_dtype is None:
        out_dtype = bias.dtype if bias is not None else torch.float16
    A8 = A8.view(torch.uint8) if A8.dtype != torch.uint8 else A8
    B8 = B8.view(torch.uint8) if B8.dtype != torch.uint8 else B8
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=A8.device)
    opt = _options(**options)
    _check(lib.fl_fused_linear_fp8(
        _dev_ptr(A8, "A8", torch.uint8), _dev_ptr(B8, "B8", torch.uint8, (K, N)), float(ab_scale),
        _dev_ptr(bias, "bias", out_dtype, (N,)), _dev_ptr(Y, "Y", out_dtype, (M, N)),
        _dev_ptr(out, "out", out_dtype, (M, N)), M, N, K, ACTS[act], _dtype_code(out_dtype), _stream(A8, stream),
        ctypes.byref(opt)))
    return out


def fused_linear_bwd(G, W, X, Y=None, act="relu", dX=None, dY=None, dbias=True, *, stream=None, workspace=None,
                     **options):
    """The backward epilogue (fl_fused_linear_bwd): D = G @ W^T with G (M,K)
    and W (N,K), then dX = D * act'(X) at the saved pre-activation X (M,N),
    for the gate also dY = D * X, and dbias = column sums of dX (fp32).
    dbias=True allocates the (N,) fp32 result, a tensor is overwritten,
    None/False skips it.  workspace: a device tensor of at least
    bwd_workspace_bytes(M, N, K, dtype) bytes, or True to allocate one with
    torch: then fl_fused_linear_bwd_ws runs and dbias is reproducible to the
    bit.  Returns (dX, dY or None, dbias or None)."""
    import torch
    lib = load_library()
    if G.dim() != 2 or W.dim() != 2 or G.shape[1] != W.shape[1]:
        raise ValueError("G must be (M,K) and W (N,K)")
    M, K = G.shape
    N = W.shape[0]
    dt = G.dtype
    if dX is None:
        dX = torch.empty((M, N), dtype=dt, device=G.device)
    if act == "glu" and dY is None:
        dY = torch.empty((M, N), dtype=dt, device=G.device)
    if dbias is True:
        dbias = torch.empty((N,), dtype=torch.float32, device=G.device)
    elif dbias is False:
        dbias = None
    opt = _options(**options)
    args = (_dev_ptr(G, "G", dt), _dev_ptr(W, "W", dt, (N, K)), _dev_ptr(X, "X", dt, (M, N)),
            _dev_ptr(Y, "Y", dt, (M, N)), _dev_ptr(dX, "dX", dt, (M, N)), _dev_ptr(dY, "dY", dt, (M, N)),
            _dev_ptr(dbias, "dbias", torch.float32, (N,)), M, N, K, ACTS[act], _dtype_code(dt), _stream(G, stream),
            ctypes.byref(opt))
    if workspace is None:
        _check(lib.fl_fused_linear_bwd(*args))
        return dX, dY, dbias
    if workspace is True:
        workspace = torch.empty((max(bwd_workspace_bytes(M, N, K, dt), 1),), dtype=torch.uint8, device=G.device)
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    _check(lib.fl_fused_linear_bwd_ws(*args, ctypes.c_void_p(workspace.data_ptr()),
                                      workspace.numel() * workspace.element_size()))
    return dX, dY, dbias


def fused_linear_bwd_noalloc(G, W, X, Y=None, act="relu", dX=None, dY=None, dbias=True, *, stream=None,
                             **options):
    """fl_fused_linear_bwd_noalloc: fused_linear_bwd with a reproducible dbias
    whose partial sums go to the library's fixed per-GPU array (nothing is
    allocated by the call; outputs not given are allocated here with torch).
    Calls that may overlap on one GPU must be serialized."""
    import torch
    lib = load_library()
    if G.dim() != 2 or W.dim() != 2 or G.shape[1] != W.shape[1]:
        raise ValueError("G must be (M,K) and W (N,K)")
    M, K = G.shape
    N = W.shape[0]
    dt = G.dtype
    if dX is None:
        dX = torch.empty((M, N), dtype=dt, device=G.device)
    if act == "glu" and dY is None:
        dY = torch.empty((M, N), dtype=dt, device=G.device)
    if dbias is True:
        dbias = torch.empty((N,), dtype=torch.float32, device=G.device)
    elif dbias is False:
        dbias = None
    opt = _options(**options)
    _check(lib.fl_fused_linear_bwd_noalloc(
        _dev_ptr(G, "G", dt), _dev_ptr(W, "W", dt, (N, K)), _dev_ptr(X, "X", dt, (M, N)), _dev_ptr(Y, "Y", dt, (M, N)),
        _dev_ptr(dX, "dX", dt, (M, N)), _dev_ptr(dY, "dY", dt, (M, N)), _dev_ptr(dbias, "dbias", torch.float32, (N,)),
        M, N, K, ACTS[act], _dtype_code(dt), _stream(G, stream), ctypes.byref(opt)))
    return dX, dY, dbias


def bwd_workspace_bytes(M, N, K, dtype):
    """Bytes of workspace fl_fused_linear_bwd_ws needs (fl_bwd_workspace_bytes)."""
    lib = load_library()
    n = ctypes.c_size_t()
    _check(lib.fl_bwd_workspace_bytes(M, N, K, _dtype_code(dtype) if not isinstance(dtype, int) else dtype,
                                      ctypes.byref(n)))
    return n.value


def gemm_nt(A, Bt, D=None, *, stream=None):
    """Unfused backward step 1: D = A @ Bt^T with Bt (N,K) row-major."""
    import torch
    lib = load_library()
    M, K = A.shape
    N = Bt.shape[0]
    dt = A.dtype
    if D is None:
        D = torch.empty((M, N), dtype=dt, device=A.device)
    _check(lib.fl_gemm_nt(_dev_ptr(A, "A", dt), _dev_ptr(Bt, "Bt", dt, (N, K)), _dev_ptr(D, "D", dt, (M, N)),
                          M, N, K, _dtype_code(dt), _stream(A, stream)))
    return D


def activation_grad(D, X, Y=None, act="relu", dX=None, dY=None, *, stream=None):
    """Unfused backward step 2: dX = D * act'(X) (gate: also dY = D * X)."""
    import torch
    lib = load_library()
    M, N = D.shape
    dt = D.dtype
    if dX is None:
        dX = torch.empty_like(D)
    if act == "glu" and dY is None:
        dY = torch.empty_like(D)
    _check(lib.fl_activation_grad(_dev_ptr(D, "D", dt), _dev_ptr(X, "X", dt, (M, N)), _dev_ptr(Y, "Y", dt, (M, N)),
                                  _dev_ptr(dX, "dX", dt, (M, N)), _dev_ptr(dY, "dY", dt, (M, N)), M, N, ACTS[act],
                                  _dtype_code(dt), _stream(D, stream)))
    return dX, dY


def column_sum(X, sums=None, *, stream=None):
    """Unfused backward step 3: sums[j] = sum_i X[i, j] (fp32)."""
    import torch
    lib = load_library()
    M, N = X.shape
    if sums is None:
        sums = torch.empty((N,), dtype=torch.float32, device=X.device)
    _check(lib.fl_column_sum(_dev_ptr(X, "X", X.dtype), _dev_ptr(sums, "sums", torch.float32, (N,)), M, N,
                             _dtype_code(X.dtype), _stream(X, stream)))
    return sums


def gemm(A, B, X=None, *, stream=None):
    """Unfused step 1: X = A@B, stored in the I/O dtype."""
    import torch
    lib = load_library()
    M, K = A.shape
    N = B.shape[1]
    dt = A.dtype
    if X is None:
        X = torch.empty((M, N), dtype=dt, device=A.device)
    _check(lib.fl_gemm(_dev_ptr(A, "A", dt), _dev_ptr(B, "B", dt, (K, N)), _dev_ptr(X, "X", dt, (M, N)),
                       M, N, K, _dtype_code(dt), _stream(A, stream)))
    return X


def bias_add(X, bias, *, stream=None):
    """Unfused step 2: X[i,j] += bias[j] in place."""
    lib = load_library()
    M, N = X.shape
    dt = X.dtype
    _check(lib.fl_bias_add(_dev_ptr(X, "X", dt), _dev_ptr(bias, "bias", dt, (N,)), M, N, _dtype_code(dt),
                           _stream(X, stream)))
    return X


def activation(X, Y=None, out=None, act="relu", *, stream=None):
    """Unfused step 3: out = act(X) (or X + X*Y for act="glu"); out may be X."""
    import torch
    lib = load_library()
    M, N = X.shape
    dt = X.dtype
    if out is None:
        out = torch.empty_like(X)
    _check(lib.fl_activation(_dev_ptr(X, "X", dt), _dev_ptr(Y, "Y", dt, (M, N)), _dev_ptr(out, "out", dt, (M, N)),
                             M, N, ACTS[act], _dtype_code(dt), _stream(X, stream)))
    return out


def tile_grid(M, N, K, dtype_code, **options):
    """(block_m, block_n, tiles_m, tiles_n) the fused kernel uses."""
    lib = load_library()
    opt = _options(**options)
    vals = [ctypes.c_int32() for _ in range(4)]
    _check(lib.fl_tile_grid(M, N, K, dtype_code, ctypes.byref(opt), *[ctypes.byref(v) for v in vals]))
    return tuple(v.value for v in vals)


def tile_of_program(program, grid, tiles_m, tiles_n, group_m, xcd_remap):
    """(m_tile, n_tile) computed by program `program` (host copy of the device map)."""
    lib = load_library()
    m, n = ctypes.c_int32(), ctypes.c_int32()
    _check(lib.fl_tile_of_program(program, grid, tiles_m, tiles_n, group_m, xcd_remap, ctypes.byref(m),
                                  ctypes.byref(n)))
    return m.value, n.value


def version():
    return load_library().fl_version()
