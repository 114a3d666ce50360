// fused_linear.hip -- host side of the C ABI declared in include/fused_linear.h:
// argument validation, tile/launch selection and kernel launches on the
// caller's stream.  All device code is in fl_kernels.hpp.
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "fl_kernels.hpp"

namespace {

thread_local char g_err[512];

fl_status fail(fl_status s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

void clear_error() { g_err[0] = '\0'; }

size_t elem_size(int dtype) { return dtype == FL_F32 ? 4 : 2; }

bool valid_dtype(int d) { return d == FL_F32 || d == FL_F16 || d == FL_BF16; }
bool valid_act(int a) { return a >= FL_ACT_NONE && a <= FL_ACT_GLU; }

bool overlaps(const void *a, size_t abytes, const void *b, size_t bbytes) {
    if (!a || !b || abytes == 0 || bbytes == 0) return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + bbytes && b0 < a0 + abytes;
}

bool aligned(const void *p, size_t n) { return ((uintptr_t)p % n) == 0; }

constexpr int64_t kMaxDim = 0x7fffffff;
// M-tiles per band of the grouped tile order: measured best of {1,2,4,8,16} at
// 4096^3 (fp16, 256x256 tiles, XCD placement on).
constexpr int kDefaultGroup = 4;

// Per-device compute-unit count, read once per device.
int cu_count() {
    static std::mutex mu;
    static int cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    std::lock_guard<std::mutex> lock(mu);
    if (cache[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cache[dev] = n;
    }
    return cache[dev];
}

// ---------------------------------------------------------- launch tables

// The fused kernels of each dtype are compiled in their own translation unit
// (fl_fused_inst.hip built once per dtype) so the build runs in parallel.
fl::fused_launcher pick_fused(int dtype, int act, bool vec, int variant, bool residual) {
    if (dtype == FL_F32) return fl::pick_fused_for<FL_F32>(act, vec, variant, residual);
    if (dtype == FL_F16) return fl::pick_fused_for<FL_F16>(act, vec, variant, residual);
    return fl::pick_fused_for<FL_BF16>(act, vec, variant, residual);
}

struct TileShape {
    int bm, bn;
    int variant;  // fl::Variant
};

// Kernel and tile for a problem (tile_cfg values as in fl_options).  fp32
// always runs the register-staged kernel.
// Automatic fp16/bf16 choice, all with 16x16x32 MFMA blocks: the width (256,
// 192 or 128) with the smallest waves * relative time of a wave, a wave of
// 256x192 tiles taking 0.79 and one of 256x128 tiles 0.55 of a 256x256 wave
// (measured at K = 4096 with the 32x32 kernels); ties go to the wider tile.
// 256 and 192 run 8-wave kernels (two waves per SIMD; 256: 1.5-14% faster
// than 4 waves on every measured shape, 192: +10% at 1024x21568x4096 and
// x3072).  192 wins where the 256-wide grid leaves its last wave mostly
// empty and the 192-wide one fills it (measured +3% on 1024x21568x4096, +6%
// on 4096x4608x4096, +10% on 3072x12288x4096 over the best power-of-two
// width).  Then, when the 256x128 grid fills both workgroup slots of every
// CU, short reductions switch to the two-per-CU kernel, whose epilogues and
// start-ups overlap the other workgroup's K loop: K <= 3072 where 256x128
// was chosen (measured +16% to +29% at K 256..1024, +4% at 3072, -2% at
// 4096 on 1024x21568), K <= 1024 where 256x192 was (+2% at 1024, -1% at
// 1280, -4% at 1536), K <= 256 where 256x256 was (+4% at 8192^2 x 256, -2%
// to -7% at 384 and 512).
constexpr int64_t kOcc2MaxK256 = 256;
constexpr int64_t kOcc2MaxK192 = 1024;
constexpr int64_t kOcc2MaxK256Fp8 = 1024;  // FP8 operands (fl_fused_linear_fp8)

// The automatic tile width (waves x relative wave time, below) and whether
// the 256x128 grid fills both workgroup slots of every CU.
struct AutoTile {
    int bn;
    bool fills_two;
};

AutoTile auto_tile(int64_t M, int64_t N) {
    const int64_t cus = cu_count();
    const int64_t tm = (M + 255) / 256;
    auto waves = [&](int64_t bn) { return (tm * ((N + bn - 1) / bn) + cus - 1) / cus; };
    // waves x time of one wave of tiles, in hundredths of a 256x256 wave
    const int64_t c256 = waves(256) * 100, c192 = waves(192) * 79, c128 = waves(128) * 55;
    const int bn = (c256 <= c192 && c256 <= c128) ? 256 : (c192 <= c128 ? 192 : 128);
    return {bn, tm * ((N + 127) / 128) >= 2 * cus};
}

fl_status tile_shape(int dtype, int64_t M, int64_t N, int64_t K, const fl_options *opt, TileShape &t) {
    const int cfg = opt ? opt->tile_cfg : 0;
    if (cfg < 0 || cfg > 15) return fail(FL_ERR_UNSUPPORTED, "tile_cfg %d is not available", cfg);
    if (dtype == FL_F32) {
        if (cfg == 2 || cfg == 6) return fail(FL_ERR_UNSUPPORTED, "tile_cfg %d (256x128) is fp16/bf16 only", cfg);
        if (cfg == 7 || cfg == 8) return fail(FL_ERR_UNSUPPORTED, "tile_cfg %d (256x192) is fp16/bf16 only", cfg);
        if (cfg >= 9) return fail(FL_ERR_UNSUPPORTED, "tile_cfg %d (16x16x32 blocks) is fp16/bf16 only", cfg);
        t = {256, 256, fl::kRegStaged};
        return FL_OK;
    }
    switch (cfg) {
    case 1: t = {256, 256, fl::kDirect64x256}; return FL_OK;
    case 2: t = {256, 128, fl::kDirect64x128}; return FL_OK;
    case 3: t = {256, 256, fl::kRegStaged}; return FL_OK;
    case 4: t = {256, 256, fl::kDirect32x256}; return FL_OK;
    case 5: t = {256, 256, fl::kDirect64x256W8}; return FL_OK;
    case 6: t = {256, 128, fl::kDirect32x128Occ2}; return FL_OK;
    case 7: t = {256, 192, fl::kDirect64x192}; return FL_OK;
    case 8: t = {256, 192, fl::kDirect32x192}; return FL_OK;
    case 9: t = {256, 256, fl::kDirect64x256M16}; return FL_OK;
    case 10: t = {256, 256, fl::kDirect64x256W8M16}; return FL_OK;
    case 11: t = {256, 192, fl::kDirect64x192M16}; return FL_OK;
    case 12: t = {256, 128, fl::kDirect64x128M16}; return FL_OK;
    case 13: t = {256, 256, fl::kDirect32x256M16}; return FL_OK;
    case 14: t = {256, 256, fl::kDirect32x256W8M16}; return FL_OK;
    case 15: t = {256, 192, fl::kDirect64x192W8M16}; return FL_OK;
    default: break;
    }
    const AutoTile at = auto_tile(M, N);
    const int bn = at.bn;
    if (at.fills_two && K <= (bn == 256 ? kOcc2MaxK256 : bn == 192 ? kOcc2MaxK192 : 3072))
        t = {256, 128, fl::kDirect32x128Occ2};
    else if (bn == 128)
        t = {256, 128, fl::kDirect64x128M16};
    else if (bn == 192)
        t = {256, 192, fl::kDirect64x192W8M16};
    else
        t = {256, 256, fl::kDirect64x256W8M16};
    return FL_OK;
}

// The sibling with 32x32 MFMA blocks of a kernel variant (the same tile):
// the FP8-operand and backward entry points choose their kernel by it.
int family32(int v) {
    switch (v) {
    case fl::kDirect64x256M16: return fl::kDirect64x256;
    case fl::kDirect64x256W8M16: return fl::kDirect64x256W8;
    case fl::kDirect32x256M16: return fl::kDirect32x256;
    case fl::kDirect32x256W8M16: return fl::kDirect64x256W8;
    case fl::kDirect64x192M16: return fl::kDirect64x192;
    case fl::kDirect64x192W8M16: return fl::kDirect64x192;
    case fl::kDirect64x128M16: return fl::kDirect64x128;
    default: return v;
    }
}

int grid_elementwise(int64_t work_items) {
    int64_t blocks = (work_items + fl::kThreads - 1) / fl::kThreads;
    const int64_t cap = (int64_t)cu_count() * 16;
    if (blocks > cap) blocks = cap;
    if (blocks < 1) blocks = 1;
    return (int)blocks;
}

fl_status check_launch(const char *what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(FL_ERR_LAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
    return FL_OK;
}

fl_status check_dims(int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N < 0 || K < 0)
        return fail(FL_ERR_INVALID_ARG, "negative size (M=%lld, N=%lld, K=%lld)", (long long)M, (long long)N,
                    (long long)K);
    if (M > kMaxDim || N > kMaxDim || K > kMaxDim)
        return fail(FL_ERR_UNSUPPORTED, "sizes above 2^31-1 are not supported");
    return FL_OK;
}

// Shared validation of the GEMM-shaped entry points.
fl_status validate_gemm(const void *A, const void *B, const void *bias, const void *R, const void *Y,
                        const void *out, int64_t M, int64_t N, int64_t K, int act, int dtype,
                        const fl_options *opt, bool out_optional = false, bool b_kn = true) {
    if (!valid_dtype(dtype)) return fail(FL_ERR_INVALID_ARG, "unknown dtype %d", dtype);
    if (!valid_act(act)) return fail(FL_ERR_INVALID_ARG, "unknown activation %d", act);
    fl_status s = check_dims(M, N, K);
    if (s != FL_OK) return s;
    if (opt) {
        if (opt->group_m < 0) return fail(FL_ERR_INVALID_ARG, "group_m must be >= 1 (0 = default)");
        if (opt->persistent != 0 && opt->persistent != 1)
            return fail(FL_ERR_INVALID_ARG, "persistent must be 0 or 1");
        if (opt->no_xcd_remap != 0 && opt->no_xcd_remap != 1)
            return fail(FL_ERR_INVALID_ARG, "no_xcd_remap must be 0 or 1");
        if (opt->debug_sync != 0 && opt->debug_sync != 1)
            return fail(FL_ERR_INVALID_ARG, "debug_sync must be 0 or 1");
        TileShape t;
        s = tile_shape(dtype, M, N, K, opt, t);
        if (s != FL_OK) return s;
    }
    const size_t es = elem_size(dtype);
    // In-tile byte offsets are 32-bit: 256 rows of A, of Y and of out must span < 2^31 bytes.
    if ((size_t)K * es * 256 >= 0x80000000ull || (size_t)N * es * 256 >= 0x80000000ull)
        return fail(FL_ERR_UNSUPPORTED, "K or N too large (256 rows must span < 2 GiB)");
    // B given as (K, N) is read through the whole K range from the tile's
    // first column with 32-bit offsets (B as (N, K), the transposed operand,
    // only through the tile's 256 rows).
    if (b_kn && (size_t)K * N * es >= 0x80000000ull)
        return fail(FL_ERR_UNSUPPORTED, "B too large (its K x N elements must span < 2 GiB)");
    const size_t a_bytes = (size_t)M * K * es, b_bytes = (size_t)K * N * es, o_bytes = (size_t)M * N * es;
    const size_t bias_bytes = bias ? (size_t)N * es : 0;
    if (!A && a_bytes) return fail(FL_ERR_INVALID_ARG, "A is NULL");
    if (!B && b_bytes) return fail(FL_ERR_INVALID_ARG, "B is NULL");
    if (!out && o_bytes && !out_optional) return fail(FL_ERR_INVALID_ARG, "out is NULL");
    if (act == FL_ACT_GLU && !Y && o_bytes) return fail(FL_ERR_INVALID_ARG, "the gate needs Y");
    if (act != FL_ACT_GLU && Y) return fail(FL_ERR_INVALID_ARG, "Y is only used by the gate (FL_ACT_GLU)");
    const void *ptrs[6] = {A, B, bias, R, Y, out};
    for (const void *p : ptrs)
        if (p && !aligned(p, es)) return fail(FL_ERR_INVALID_ARG, "pointer %p is not aligned to the element size", p);
    if (overlaps(out, o_bytes, A, a_bytes)) return fail(FL_ERR_INVALID_ARG, "out overlaps A");
    if (overlaps(out, o_bytes, B, b_bytes)) return fail(FL_ERR_INVALID_ARG, "out overlaps B");
    if (overlaps(out, o_bytes, bias, bias_bytes)) return fail(FL_ERR_INVALID_ARG, "out overlaps bias");
    if (Y && Y != out && overlaps(out, o_bytes, Y, o_bytes))
        return fail(FL_ERR_INVALID_ARG, "Y partially overlaps out (only Y == out is allowed)");
    if (R && R != out && overlaps(out, o_bytes, R, o_bytes))
        return fail(FL_ERR_INVALID_ARG, "R partially overlaps out (only R == out is allowed)");
    return FL_OK;
}

fl_status launch_gemm(const void *A, const void *B, const void *bias, const void *R, const void *Y, void *out,
                      int64_t M, int64_t N, int64_t K, int act, int dtype, void *stream, const fl_options *opt,
                      int qfmt = -1, float scale = 1.0f, bool fp8_in = false, float ab_scale = 1.0f,
                      const void *Xs = nullptr, void *dY = nullptr, float *dbias = nullptr, bool bwd = false,
                      float *dbias_part = nullptr) {
    if (M == 0 || N == 0) return FL_OK;
    TileShape t;
    fl_status s = tile_shape(dtype, M, N, K, opt, t);
    if (s != FL_OK) return s;
    const int64_t tiles_m = (M + t.bm - 1) / t.bm, tiles_n = (N + t.bn - 1) / t.bn;
    if (tiles_m * tiles_n > kMaxDim) return fail(FL_ERR_UNSUPPORTED, "too many output tiles");
    const int es = (int)elem_size(dtype);
    const int vec = 16 / es;
    // The direct-to-LDS kernels take any alignment; the register-staged
    // kernels need 16-byte aligned rows for their vector path.
    const bool aligned_rows = (K % vec == 0) && (N % vec == 0) && aligned(A, 16) && aligned(B, 16) &&
                              aligned(out, 16) && (!bias || aligned(bias, 16)) && (!Y || aligned(Y, 16)) &&
                              (!R || aligned(R, 16));
    fl::GemmArgs a;
    a.A = A;
    a.B = B;
    a.bias = bias;
    a.Y = Y;
    a.R = R;
    a.scale = scale;
    const int64_t out_row_bytes = N * (qfmt >= 0 ? 1 : es);
    a.stream_out = (out_row_bytes % 128 == 0) && aligned(out, 128);
    a.ab_scale = ab_scale;
    a.Xs = Xs;
    a.dY = dY;
    a.dbias = dbias;
    a.dbias_part = dbias_part;
    a.out = out;
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.tiles_m = (int)tiles_m;
    a.tiles_n = (int)tiles_n;
    a.group = (opt && opt->group_m > 0) ? opt->group_m : kDefaultGroup;
    a.xcd_remap = (opt && opt->no_xcd_remap) ? 0 : 1;
    a.persistent = (opt && opt->persistent) ? 1 : 0;
    a.tile_count = opt ? opt->debug_tile_count : nullptr;
    a.debug_sync = (opt && opt->debug_sync) ? 1 : 0;
    const int ntiles = (int)(tiles_m * tiles_n);
    int grid = ntiles;
    if (a.persistent) {
        const int slots = cu_count();
        grid = ntiles < slots ? ntiles : slots;
    }
    if (bwd) {
        const fl::fused_launcher f = dtype == FL_F16 ? fl::pick_bwd_for<FL_F16>(act, t.variant)
                                                     : fl::pick_bwd_for<FL_BF16>(act, t.variant);
        if (!f) return fail(FL_ERR_UNSUPPORTED, "the backward epilogue is built for tile_cfg 0, 2, 5, 10 and 12 only");
        f(a, grid, static_cast<hipStream_t>(stream));
        return check_launch("fused_linear_bwd");
    }
    if (fp8_in) {
        const fl::fused_launcher f = dtype == FL_F16 ? fl::pick_fp8_for<FL_F16>(act, t.variant)
                                                     : fl::pick_fp8_for<FL_BF16>(act, t.variant);
        if (!f) return fail(FL_ERR_UNSUPPORTED, "FP8 inputs are built for tile_cfg 0, 1, 2, 5, 6, 7 and 12 only");
        f(a, grid, static_cast<hipStream_t>(stream));
        return check_launch("fused_linear_fp8");
    }
    if (qfmt >= 0) {
        const fl::fused_launcher q = dtype == FL_F16 ? fl::pick_quant_for<FL_F16>(act, t.variant, qfmt)
                                                     : fl::pick_quant_for<FL_BF16>(act, t.variant, qfmt);
        if (!q) return fail(FL_ERR_UNSUPPORTED, "quantized output is built for tile_cfg 0, 2, 5, 6, 7, 10, 11, 12 and 15 only");
        q(a, grid, static_cast<hipStream_t>(stream));
        return check_launch("fused_linear_quant");
    }
    const bool use_vec = t.variant != fl::kRegStaged || aligned_rows;
    pick_fused(dtype, act, use_vec, t.variant, R != nullptr)(a, grid, static_cast<hipStream_t>(stream));
    return check_launch("fused_linear");
}

// out[c] = the sum of column c of the rows x n partial sums, added in row
// order from 0 (the bias gradient from the backward tiles' partial column
// sums: the same bits whatever order the tiles ran in).
// Rows are loaded 16 at a time ahead of their additions, so a thread waits
// for memory once per 16 rows instead of once per row.
__global__ void sum_rows_f32_kernel(const float *part, int64_t rows, int64_t n, float *out) {
    for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < n; c += (int64_t)gridDim.x * blockDim.x) {
        float acc = 0.0f;
        int64_t r = 0;
        for (; r + 16 <= rows; r += 16) {
            float v[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) v[j] = part[(r + j) * n + c];
#pragma unroll
            for (int j = 0; j < 16; ++j) acc += v[j];
        }
        for (; r < rows; ++r) acc += part[r * n + c];
        out[c] = acc;
    }
}

// Zeroes n floats (the bias gradient before the tiles add into it); a
// kernel rather than a memset, so that a captured graph replays it as work.
__global__ void zero_f32_kernel(float *p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0.0f;
}

// The tile choice of the transposed-B kernels: the 8-wave 256x256 kernel
// with 16x16x32 blocks where the forward choice is 256x256, else 256x128
// with 32x32x16 blocks (16% faster there than its 16x16 sibling, whose
// accumulators the compiler moves between registers in the K loop:
// measured on the gate's backward, 1024x21568x4096).
fl_options bwd_tiles(int dtype, int64_t M, int64_t N, int64_t K) {
    fl_options o{};
    TileShape t;
    tile_shape(dtype, M, N, K, &o, t);
    o.tile_cfg = family32(t.variant) == fl::kDirect64x256W8 ? 10 : 2;
    return o;
}

template <int DT, int ACT>
void launch_ag(bool vec, int grid, hipStream_t st, const void *D, const void *X, const void *Y, void *dX, void *dY,
               int64_t total) {
    if (vec)
        hipLaunchKernelGGL((fl::activation_grad_kernel<DT, ACT, true>), dim3(grid), dim3(fl::kThreads), 0, st, D, X, Y,
                           dX, dY, total);
    else
        hipLaunchKernelGGL((fl::activation_grad_kernel<DT, ACT, false>), dim3(grid), dim3(fl::kThreads), 0, st, D, X, Y,
                           dX, dY, total);
}

template <int DT>
void launch_ag_act(int act, bool vec, int grid, hipStream_t st, const void *D, const void *X, const void *Y, void *dX,
                   void *dY, int64_t total) {
    switch (act) {
    case FL_ACT_NONE: launch_ag<DT, FL_ACT_NONE>(vec, grid, st, D, X, Y, dX, dY, total); break;
    case FL_ACT_RELU: launch_ag<DT, FL_ACT_RELU>(vec, grid, st, D, X, Y, dX, dY, total); break;
    case FL_ACT_GELU_TANH: launch_ag<DT, FL_ACT_GELU_TANH>(vec, grid, st, D, X, Y, dX, dY, total); break;
    default: launch_ag<DT, FL_ACT_GLU>(vec, grid, st, D, X, Y, dX, dY, total); break;
    }
}

fl_status launch_activation_grad(int dtype, int act, bool vec, int grid, hipStream_t st, const void *D, const void *X,
                                 const void *Y, void *dX, void *dY, int64_t total) {
    if (dtype == FL_F16)
        launch_ag_act<FL_F16>(act, vec, grid, st, D, X, Y, dX, dY, total);
    else
        launch_ag_act<FL_BF16>(act, vec, grid, st, D, X, Y, dX, dY, total);
    return FL_OK;
}

template <int DT>
void launch_column_sum(bool vec, dim3 grid, hipStream_t st, const void *X, float *sums, int64_t M, int64_t N) {
    if (vec)
        hipLaunchKernelGGL((fl::column_sum_kernel<DT, true>), grid, dim3(fl::kThreads), 0, st, X, sums, M, N);
    else
        hipLaunchKernelGGL((fl::column_sum_kernel<DT, false>), grid, dim3(fl::kThreads), 0, st, X, sums, M, N);
}

}  // namespace

extern "C" {

fl_status fl_fused_linear_ex(const void *A, const void *B, const void *bias, const void *Y, void *out, int64_t M,
                             int64_t N, int64_t K, fl_act act, fl_dtype dtype, void *stream,
                             const fl_options *opt) {
    clear_error();
    fl_status s = validate_gemm(A, B, bias, nullptr, Y, out, M, N, K, act, dtype, opt);
    if (s != FL_OK) return s;
    return launch_gemm(A, B, bias, nullptr, Y, out, M, N, K, act, dtype, stream, opt);
}

fl_status fl_fused_linear_residual(const void *A, const void *B, const void *bias, const void *R, const void *Y,
                                   void *out, int64_t M, int64_t N, int64_t K, fl_act act, fl_dtype dtype,
                                   void *stream, const fl_options *opt) {
    clear_error();
    if (!R && M > 0 && N > 0) return fail(FL_ERR_INVALID_ARG, "R is NULL (use fl_fused_linear without a residual)");
    fl_status s = validate_gemm(A, B, bias, R, Y, out, M, N, K, act, dtype, opt);
    if (s != FL_OK) return s;
    return launch_gemm(A, B, bias, R, Y, out, M, N, K, act, dtype, stream, opt);
}

fl_status fl_fused_linear(const void *A, const void *B, const void *bias, const void *Y, void *out, int64_t M,
                          int64_t N, int64_t K, fl_act act, fl_dtype dtype, void *stream) {
    return fl_fused_linear_ex(A, B, bias, Y, out, M, N, K, act, dtype, stream, nullptr);
}

fl_status fl_fused_linear_quant(const void *A, const void *B, const void *bias, const void *Y, void *out_q,
                                float scale, int64_t M, int64_t N, int64_t K, fl_act act, fl_dtype dtype,
                                fl_qformat qfmt, void *stream, const fl_options *opt) {
    clear_error();
    if (qfmt != FL_Q_FP8_E4M3 && qfmt != FL_Q_INT8) return fail(FL_ERR_INVALID_ARG, "unknown qformat %d", (int)qfmt);
    if (!(scale == scale) || scale - scale != 0.0f) return fail(FL_ERR_INVALID_ARG, "scale must be finite");
    if (dtype == FL_F32) return fail(FL_ERR_UNSUPPORTED, "quantized output takes fp16 or bf16 inputs");
    // Validate the inputs as for a 16-bit output, with out checked apart:
    // out_q holds M*N one-byte codes and may not overlap any input.
    fl_status s = validate_gemm(A, B, bias, nullptr, Y, nullptr, M, N, K, act, dtype, opt, /*out_optional=*/true);
    if (s != FL_OK) return s;
    const size_t q_bytes = (size_t)M * N;
    if (!out_q && q_bytes) return fail(FL_ERR_INVALID_ARG, "out is NULL");
    const size_t es = elem_size(dtype);
    if (overlaps(out_q, q_bytes, A, (size_t)M * K * es)) return fail(FL_ERR_INVALID_ARG, "out overlaps A");
    if (overlaps(out_q, q_bytes, B, (size_t)K * N * es)) return fail(FL_ERR_INVALID_ARG, "out overlaps B");
    if (overlaps(out_q, q_bytes, bias, bias ? (size_t)N * es : 0))
        return fail(FL_ERR_INVALID_ARG, "out overlaps bias");
    if (overlaps(out_q, q_bytes, Y, Y ? (size_t)M * N * es : 0)) return fail(FL_ERR_INVALID_ARG, "out overlaps Y");
    return launch_gemm(A, B, bias, nullptr, Y, out_q, M, N, K, act, dtype, stream, opt, (int)qfmt, scale);
}

fl_status fl_fused_linear_fp8(const void *A8, const void *B8, float ab_scale, const void *bias, const void *Y,
                              void *out, int64_t M, int64_t N, int64_t K, fl_act act, fl_dtype out_dtype, void *stream,
                              const fl_options *opt) {
    clear_error();
    if (!(ab_scale == ab_scale) || ab_scale - ab_scale != 0.0f) return fail(FL_ERR_INVALID_ARG, "ab_scale must be finite");
    if (out_dtype == FL_F32) return fail(FL_ERR_UNSUPPORTED, "FP8 inputs produce fp16 or bf16 outputs");
    // Bias, Y and out are checked as for a 16-bit layer (A and B apart: one
    // byte per element).
    fl_status s = validate_gemm(nullptr, nullptr, bias, nullptr, Y, out, M, N, 0, act, out_dtype, opt);
    if (s != FL_OK) return s;
    s = check_dims(M, N, K);
    if (s != FL_OK) return s;
    // A partial last dword of B may hold its last three codes; they must lie
    // in its last row, which the kernel's last K stage patches.
    if (N > 0 && N < 3) return fail(FL_ERR_UNSUPPORTED, "FP8 inputs need N >= 3");
    if (!aligned(A8, 16) || !aligned(B8, 16)) return fail(FL_ERR_INVALID_ARG, "A8 and B8 must be 16-byte aligned");
    if (opt) {
        TileShape t;
        s = tile_shape(FL_F16, M, N, K, opt, t);
        if (s != FL_OK) return s;
    }
    const size_t a_bytes = (size_t)M * K, b_bytes = (size_t)K * N, o_bytes = (size_t)M * N * elem_size(out_dtype);
    if (!A8 && a_bytes) return fail(FL_ERR_INVALID_ARG, "A is NULL");
    if (!B8 && b_bytes) return fail(FL_ERR_INVALID_ARG, "B is NULL");
    if (K * 256 >= 0x80000000ll) return fail(FL_ERR_UNSUPPORTED, "K too large (256 rows must span < 2 GiB)");
    if (b_bytes >= 0x80000000ull) return fail(FL_ERR_UNSUPPORTED, "B too large (its K x N bytes must span < 2 GiB)");
    if (overlaps(out, o_bytes, A8, a_bytes)) return fail(FL_ERR_INVALID_ARG, "out overlaps A");
    if (overlaps(out, o_bytes, B8, b_bytes)) return fail(FL_ERR_INVALID_ARG, "out overlaps B");
    fl_options o = opt ? *opt : fl_options{};
    if (o.tile_cfg == 0) {
        // 32x32x64 blocks in the forward choice's width: the 8-wave 256x256
        // kernel, 256x192, or 256x128.  An FP8 K loop takes about half the
        // time of a 16-bit one of the same K, so the two-per-CU kernel, whose
        // epilogues overlap the other workgroup's K loop, pays off up to
        // longer reductions than in 16 bits: K <= 1024 where the width is
        // 256 (measured on 8192^2: +27% at K 256, +6% at 1024, -5% at
        // 2048), K <= 3072 where it is 192 (on 1024x21568: +17% at 512, +4%
        // at 3072, -3% at 4096) or 128.  The 16x16x128 kernel (256x128) is
        // an option: no faster than the 32x32x64 one of the same tile, where
        // 16-bit blocks of 16x16 gain from their lower power draw.
        const AutoTile at = auto_tile(M, N);
        if (at.fills_two && K <= (at.bn == 256 ? kOcc2MaxK256Fp8 : 3072))
            o.tile_cfg = 6;
        else
            o.tile_cfg = at.bn == 256 ? 5 : at.bn == 192 ? 7 : 2;
    }
    return launch_gemm(A8, B8, bias, nullptr, Y, out, M, N, K, act, out_dtype, stream, &o, -1, 1.0f, true, ab_scale);
}

// Bytes of the backward's partial column sums: two rows (one per wave row
// of a tile) per 256-row tile row, N fp32 values each.
size_t bwd_part_bytes(int64_t M, int64_t N) {
    if (M <= 0 || N <= 0) return 0;
    return (size_t)2 * (size_t)((M + 255) / 256) * (size_t)N * sizeof(float);
}

// The backward epilogue; with `part` (bwd_part_bytes of device memory) the
// tiles write partial column sums there and one more pass adds them into
// dbias in a fixed order, else the tiles add into a zeroed dbias with
// atomics.  `ws` is the workspace argument as the caller gave it (checked
// here when part is used).  check_only: validate every other argument and
// return before any launch.
fl_status bwd_impl(const void *G, const void *W, const void *X, const void *Y, void *dX, void *dY, float *dbias,
                   int64_t M, int64_t N, int64_t K, fl_act act, fl_dtype dtype, void *stream, const fl_options *opt,
                   bool deterministic, void *ws, size_t ws_bytes, bool check_only = false) {
    if (dtype == FL_F32) return fail(FL_ERR_UNSUPPORTED, "the backward epilogue is built for fp16 and bf16");
    // G plays A (M,K) and W (N,K) has B's size; X is checked as a residual
    // would be (it may be dX itself), Y as the gate's operand.
    fl_status s = validate_gemm(G, W, nullptr, X, Y, dX, M, N, K, act, dtype, opt, false, /*b_kn=*/false);
    if (s != FL_OK) return s;
    const size_t es = elem_size(dtype);
    const size_t g_bytes = (size_t)M * K * es, w_bytes = (size_t)N * K * es, o_bytes = (size_t)M * N * es;
    if (!X && o_bytes) return fail(FL_ERR_INVALID_ARG, "X (the saved pre-activation) is NULL");
    if (act == FL_ACT_GLU && !dY && o_bytes) return fail(FL_ERR_INVALID_ARG, "the gate's backward needs dY");
    if (act != FL_ACT_GLU && dY) return fail(FL_ERR_INVALID_ARG, "dY is only written for the gate (FL_ACT_GLU)");
    if (overlaps(X, o_bytes, G, g_bytes) || overlaps(X, o_bytes, W, w_bytes))
        return fail(FL_ERR_INVALID_ARG, "X overlaps G or W");
    if (dY) {
        if (!aligned(dY, es)) return fail(FL_ERR_INVALID_ARG, "dY is not aligned to the element size");
        const void *others[4] = {G, W, X, dX};
        const size_t sizes[4] = {g_bytes, w_bytes, o_bytes, o_bytes};
        for (int i = 0; i < 4; ++i)
            if (overlaps(dY, o_bytes, others[i], sizes[i]))
                return fail(FL_ERR_INVALID_ARG, "dY overlaps G, W, X or dX");
        if (dY != Y && overlaps(dY, o_bytes, Y, o_bytes))
            return fail(FL_ERR_INVALID_ARG, "dY partially overlaps Y (only dY == Y is allowed)");
    }
    if (dbias) {
        if (!aligned(dbias, 4)) return fail(FL_ERR_INVALID_ARG, "dbias is not 4-byte aligned");
        const size_t db_bytes = (size_t)N * 4;
        const void *others[5] = {G, W, X, Y, dX};
        const size_t sizes[5] = {g_bytes, w_bytes, o_bytes, Y ? o_bytes : 0, o_bytes};
        for (int i = 0; i < 5; ++i)
            if (overlaps(dbias, db_bytes, others[i], sizes[i])) return fail(FL_ERR_INVALID_ARG, "dbias overlaps an operand");
        if (dY && overlaps(dbias, db_bytes, dY, o_bytes)) return fail(FL_ERR_INVALID_ARG, "dbias overlaps dY");
    }
    fl_options o = opt ? *opt : fl_options{};
    if (o.tile_cfg == 0) {
        TileShape t;
        tile_shape(dtype, M, N, K, &o, t);
        o.tile_cfg = family32(t.variant) == fl::kDirect64x256W8 ? 10 : 2;
    } else if (o.tile_cfg != 2 && o.tile_cfg != 5 && o.tile_cfg != 10 && o.tile_cfg != 12) {
        return fail(FL_ERR_UNSUPPORTED, "the backward epilogue is built for tile_cfg 0, 2, 5, 10 and 12 only");
    }
    if (check_only) return FL_OK;  // the caller checks or supplies the workspace itself
    float *part = nullptr;
    const size_t need = bwd_part_bytes(M, N);
    if (deterministic && dbias && need) {
        if (!ws) return fail(FL_ERR_INVALID_ARG, "workspace is NULL (%zu bytes needed)", need);
        if (ws_bytes < need)
            return fail(FL_ERR_INVALID_ARG, "workspace of %zu bytes is too small (%zu bytes needed)", ws_bytes, need);
        if (!aligned(ws, 4)) return fail(FL_ERR_INVALID_ARG, "workspace is not 4-byte aligned");
        const size_t es = elem_size(dtype);
        const size_t g_bytes = (size_t)M * K * es, w_bytes = (size_t)N * K * es, o_bytes = (size_t)M * N * es;
        const void *others[7] = {G, W, X, Y, dX, dY, dbias};
        const size_t sizes[7] = {g_bytes, w_bytes, o_bytes, Y ? o_bytes : 0, o_bytes, dY ? o_bytes : 0,
                                 (size_t)N * 4};
        for (int i = 0; i < 7; ++i)
            if (overlaps(ws, need, others[i], sizes[i])) return fail(FL_ERR_INVALID_ARG, "workspace overlaps an operand");
        part = static_cast<float *>(ws);
    }
    if (part) {
        // the tiles write every partial sum; one pass then adds them in order
        fl_status s2 = launch_gemm(G, W, nullptr, nullptr, Y, dX, M, N, K, act, dtype, stream, &o, -1, 1.0f, false,
                                   1.0f, X, dY, dbias, true, part);
        if (s2 != FL_OK) return s2;
        hipLaunchKernelGGL(sum_rows_f32_kernel, dim3(grid_elementwise(N)), dim3(fl::kThreads), 0,
                           static_cast<hipStream_t>(stream), part, (int64_t)(need / ((size_t)N * 4)), (int64_t)N,
                           dbias);
        return check_launch("fused_linear_bwd (dbias sum)");
    }
    // dbias is a sum over every tile row: zero it first (a fill kernel on
    // the same stream), then the tiles add into it.
    if (dbias && N > 0) {
        const int blocks = grid_elementwise(N);
        hipLaunchKernelGGL(zero_f32_kernel, dim3(blocks), dim3(fl::kThreads), 0, static_cast<hipStream_t>(stream),
                           dbias, (int64_t)N);
        s = check_launch("fused_linear_bwd (dbias fill)");
        if (s != FL_OK) return s;
    }
    if (M == 0 || N == 0) return FL_OK;
    return launch_gemm(G, W, nullptr, nullptr, Y, dX, M, N, K, act, dtype, stream, &o, -1, 1.0f, false, 1.0f, X, dY,
                       dbias, true);
}

fl_status fl_fused_linear_bwd(const void *G, const void *W, const void *X, const void *Y, void *dX, void *dY,
                              float *dbias, int64_t M, int64_t N, int64_t K, fl_act act, fl_dtype dtype,
                              void *stream, const fl_options *opt) {
    clear_error();
    return bwd_impl(G, W, X, Y, dX, dY, dbias, M, N, K, act, dtype, stream, opt, false, nullptr, 0);
}

fl_status fl_bwd_workspace_bytes(int64_t M, int64_t N, int64_t K, fl_dtype dtype, size_t *bytes) {
    clear_error();
    if (!bytes) return fail(FL_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = 0;
    if (dtype != FL_F16 && dtype != FL_BF16)
        return fail(dtype == FL_F32 ? FL_ERR_UNSUPPORTED : FL_ERR_INVALID_ARG,
                    "the backward epilogue is built for fp16 and bf16");
    const fl_status s = check_dims(M, N, K);
    if (s != FL_OK) return s;
    *bytes = bwd_part_bytes(M, N);
    return FL_OK;
}

fl_status fl_fused_linear_bwd_ws(const void *G, const void *W, const void *X, const void *Y, void *dX, void *dY,
                                 float *dbias, int64_t M, int64_t N, int64_t K, fl_act act, fl_dtype dtype,
                                 void *stream, const fl_options *opt, void *workspace, size_t workspace_bytes) {
    clear_error();
    return bwd_impl(G, W, X, Y, dX, dY, dbias, M, N, K, act, dtype, stream, opt, true, workspace, workspace_bytes);
}

// The partial column sums of fl_fused_linear_bwd_noalloc live here: one
// fixed array per GPU, held until the process ends.  In host code this name
// is only a stand-in for the symbol; the device address of each GPU's copy
// comes from hipGetSymbolAddress (scratch_on_current_device) and only that
// address is passed to kernels.
constexpr size_t kNoAllocScratchBytes = size_t(8) << 20;
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_addr[kMaxScratchDevices];

// The device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
fl_status scratch_on_current_device(void **addr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(FL_ERR_LAUNCH, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxScratchDevices)
        return fail(FL_ERR_UNSUPPORTED, "device %d: the static scratch serves devices 0..%d", dev,
                    kMaxScratchDevices - 1);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(FL_ERR_LAUNCH, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                        hipGetErrorString(e));
        g_scratch_addr[dev] = p;
    }
    *addr = g_scratch_addr[dev];
    return FL_OK;
}
}  // namespace

fl_status fl_fused_linear_bwd_noalloc(const void *G, const void *W, const void *X, const void *Y, void *dX,
                                      void *dY, float *dbias, int64_t M, int64_t N, int64_t K, fl_act act,
                                      fl_dtype dtype, void *stream, const fl_options *opt) {
    clear_error();
    const fl_status s = check_dims(M, N, K);
    if (s != FL_OK) return s;
    const size_t need = dbias ? bwd_part_bytes(M, N) : 0;
    if (need > kNoAllocScratchBytes)
        return fail(FL_ERR_UNSUPPORTED,
                    "fl_fused_linear_bwd_noalloc: dbias of this shape needs %zu bytes of scratch; the static scratch "
                    "holds %zu (2 * ceil(M/256) * N * 4 bytes must fit)",
                    need, kNoAllocScratchBytes);
    void *ws = nullptr;
    if (need) {
        // every other argument is checked before the first HIP call
        const fl_status v = bwd_impl(G, W, X, Y, dX, dY, dbias, M, N, K, act, dtype, nullptr, opt, true, nullptr,
                                     0, /*check_only=*/true);
        if (v != FL_OK) return v;
        const fl_status a = scratch_on_current_device(&ws);
        if (a != FL_OK) return a;
    }
    return bwd_impl(G, W, X, Y, dX, dY, dbias, M, N, K, act, dtype, stream, opt, true, ws, kNoAllocScratchBytes);
}

fl_status fl_gemm_nt(const void *A, const void *Bt, void *D, int64_t M, int64_t N, int64_t K, fl_dtype dtype,
                     void *stream) {
    clear_error();
    if (dtype == FL_F32) return fail(FL_ERR_UNSUPPORTED, "the transposed-B product is built for fp16 and bf16");
    fl_status s = validate_gemm(A, Bt, nullptr, nullptr, nullptr, D, M, N, K, FL_ACT_NONE, dtype, nullptr, false,
                                /*b_kn=*/false);
    if (s != FL_OK) return s;
    if (M == 0 || N == 0) return FL_OK;
    const fl_options o = bwd_tiles(dtype, M, N, K);
    return launch_gemm(A, Bt, nullptr, nullptr, nullptr, D, M, N, K, FL_ACT_NONE, dtype, stream, &o, -1, 1.0f, false,
                       1.0f, nullptr, nullptr, nullptr, true);
}

fl_status fl_activation_grad(const void *D, const void *X, const void *Y, void *dX, void *dY, int64_t M, int64_t N,
                             fl_act act, fl_dtype dtype, void *stream) {
    clear_error();
    if (!valid_dtype(dtype)) return fail(FL_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
    if (!valid_act(act)) return fail(FL_ERR_INVALID_ARG, "unknown activation %d", (int)act);
    if (dtype == FL_F32) return fail(FL_ERR_UNSUPPORTED, "the backward passes are built for fp16 and bf16");
    fl_status s = check_dims(M, N, 0);
    if (s != FL_OK) return s;
    const size_t es = elem_size(dtype), bytes = (size_t)M * N * es;
    if (bytes == 0) return FL_OK;
    if (!D || !X || !dX) return fail(FL_ERR_INVALID_ARG, "D, X and dX must not be NULL");
    if (act == FL_ACT_GLU && (!Y || !dY)) return fail(FL_ERR_INVALID_ARG, "the gate's backward needs Y and dY");
    if (act != FL_ACT_GLU && (Y || dY)) return fail(FL_ERR_INVALID_ARG, "Y and dY are only used by the gate");
    const void *ptrs[5] = {D, X, Y, dX, dY};
    for (const void *p : ptrs)
        if (p && !aligned(p, es)) return fail(FL_ERR_INVALID_ARG, "pointer %p is not aligned to the element size", p);
    // dX may be D, dY may be Y; no other overlap among inputs and outputs
    if (dX != D && overlaps(dX, bytes, D, bytes)) return fail(FL_ERR_INVALID_ARG, "dX partially overlaps D");
    if (overlaps(dX, bytes, X, bytes) || (Y && overlaps(dX, bytes, Y, bytes)))
        return fail(FL_ERR_INVALID_ARG, "dX overlaps X or Y");
    if (dY) {
        if (dY != Y && overlaps(dY, bytes, Y, bytes)) return fail(FL_ERR_INVALID_ARG, "dY partially overlaps Y");
        if (overlaps(dY, bytes, D, bytes) || overlaps(dY, bytes, X, bytes) || overlaps(dY, bytes, dX, bytes))
            return fail(FL_ERR_INVALID_ARG, "dY overlaps D, X or dX");
    }
    const bool vec = aligned(D, 16) && aligned(X, 16) && aligned(dX, 16) && (!Y || aligned(Y, 16)) &&
                     (!dY || aligned(dY, 16));
    const int64_t total = (int64_t)(bytes / es);
    const int grid = grid_elementwise(vec ? total / (16 / (int64_t)es) + 1 : total);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const fl_status ls = launch_activation_grad(dtype, act, vec, grid, st, D, X, Y, dX, dY, total);
    if (ls != FL_OK) return ls;
    return check_launch("activation_grad");
}

fl_status fl_column_sum(const void *X, float *sums, int64_t M, int64_t N, fl_dtype dtype, void *stream) {
    clear_error();
    if (!valid_dtype(dtype)) return fail(FL_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
    if (dtype == FL_F32) return fail(FL_ERR_UNSUPPORTED, "the backward passes are built for fp16 and bf16");
    fl_status s = check_dims(M, N, 0);
    if (s != FL_OK) return s;
    if (N == 0) return FL_OK;
    const size_t es = elem_size(dtype), bytes = (size_t)M * N * es;
    if (!sums) return fail(FL_ERR_INVALID_ARG, "sums is NULL");
    if (!X && bytes) return fail(FL_ERR_INVALID_ARG, "X is NULL");
    if (!aligned(sums, 4) || (X && !aligned(X, es))) return fail(FL_ERR_INVALID_ARG, "misaligned pointer");
    if (overlaps(sums, (size_t)N * 4, X, bytes)) return fail(FL_ERR_INVALID_ARG, "sums overlaps X");
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(zero_f32_kernel, dim3(grid_elementwise(N)), dim3(fl::kThreads), 0, st, sums, (int64_t)N);
    s = check_launch("column_sum (fill)");
    if (s != FL_OK || M == 0) return s;
    const bool vec = (N % 8 == 0) && aligned(X, 16);
    const int64_t cpt = vec ? 8 : 1;
    const int64_t bands = (M + fl::kColRows - 1) / fl::kColRows;
    const dim3 grid((unsigned)((N / cpt + fl::kThreads - 1) / fl::kThreads), (unsigned)(bands < 4096 ? bands : 4096));
    if (dtype == FL_F16)
        launch_column_sum<FL_F16>(vec, grid, st, X, sums, M, N);
    else
        launch_column_sum<FL_BF16>(vec, grid, st, X, sums, M, N);
    return check_launch("column_sum");
}

fl_status fl_gemm(const void *A, const void *B, void *X, int64_t M, int64_t N, int64_t K, fl_dtype dtype,
                  void *stream) {
    clear_error();
    fl_status s = validate_gemm(A, B, nullptr, nullptr, nullptr, X, M, N, K, FL_ACT_NONE, dtype, nullptr);
    if (s != FL_OK) return s;
    return launch_gemm(A, B, nullptr, nullptr, nullptr, X, M, N, K, FL_ACT_NONE, dtype, stream, nullptr);
}

fl_status fl_bias_add(void *X, const void *bias, int64_t M, int64_t N, fl_dtype dtype, void *stream) {
    clear_error();
    if (!valid_dtype(dtype)) return fail(FL_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
    fl_status s = check_dims(M, N, 0);
    if (s != FL_OK) return s;
    const size_t es = elem_size(dtype);
    const size_t x_bytes = (size_t)M * N * es;
    if (!x_bytes) return FL_OK;
    if (!X) return fail(FL_ERR_INVALID_ARG, "X is NULL");
    if (!bias) return fail(FL_ERR_INVALID_ARG, "bias is NULL");
    if (!aligned(X, es) || !aligned(bias, es)) return fail(FL_ERR_INVALID_ARG, "pointer not aligned to element size");
    if (overlaps(X, x_bytes, bias, (size_t)N * es)) return fail(FL_ERR_INVALID_ARG, "X overlaps bias");
    const int vec = 16 / (int)es;
    const bool v = (N % vec == 0) && aligned(X, 16) && aligned(bias, 16);
    const int64_t items = v ? M * N / vec : M * N;
    const int grid = grid_elementwise(items);
    hipStream_t st = static_cast<hipStream_t>(stream);
#define FL_BIAS_LAUNCH(DT)                                                                          \
    if (v)                                                                                          \
        hipLaunchKernelGGL((fl::bias_add_kernel<DT, true>), dim3(grid), dim3(fl::kThreads), 0, st, X, bias, M, N); \
    else                                                                                            \
        hipLaunchKernelGGL((fl::bias_add_kernel<DT, false>), dim3(grid), dim3(fl::kThreads), 0, st, X, bias, M, N);
    if (dtype == FL_F32) {
        FL_BIAS_LAUNCH(FL_F32)
    } else if (dtype == FL_F16) {
        FL_BIAS_LAUNCH(FL_F16)
    } else {
        FL_BIAS_LAUNCH(FL_BF16)
    }
#undef FL_BIAS_LAUNCH
    return check_launch("bias_add");
}

}  // extern "C"

namespace {

template <int DT, int ACT>
void launch_act(bool v, int grid, hipStream_t st, const void *X, const void *Y, void *out, int64_t total) {
    if (v)
        hipLaunchKernelGGL((fl::activation_kernel<DT, ACT, true>), dim3(grid), dim3(fl::kThreads), 0, st, X, Y, out,
                           total);
    else
        hipLaunchKernelGGL((fl::activation_kernel<DT, ACT, false>), dim3(grid), dim3(fl::kThreads), 0, st, X, Y, out,
                           total);
}

template <int DT>
void launch_act_dt(int act, bool v, int grid, hipStream_t st, const void *X, const void *Y, void *out,
                   int64_t total) {
    switch (act) {
    case FL_ACT_NONE: launch_act<DT, FL_ACT_NONE>(v, grid, st, X, Y, out, total); break;
    case FL_ACT_RELU: launch_act<DT, FL_ACT_RELU>(v, grid, st, X, Y, out, total); break;
    case FL_ACT_GELU_TANH: launch_act<DT, FL_ACT_GELU_TANH>(v, grid, st, X, Y, out, total); break;
    default: launch_act<DT, FL_ACT_GLU>(v, grid, st, X, Y, out, total); break;
    }
}

}  // namespace

extern "C" {

fl_status fl_activation(const void *X, const void *Y, void *out, int64_t M, int64_t N, fl_act act, fl_dtype dtype,
                        void *stream) {
    clear_error();
    if (!valid_dtype(dtype)) return fail(FL_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
    if (!valid_act(act)) return fail(FL_ERR_INVALID_ARG, "unknown activation %d", (int)act);
    fl_status s = check_dims(M, N, 0);
    if (s != FL_OK) return s;
    const size_t es = elem_size(dtype);
    const size_t bytes = (size_t)M * N * es;
    if (act == FL_ACT_GLU && !Y && bytes) return fail(FL_ERR_INVALID_ARG, "the gate needs Y");
    if (act != FL_ACT_GLU && Y) return fail(FL_ERR_INVALID_ARG, "Y is only used by the gate (FL_ACT_GLU)");
    if (!bytes) return FL_OK;
    if (!X || !out) return fail(FL_ERR_INVALID_ARG, "X or out is NULL");
    if (!aligned(X, es) || !aligned(out, es) || (Y && !aligned(Y, es)))
        return fail(FL_ERR_INVALID_ARG, "pointer not aligned to element size");
    if (X != out && overlaps(X, bytes, out, bytes))
        return fail(FL_ERR_INVALID_ARG, "X partially overlaps out (only X == out is allowed)");
    if (Y && Y != out && overlaps(Y, bytes, out, bytes))
        return fail(FL_ERR_INVALID_ARG, "Y partially overlaps out (only Y == out is allowed)");
    const int vec = 16 / (int)es;
    const bool v = aligned(X, 16) && aligned(out, 16) && (!Y || aligned(Y, 16));
    const int64_t total = M * N;
    const int grid = grid_elementwise(v ? total / vec + 1 : total);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (dtype == FL_F32)
        launch_act_dt<FL_F32>(act, v, grid, st, X, Y, out, total);
    else if (dtype == FL_F16)
        launch_act_dt<FL_F16>(act, v, grid, st, X, Y, out, total);
    else
        launch_act_dt<FL_BF16>(act, v, grid, st, X, Y, out, total);
    return check_launch("activation");
}

fl_status fl_tile_grid(int64_t M, int64_t N, int64_t K, fl_dtype dtype, const fl_options *opt, int32_t *block_m,
                       int32_t *block_n, int32_t *tiles_m, int32_t *tiles_n) {
    clear_error();
    if (!valid_dtype(dtype)) return fail(FL_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
    fl_status s = check_dims(M, N, K);
    if (s != FL_OK) return s;
    TileShape t;
    s = tile_shape(dtype, M, N, K, opt, t);
    if (s != FL_OK) return s;
    if (!block_m || !block_n || !tiles_m || !tiles_n) return fail(FL_ERR_INVALID_ARG, "NULL output pointer");
    *block_m = t.bm;
    *block_n = t.bn;
    *tiles_m = (int32_t)((M + t.bm - 1) / t.bm);
    *tiles_n = (int32_t)((N + t.bn - 1) / t.bn);
    return FL_OK;
}

fl_status fl_tile_of_program(int32_t program, int32_t grid, int32_t tiles_m, int32_t tiles_n, int32_t group_m,
                             int32_t xcd_remap, int32_t *m_tile, int32_t *n_tile) {
    clear_error();
    if (tiles_m <= 0 || tiles_n <= 0 || group_m <= 0 || grid <= 0 || !m_tile || !n_tile)
        return fail(FL_ERR_INVALID_ARG, "bad tile-map arguments");
    if ((int64_t)tiles_m * tiles_n > kMaxDim) return fail(FL_ERR_UNSUPPORTED, "too many tiles");
    if (grid != tiles_m * tiles_n) return fail(FL_ERR_INVALID_ARG, "grid must equal tiles_m*tiles_n");
    if (program < 0 || program >= grid) return fail(FL_ERR_INVALID_ARG, "program out of range");
    const int pid = xcd_remap ? fl::xcd_logical(program, grid) : program;
    int m, n;
    fl::grouped_tile(pid, tiles_m, tiles_n, group_m, m, n);
    *m_tile = m;
    *n_tile = n;
    return FL_OK;
}

const char *fl_status_string(fl_status s) {
    switch (s) {
    case FL_OK: return "ok";
    case FL_ERR_INVALID_ARG: return "invalid argument";
    case FL_ERR_UNSUPPORTED: return "unsupported";
    case FL_ERR_LAUNCH: return "launch failed";
    default: return "unknown status";
    }
}

const char *fl_last_error(void) { return g_err; }

int fl_version(void) { return 10100; }

}  // extern "C"
