// fl_kernels.hpp -- gfx950 device code of the fused linear layer.
//
// out = act(A@B + bias): one MFMA GEMM per output tile whose epilogue runs on
// the fp32 accumulator registers after the whole K loop ("Epilogue concept",
// "Where the accumulator is finally correct"), plus the elementwise passes of
// the unfused chain ("Triton: Fused Matmul + Bias + ReLU", "The HBM traffic").
//
// Tile design (CDNA4, 64-wide waves, 160 KB LDS per CU):
//   * 256 threads = 4 waves in a 2x2 arrangement; each wave owns a 128x128
//     piece of the 256x256 output tile as 4x4 blocks of 32x32 MFMA
//     accumulators (16 fp32 per lane each, 256 per lane in total).
//   * Per K stage each tile row holds 128 bytes of K (64 fp16/bf16 or 32 fp32
//     values) as 8 chunks of 16 bytes.  A rows are K-contiguous in memory and
//     are copied as they are; B is N-contiguous, so each thread loads a square
//     block (8x8 halves or 4x4 floats) and transposes it in registers, which
//     makes B's LDS rows K-contiguous too.  Both operands are then read with
//     one 16-byte LDS read per lane per MFMA operand.
//   * LDS chunk placement is XOR-swizzled, chunk ^ ((row ^ row>>3) & 7), so
//     the 16-byte operand reads of 8 (or 16) consecutive lanes and the
//     transposed B writes hit distinct banks.
//   * Two LDS stages (2 x 64 KB): the next stage's global loads are in
//     flight in registers while the current stage's MFMAs run, and are
//     written to the other LDS stage afterwards; one barrier per stage.
//   * MFMA operands are swapped (B fragment first) so that the 32x32
//     accumulator layout puts 4 consecutive output columns of one output row
//     in each lane: the epilogue loads bias/Y and stores out 4 elements at a
//     time.
//   * Programs map to tiles through the grouped order of "Tiles and grouped
//     ownership" (band height min(group, tiles_m - first_m)), after an
//     optional XCD placement step: workgroups are dispatched round-robin over
//     the 8 XCDs, so consecutive program ids are regrouped so that each XCD
//     receives a contiguous run of grouped tiles and its own L2 serves the
//     shared A rows and B columns ("Optimizing GEMM + Activation on CDNA4
//     with TLX", "Version 2", L2 locality).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fused_linear.h"

namespace fl {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int v2u32_t __attribute__((ext_vector_type(2)));
typedef unsigned int v4u32_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kInFp8 = 3;  // A/B element type "OCP FP8 E4M3 codes" (template argument, not an fl_dtype)
constexpr int kChunks = 8;  // 16-byte chunks of K per LDS row per stage
constexpr int kNumXcd = 8;

// ------------------------------------------------------------ element types

template <int DT> struct Io;
template <> struct Io<FL_F32> {
    using raw = float;
    static constexpr int size = 4;
    __device__ static float to_f32(raw v) { return v; }
    __device__ static raw from_f32(float v) { return v; }
};
template <> struct Io<FL_F16> {
    using raw = uint16_t;
    static constexpr int size = 2;
    __device__ static float to_f32(raw v) { return (float)__builtin_bit_cast(_Float16, v); }
    __device__ static raw from_f32(float v) { return __builtin_bit_cast(uint16_t, (_Float16)v); }
    // a in the low half, b in the high half: one v_cvt_pk_f16_f32 (round to
    // nearest even, as the scalar conversion)
    __device__ static uint32_t pack2(float a, float b) {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, f16x2_t));
    }
};
template <> struct Io<FL_BF16> {
    using raw = uint16_t;
    static constexpr int size = 2;
    __device__ static float to_f32(raw v) { return __builtin_bit_cast(float, (uint32_t)v << 16); }
    __device__ static raw from_f32(float v) { return __builtin_bit_cast(uint16_t, (__bf16)v); }
    __device__ static uint32_t pack2(float a, float b) {  // one v_cvt_pk_bf16_f32
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
    }
};

// ------------------------------------------------------------- epilogue ops

// The activation applied to x = acc + bias (y is the gate operand), in fp32.
// GELU(tanh): with tanh(u) = 2 sigmoid(2u) - 1 the tanh form becomes
// x * sigmoid(2u) = x / (1 + 2^(-2u log2 e)), u = sqrt(2/pi) (x + 0.044715 x^3);
// one v_exp_f32 and one v_rcp_f32.  x -> -inf gives x * 0, x -> +inf gives x.
template <int ACT>
__device__ __forceinline__ float activate_math(float x, float y) {
    if constexpr (ACT == FL_ACT_RELU) {
        return __builtin_fmaxf(x, 0.0f);  // branchless clamp, float literal
    } else if constexpr (ACT == FL_ACT_GELU_TANH) {
        constexpr float k2u = 2.0f * 0.7978845608028654f * 1.4426950408889634f;
        float u = x * __builtin_fmaf(0.044715f * x, x, 1.0f);
        float e = __builtin_amdgcn_exp2f(-k2u * u);
        return x * __builtin_amdgcn_rcpf(1.0f + e);
    } else if constexpr (ACT == FL_ACT_GLU) {
        return __builtin_fmaf(x, y, x);  // X + X*Y as one fma
    } else {
        return x;
    }
}

// Derivative of the activation at x (the gate: d(X + X*Y)/dX = 1 + Y), in
// fp32, for the backward epilogue.  GELU(tanh) with s = sigmoid(2u) (the
// form used above): g = x s, so g' = s + x s (1 - s) 2 u', u' = sqrt(2/pi)
// (1 + 3 * 0.044715 x^2).  ReLU: 0 at x = 0.
template <int ACT>
__device__ __forceinline__ float activate_grad(float x, float y) {
    float r;
    if constexpr (ACT == FL_ACT_RELU) {
        r = x > 0.0f ? 1.0f : 0.0f;
    } else if constexpr (ACT == FL_ACT_GELU_TANH) {
        constexpr float kc = 0.7978845608028654f;
        constexpr float k2u = 2.0f * kc * 1.4426950408889634f;
        const float u = x * __builtin_fmaf(0.044715f * x, x, 1.0f);
        const float s = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-k2u * u));
        const float du2 = 2.0f * kc * __builtin_fmaf(3.0f * 0.044715f * x, x, 1.0f);
        r = __builtin_fmaf(x * s * (1.0f - s), du2, s);
    } else if constexpr (ACT == FL_ACT_GLU) {
        r = 1.0f + y;
    } else {
        r = 1.0f;
    }
    return r;
}

// The epilogue value, held as an fp32 register before any cast.  Without the
// empty asm the compiler may fold a following cast to a 16-bit type into the
// last fma (v_fma_mix with a 16-bit result rounds once where fp32 math and a
// cast round twice), differently from one kernel to the next; with it every
// kernel rounds to fp32 first and then casts once.
template <int ACT>
__device__ __forceinline__ float activate(float x, float y) {
    float r = activate_math<ACT>(x, y);
    asm("" : "+v"(r));
    return r;
}

// The quantized store ("Triton: Fused Matmul + Bias + ReLU (Epilogue
// Fusion)", "Variants": the value is scaled, limited and written as 8-bit codes):
// four epilogue values times the scale, in fp32, packed as four one-byte
// codes (first value in the low byte).  FP8: clamp to the largest finite
// E4M3 value 448, then the hardware conversion (round to nearest even, OCP
// E4M3); int8: round to nearest even, clamp to [-128, 127].
template <int QF>
__device__ __forceinline__ uint32_t quantize4(const float (&v)[4], float scale) {
    float u[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) u[e] = v[e] * scale;
    if constexpr (QF == FL_Q_FP8_E4M3) {
#pragma unroll
        for (int e = 0; e < 4; ++e) u[e] = __builtin_fminf(__builtin_fmaxf(u[e], -448.0f), 448.0f);
        int w = __builtin_amdgcn_cvt_pk_fp8_f32(u[0], u[1], 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(u[2], u[3], w, true);
        return (uint32_t)w;
    } else {
        uint32_t w = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float r = __builtin_fminf(__builtin_fmaxf(__builtin_rintf(u[e]), -128.0f), 127.0f);
            w |= ((uint32_t)(int)r & 0xffu) << (8 * e);
        }
        return w;
    }
}

// ------------------------------------------------------------- tile order

// Grouped program -> (m_tile, n_tile): bands of `group` M-tiles are swept
// column by column; the last band may be shorter.
__host__ __device__ inline void grouped_tile(int pid, int tiles_m, int tiles_n, int group,
                                             int &m_tile, int &n_tile) {
    const int per_band = group * tiles_n;
    const int band = pid / per_band;
    const int first_m = band * group;
    const int rest = tiles_m - first_m;
    const int height = rest < group ? rest : group;
    const int r = pid - band * per_band;
    m_tile = first_m + r % height;
    n_tile = r / height;
}

// Program b of a grid of n runs on XCD b % 8.  Return the logical index that
// gives XCD x the contiguous run [start(x), start(x) + count(x)).
__host__ __device__ inline int xcd_logical(int b, int n) {
    const int q = n / kNumXcd, r = n % kNumXcd;
    const int x = b % kNumXcd, i = b / kNumXcd;
    return x * q + (x < r ? x : r) + i;
}

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row ^ (row >> 3)) & 7); }

// ------------------------------------------------------------ buffer access

// Raw buffer resource (gfx9 family word 3: 32-bit data format).  A lane whose
// byte offset is at or beyond num_records reads zero and its store is
// dropped, so masked loads/stores need no branches: invalid lanes use kOob.
constexpr uint32_t kOob = 0x80000000u;
constexpr uint32_t kRsrcWord3 = 0x00020000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, size_t bytes) {
    const int n = bytes > 0x7fffffffull ? 0x7fffffff : (int)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, n, (int)kRsrcWord3);
}

template <int SIZE> struct RawBits;
template <> struct RawBits<2> { using T = uint16_t; };
template <> struct RawBits<4> { using T = uint32_t; };

template <int SIZE>
__device__ __forceinline__ typename RawBits<SIZE>::T load_elem(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    if constexpr (SIZE == 2)
        return (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
    else
        return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

template <int SIZE>
__device__ __forceinline__ void store_elem(typename RawBits<SIZE>::T v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
    if constexpr (SIZE == 2)
        __builtin_amdgcn_raw_buffer_store_b16(v, r, off, 0, 0);
    else
        __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, 0);
}

// ------------------------------------------------------------- fused GEMM

struct GemmArgs {
    const void *A;
    const void *B;
    const void *bias;  // may be null
    const void *Y;     // gate operand or null
    const void *R;     // residual (M,N) added before the activation, or null
    float scale;       // quantized output: codes of (epilogue value) * scale
    int stream_out;    // nonzero: every output row starts on a 128-byte line (streaming stores)
    float ab_scale;    // FP8 inputs: accumulator scale (product of A's and B's per-tensor scales)
    const void *Xs;    // backward: the saved pre-activation X (M,N); B is then (N,K) row-major
    void *dY;          // backward, gate: the second output D*X (M,N)
    float *dbias;      // backward: column sums of dX (N,), fp32, added to atomically
    float *dbias_part; // backward, or null: per (tile row, wave row) column sums of dX, (2*tiles_m, N)
                       // fp32, written instead of the atomics (dbias is left alone then)
    void *out;
    int M, N, K;
    int tiles_m, tiles_n, group;
    int xcd_remap;
    int persistent;   // nonzero: loop over tiles with stride gridDim.x
    uint32_t *tile_count;
    int debug_sync;   // nonzero: an extra full wait and barrier in every K stage (same results)
};

template <int DT, int ACT, bool VECTOR>
struct FusedTile {
    using io = Io<DT>;
    using raw = typename io::raw;
    using bits = typename RawBits<io::size>::T;
    static constexpr int ES = io::size;
    static constexpr int VEC = 16 / ES;                // elements per 16-byte chunk
    static constexpr int BKE = VEC * kChunks;          // K elements per stage
    static constexpr int BM = 256, BN = 256;
    static constexpr int STAGE = (BM + BN) * kChunks;  // u32x4 per stage
    static constexpr int BLK_PER_KROW = BN / VEC;      // B blocks across N
    static constexpr int BLK_PER_THREAD = kChunks * BLK_PER_KROW / kThreads;
    static_assert(BLK_PER_THREAD * VEC == 8, "8 B chunks per thread");

    // --- global -> registers (one stage) ---
    // Buffers are rebased at the stage origin, so every in-tile byte offset
    // fits 32 bits (256 * K * ES and 64 * N * ES are below 2^31, checked on
    // the host).  Out-of-range chunks/elements read as zero.
    __device__ __forceinline__ static void load_stage(const GemmArgs &a, int m0, int n0, int k0, int tid,
                                                      u32x4_t (&ra)[8], u32x4_t (&rb)[8]) {
        const size_t a_org = (size_t)m0 * a.K + k0;
        const size_t b_org = (size_t)k0 * a.N + n0;
        const __amdgpu_buffer_rsrc_t rA =
            make_rsrc(static_cast<const char *>(a.A) + a_org * ES, ((size_t)a.M * a.K - a_org) * ES);
        const __amdgpu_buffer_rsrc_t rB =
            make_rsrc(static_cast<const char *>(a.B) + b_org * ES, ((size_t)a.K * a.N - b_org) * ES);
        const int ca = tid & 7, r0 = tid >> 3;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int row = r0 + 32 * i;
            const bool row_ok = m0 + row < a.M;
            if constexpr (VECTOR) {
                const bool ok = row_ok && (k0 + ca * VEC < a.K);
                const uint32_t off = ok ? (uint32_t)(row * a.K + ca * VEC) * ES : kOob;
                ra[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rA, off, 0, 0));
            } else {
                bits e[VEC];
#pragma unroll
                for (int t = 0; t < VEC; ++t) {
                    const bool ok = row_ok && (k0 + ca * VEC + t < a.K);
                    const uint32_t off = ok ? (uint32_t)(row * a.K + ca * VEC + t) * ES : kOob;
                    e[t] = load_elem<ES>(rA, off);
                }
                ra[i] = __builtin_bit_cast(u32x4_t, e);
            }
        }
#pragma unroll
        for (int j = 0; j < BLK_PER_THREAD; ++j) {
            const int b = tid + kThreads * j;
            const int kb = b / BLK_PER_KROW, nb = b % BLK_PER_KROW;
            if constexpr (VECTOR) {
                // rows of the block as stored in memory (N-contiguous); transposed later
                const bool col_ok = n0 + nb * VEC < a.N;
#pragma unroll
                for (int r = 0; r < VEC; ++r) {
                    const int kr = kb * VEC + r;
                    const bool ok = col_ok && (k0 + kr < a.K);
                    const uint32_t off = ok ? (uint32_t)(kr * a.N + nb * VEC) * ES : kOob;
                    rb[j * VEC + r] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rB, off, 0, 0));
                }
            } else {
                // element loads land directly in K-contiguous order
#pragma unroll
                for (int c = 0; c < VEC; ++c) {
                    bits e[VEC];
                    const bool col_ok = n0 + nb * VEC + c < a.N;
#pragma unroll
                    for (int r = 0; r < VEC; ++r) {
                        const int kr = kb * VEC + r;
                        const bool ok = col_ok && (k0 + kr < a.K);
                        const uint32_t off = ok ? (uint32_t)(kr * a.N + nb * VEC + c) * ES : kOob;
                        e[r] = load_elem<ES>(rB, off);
                    }
                    rb[j * VEC + c] = __builtin_bit_cast(u32x4_t, e);
                }
            }
        }
    }

    // --- registers -> LDS (one stage), transposing B blocks ---
    __device__ __forceinline__ static void store_stage(u32x4_t *s, int tid, const u32x4_t (&ra)[8],
                                                       const u32x4_t (&rb)[8]) {
        const int ca = tid & 7, r0 = tid >> 3;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int row = r0 + 32 * i;
            s[row * kChunks + swz(row, ca)] = ra[i];
        }
        u32x4_t *sb = s + BM * kChunks;
#pragma unroll
        for (int j = 0; j < BLK_PER_THREAD; ++j) {
            const int b = tid + kThreads * j;
            const int kb = b / BLK_PER_KROW, nb = b % BLK_PER_KROW;
            u32x4_t t[VEC];
            if constexpr (VECTOR) {
                if constexpr (VEC == 8) {
                    // 8x8 halves: t[c] holds column c of the block (8 k values)
#pragma unroll
                    for (int c = 0; c < 8; ++c) {
#pragma unroll
                        for (int d = 0; d < 4; ++d) {
                            const uint32_t lo = rb[j * 8 + 2 * d][c >> 1];
                            const uint32_t hi = rb[j * 8 + 2 * d + 1][c >> 1];
                            t[c][d] = (c & 1) ? ((lo >> 16) | (hi & 0xffff0000u))
                                              : ((lo & 0xffffu) | (hi << 16));
                        }
                    }
                } else {
                    // 4x4 floats
#pragma unroll
                    for (int c = 0; c < 4; ++c)
#pragma unroll
                        for (int r = 0; r < 4; ++r) t[c][r] = rb[j * 4 + r][c];
                }
            } else {
#pragma unroll
                for (int c = 0; c < VEC; ++c) t[c] = rb[j * VEC + c];
            }
#pragma unroll
            for (int c = 0; c < VEC; ++c) {
                const int row = nb * VEC + c;
                sb[row * kChunks + swz(row, kb)] = t[c];
            }
        }
    }

    // --- MFMAs over one LDS stage ---
    __device__ __forceinline__ static void compute_stage(const u32x4_t *s, int wm, int wn, int lane,
                                                         f32x16_t (&acc)[4][4]) {
        const int lrow = lane & 31, lg = lane >> 5;
        const u32x4_t *sa = s;
        const u32x4_t *sb = s + BM * kChunks;
#pragma unroll
        for (int kk = 0; kk < kChunks / 2; ++kk) {
            u32x4_t af[4], bf[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ar = wm * 128 + i * 32 + lrow;
                af[i] = sa[ar * kChunks + swz(ar, kk * 2 + lg)];
                const int br = wn * 128 + i * 32 + lrow;
                bf[i] = sb[br * kChunks + swz(br, kk * 2 + lg)];
            }
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
                for (int ni = 0; ni < 4; ++ni) {
                    if constexpr (DT == FL_F16) {
                        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                            __builtin_bit_cast(f16x8_t, bf[ni]), __builtin_bit_cast(f16x8_t, af[mi]),
                            acc[mi][ni], 0, 0, 0);
                    } else if constexpr (DT == FL_BF16) {
                        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            __builtin_bit_cast(bf16x8_t, bf[ni]), __builtin_bit_cast(bf16x8_t, af[mi]),
                            acc[mi][ni], 0, 0, 0);
                    } else {
                        // Reinterpret whole vectors: bit_cast of a single
                        // ext-vector element miscompiles (always element 0).
                        const f32x4_t bv = __builtin_bit_cast(f32x4_t, bf[ni]);
                        const f32x4_t av = __builtin_bit_cast(f32x4_t, af[mi]);
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x2f32(bv[e], av[e], acc[mi][ni], 0, 0, 0);
                    }
                }
            }
        }
    }

    // Raw bits of 4 consecutive elements (8 bytes for fp16/bf16, 16 for fp32).
    using quad_t = typename std::conditional<ES == 2, u32x2_t, u32x4_t>::type;

    // Load 4 consecutive elements at byte offset off: one 8- or 16-byte access
    // when all 4 are in range on the vector path, else element by element
    // (elements past `valid`, or the whole group when off is kOob, read 0).
    __device__ __forceinline__ static quad_t load4(__amdgpu_buffer_rsrc_t r, uint32_t off, int valid) {
        if (VECTOR && valid >= 4) {
            if constexpr (ES == 2)
                return __builtin_bit_cast(quad_t, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
            else
                return __builtin_bit_cast(quad_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
        } else {
            bits e[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) e[i] = load_elem<ES>(r, i < valid ? off + i * ES : kOob);
            return __builtin_bit_cast(quad_t, e);
        }
    }

    __device__ __forceinline__ static float elem_f32(const quad_t &q, int i) {
        if constexpr (ES == 2)
            return io::to_f32(raw((i & 1) ? (q[i >> 1] >> 16) : (q[i >> 1] & 0xffffu)));
        else
            return __builtin_bit_cast(f32x4_t, q)[i];
    }

    // --- epilogue: bias, activation, one conversion, one masked store ---
    // Lane (lrow, lg) of wave (wm, wn) holds, for block (mi, ni) and group q,
    // out[m0 + wm*128 + mi*32 + lrow][n0 + wn*128 + ni*32 + q*8 + lg*4 + 0..3]
    // in acc[mi][ni][q*4 + 0..3].  Offsets are relative to (m0, n0).
    // gfx9 counts stores in vmcnt, so a load issued after a store makes its
    // consumer wait for that store too.  The bias of all 16 column groups is
    // therefore loaded before any store, and the gate operand of row block
    // mi+1 is loaded before the stores of row block mi.
    __device__ __forceinline__ static void epilogue(const GemmArgs &a, int m0, int n0, int wm, int wn, int lane,
                                                    const f32x16_t (&acc)[4][4]) {
        const size_t o_org = (size_t)m0 * a.N + n0;
        const size_t o_bytes = ((size_t)a.M * a.N - o_org) * ES;
        const __amdgpu_buffer_rsrc_t rO = make_rsrc(static_cast<char *>(a.out) + o_org * ES, o_bytes);
        const __amdgpu_buffer_rsrc_t rY =
            make_rsrc(a.Y ? static_cast<const char *>(a.Y) + o_org * ES : nullptr, a.Y ? o_bytes : 0);
        const bool has_r = a.R != nullptr;
        const __amdgpu_buffer_rsrc_t rR =
            make_rsrc(has_r ? static_cast<const char *>(a.R) + o_org * ES : nullptr, has_r ? o_bytes : 0);
        const __amdgpu_buffer_rsrc_t rBias =
            make_rsrc(a.bias ? static_cast<const char *>(a.bias) + (size_t)n0 * ES : nullptr,
                      a.bias ? (size_t)(a.N - n0) * ES : 0);
        const int lrow = lane & 31, lg = lane >> 5;
        int col[16], valid[16];
#pragma unroll
        for (int g = 0; g < 16; ++g) {
            col[g] = wn * 128 + (g >> 2) * 32 + (g & 3) * 8 + lg * 4;  // g = ni*4 + q
            valid[g] = a.N - n0 - col[g];
        }
        quad_t bq[16];
#pragma unroll
        for (int g = 0; g < 16; ++g) {
            bq[g] = quad_t{};
            if (a.bias) bq[g] = load4(rBias, valid[g] > 0 ? (uint32_t)col[g] * ES : kOob, valid[g]);
        }
        auto offset = [&](int mi, int g) -> uint32_t {
            const int row = wm * 128 + mi * 32 + lrow;
            return (m0 + row < a.M && valid[g] > 0) ? (uint32_t)(row * a.N + col[g]) * ES : kOob;
        };
        quad_t yq[2][16];
        if constexpr (ACT == FL_ACT_GLU) {
#pragma unroll
            for (int g = 0; g < 16; ++g) yq[0][g] = load4(rY, offset(0, g), valid[g]);
        }
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            if constexpr (ACT == FL_ACT_GLU) {
                if (mi + 1 < 4) {
#pragma unroll
                    for (int g = 0; g < 16; ++g) yq[(mi + 1) & 1][g] = load4(rY, offset(mi + 1, g), valid[g]);
                }
            }
#pragma unroll
            for (int g = 0; g < 16; ++g) {
                const int ni = g >> 2, q = g & 3;
                const uint32_t off = offset(mi, g);
                // residual of this group, read (like Y) before this row block's stores
                quad_t rq = quad_t{};
                if (has_r) rq = load4(rR, off, valid[g]);
                bits o[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float y = (ACT == FL_ACT_GLU) ? elem_f32(yq[mi & 1][g], e) : 0.0f;
                    float x = acc[mi][ni][q * 4 + e] + elem_f32(bq[g], e);
                    if (has_r) x += elem_f32(rq, e);
                    o[e] = __builtin_bit_cast(bits, io::from_f32(activate<ACT>(x, y)));
                }
                if (VECTOR && valid[g] >= 4) {
                    if constexpr (ES == 2) {
                        u32x2_t w;
                        w[0] = (uint32_t)o[0] | ((uint32_t)o[1] << 16);
                        w[1] = (uint32_t)o[2] | ((uint32_t)o[3] << 16);
                        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2u32_t, w), rO, off, 0, 0);
                    } else {
                        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u32_t, o), rO, off, 0, 0);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) store_elem<ES>(o[e], rO, e < valid[g] ? off + e * ES : kOob);
                }
            }
            // One row block at a time: without this the scheduler reads
            // every accumulator out of the AGPRs up front and spills.
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    __device__ __forceinline__ static void run_tile(const GemmArgs &a, int pid, u32x4_t *smem) {
        const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
        const int wm = wave >> 1, wn = wave & 1;
        int tm, tn;
        grouped_tile(pid, a.tiles_m, a.tiles_n, a.group, tm, tn);
        const int m0 = tm * BM, n0 = tn * BN;

        f32x16_t acc[4][4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int ni = 0; ni < 4; ++ni)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[mi][ni][e] = 0.0f;

        const int nk = (a.K + BKE - 1) / BKE;
        if (nk > 0) {
            u32x4_t ra[8], rb[8];
            load_stage(a, m0, n0, 0, tid, ra, rb);
            store_stage(smem, tid, ra, rb);
            __syncthreads();
            for (int kt = 0; kt < nk; ++kt) {
                u32x4_t *cur = smem + (kt & 1) * STAGE;
                u32x4_t *nxt = smem + ((kt + 1) & 1) * STAGE;
                const bool more = kt + 1 < nk;
                if (more) load_stage(a, m0, n0, (kt + 1) * BKE, tid, ra, rb);
                compute_stage(cur, wm, wn, lane, acc);
                if (more) store_stage(nxt, tid, ra, rb);
                __syncthreads();
                if (a.debug_sync) __syncthreads();
            }
        }
        epilogue(a, m0, n0, wm, wn, lane, acc);
        if (a.tile_count && tid == 0) atomicAdd(&a.tile_count[tm * a.tiles_n + tn], 1u);
    }
};

template <int DT, int ACT, bool VECTOR>
__global__ void __launch_bounds__(kThreads, 1) fused_linear_kernel(GemmArgs a) {
    using T = FusedTile<DT, ACT, VECTOR>;
    __shared__ u32x4_t smem[2 * T::STAGE];
    const int ntiles = a.tiles_m * a.tiles_n;
    if (!a.persistent) {
        const int pid = a.xcd_remap ? xcd_logical(blockIdx.x, gridDim.x) : (int)blockIdx.x;
        T::run_tile(a, pid, smem);
    } else {
        const int G = gridDim.x;
        const int slot = a.xcd_remap ? xcd_logical(blockIdx.x, G) : (int)blockIdx.x;
        for (int base = 0; base < ntiles; base += G) {
            const int pid = base + slot;
            if (pid < ntiles) T::run_tile(a, pid, smem);
            __syncthreads();  // LDS of this tile is dead before the next one loads
        }
    }
}

// ------------------------------------------------------ unfused elementwise

// X[i,j] += bias[j] in place, rounded once to dtype.  VECTOR: N % VEC == 0
// and 16-byte aligned pointers, so a 16-byte chunk never crosses a row.
template <int DT, bool VECTOR>
__global__ void __launch_bounds__(kThreads) bias_add_kernel(void *Xv, const void *biasv, int64_t M,
                                                           int64_t N) {
    using io = Io<DT>;
    using raw = typename io::raw;
    constexpr int VEC = 16 / io::size;
    raw *X = static_cast<raw *>(Xv);
    const raw *bias = static_cast<const raw *>(biasv);
    const int64_t total = M * N;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    if constexpr (VECTOR) {
        const int64_t nchunks = total / VEC;
        for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < nchunks; c += stride) {
            const int64_t e0 = c * VEC;
            const int64_t n = e0 % N;
            u32x4_t xv = *reinterpret_cast<const u32x4_t *>(X + e0);
            const u32x4_t bv = *reinterpret_cast<const u32x4_t *>(bias + n);
            raw xs[VEC], bs[VEC], os[VEC];
            __builtin_memcpy(xs, &xv, 16);
            __builtin_memcpy(bs, &bv, 16);
#pragma unroll
            for (int t = 0; t < VEC; ++t) os[t] = io::from_f32(io::to_f32(xs[t]) + io::to_f32(bs[t]));
            __builtin_memcpy(&xv, os, 16);
            *reinterpret_cast<u32x4_t *>(X + e0) = xv;
        }
    } else {
        for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += stride)
            X[e] = io::from_f32(io::to_f32(X[e]) + io::to_f32(bias[e % N]));
    }
}

// The unfused backward chain's second pass, elementwise: dX = D * act'(X)
// and, for the gate, dY = D * X, each rounded once to the I/O dtype (D may be
// dX and Y may be dY: each element is read before it is written, by the same
// thread).  VECTOR: 16-byte aligned pointers; the tail that does not fill a
// chunk is done element by element.
template <int DT, int ACT, bool VECTOR>
__global__ void __launch_bounds__(kThreads) activation_grad_kernel(const void *Dv, const void *Xv, const void *Yv,
                                                                   void *dXv, void *dYv, int64_t total) {
    using io = Io<DT>;
    using raw = typename io::raw;
    constexpr int VEC = 16 / io::size;
    const raw *D = static_cast<const raw *>(Dv);
    const raw *X = static_cast<const raw *>(Xv);
    const raw *Y = static_cast<const raw *>(Yv);
    raw *dX = static_cast<raw *>(dXv);
    raw *dY = static_cast<raw *>(dYv);
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    auto one = [&](raw d16, raw x16, raw y16, raw &dx16, raw &dy16) {
        const float d = io::to_f32(d16), x = io::to_f32(x16);
        float dx = d * activate_grad<ACT>(x, ACT == FL_ACT_GLU ? io::to_f32(y16) : 0.0f);
        asm("" : "+v"(dx));
        dx16 = io::from_f32(dx);
        float dy = d * x;
        asm("" : "+v"(dy));
        dy16 = io::from_f32(dy);
    };
    int64_t done = 0;
    if constexpr (VECTOR) {
        const int64_t nchunks = total / VEC;
        for (int64_t c = gid; c < nchunks; c += stride) {
            const u32x4_t dv = *reinterpret_cast<const u32x4_t *>(D + c * VEC);
            const u32x4_t xv = *reinterpret_cast<const u32x4_t *>(X + c * VEC);
            u32x4_t yv = {0u, 0u, 0u, 0u};
            if constexpr (ACT == FL_ACT_GLU) yv = *reinterpret_cast<const u32x4_t *>(Y + c * VEC);
            raw ds[VEC], xs[VEC], ys[VEC], ox[VEC], oy[VEC];
            __builtin_memcpy(ds, &dv, 16);
            __builtin_memcpy(xs, &xv, 16);
            __builtin_memcpy(ys, &yv, 16);
#pragma unroll
            for (int t = 0; t < VEC; ++t) one(ds[t], xs[t], ys[t], ox[t], oy[t]);
            u32x4_t o;
            __builtin_memcpy(&o, ox, 16);
            *reinterpret_cast<u32x4_t *>(dX + c * VEC) = o;
            if constexpr (ACT == FL_ACT_GLU) {
                __builtin_memcpy(&o, oy, 16);
                *reinterpret_cast<u32x4_t *>(dY + c * VEC) = o;
            }
        }
        done = nchunks * VEC;
    }
    for (int64_t e = done + gid; e < total; e += stride) {
        raw ox, oy;
        one(D[e], X[e], ACT == FL_ACT_GLU ? Y[e] : raw(0), ox, oy);
        dX[e] = ox;
        if constexpr (ACT == FL_ACT_GLU) dY[e] = oy;
    }
}

// The unfused backward chain's third pass: sums[j] += the fp32 sum of X[i, j]
// over rows (sums zeroed first by the caller).  Block (bx, by) takes
// kThreads column groups of CPT columns (one 16-byte load per row when
// VECTOR) and the bands of kColRows rows by, by + gridDim.y, ...; one fp32
// atomic per column and block, so the order of the additions is not fixed.
constexpr int kColRows = 64;  // rows per band
template <int DT, bool VECTOR>
__global__ void __launch_bounds__(kThreads) column_sum_kernel(const void *Xv, float *sums, int64_t M, int64_t N) {
    using io = Io<DT>;
    using raw = typename io::raw;
    constexpr int CPT = VECTOR ? 16 / io::size : 1;  // columns per thread
    const raw *X = static_cast<const raw *>(Xv);
    const int64_t j0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * CPT;
    if (j0 >= N) return;
    float acc[CPT];
#pragma unroll
    for (int t = 0; t < CPT; ++t) acc[t] = 0.0f;
    for (int64_t band = blockIdx.y; band * kColRows < M; band += gridDim.y) {
        const int64_t r0 = band * kColRows, r1 = r0 + kColRows < M ? r0 + kColRows : M;
#pragma unroll 8
        for (int64_t i = r0; i < r1; ++i) {
            if constexpr (VECTOR) {
                const u32x4_t v = *reinterpret_cast<const u32x4_t *>(X + i * N + j0);
                raw xs[CPT];
                __builtin_memcpy(xs, &v, 16);
#pragma unroll
                for (int t = 0; t < CPT; ++t) acc[t] += io::to_f32(xs[t]);
            } else {
                acc[0] += io::to_f32(X[i * N + j0]);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < CPT; ++t) unsafeAtomicAdd(sums + j0 + t, acc[t]);
}

// out = act(X[, Y]) elementwise.  VECTOR: 16-byte aligned pointers; the
// tail that does not fill a chunk is done element by element.
template <int DT, int ACT, bool VECTOR>
__global__ void __launch_bounds__(kThreads) activation_kernel(const void *Xv, const void *Yv, void *outv,
                                                             int64_t total) {
    using io = Io<DT>;
    using raw = typename io::raw;
    constexpr int VEC = 16 / io::size;
    const raw *X = static_cast<const raw *>(Xv);
    const raw *Y = static_cast<const raw *>(Yv);
    raw *out = static_cast<raw *>(outv);
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    int64_t done = 0;
    if constexpr (VECTOR) {
        const int64_t nchunks = total / VEC;
        for (int64_t c = gid; c < nchunks; c += stride) {
            const u32x4_t xv = *reinterpret_cast<const u32x4_t *>(X + c * VEC);
            u32x4_t yv = {0u, 0u, 0u, 0u};
            if constexpr (ACT == FL_ACT_GLU) yv = *reinterpret_cast<const u32x4_t *>(Y + c * VEC);
            raw xs[VEC], ys[VEC], os[VEC];
            __builtin_memcpy(xs, &xv, 16);
            __builtin_memcpy(ys, &yv, 16);
#pragma unroll
            for (int t = 0; t < VEC; ++t)
                os[t] = io::from_f32(activate<ACT>(io::to_f32(xs[t]), ACT == FL_ACT_GLU ? io::to_f32(ys[t]) : 0.f));
            u32x4_t ov;
            __builtin_memcpy(&ov, os, 16);
            *reinterpret_cast<u32x4_t *>(out + c * VEC) = ov;
        }
        done = nchunks * VEC;
    }
    for (int64_t e = done + gid; e < total; e += stride) {
        const float y = (ACT == FL_ACT_GLU) ? io::to_f32(Y[e]) : 0.f;
        out[e] = io::from_f32(activate<ACT>(io::to_f32(X[e]), y));
    }
}

// ------------------------------------------------------------ launchers

typedef void (*fused_launcher)(const GemmArgs &, int grid, hipStream_t);

// Kernel variants (selected on the host, see fused_linear.hip).
enum Variant {
    kRegStaged = 1,     // FusedTile: register-staged loads, 256x256, any dtype; `vec` picks the load path
    kDirect64x256 = 0,  // Dma16 BK 64, 256x256 (fp16/bf16)
    kDirect32x256 = 2,  // Dma16 BK 32, 256x256
    kDirect64x128 = 4,  // Dma16 BK 64, 256x128
    kDirect64x256W8 = 5,  // Dma16 BK 64, 256x256, 8 waves (two per SIMD)
    kDirect32x128Occ2 = 6,  // Dma16 BK 32, 256x128, two workgroups per CU
    kDirect64x192 = 7,  // Dma16 BK 64, 256x192 (a width that is not a power of two), 4 waves
    kDirect32x192 = 8,  // Dma16 BK 32, 256x192, 4 waves
    kDirect64x256M16 = 9,     // Dma16 BK 64, 256x256, 4 waves, 16x16x32 MFMA blocks
    kDirect64x256W8M16 = 10,  // Dma16 BK 64, 256x256, 8 waves, 16x16x32 MFMA blocks
    kDirect64x192M16 = 11,    // Dma16 BK 64, 256x192, 4 waves, 16x16x32 MFMA blocks
    kDirect64x128M16 = 12,    // Dma16 BK 64, 256x128, 4 waves, 16x16x32 MFMA blocks
    kDirect32x256M16 = 13,    // Dma16 BK 32 (five-stage ring), 256x256, 4 waves, 16x16x32 MFMA blocks
    kDirect32x256W8M16 = 14,  // Dma16 BK 32 (five-stage ring), 256x256, 8 waves, 16x16x32 MFMA blocks
    kDirect64x192W8M16 = 15,  // Dma16 BK 64, 256x192, 8 waves (48 columns each), 16x16x32 MFMA blocks
};

// Returns the launcher of the fused kernel for (DT, act, variant, residual);
// defined in the per-dtype instantiation unit.  The register-staged kernels
// test a.R at run time; the direct ones are compiled with or without it.
template <int DT>
fused_launcher pick_fused_for(int act, bool vec, int variant, bool residual);

// The backward-epilogue kernel for (DT, act, variant), or null where none is
// built (defined in the per-dtype backward instantiation unit).
template <int DT>
fused_launcher pick_bwd_for(int act, int variant);

// Launcher of the quantized-output kernel for (DT, act, variant, qfmt), or
// nullptr when that variant has none; defined in the per-dtype quantized
// instantiation unit (fp16/bf16 only).
template <int DT>
fused_launcher pick_quant_for(int act, int variant, int qfmt);

// Launcher of the FP8-input kernel with output dtype DT for (act, variant),
// or nullptr when that variant has none; defined in the per-output-dtype
// FP8 instantiation unit.
template <int DT>
fused_launcher pick_fp8_for(int act, int variant);

}  // namespace fl
