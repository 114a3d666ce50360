/*
 * fused_linear.h -- C ABI of the gfx950 fused linear layer
 *
 *     out = act(A @ B + bias)
 *
 * computed by one tiled MFMA GEMM whose epilogue runs on the fp32
 * accumulators after the whole K reduction: a per-column bias broadcast over
 * rows, then ReLU, GELU(tanh) or the gate X + X*Y, then one conversion to the
 * I/O dtype and one store.
 *
 * Definitions followed (page title, section):
 *   - "Triton: Fused Matmul + Bias + ReLU (Epilogue Fusion)": the opening
 *     formula out[i,j] = max(0, sum_k A[i,k] B[k,j] + bias[j]); the bias is per
 *     column, broadcast across rows, added once after the K loop.
 *   - "Epilogue concept", "Where the accumulator is finally correct": the
 *     epilogue transforms the accumulator after the K loop, then one store.
 *   - "I3. Fuse a GEMM epilogue and change tile scheduling": fp32 accumulate,
 *     epilogue in fp32, conversion to the input dtype only at the store;
 *     K = 0 still runs the epilogue ("Implement in stages"); grouped
 *     program-id ownership with a short final group ("Tiles and grouped
 *     ownership").
 *   - "Optimizing GEMM + Activation on CDNA4 with TLX", "The GLU Block":
 *     X = A@B + bias, out = X + X*Y; the unfused path writes X and reads it
 *     back, which the separate entry points below reproduce.
 *   - GELU(tanh) is named as a fusable activation on the first page but not
 *     written out; the tanh approximation of Hendrycks & Gimpel (2016),
 *     0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))), is used.
 *
 * Conventions shared by every entry point:
 *   Layout     Row-major, contiguous: A is (M,K) with row stride K, B is (K,N)
 *              with row stride N, Y/X/out are (M,N) with row stride N, bias is
 *              (N,).  Strides are not supported.
 *   Dtypes     A, B, bias, Y and out all use `dtype`; accumulation and the
 *              epilogue are fp32; the single store rounds to nearest even.
 *   Ownership  Every data pointer is a caller-owned DEVICE pointer.  The
 *              library never allocates, frees or copies host<->device memory.
 *   Async      Work is enqueued on `stream` (a hipStream_t; NULL = the null
 *              stream) and the call returns; the library never synchronises.
 *              Buffers must stay alive until the work has finished.
 *   Aliasing   out must not overlap A, B or bias.  Y may be exactly out (each
 *              element is read before it is written) but must not partially
 *              overlap it.
 *   Shapes     M, N, K >= 0 and <= 2^31-1.  M == 0 or N == 0 returns FL_OK
 *              without launching.  K == 0 is valid: out = act(bias) on every
 *              row (bias NULL counts as zero).  Offsets inside a tile are
 *              32-bit: 256 rows of A and of out (256*K and 256*N elements)
 *              and the whole of B (K*N elements; not the transposed operand
 *              of the backward entries) must each span less than 2 GiB, else
 *              FL_ERR_UNSUPPORTED.
 *   Alignment  Pointers must be aligned to the element size.  The
 *              direct-to-LDS kernels (fp16/bf16, FP8 operands) take any such
 *              pointers and any K and N with the same code.  The
 *              register-staged kernel (fp32, tile_cfg 3) takes its
 *              vector-load path for 16-byte aligned pointers with K and N
 *              multiples of 16 bytes / element size, its element path
 *              otherwise; both produce the same results.
 *   Errors     Arguments are validated before any HIP call; a bad argument
 *              returns FL_ERR_INVALID_ARG (or FL_ERR_UNSUPPORTED for a
 *              well-formed request the library does not implement) with no
 *              launch and no write, and sets a thread-local message readable
 *              with fl_last_error().  A failed launch returns FL_ERR_LAUNCH.
 *   Threads    Stateless apart from the thread-local error message and a
 *              per-device cache of the compute-unit count; safe to call from
 *              several host threads.
 */
#ifndef FUSED_LINEAR_H
#define FUSED_LINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FL_F32 = 0, FL_F16 = 1, FL_BF16 = 2 } fl_dtype;

typedef enum {
    FL_ACT_NONE = 0,      /* out = X                                  */
    FL_ACT_RELU = 1,      /* out = max(X, 0)                          */
    FL_ACT_GELU_TANH = 2, /* out = 0.5 X (1 + tanh(sqrt(2/pi)(X + 0.044715 X^3))) */
    FL_ACT_GLU = 3        /* out = X + X*Y  (the gate; needs Y)       */
} fl_act;

/* One-byte output codes of fl_fused_linear_quant. */
typedef enum {
    FL_Q_FP8_E4M3 = 0, /* OCP FP8 E4M3 (largest finite 448, no infinities) */
    FL_Q_INT8 = 1      /* two's-complement int8 */
} fl_qformat;

typedef enum {
    FL_OK = 0,
    FL_ERR_INVALID_ARG = 1,
    FL_ERR_UNSUPPORTED = 2,
    FL_ERR_LAUNCH = 3
} fl_status;

/* Tuning and debug options of fl_fused_linear_ex.  Zero-initialise and set
 * what you need; every field's zero means "default". */
typedef struct {
    int32_t group_m;    /* M-tiles per band of the grouped program map; 0 = 4.
                           1 gives row-major tile order. */
    int32_t persistent; /* 0 = one workgroup per output tile; 1 = a grid sized
                           to the GPU whose workgroups loop over tiles. */
    int32_t tile_cfg;   /* Kernel and tile.  0 = automatic: fp32 runs the
                           register-staged 256x256 kernel; fp16/bf16 run the
                           direct-to-LDS kernel with 16x16x32 MFMA blocks and
                           256x256 tiles (8 waves, as 10), 256x192 (8 waves,
                           as 15) or 256x128 (as 12), whichever takes the
                           fewest waves x relative wave time on this GPU's
                           compute units; short reductions (K <= 3072 for a
                           256x128 choice, K <= 1024 for 256x192, K <= 256
                           for 256x256) whose 256x128 grid fills two
                           workgroups per compute unit run as 6.  The
                           quantized-output, FP8-operand and backward entry
                           points state their own automatic choices.
                           Variants with 32x32x16 MFMA blocks: 1 = 256x256
                           direct, 4 waves (fp16/bf16; fp32 as 0); 2 =
                           256x128 direct (fp16/bf16 only); 3 =
                           register-staged 256x256 for any dtype; 4 =
                           256x256 direct with 32-deep K stages; 5 = 256x256
                           direct with 8 waves (two per SIMD, 128x64 each;
                           fp16/bf16; fp32 as 0); 6 = 256x128 direct with
                           32-deep K stages and two workgroups per compute
                           unit (fp16/bf16 only); 7 and 8 = 256x192 direct
                           (a tile width that is not a power of two, 4 waves
                           of 128x96) with 64- and 32-deep K stages
                           (fp16/bf16 only).  Variants with 16x16x32 MFMA
                           blocks (fp16/bf16 only): 9 = 256x256, 4 waves;
                           10 = 256x256, 8 waves; 11 = 256x192, 4 waves; 12 =
                           256x128; 13 and 14 = 256x256 with 4 and 8 waves
                           and 32-deep K stages in a five-stage ring; 15 =
                           256x192, 8 waves (128x48 each).  All variants of
                           one MFMA shape give bit-identical results; the
                           two shapes sum each output in a different order
                           (both within the stated tolerance, and equal
                           wherever the arithmetic is exact).  Any other
                           value, or a variant the problem does not allow,
                           is FL_ERR_UNSUPPORTED. */
    int32_t no_xcd_remap; /* 0 = place neighbouring tiles on one XCD; 1 = off */
    uint32_t *debug_tile_count; /* NULL, or a device array of tiles_m*tiles_n
                           counters (see fl_tile_grid); each output tile adds
                           one when it is written.  Caller zeroes it. */
    int32_t debug_sync; /* 0 = normal; 1 = a debugging schedule: every K
                           stage also waits for all of its wave's copies and
                           meets the other waves at an extra barrier.  It
                           changes timing only, so the results are the same
                           bits as with 0 (a test checks this); slower. */
} fl_options;

/*
 * out = act(A@B + bias).
 *   A     (M,K) device pointer; may be NULL only if M*K == 0.
 *   B     (K,N) device pointer; may be NULL only if K*N == 0.
 *   bias  (N,) device pointer, or NULL for no bias.
 *   Y     (M,N) device pointer, required when act == FL_ACT_GLU and NULL
 *         otherwise (a non-NULL Y with another act is FL_ERR_INVALID_ARG).
 *   out   (M,N) device pointer.
 *   stream  hipStream_t to enqueue on.
 * Uses the default options (grouped map with 4 M-tiles per band, automatic
 * tile size, XCD-aware placement).
 */
fl_status fl_fused_linear(const void *A, const void *B, const void *bias,
                          const void *Y, void *out, int64_t M, int64_t N,
                          int64_t K, fl_act act, fl_dtype dtype, void *stream);

/* As fl_fused_linear, with explicit options (opt may be NULL = defaults).
 * Results are bitwise identical for every group_m, persistent,
 * no_xcd_remap and debug_sync setting: they change which workgroup computes
 * a tile, or when, never the arithmetic of the tile.  The tile_cfg variants
 * of one MFMA shape sum each output in the same order and give the same
 * bits; the 32x32x16 and 16x16x32 shapes sum in different orders (see
 * tile_cfg). */
fl_status fl_fused_linear_ex(const void *A, const void *B, const void *bias,
                             const void *Y, void *out, int64_t M, int64_t N,
                             int64_t K, fl_act act, fl_dtype dtype,
                             void *stream, const fl_options *opt);

/*
 * out = act(A@B + bias + R): the fused linear layer with a same-shape
 * residual R added to the accumulator after the K reduction, before the
 * activation ("Triton: Fused Matmul + Bias + ReLU (Epilogue Fusion)",
 * "Variants": the residual tile is loaded after the K loop under the same
 * mask as the store).  In fp32: (acc + bias) + R, then act, then one
 * rounding to dtype.
 *   R     (M,N) device pointer in dtype, row stride N; must not be NULL
 *         (unless M*N == 0).  R may be exactly out (each element is read
 *         before it is written) but must not partially overlap it.
 *   Every other argument, option and error as fl_fused_linear_ex; act may
 *   be any activation, including the gate (then Y is required too:
 *   out = X + X*Y with X = A@B + bias + R).
 */
fl_status fl_fused_linear_residual(const void *A, const void *B,
                                   const void *bias, const void *R,
                                   const void *Y, void *out, int64_t M,
                                   int64_t N, int64_t K, fl_act act,
                                   fl_dtype dtype, void *stream,
                                   const fl_options *opt);

/*
 * out_q = Q(scale * act(A@B + bias)): the fused linear layer with a
 * quantized store ("Triton: Fused Matmul + Bias + ReLU (Epilogue Fusion)",
 * "Variants": the epilogue value is scaled, limited to the code's range and
 * written as 8-bit integer or FP8 codes).  The epilogue value is the
 * fp32 one fl_fused_linear would round to dtype; it is multiplied by scale
 * in fp32 and
 *   FL_Q_FP8_E4M3: clamped to [-448, 448] and rounded to nearest even on the
 *                  OCP E4M3 grid (subnormals kept);
 *   FL_Q_INT8:     rounded to nearest even and clamped to [-128, 127].
 *   out_q  (M,N) device pointer to M*N bytes (row stride N); must not overlap
 *          A, B, bias or Y.
 *   scale  finite fp32 (a per-tensor output scale).
 *   dtype  FL_F16 or FL_BF16 (FL_F32 inputs are FL_ERR_UNSUPPORTED).
 *   opt    as fl_fused_linear_ex, with tile_cfg 0 (the automatic choice of
 *          fl_fused_linear_ex), 2, 5, 6, 7, 10, 11, 12 or 15; other values
 *          are FL_ERR_UNSUPPORTED.
 * Errors as fl_fused_linear_ex; an unknown qfmt or a non-finite scale is
 * FL_ERR_INVALID_ARG.
 */
fl_status fl_fused_linear_quant(const void *A, const void *B,
                                const void *bias, const void *Y, void *out_q,
                                float scale, int64_t M, int64_t N, int64_t K,
                                fl_act act, fl_dtype dtype, fl_qformat qfmt,
                                void *stream, const fl_options *opt);

/*
 * out = act(ab_scale * (A8 @ B8) + bias): the fused linear layer with FP8
 * operands ("Optimizing GEMM + Activation on CDNA4 with TLX", "Future Work":
 * the projection in FP8, which CDNA4's matrix cores run at twice the 16-bit
 * rate and which halves the operand traffic).  A8 (M,K) and B8 (K,N) are OCP
 * FP8 E4M3 codes, row-major; the products are summed in fp32 by the
 * matrix cores' scaled FP8 instructions (32x32x64 or 16x16x128 blocks, no
 * block scales), the sum is multiplied by ab_scale (the product of the two
 * per-tensor scales) in fp32, then bias, activation (the gate with Y), one
 * rounding to out_dtype and one store, as fl_fused_linear.
 *   A8, B8    device pointers to M*K and K*N bytes, 16-byte aligned.
 *   ab_scale  finite fp32.
 *   bias, Y, out  in out_dtype (FL_F16 or FL_BF16; FL_F32 is
 *             FL_ERR_UNSUPPORTED), conventions as fl_fused_linear.
 *   Any M and K; N of 1 or 2 is FL_ERR_UNSUPPORTED (rows of B of 1 or 2
 *             bytes), any other N is served.
 *   opt       tile_cfg 0 (automatic: the tile width fl_fused_linear would
 *             choose, 256, 192 or 128, with 32x32x64 blocks; where the
 *             256x128 grid fills two workgroups per compute unit and K <=
 *             1024 (width 256) or K <= 3072 (192 or 128), the two-per-CU
 *             256x128 kernel), 1, 2, 5, 6 or 7 (32x32x64 blocks,
 *             bit-identical to one another; 6 is the two-per-CU kernel with
 *             64-deep stages) or 12 (16x16x128 blocks, 256x128 tiles: the
 *             same products summed in another order); others are
 *             FL_ERR_UNSUPPORTED.
 */
fl_status fl_fused_linear_fp8(const void *A8, const void *B8, float ab_scale,
                              const void *bias, const void *Y, void *out,
                              int64_t M, int64_t N, int64_t K, fl_act act,
                              fl_dtype out_dtype, void *stream,
                              const fl_options *opt);

/*
 * The backward epilogue ("Optimizing GEMM + Activation on CDNA4 with TLX",
 * "Future Work": the same epilogue fusion applied to the backward pass).  For
 * a layer out = act(X), X = A@B + bias, whose output is multiplied by a
 * weight W (N,K) in the next product, the loss gradient reaching out is
 * D = G @ W^T (G (M,K): the gradient at that product's output).  One launch
 * computes D with fp32 accumulation (W read as its transpose, K-contiguous:
 * no transposed copy is made) and in its epilogue
 *   dX = D * act'(X)     (ReLU: 1 where X > 0, else 0; GELU(tanh): its
 *                          derivative; none: 1; gate X + X*Y: 1 + Y),
 *   dY = D * X           (the gate only),
 *   dbias = sum over the M rows of dX (fp32, before dX is rounded),
 * then one rounding of dX and dY to dtype.
 *   G      (M,K) device pointer, dtype.
 *   W      (N,K) row-major device pointer, dtype.
 *   X      (M,N) the saved pre-activation, dtype; may equal dX (read before
 *          it is overwritten), must not otherwise overlap an output.
 *   Y      (M,N) the gate's operand, for FL_ACT_GLU only (NULL otherwise).
 *   dX     (M,N) output, dtype.
 *   dY     (M,N) output for FL_ACT_GLU (may equal Y), NULL otherwise.
 *   dbias  (N,) fp32 device buffer, or NULL for no bias gradient.  It is
 *          overwritten: a fill kernel zeroes it on `stream`, then every
 *          output tile adds its column sums with fp32 atomics, so its last
 *          bits may differ from run to run (the order of the additions is
 *          not fixed; fl_fused_linear_bwd_ws fixes it); dX and dY are
 *          deterministic.
 *   dtype  FL_F16 or FL_BF16 (FL_F32 is FL_ERR_UNSUPPORTED).
 *   opt    tile_cfg 0 (automatic: the 8-wave 256x256 kernel with 16x16x32
 *          MFMA blocks (10) where the forward choice is 256 wide, 256x128
 *          with 32x32x16 blocks (2) elsewhere), 10 and 12 (16x16x32
 *          blocks), or 5 and 2 (32x32x16 blocks); others are
 *          FL_ERR_UNSUPPORTED.
 *          group_m, persistent and no_xcd_remap as for fl_fused_linear_ex.
 * Alignment, sizes and errors as fl_fused_linear_ex; M = 0 or N = 0 writes
 * nothing but a zero dbias; K = 0 gives zeros.
 */
fl_status fl_fused_linear_bwd(const void *G, const void *W, const void *X,
                              const void *Y, void *dX, void *dY,
                              float *dbias, int64_t M, int64_t N, int64_t K,
                              fl_act act, fl_dtype dtype, void *stream,
                              const fl_options *opt);

/* The backward epilogue ("Optimizing GEMM + Activation on CDNA4 with TLX",
 * "Future Work", as fl_fused_linear_bwd) with a bias gradient that is the
 * same to the bit from run to run and whatever order the tiles run in
 * (fl_fused_linear_bwd's atomics fix neither).  Same arguments, outputs and errors as
 * fl_fused_linear_bwd, plus a caller-owned device workspace: each 256-row
 * tile row writes two rows of fp32 partial column sums of dX (one per
 * 128-row half, each summed in a fixed order) into
 * workspace[(2*tile_row + half) * N + column], then one more launch on
 * `stream` sets dbias[c] to those rows added in row order.  dX and dY are
 * bit-identical to fl_fused_linear_bwd's; dbias agrees with it within the
 * rounding of an fp32 sum (the tolerance fl_fused_linear_bwd states) and
 * is bit-identical between tile_cfg values of one MFMA shape (10 and 12;
 * 5 and 2).
 *   workspace        device memory of at least fl_bwd_workspace_bytes(M,
 *                    N, K, dtype) bytes, 4-byte aligned, overlapping no
 *                    operand; only read and written by this call's
 *                    launches on `stream` (its contents afterwards are
 *                    unspecified).  Unused (may be NULL) when dbias is
 *                    NULL or M or N is 0.
 *   workspace_bytes  its size; FL_ERR_INVALID_ARG (no launch) when smaller
 *                    than needed, NULL, misaligned or overlapping.
 */
fl_status fl_fused_linear_bwd_ws(const void *G, const void *W, const void *X,
                                 const void *Y, void *dX, void *dY,
                                 float *dbias, int64_t M, int64_t N, int64_t K,
                                 fl_act act, fl_dtype dtype, void *stream,
                                 const fl_options *opt, void *workspace,
                                 size_t workspace_bytes);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops, harnesses that forbid hipMalloc):
 * fl_fused_linear_bwd_ws with the library's own workspace, a fixed 8 MiB
 * device array per GPU (held until the process ends), so nothing is
 * allocated, here or by the caller.  Same arguments, results and errors as
 * fl_fused_linear_bwd_ws without the workspace; a dbias whose partial sums
 * need more than 8 MiB (2 * ceil(M/256) * N * 4 bytes, e.g. M = 16384 with
 * N = 16384 still fits) is FL_ERR_UNSUPPORTED with no launch.  On its first
 * call on a device the library looks up that device's copy of the array
 * (FL_ERR_LAUNCH if the lookup fails).  Every call on one GPU uses the same
 * array and leaves its partial sums there; a call writes every partial sum
 * it reads before reading it, so nothing needs clearing between calls.
 * Calls that may overlap on one GPU (two streams, two threads) race on the
 * array and must be serialized by the caller.
 */
fl_status fl_fused_linear_bwd_noalloc(const void *G, const void *W,
                                      const void *X, const void *Y, void *dX,
                                      void *dY, float *dbias, int64_t M,
                                      int64_t N, int64_t K, fl_act act,
                                      fl_dtype dtype, void *stream,
                                      const fl_options *opt);

/* Bytes of workspace fl_fused_linear_bwd_ws needs for an (M,N) output:
 * 2 * ceil(M/256) * N * 4 (0 when M or N is 0).  FL_ERR_INVALID_ARG for a
 * NULL `bytes`, negative sizes or an unknown dtype, FL_ERR_UNSUPPORTED for
 * fp32 and sizes above 2^31-1. */
fl_status fl_bwd_workspace_bytes(int64_t M, int64_t N, int64_t K,
                                 fl_dtype dtype, size_t *bytes);

/* The unfused backward chain, for comparison with fl_fused_linear_bwd: one
 * launch per step, each storing its result in dtype (so D and dX round-trip
 * through memory), together round(round(D) * act'(X)) and the fp32 column
 * sums of the stored dX. */

/* D = A @ Bt^T: A (M,K), Bt (N,K) row-major (B given as its transpose), D
 * (M,N), dtype FL_F16 or FL_BF16 (FL_F32 is FL_ERR_UNSUPPORTED); the
 * backward kernel with no epilogue work.  Conventions as fl_gemm. */
fl_status fl_gemm_nt(const void *A, const void *Bt, void *D, int64_t M,
                     int64_t N, int64_t K, fl_dtype dtype, void *stream);

/* dX = D * act'(X) elementwise, and for FL_ACT_GLU also dY = D * X (Y and
 * dY NULL for the other activations).  All (M,N) in dtype (FL_F16 or
 * FL_BF16); dX may equal D and dY may equal Y, no other overlap. */
fl_status fl_activation_grad(const void *D, const void *X, const void *Y,
                             void *dX, void *dY, int64_t M, int64_t N,
                             fl_act act, fl_dtype dtype, void *stream);

/* sums[j] = sum over i of X[i,j] in fp32: X (M,N) in dtype (FL_F16 or
 * FL_BF16), sums (N,) fp32, overwritten (zeroed by a fill kernel, then
 * added to with fp32 atomics, so its last bits may differ from run to
 * run). */
fl_status fl_column_sum(const void *X, float *sums, int64_t M, int64_t N,
                        fl_dtype dtype, void *stream);

/* The unfused chain ("Triton: Fused Matmul + Bias + ReLU", "The HBM
 * traffic": GEMM writes X, a bias pass reads and writes it, an activation
 * pass reads and writes it).  Each call is one launch and stores its result
 * in dtype.  Together they compute round(act(round(round(A@B) + bias))). */

/* X = A@B, the fused kernel with no bias and no activation. */
fl_status fl_gemm(const void *A, const void *B, void *X, int64_t M,
                  int64_t N, int64_t K, fl_dtype dtype, void *stream);

/* X[i,j] += bias[j] in place (X is (M,N); bias (N,) must not be NULL). */
fl_status fl_bias_add(void *X, const void *bias, int64_t M, int64_t N,
                      fl_dtype dtype, void *stream);

/* out = act(X) elementwise (out may equal X); Y (M,N) is required for
 * FL_ACT_GLU (out = X + X*Y) and must be NULL otherwise.  FL_ACT_NONE copies. */
fl_status fl_activation(const void *X, const void *Y, void *out, int64_t M,
                        int64_t N, fl_act act, fl_dtype dtype, void *stream);

/* Tile grid fl_fused_linear_ex would use for this problem.  Writes the tile
 * shape and the number of tiles along M and N.  The automatic choice reads
 * the current device's compute-unit count once (256 when no device is
 * available); no other HIP call is made. */
fl_status fl_tile_grid(int64_t M, int64_t N, int64_t K, fl_dtype dtype,
                       const fl_options *opt, int32_t *block_m,
                       int32_t *block_n, int32_t *tiles_m, int32_t *tiles_n);

/* Grouped program-id -> tile map used on the device, evaluated on the host
 * for tests ("Tiles and grouped ownership").  xcd_remap selects whether the
 * XCD placement step is applied first.  grid is the number of programs. */
fl_status fl_tile_of_program(int32_t program, int32_t grid, int32_t tiles_m,
                             int32_t tiles_n, int32_t group_m,
                             int32_t xcd_remap, int32_t *m_tile,
                             int32_t *n_tile);

const char *fl_status_string(fl_status s);
const char *fl_last_error(void); /* thread-local; "" when none */
int fl_version(void);            /* major*10000 + minor*100 + patch */

#ifdef __cplusplus
}
#endif

#endif /* FUSED_LINEAR_H */
