/*
 * fused_linear_oracle.c -- plain FP64 CPU oracle for out = act(A@B + bias).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or
 * calls this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header, table or helper with
 * the HIP library: it has its own fp16/bf16 decoders and encoders, its own
 * tile map and its own GELU.
 *
 * What it computes (the plain definition, written out, no blocking, no
 * fusion, no reordering):
 *   X[i,j]   = sum_k A[i,k] * B[k,j]              (FP64, k ascending)
 *   X[i,j]  += bias[j]                            (once, by column)
 *   X[i,j]  += R[i,j]                             (residual, when given)
 *   out[i,j] = act(X[i,j]) (or X + X*Y for the gate)
 *   out      = round_to_nearest_even(out, dtype)  (once, at the end)
 *
 * Sources (page title, section):
 *   - "Triton: Fused Matmul + Bias + ReLU (Epilogue Fusion)", opening formula
 *     and the note under it: per-column bias broadcast over rows, added once
 *     after the K loop, then max(0, .).
 *   - "Epilogue concept", "Where the accumulator is finally correct": the
 *     loop nest acc=0; acc += A*B over k; epilogue; one store.
 *   - "I3. Fuse a GEMM epilogue and change tile scheduling", intro and
 *     "Why the baseline uses FP32": the correctness reference is an FP64
 *     GEMM+bias+activation rounded once at the end; the output dtype is the
 *     input dtype.  "Tiles and grouped ownership": the grouped program-id map
 *     with actual_group = min(GROUP, tiles_m - first_m).
 *   - "Optimizing GEMM + Activation on CDNA4 with TLX", "The GLU Block":
 *     X = A@B + bias, out = X + X*Y.
 *   - "Triton: Fused Matmul + Bias + ReLU (Epilogue Fusion)", "Variants":
 *     a residual of the output's shape is summed into the accumulator after
 *     the K loop, ahead of the activation; and the quantized output: the
 *     epilogue value times a scale, limited to the target range and
 *     converted to int8 or FP8 codes as it is stored (see
 *     orc_fused_linear_quant).
 *   - "Optimizing GEMM + Activation on CDNA4 with TLX", "Future Work" (FP8
 *     precision): the projection itself in FP8, i.e. A and B as OCP E4M3
 *     codes with a per-tensor scale, fp32 accumulation, and the same
 *     epilogue in the 16-bit output dtype (see orc_fused_linear_fp8).
 *   - "Optimizing GEMM + Activation on CDNA4 with TLX", "Future Work":
 *     the epilogue fusion carried over to the backward pass (see
 *     orc_fused_linear_bwd; the derivatives follow from the forward
 *     definitions by the chain rule).
 *   - GELU: the pages name it as a fusable activation but print no formula;
 *     this file uses the tanh form of Hendrycks & Gimpel (2016),
 *     0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))), with libm tanh.
 *
 * Rounding: round-to-nearest, ties-to-even (the IEEE default; the pages do
 * not name a mode), computed directly from FP64 with rint(), including
 * subnormals and overflow to infinity.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2 };
enum { ORC_NONE = 0, ORC_RELU = 1, ORC_GELU_TANH = 2, ORC_GLU = 3 };

/* ---------------------------------------------------------------- decode */

static double dec_f16(uint16_t h) {
    int s = (h >> 15) & 1, e = (h >> 10) & 0x1f, m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24); /* subnormal: m * 2^-14 * 2^-10 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m + 1024), e - 25); /* (1 + m/2^10) * 2^(e-15) */
    return s ? -v : v;
}

static double dec_bf16(uint16_t b) {
    /* bf16 is the top half of a binary32: widen the bit pattern. */
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

static double dec_one(int dtype, const void *p, int64_t i) {
    if (dtype == ORC_F32) return (double)((const float *)p)[i];
    if (dtype == ORC_F16) return dec_f16(((const uint16_t *)p)[i]);
    return dec_bf16(((const uint16_t *)p)[i]);
}

int orc_decode(int dtype, const void *src, int64_t n, double *dst) {
    if (dtype < 0 || dtype > 2 || n < 0) return 1;
    for (int64_t i = 0; i < n; ++i) dst[i] = dec_one(dtype, src, i);
    return 0;
}

/* ---------------------------------------------------------------- encode */

/* Round x to a binary format with p significand bits (implicit bit included),
 * minimum normal exponent emin and maximum exponent emax; RNE; overflow to
 * +-inf.  Returns the rounded value as a double (exactly representable). */
static double round_fmt(double x, int p, int emin, int emax) {
    if (x == 0.0 || isnan(x) || isinf(x)) return x;
    int e2;
    frexp(x, &e2);              /* x = f * 2^e2, 0.5 <= |f| < 1 */
    int E = e2 - 1;             /* unbiased exponent of x */
    if (E < emin) E = emin;     /* below the normal range the quantum is fixed */
    int q = E - (p - 1);        /* exponent of one unit in the last place */
    double r = ldexp(rint(ldexp(x, -q)), q);
    if (fabs(r) >= ldexp(1.0, emax + 1)) return copysign(INFINITY, x);
    return r;
}

static uint16_t enc_small(double x, int ebits, int mbits) {
    /* x must already be rounded to the format. */
    int bias = (1 << (ebits - 1)) - 1;
    int emin = 1 - bias;
    uint16_t s = signbit(x) ? 1 : 0;
    uint16_t sign = (uint16_t)(s << (ebits + mbits));
    uint16_t expmask = (uint16_t)(((1 << ebits) - 1) << mbits);
    if (isnan(x)) return (uint16_t)(expmask | (1 << (mbits - 1)));
    if (isinf(x)) return (uint16_t)(sign | expmask);
    double a = fabs(x);
    if (a == 0.0) return sign;
    int e2;
    frexp(a, &e2);
    int E = e2 - 1;
    if (E < emin) { /* subnormal */
        uint16_t m = (uint16_t)ldexp(a, -(emin - mbits));
        return (uint16_t)(sign | m);
    }
    uint16_t m = (uint16_t)(ldexp(a, mbits - E) - ldexp(1.0, mbits));
    return (uint16_t)(sign | ((E + bias) << mbits) | m);
}

static void enc_one(int dtype, double x, void *p, int64_t i) {
    if (dtype == ORC_F32) {
        ((float *)p)[i] = (float)round_fmt(x, 24, -126, 127); /* exact */
    } else if (dtype == ORC_F16) {
        ((uint16_t *)p)[i] = enc_small(round_fmt(x, 11, -14, 15), 5, 10);
    } else {
        ((uint16_t *)p)[i] = enc_small(round_fmt(x, 8, -126, 127), 8, 7);
    }
}

int orc_encode(int dtype, const double *src, int64_t n, void *dst) {
    if (dtype < 0 || dtype > 2 || n < 0) return 1;
    for (int64_t i = 0; i < n; ++i) enc_one(dtype, src[i], dst, i);
    return 0;
}

/* ------------------------------------------------------ quantized output */

enum { ORC_Q_FP8_E4M3 = 0, ORC_Q_INT8 = 1 };

/* OCP FP8 E4M3 ("e4m3fn": exponent bias 7, 3 mantissa bits, subnormals,
 * largest finite 448, no infinities, S.1111.111 = NaN).  Saturating: |u| >=
 * 448 gives +-448; otherwise round to nearest, ties to even, on the format's
 * grid (subnormal quantum 2^-9). */
static uint8_t enc_e4m3(double u) {
    if (isnan(u)) return 0x7f;
    if (u >= 448.0) return 0x7e;
    if (u <= -448.0) return 0xfe;
    double r = round_fmt(u, 4, -6, 8); /* |r| <= 448 here: 464 is the first tie above */
    return (uint8_t)enc_small(r, 4, 3);
}

static double dec_e4m3(uint8_t c) {
    int s = c >> 7, e = (c >> 3) & 0xf, m = c & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        v = ldexp((double)m, -9); /* m/8 * 2^-6 */
    else
        v = ldexp((double)(m + 8), e - 10); /* (1 + m/8) * 2^(e-7) */
    return s ? -v : v;
}

/* int8: round to nearest, ties to even, then clamp to [-128, 127]. */
static uint8_t enc_i8(double u) {
    double r = rint(u);
    if (r > 127.0) r = 127.0;
    if (r < -128.0) r = -128.0;
    return (uint8_t)(int8_t)r;
}

static uint8_t quantize(int qfmt, double u) { return qfmt == ORC_Q_INT8 ? enc_i8(u) : enc_e4m3(u); }

static double dequantize(int qfmt, uint8_t c) { return qfmt == ORC_Q_INT8 ? (double)(int8_t)c : dec_e4m3(c); }

int orc_quantize(int qfmt, const double *src, int64_t n, uint8_t *dst) {
    if (qfmt < 0 || qfmt > 1 || n < 0) return 1;
    for (int64_t i = 0; i < n; ++i) dst[i] = quantize(qfmt, src[i]);
    return 0;
}

int orc_dequantize(int qfmt, const uint8_t *src, int64_t n, double *dst) {
    if (qfmt < 0 || qfmt > 1 || n < 0) return 1;
    for (int64_t i = 0; i < n; ++i) dst[i] = dequantize(qfmt, src[i]);
    return 0;
}

/* The value a quantized store decides on, in the kernel's precision: the
 * epilogue value v rounded to binary32, times the scale rounded to binary32
 * (the product of two binary32 numbers is exact in FP64, so the second
 * rounding is that of a binary32 multiply). */
static double quant_input(double v, float scale) {
    float t = (float)v;
    return (double)(float)((double)t * (double)scale);
}

/* ------------------------------------------------------------ activation */

double orc_gelu_tanh(double x) {
    const double c = sqrt(2.0 / M_PI);
    return 0.5 * x * (1.0 + tanh(c * (x + 0.044715 * x * x * x)));
}

static double apply_act(int act, double x, double y) {
    switch (act) {
    case ORC_RELU: return x > 0.0 ? x : 0.0;  /* max(0, x) */
    case ORC_GELU_TANH: return orc_gelu_tanh(x);
    case ORC_GLU: return x + x * y;           /* the gate X + X*Y */
    default: return x;
    }
}

/* ------------------------------------------------------- fused reference */

/* One output row i of X = A@B (FP64, k ascending), into acc[0..N). */
static void row_product(const double *A64row, const double *B64, double *acc,
                        int64_t N, int64_t K) {
    for (int64_t j = 0; j < N; ++j) acc[j] = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        double a = A64row[k];
        const double *b = B64 + k * N;
        for (int64_t j = 0; j < N; ++j) acc[j] += a * b[j];
    }
}

static int check_args(int dtype, int act, const void *A, const void *B,
                      const void *Y, const void *out, int64_t M, int64_t N,
                      int64_t K) {
    if (dtype < 0 || dtype > 2 || act < 0 || act > 3) return 1;
    if (M < 0 || N < 0 || K < 0) return 1;
    if (!out && M * N > 0) return 1;
    if ((!A && M * K > 0) || (!B && K * N > 0)) return 1;
    if (act == ORC_GLU && !Y && M * N > 0) return 1;
    return 0;
}

/*
 * out (nrows x N, dtype) = round(act(A[rows]@B + bias + R)).
 * rows == NULL computes every row (nrows must equal M).  bias and the
 * residual R (M, N) may be NULL (count as zero).  Y is (M, N) and read only
 * for the gate.  x_out, when not
 * NULL, receives the unrounded FP64 value after the epilogue (nrows x N).
 * unfused != 0 switches to the three-stage chain that rounds after every
 * stage: round(act(round(round(A@B) + bias))), which is what separate
 * GEMM, bias and activation kernels each storing in dtype compute.
 */
static int run(int dtype, int act, const void *A, const void *B,
               const void *bias, const void *R, const void *Y, void *out,
               int64_t M, int64_t N, int64_t K, const int64_t *rows,
               int64_t nrows, int nthreads, double *x_out, int unfused,
               int qfmt, float scale) {
    if (check_args(dtype, act, A, B, Y, out, M, N, K)) return 1;
    if (unfused && R) return 1; /* the chain has no residual stage */
    if (!rows) nrows = M;
    if (nrows < 0) return 1;
    if (rows)
        for (int64_t r = 0; r < nrows; ++r)
            if (rows[r] < 0 || rows[r] >= M) return 1;
    if (nrows == 0 || N == 0) return 0;

    double *B64 = (double *)malloc(sizeof(double) * (size_t)(K * N + 1));
    double *bias64 = (double *)malloc(sizeof(double) * (size_t)N);
    if (!B64 || !bias64) { free(B64); free(bias64); return 2; }
    orc_decode(dtype, B, K * N, B64);
    for (int64_t j = 0; j < N; ++j) bias64[j] = bias ? dec_one(dtype, bias, j) : 0.0;

    int status = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel
    {
        double *acc = (double *)malloc(sizeof(double) * (size_t)N);
        double *arow = (double *)malloc(sizeof(double) * (size_t)(K + 1));
        if (!acc || !arow) {
#pragma omp atomic write
            status = 2;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t r = 0; r < nrows; ++r) {
                int64_t i = rows ? rows[r] : r;
                for (int64_t k = 0; k < K; ++k) arow[k] = dec_one(dtype, A, i * K + k);
                row_product(arow, B64, acc, N, K);
                for (int64_t j = 0; j < N; ++j) {
                    double y = (act == ORC_GLU) ? dec_one(dtype, Y, i * N + j) : 0.0;
                    double x = acc[j], v;
                    if (!unfused) {
                        double res = R ? dec_one(dtype, R, i * N + j) : 0.0;
                        v = apply_act(act, x + bias64[j] + res, y);
                    } else {
                        double tmp[1];
                        uint16_t h[2];
                        float f[1];
                        void *slot = (dtype == ORC_F32) ? (void *)f : (void *)h;
                        /* stage 1: the GEMM stores X in dtype */
                        tmp[0] = x; orc_encode(dtype, tmp, 1, slot); orc_decode(dtype, slot, 1, tmp);
                        /* stage 2: the bias pass stores X + bias in dtype */
                        tmp[0] = tmp[0] + bias64[j]; orc_encode(dtype, tmp, 1, slot); orc_decode(dtype, slot, 1, tmp);
                        /* stage 3: the activation pass */
                        v = apply_act(act, tmp[0], y);
                    }
                    if (qfmt >= 0) {
                        double u = quant_input(v, scale);
                        if (x_out) x_out[r * N + j] = u;
                        ((uint8_t *)out)[r * N + j] = quantize(qfmt, u);
                        continue;
                    }
                    if (x_out) x_out[r * N + j] = v;
                    enc_one(dtype, v, out, r * N + j);
                }
            }
        }
        free(acc);
        free(arow);
    }
    free(B64);
    free(bias64);
    return status;
}

int orc_fused_linear(int dtype, int act, const void *A, const void *B,
                     const void *bias, const void *R, const void *Y, void *out,
                     int64_t M, int64_t N, int64_t K, const int64_t *rows,
                     int64_t nrows, int nthreads, double *x_out) {
    return run(dtype, act, A, B, bias, R, Y, out, M, N, K, rows, nrows, nthreads, x_out, 0, -1, 1.0f);
}

/*
 * Quantized output: out (nrows x N bytes) = Q(fp32(fp32(act(A@B + bias)) *
 * scale)), Q = saturating RNE to FP8 E4M3 (qfmt 0) or RNE + clamp to int8
 * (qfmt 1).  The activation and everything before it are as in
 * orc_fused_linear (FP64, no residual); x_out, when not NULL, receives the
 * binary32 value Q decides on.
 */
int orc_fused_linear_quant(int dtype, int act, const void *A, const void *B,
                           const void *bias, const void *Y, void *out,
                           int64_t M, int64_t N, int64_t K, int qfmt,
                           float scale, const int64_t *rows, int64_t nrows,
                           int nthreads, double *x_out) {
    if (qfmt < 0 || qfmt > 1 || !isfinite(scale)) return 1;
    return run(dtype, act, A, B, bias, NULL, Y, out, M, N, K, rows, nrows, nthreads, x_out, 0, qfmt, scale);
}

int orc_unfused_chain(int dtype, int act, const void *A, const void *B,
                      const void *bias, const void *Y, void *out, int64_t M,
                      int64_t N, int64_t K, const int64_t *rows, int64_t nrows,
                      int nthreads, double *x_out) {
    return run(dtype, act, A, B, bias, NULL, Y, out, M, N, K, rows, nrows, nthreads, x_out, 1, -1, 1.0f);
}

/* Single output element (i, j), FP64, unrounded:
 * act(sum_k A[i,k]B[k,j] + bias[j] + R[i,j]). */
int orc_element(int dtype, int act, const void *A, const void *B,
                const void *bias, const void *R, const void *Y, int64_t M,
                int64_t N, int64_t K, int64_t i, int64_t j, double *value) {
    if (check_args(dtype, act, A, B, Y, value, M, N, K)) return 1;
    if (i < 0 || i >= M || j < 0 || j >= N) return 1;
    double x = 0.0;
    for (int64_t k = 0; k < K; ++k)
        x += dec_one(dtype, A, i * K + k) * dec_one(dtype, B, k * N + j);
    x += bias ? dec_one(dtype, bias, j) : 0.0;
    x += R ? dec_one(dtype, R, i * N + j) : 0.0;
    double y = (act == ORC_GLU) ? dec_one(dtype, Y, i * N + j) : 0.0;
    *value = apply_act(act, x, y);
    return 0;
}

/* ---------------------------------------------------------- FP8 inputs */

/*
 * out (nrows x N, out_dtype) = round(act(ab_scale * (A8[rows] @ B8) + bias)):
 * A8 (M,K) and B8 (K,N) are OCP FP8 E4M3 codes (decoded exactly), ab_scale
 * is the product of the two per-tensor scales, bias and Y are in out_dtype
 * (fp16 or bf16).  FP64 throughout, rounded once.  x_out, when not NULL,
 * receives the unrounded epilogue value.
 */
int orc_fused_linear_fp8(int out_dtype, int act, const uint8_t *A8,
                         const uint8_t *B8, double ab_scale, const void *bias,
                         const void *Y, void *out, int64_t M, int64_t N,
                         int64_t K, const int64_t *rows, int64_t nrows,
                         int nthreads, double *x_out) {
    if (out_dtype < 0 || out_dtype > 2 || act < 0 || act > 3) return 1;
    if (M < 0 || N < 0 || K < 0 || !isfinite(ab_scale)) return 1;
    if ((!A8 && M * K > 0) || (!B8 && K * N > 0) || (!out && M * N > 0)) return 1;
    if (act == ORC_GLU && !Y && M * N > 0) return 1;
    if (!rows) nrows = M;
    if (nrows < 0) return 1;
    if (rows)
        for (int64_t r = 0; r < nrows; ++r)
            if (rows[r] < 0 || rows[r] >= M) return 1;
    if (nrows == 0 || N == 0) return 0;
    double *B64 = (double *)malloc(sizeof(double) * (size_t)(K * N + 1));
    if (!B64) return 2;
    for (int64_t i = 0; i < K * N; ++i) B64[i] = dec_e4m3(B8[i]);
    int status = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel
    {
        double *acc = (double *)malloc(sizeof(double) * (size_t)N);
        double *arow = (double *)malloc(sizeof(double) * (size_t)(K + 1));
        if (!acc || !arow) {
#pragma omp atomic write
            status = 2;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t r = 0; r < nrows; ++r) {
                int64_t i = rows ? rows[r] : r;
                for (int64_t k = 0; k < K; ++k) arow[k] = dec_e4m3(A8[i * K + k]);
                row_product(arow, B64, acc, N, K);
                for (int64_t j = 0; j < N; ++j) {
                    double x = acc[j] * ab_scale + (bias ? dec_one(out_dtype, bias, j) : 0.0);
                    double y = (act == ORC_GLU) ? dec_one(out_dtype, Y, i * N + j) : 0.0;
                    double v = apply_act(act, x, y);
                    if (x_out) x_out[r * N + j] = v;
                    enc_one(out_dtype, v, out, r * N + j);
                }
            }
        }
        free(acc);
        free(arow);
    }
    free(B64);
    return status;
}

/* ---------------------------------------------------- backward epilogue */

/* Derivative of the tanh-form GELU, from the product and chain rules:
 * with u = c (x + a x^3) and t = tanh(u),
 * g'(x) = 0.5 (1 + t) + 0.5 x (1 - t^2) c (1 + 3 a x^2). */
double orc_gelu_tanh_grad(double x) {
    const double c = sqrt(2.0 / M_PI), a = 0.044715;
    const double t = tanh(c * (x + a * x * x * x));
    return 0.5 * (1.0 + t) + 0.5 * x * (1.0 - t * t) * c * (1.0 + 3.0 * a * x * x);
}

/* d act(x) / dx; for the gate X + X*Y the derivative in X is 1 + Y.  ReLU's
 * derivative is taken as 0 at x = 0 (max(0, x) has no derivative there; the
 * usual subgradient choice). */
static double act_grad(int act, double x, double y) {
    switch (act) {
    case ORC_RELU: return x > 0.0 ? 1.0 : 0.0;
    case ORC_GELU_TANH: return orc_gelu_tanh_grad(x);
    case ORC_GLU: return 1.0 + y;
    default: return 1.0;
    }
}

/*
 * Backward of out = act(X) fused into the epilogue of the GEMM that brings
 * its incoming gradient ("Optimizing GEMM + Activation on CDNA4 with TLX",
 * "Future Work": the same epilogue fusion in the backward pass).  For a
 * layer whose output feeds a product with a weight W (N, K) row-major (the
 * next layer's B, so its transpose is taken), the gradient of the loss with
 * respect to out is D = G @ W^T, G (M, K) the gradient at the next layer's
 * pre-activation.  By the chain rule
 *   D[i,j]   = sum_k G[i,k] * W[j,k]        (FP64, k ascending)
 *   dX[i,j]  = D[i,j] * act'(X[i,j])        (X: the saved pre-activation)
 *   dY[i,j]  = D[i,j] * X[i,j]              (the gate only: d(X + X*Y)/dY)
 *   dbias[j] = sum_i dX[i,j]                (X = A@B + bias, so the bias
 *                                            gradient is dX summed over rows;
 *                                            FP64 sum of unrounded dX)
 * dX and dY are rounded once to dtype.  rows / nrows select output rows as
 * in orc_fused_linear; dbias then sums the selected rows only.  dx_out, when
 * not NULL, receives the unrounded dX (nrows x N).
 */
static int run_bwd(int dtype, int act, const void *G, const void *W,
                   const void *X, const void *Y, void *dX, void *dY,
                   double *dbias, int64_t M, int64_t N, int64_t K,
                   const int64_t *rows, int64_t nrows, int nthreads,
                   double *dx_out, int unfused) {
    if (dtype < 0 || dtype > 2 || act < 0 || act > 3) return 1;
    if (M < 0 || N < 0 || K < 0) return 1;
    if ((!G && M * K > 0) || (!W && N * K > 0) || (!X && M * N > 0) || (!dX && M * N > 0)) return 1;
    if (act == ORC_GLU && (!Y || !dY) && M * N > 0) return 1;
    if (!rows) nrows = M;
    if (nrows < 0) return 1;
    if (rows)
        for (int64_t r = 0; r < nrows; ++r)
            if (rows[r] < 0 || rows[r] >= M) return 1;
    if (dbias)
        for (int64_t j = 0; j < N; ++j) dbias[j] = 0.0;
    if (nrows == 0 || N == 0) return 0;
    double *W64 = (double *)malloc(sizeof(double) * (size_t)(N * K + 1));
    double *D = (double *)malloc(sizeof(double) * (size_t)(nrows * N));
    if (!W64 || !D) { free(W64); free(D); return 2; }
    orc_decode(dtype, W, N * K, W64);
    int status = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel
    {
        double *grow = (double *)malloc(sizeof(double) * (size_t)(K + 1));
        if (!grow) {
#pragma omp atomic write
            status = 2;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t r = 0; r < nrows; ++r) {
                int64_t i = rows ? rows[r] : r;
                for (int64_t k = 0; k < K; ++k) grow[k] = dec_one(dtype, G, i * K + k);
                for (int64_t j = 0; j < N; ++j) {
                    double d = 0.0;
                    const double *w = W64 + j * K;
                    for (int64_t k = 0; k < K; ++k) d += grow[k] * w[k];
                    const double x = dec_one(dtype, X, i * N + j);
                    const double y = (act == ORC_GLU) ? dec_one(dtype, Y, i * N + j) : 0.0;
                    if (unfused) {
                        /* the chain stores D in dtype before the elementwise pass */
                        double t[1] = {d};
                        uint16_t h[2];
                        float f[1];
                        void *slot = (dtype == ORC_F32) ? (void *)f : (void *)h;
                        orc_encode(dtype, t, 1, slot);
                        orc_decode(dtype, slot, 1, t);
                        d = t[0];
                    }
                    double dx = d * act_grad(act, x, y);
                    if (act == ORC_GLU) enc_one(dtype, d * x, dY, r * N + j);
                    enc_one(dtype, dx, dX, r * N + j);
                    if (unfused) dx = dec_one(dtype, dX, r * N + j); /* the sums read the stored dX */
                    D[r * N + j] = dx;
                    if (dx_out) dx_out[r * N + j] = dx;
                }
            }
        }
        free(grow);
    }
    /* the column sums in row order, one thread, so the result does not
       depend on the thread count */
    if (dbias && status == 0)
        for (int64_t r = 0; r < nrows; ++r)
            for (int64_t j = 0; j < N; ++j) dbias[j] += D[r * N + j];
    free(W64);
    free(D);
    return status;
}

int orc_fused_linear_bwd(int dtype, int act, const void *G, const void *W,
                         const void *X, const void *Y, void *dX, void *dY,
                         double *dbias, int64_t M, int64_t N, int64_t K,
                         const int64_t *rows, int64_t nrows, int nthreads,
                         double *dx_out) {
    return run_bwd(dtype, act, G, W, X, Y, dX, dY, dbias, M, N, K, rows, nrows, nthreads, dx_out, 0);
}

/*
 * The unfused backward chain (a product, an elementwise pass, a column sum,
 * each storing its result): D is rounded to dtype before the elementwise
 * pass, dX = round(round(D) * act'(X)), dY = round(round(D) * X), and dbias
 * sums the stored (rounded) dX.  dx_out receives the rounded dX as FP64.
 */
int orc_unfused_bwd_chain(int dtype, int act, const void *G, const void *W,
                          const void *X, const void *Y, void *dX, void *dY,
                          double *dbias, int64_t M, int64_t N, int64_t K,
                          const int64_t *rows, int64_t nrows, int nthreads,
                          double *dx_out) {
    return run_bwd(dtype, act, G, W, X, Y, dX, dY, dbias, M, N, K, rows, nrows, nthreads, dx_out, 1);
}

/* --------------------------------------------------------------- tile map */

/*
 * Grouped program-id -> (m_tile, n_tile) map ("Tiles and grouped
 * ownership"): programs sweep a band of `group` M-tiles down each N column
 * before moving right; the last band may hold fewer M-tiles, so the band
 * height is min(group, tiles_m - first_m) before the remainder/quotient.
 */
int orc_tile_of_pid(int64_t pid, int64_t tiles_m, int64_t tiles_n,
                    int64_t group, int64_t *m_tile, int64_t *n_tile) {
    if (tiles_m <= 0 || tiles_n <= 0 || group <= 0) return 1;
    if (pid < 0 || pid >= tiles_m * tiles_n) return 1;
    int64_t per_band = group * tiles_n;
    int64_t band = pid / per_band;
    int64_t first_m = band * group;
    int64_t height = tiles_m - first_m;
    if (height > group) height = group;
    int64_t r = pid % per_band;
    *m_tile = first_m + r % height;
    *n_tile = r / height;
    return 0;
}

int orc_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
