/*
 * oracle.c -- plain, slow, obviously correct CPU reference for the dense GEMM
 * C = A * B (row-major A of M x K, row-major B of K x N).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call
 * this file; only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark do.  It shares no code, header or table with the GPU library.
 *
 * What it computes (the plain definition, no blocking, no reordering):
 *   - "[CUDA 优化实战] hgemm - 超越 cuBLAS", sections 0-1: C = A*B with A and B
 *     both row-major ("A/B 都行优先"), half-precision (fp16 or bf16) inputs and
 *     an fp32 accumulator; the reference here accumulates in fp64 and never
 *     rounds the result, so the tests compare the GPU output against the exact
 *     sum up to fp64 rounding.
 *   - "CUDA GEMM 优化实践笔记", register-tiling section: the fp32 SGEMM with the
 *     same row-major indexing A[row*K + col], B[row*N + col].
 *   - "深度学习加速核心：GEMM优化从分块到TensorCore的实战解析", section 4.3: FP8
 *     (E4M3) operands, each 64x64 sub-block multiplied by its own scale factor;
 *     section 5.2 (third pitfall): the scales are 32-bit floats.
 *
 *   - the same section 4.3 and section 5.2: the quantiser that produces such
 *     operands (orc_quantize_fp8 below): one 32-bit scale per 32x32 or 64x64
 *     block, the block's largest magnitude over the largest FP8 value, and each
 *     element divided by its block's scale and stored as FP8 (E4M3 or E5M2).
 *
 * Every input is decoded bit by bit to an exact double by the decoders below
 * (they do not use compiler half/bfloat/fp8 types).  The sum for each entry runs
 * over k = 0 .. K-1 in ascending order.  Build with -ffp-contract=off and no
 * fast-math so that each step is one IEEE multiply and one IEEE add in fp64.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- decoders */

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double orc_f16_to_f64(uint16_t h)
{
    int s = (h >> 15) & 1, e = (h >> 10) & 0x1f, f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);                 /* subnormal: f * 2^(1-15-10) */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(0x400 | f), e - 25);    /* (1.f) * 2^(e-15), as an integer * 2^(e-15-10) */
    return s ? -v : v;
}

/* bfloat16: the upper half of an IEEE binary32: 1 sign, 8 exponent (bias 127), 7 fraction. */
double orc_bf16_to_f64(uint16_t b)
{
    int s = (b >> 15) & 1, e = (b >> 7) & 0xff, f = b & 0x7f;
    double v;
    if (e == 0)
        v = ldexp((double)f, -133);                /* subnormal: f * 2^(1-127-7) */
    else if (e == 255)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(0x80 | f), e - 134);    /* (128+f) * 2^(e-127-7) */
    return s ? -v : v;
}

/* OCP FP8 E4M3 ("E4M3FN"): 1 sign, 4 exponent (bias 7), 3 mantissa; no infinities;
 * S.1111.111 is NaN; largest finite magnitude 448; subnormals down to 2^-9. */
double orc_e4m3_to_f64(uint8_t q)
{
    int s = (q >> 7) & 1, e = (q >> 3) & 0xf, m = q & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);                  /* subnormal: m * 2^(1-7-3) */
    else
        v = ldexp((double)(8 | m), e - 10);        /* (8+m) * 2^(e-7-3) */
    return s ? -v : v;
}

/* OCP FP8 E5M2: 1 sign, 5 exponent (bias 15), 2 mantissa, IEEE-like: exponent
 * 31 holds the infinities (mantissa 0) and NaNs; largest finite magnitude 57344;
 * subnormals down to 2^-16. */
double orc_e5m2_to_f64(uint8_t q)
{
    int s = (q >> 7) & 1, e = (q >> 2) & 0x1f, m = q & 3;
    double v;
    if (e == 31)
        v = m ? NAN : INFINITY;
    else if (e == 0)
        v = ldexp((double)m, -16);                 /* subnormal: m * 2^(1-15-2) */
    else
        v = ldexp((double)(4 | m), e - 17);        /* (4+m) * 2^(e-15-2) */
    return s ? -v : v;
}

/* IEEE binary32 from its bit pattern, built from the fields as well. */
double orc_f32_to_f64(uint32_t u)
{
    int s = (u >> 31) & 1, e = (u >> 23) & 0xff;
    uint32_t f = u & 0x7fffff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -149);                /* subnormal: f * 2^(1-127-23) */
    else if (e == 255)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(0x800000u | f), e - 150);
    return s ? -v : v;
}

void orc_decode_f16(const uint16_t *in, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; i++) out[i] = orc_f16_to_f64(in[i]);
}
void orc_decode_bf16(const uint16_t *in, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; i++) out[i] = orc_bf16_to_f64(in[i]);
}
void orc_decode_e4m3(const uint8_t *in, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; i++) out[i] = orc_e4m3_to_f64(in[i]);
}
void orc_decode_e5m2(const uint8_t *in, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; i++) out[i] = orc_e5m2_to_f64(in[i]);
}

void orc_decode_f32(const uint32_t *in, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; i++) out[i] = orc_f32_to_f64(in[i]);
}

/* ------------------------------------------------------ operand decoding */

enum { ORC_F16 = 0, ORC_BF16 = 1, ORC_F32 = 2, ORC_FP8 = 3 };

/* Block edge of the FP8 scale grid (64x64 sub-blocks). */
#define ORC_SCALE_BLOCK 64

/* Value of element (r, c) of a row-major operand with leading dimension ld.
 * For FP8, scale is the row-major grid of per-block fp32 scales with
 * scale_cols columns, and the element is e4m3(q) * scale[r/64][c/64]. */
static double operand_at(int dtype, const void *p, int64_t ld, int64_t r, int64_t c,
                         const float *scale, int64_t scale_cols)
{
    int64_t idx = r * ld + c;
    switch (dtype) {
    case ORC_F16:  return orc_f16_to_f64(((const uint16_t *)p)[idx]);
    case ORC_BF16: return orc_bf16_to_f64(((const uint16_t *)p)[idx]);
    case ORC_F32:  return orc_f32_to_f64(((const uint32_t *)p)[idx]);
    default: {
        uint32_t sbits;
        float s = scale[(r / ORC_SCALE_BLOCK) * scale_cols + (c / ORC_SCALE_BLOCK)];
        memcpy(&sbits, &s, 4);
        return orc_e4m3_to_f64(((const uint8_t *)p)[idx]) * orc_f32_to_f64(sbits);
    }
    }
}

/* Decode a rows x cols operand into a dense fp64 array (leading dimension cols). */
static void decode_operand(int dtype, const void *p, int64_t ld, int64_t rows, int64_t cols,
                           const float *scale, double *out)
{
    int64_t scale_cols = (cols + ORC_SCALE_BLOCK - 1) / ORC_SCALE_BLOCK;
    for (int64_t r = 0; r < rows; r++)
        for (int64_t c = 0; c < cols; c++)
            out[r * cols + c] = operand_at(dtype, p, ld, r, c, scale, scale_cols);
}

/* ------------------------------------------------------------ the product */

typedef struct {
    const double *a, *b;   /* M x K and K x N, dense */
    double *c;             /* M x N, leading dimension ldc */
    int64_t n, k, ldc, row0, row1;
} rows_job;

/* C[i][j] = sum_{k=0}^{K-1} A[i][k] * B[k][j] for rows row0 <= i < row1.
 * The i-k-j loop order adds the terms of every entry in ascending k, exactly
 * like the textbook i-j-k triple loop; it only visits memory in rows. */
static void *rows_worker(void *arg)
{
    const rows_job *job = (const rows_job *)arg;
    for (int64_t i = job->row0; i < job->row1; i++) {
        double *ci = job->c + i * job->ldc;
        for (int64_t j = 0; j < job->n; j++) ci[j] = 0.0;
        for (int64_t kk = 0; kk < job->k; kk++) {
            double aik = job->a[i * job->k + kk];
            const double *bk = job->b + kk * job->n;
            for (int64_t j = 0; j < job->n; j++) ci[j] = ci[j] + aik * bk[j];
        }
    }
    return NULL;
}

static int run_rows(const double *a, const double *b, double *c, int64_t m, int64_t n, int64_t k,
                    int64_t ldc, int nthreads)
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (m < nthreads) nthreads = m > 0 ? (int)m : 1;
    pthread_t tid[256];
    int running[256];
    rows_job jobs[256];
    int64_t per = (m + nthreads - 1) / nthreads;
    for (int t = 0; t < nthreads; t++) {
        jobs[t].a = a; jobs[t].b = b; jobs[t].c = c;
        jobs[t].n = n; jobs[t].k = k; jobs[t].ldc = ldc;
        jobs[t].row0 = t * per < m ? t * per : m;
        jobs[t].row1 = (t + 1) * per < m ? (t + 1) * per : m;
        running[t] = nthreads > 1 && pthread_create(&tid[t], NULL, rows_worker, &jobs[t]) == 0;
        if (!running[t]) rows_worker(&jobs[t]);   /* single thread, or no thread: do the rows here */
    }
    for (int t = 0; t < nthreads; t++)
        if (running[t]) pthread_join(tid[t], NULL);
    return 0;
}

/*
 * Full reference product.  A: M x K (leading dimension lda), B: K x N (ldb),
 * raw bits of the given dtype; for FP8 scale_a is the ceil(M/64) x ceil(K/64)
 * grid and scale_b the ceil(K/64) x ceil(N/64) grid, both row-major fp32.
 * out: M x N fp64 with leading dimension ldo (the exact sum, not rounded).
 * Returns 0, or -1 on a bad argument / allocation failure.
 */
int orc_gemm(int dtype, const void *A, const void *B, const float *scale_a, const float *scale_b,
             int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, double *out, int64_t ldo,
             int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || lda < K || ldb < N || ldo < N) return -1;
    if (dtype == ORC_FP8 && K > 0 && (!scale_a || !scale_b)) return -1;
    if (M == 0 || N == 0) return 0;
    double *a = (double *)malloc(sizeof(double) * (size_t)(M * (K > 0 ? K : 1)));
    double *b = (double *)malloc(sizeof(double) * (size_t)((K > 0 ? K : 1) * N));
    if (!a || !b) { free(a); free(b); return -1; }
    decode_operand(dtype, A, lda, M, K, scale_a, a);
    decode_operand(dtype, B, ldb, K, N, scale_b, b);
    run_rows(a, b, out, M, N, K, ldo, nthreads);
    free(a);
    free(b);
    return 0;
}

/*
 * The same sum for a list of entries (rows[t], cols[t]) only, decoding the
 * operands on the fly: used to check products too large to form in full.
 */
int orc_gemm_entries(int dtype, const void *A, const void *B, const float *scale_a,
                     const float *scale_b, int64_t M, int64_t N, int64_t K, int64_t lda,
                     int64_t ldb, const int64_t *rows, const int64_t *cols, int64_t count,
                     double *out)
{
    if (M < 0 || N < 0 || K < 0 || lda < K || ldb < N) return -1;
    int64_t sa_cols = (K + ORC_SCALE_BLOCK - 1) / ORC_SCALE_BLOCK;
    int64_t sb_cols = (N + ORC_SCALE_BLOCK - 1) / ORC_SCALE_BLOCK;
    for (int64_t t = 0; t < count; t++) {
        int64_t i = rows[t], j = cols[t];
        if (i < 0 || i >= M || j < 0 || j >= N) return -1;
        double acc = 0.0;
        for (int64_t kk = 0; kk < K; kk++)
            acc = acc + operand_at(dtype, A, lda, i, kk, scale_a, sa_cols) *
                            operand_at(dtype, B, ldb, kk, j, scale_b, sb_cols);
        out[t] = acc;
    }
    return 0;
}

/* -------------------------------------------------------- FP8 quantiser */

/* "深度学习加速核心：GEMM优化从分块到TensorCore的实战解析", section 4.3 (FP8
 * operands with one scale per 32x32 or 64x64 sub-block) and section 5.2, third
 * pitfall (32-bit scales).  Reading of the steps, all in fp32 arithmetic:
 *   amax = largest |x| of the block (elements inside the matrix only),
 *   s    = amax / F with F the largest finite FP8 value (448 for E4M3, 57344
 *          for E5M2), one IEEE division; s = 1 when amax = 0,
 *   y    = x / s, one IEEE division per element, clamped to [-F, F],
 *   q    = the FP8 value nearest to y, ties to the even mantissa, sign kept
 *          (also when y rounds to zero).
 * Inputs must be finite. */
#define ORC_FP8_E4M3 0
#define ORC_FP8_E5M2 1

/* Nearest FP8 code to a finite y with |y| <= F, ties to even. */
uint8_t orc_fp8_encode(float y, int fmt)
{
    const int mbits = fmt == ORC_FP8_E4M3 ? 3 : 2;
    const int bias = fmt == ORC_FP8_E4M3 ? 7 : 15;
    const int emin = 1 - bias;                     /* exponent of the smallest normal */
    const uint8_t sign = signbit(y) ? 0x80 : 0;
    const double a = fabs((double)y);
    int e = emin;                                  /* binade of a; the subnormals share emin's spacing */
    if (a > 0) {
        int ex;
        frexp(a, &ex);                             /* a = f * 2^ex, f in [1/2, 1) */
        if (ex - 1 > e) e = ex - 1;
    }
    const double quantum = ldexp(1.0, e - mbits);  /* spacing of the FP8 values there */
    double n = rint(a / quantum);                  /* exact quotient; rint: nearest, ties to even */
    if (n >= ldexp(1.0, mbits + 1)) {              /* rounded up to the next binade's first value */
        e += 1;
        n = ldexp(1.0, mbits);
    }
    int expfield, mant;
    if (n < ldexp(1.0, mbits)) {                   /* subnormal (e == emin) */
        expfield = 0;
        mant = (int)n;
    } else {
        expfield = e + bias;
        mant = (int)n - (1 << mbits);
    }
    return (uint8_t)(sign | (expfield << mbits) | mant);
}

void orc_fp8_encode_array(const float *y, int64_t n, int fmt, uint8_t *out)
{
    for (int64_t i = 0; i < n; i++) out[i] = orc_fp8_encode(y[i], fmt);
}

static float input_f32(int dtype, const void *X, int64_t ld, int64_t r, int64_t c)
{
    if (dtype == ORC_BF16) return (float)orc_bf16_to_f64(((const uint16_t *)X)[r * ld + c]);
    uint32_t u;
    memcpy(&u, (const uint32_t *)X + r * ld + c, 4);
    return (float)orc_f32_to_f64(u);
}

/* X: rows x cols, row-major with leading dimension ldx, fp32 (ORC_F32) or bf16
 * (ORC_BF16) bits.  Q: rows x cols FP8 codes, leading dimension ldq.  scales:
 * ceil(rows/block) x ceil(cols/block) fp32, row-major and contiguous.
 * Returns 0, or -1 for arguments it does not handle. */
int orc_quantize_fp8(int dtype, const void *X, int64_t rows, int64_t cols, int64_t ldx,
                     int block, int fmt, uint8_t *Q, int64_t ldq, float *scales)
{
    if ((dtype != ORC_F32 && dtype != ORC_BF16) || (block != 32 && block != 64) ||
        (fmt != ORC_FP8_E4M3 && fmt != ORC_FP8_E5M2) || rows < 0 || cols < 0 ||
        ldx < cols || ldq < cols)
        return -1;
    const float fmax = fmt == ORC_FP8_E4M3 ? 448.0f : 57344.0f;
    const int64_t br = (rows + block - 1) / block, bc = (cols + block - 1) / block;
    for (int64_t bi = 0; bi < br; bi++)
        for (int64_t bj = 0; bj < bc; bj++) {
            const int64_t r0 = bi * block, c0 = bj * block;
            const int64_t r1 = r0 + block < rows ? r0 + block : rows;
            const int64_t c1 = c0 + block < cols ? c0 + block : cols;
            float amax = 0.0f;
            for (int64_t r = r0; r < r1; r++)
                for (int64_t c = c0; c < c1; c++) {
                    const float a = fabsf(input_f32(dtype, X, ldx, r, c));
                    if (a > amax) amax = a;
                }
            const float s = amax > 0.0f ? amax / fmax : 1.0f;
            scales[bi * bc + bj] = s;
            for (int64_t r = r0; r < r1; r++)
                for (int64_t c = c0; c < c1; c++) {
                    float y = input_f32(dtype, X, ldx, r, c) / s;
                    if (y > fmax) y = fmax;
                    if (y < -fmax) y = -fmax;
                    Q[r * ldq + c] = orc_fp8_encode(y, fmt);
                }
        }
    return 0;
}

/* ---------------------------------------------------- fused epilogue */

/* The step after the product, applied entry by entry to the exact sum:
 *   out[i][j] = act( alpha * prod[i][j] + beta * c(i, j) + bias[j] )
 * "深度学习加速核心：GEMM优化从分块到TensorCore的实战解析", section 1.1: a
 * fully connected layer is a matrix product plus a bias, one bias value per
 * output feature, i.e. per column j of C (C = X * W with X of batch x inputs and
 * W of inputs x outputs).  "[CUDA 优化实战] hgemm - 超越 cuBLAS", section 5: the
 * vendor kernel it compares against carries a relu in its epilogue, so the
 * activation is max(v, 0) applied last.  alpha and beta are the usual scales
 * of the product and of the C already in memory; the pages name neither, so
 * their reading is the plain BLAS one: c(i, j) is the prior output value decoded
 * from the output type's bits (row-major, leading dimension ldc) and it is read
 * only when beta != 0, so a C that holds garbage (even NaN) is fine then.
 * bias may be NULL (no bias).  act: 0 = none, 1 = relu.
 * prod and out are M x N fp64 with leading dimension N (out may be prod).
 * out_dtype: ORC_F16, ORC_BF16 or ORC_F32.  Returns 0, or -1 on bad arguments. */
int orc_epilogue(int out_dtype, const double *prod, int64_t M, int64_t N, double alpha,
                 double beta, const void *c_bits, int64_t ldc, const float *bias, int act,
                 double *out)
{
    if (M < 0 || N < 0 || ldc < N || (act != 0 && act != 1)) return -1;
    if (out_dtype != ORC_F16 && out_dtype != ORC_BF16 && out_dtype != ORC_F32) return -1;
    if (beta != 0.0 && !c_bits && M > 0 && N > 0) return -1;
    for (int64_t i = 0; i < M; i++)
        for (int64_t j = 0; j < N; j++) {
            double v = alpha * prod[i * N + j];
            if (beta != 0.0) v = v + beta * operand_at(out_dtype, c_bits, ldc, i, j, NULL, 0);
            if (bias) {
                uint32_t bbits;
                memcpy(&bbits, &bias[j], 4);
                v = v + orc_f32_to_f64(bbits);
            }
            if (act == 1 && !(v > 0.0)) v = 0.0;
            out[i * N + j] = v;
        }
    return 0;
}

/* ------------------------------------------------- convolution (direct) */

/* "深度学习加速核心：GEMM优化从分块到TensorCore的实战解析" section 1.1: a
 * convolution is a GEMM once every output position's receptive field is laid
 * out as one row of a large matrix (im2col).  The oracle computes the
 * convolution itself, by its definition, not through that matrix:
 *   Y[n][oh][ow][co] = sum over kh < KH, kw < KW, ci < C_in of
 *                      X[n][oh*sh - ph + kh*dh][ow*sw - pw + kw*dw][ci] * Wt[kh][kw][ci][co]
 * with X read as 0 outside the H x W image (zero padding).  Layouts (the pages
 * fix none; channels-last is the plain reading for a GEMM whose rows are output
 * positions): X is NHWC, Wt is KH x KW x C_in x C_out ("HWIO"), Y is NHWC,
 * all dense.  Output size: Ho = (H + 2 ph - dh (KH-1) - 1) / sh + 1 (floor),
 * likewise Wo.  geom = {n, h, w, c_in, c_out, kh, kw, sh, sw, ph, pw, dh, dw}.
 * The sum runs over (kh, kw, ci) in that nesting, ascending, in fp64.
 * dtype: ORC_F16, ORC_BF16 or ORC_F32 for X and Wt.  out: n*Ho*Wo*C_out. */
static int conv_geometry(const int64_t *g, int64_t *ho, int64_t *wo)
{
    for (int i = 0; i < 13; i++)
        if (g[i] < 0) return -1;
    if (g[5] < 1 || g[6] < 1 || g[7] < 1 || g[8] < 1 || g[11] < 1 || g[12] < 1) return -1;
    const int64_t eh = g[1] + 2 * g[9] - g[11] * (g[5] - 1) - 1;
    const int64_t ew = g[2] + 2 * g[10] - g[12] * (g[6] - 1) - 1;
    *ho = eh < 0 ? 0 : eh / g[7] + 1;
    *wo = ew < 0 ? 0 : ew / g[8] + 1;
    return 0;
}

int orc_conv2d_output_size(const int64_t *geom, int64_t *ho, int64_t *wo)
{
    return conv_geometry(geom, ho, wo);
}

int orc_conv2d_nhwc(int dtype, const void *X, const void *Wt, const int64_t *geom, double *out)
{
    int64_t ho, wo;
    if (conv_geometry(geom, &ho, &wo) != 0) return -1;
    if (dtype != ORC_F16 && dtype != ORC_BF16 && dtype != ORC_F32) return -1;
    const int64_t N = geom[0], H = geom[1], W = geom[2], CI = geom[3], CO = geom[4];
    const int64_t KH = geom[5], KW = geom[6], SH = geom[7], SW = geom[8];
    const int64_t PH = geom[9], PW = geom[10], DH = geom[11], DW = geom[12];
    for (int64_t n = 0; n < N; n++)
        for (int64_t oh = 0; oh < ho; oh++)
            for (int64_t ow = 0; ow < wo; ow++)
                for (int64_t co = 0; co < CO; co++) {
                    double acc = 0.0;
                    for (int64_t kh = 0; kh < KH; kh++) {
                        const int64_t ih = oh * SH - PH + kh * DH;
                        for (int64_t kw = 0; kw < KW; kw++) {
                            const int64_t iw = ow * SW - PW + kw * DW;
                            for (int64_t ci = 0; ci < CI; ci++) {
                                double x = 0.0;
                                if (ih >= 0 && ih < H && iw >= 0 && iw < W)
                                    x = operand_at(dtype, X, CI, (n * H + ih) * W + iw, ci, NULL, 0);
                                const double wv =
                                    operand_at(dtype, Wt, CO, (kh * KW + kw) * CI + ci, co, NULL, 0);
                                acc = acc + x * wv;
                            }
                        }
                    }
                    out[((n * ho + oh) * wo + ow) * CO + co] = acc;
                }
    return 0;
}

/* The im2col matrix itself (raw element bits, esize 2 or 4 bytes): row
 * (n, oh, ow), column (kh, kw, ci), i.e.
 *   col[((n*Ho + oh)*Wo + ow) * ldcol + (kh*KW + kw)*C_in + ci]
 *     = X[n][oh*sh - ph + kh*dh][ow*sw - pw + kw*dw][ci], or 0 outside the image.
 * The convolution is then col (M x K) times Wt seen as (KH*KW*C_in) x C_out. */
int orc_im2col_nhwc(int esize, const void *X, const int64_t *geom, void *col, int64_t ldcol)
{
    int64_t ho, wo;
    if (conv_geometry(geom, &ho, &wo) != 0 || (esize != 2 && esize != 4)) return -1;
    const int64_t N = geom[0], H = geom[1], W = geom[2], CI = geom[3];
    const int64_t KH = geom[5], KW = geom[6], SH = geom[7], SW = geom[8];
    const int64_t PH = geom[9], PW = geom[10], DH = geom[11], DW = geom[12];
    if (ldcol < KH * KW * CI) return -1;
    for (int64_t n = 0; n < N; n++)
        for (int64_t oh = 0; oh < ho; oh++)
            for (int64_t ow = 0; ow < wo; ow++) {
                const int64_t row = (n * ho + oh) * wo + ow;
                for (int64_t kh = 0; kh < KH; kh++)
                    for (int64_t kw = 0; kw < KW; kw++) {
                        const int64_t ih = oh * SH - PH + kh * DH, iw = ow * SW - PW + kw * DW;
                        const int inside = ih >= 0 && ih < H && iw >= 0 && iw < W;
                        for (int64_t ci = 0; ci < CI; ci++) {
                            const int64_t dst = row * ldcol + (kh * KW + kw) * CI + ci;
                            const int64_t src = ((n * H + ih) * W + iw) * CI + ci;
                            if (esize == 2)
                                ((uint16_t *)col)[dst] = inside ? ((const uint16_t *)X)[src] : 0;
                            else
                                ((uint32_t *)col)[dst] = inside ? ((const uint32_t *)X)[src] : 0;
                        }
                    }
            }
    return 0;
}
