/*
 * libgemm -- dense GEMM C = A * B on AMD Instinct MI355X (gfx950).
 *
 * The operation (the four GEMM entry points):
 *   C[i*ldc + j] = round_out( sum_{k<K} a(i,k) * b(k,j) )   for 0 <= i < M, 0 <= j < N,
 * with a(i,k) = A[i*lda + k] and b(k,j) = B[k*ldb + j]: A is M x K and B is K x N,
 * both row-major, as in "[CUDA 优化实战] hgemm - 超越 cuBLAS" sections 0-1 (both
 * operands row-major, fp16/bf16 inputs, fp32 accumulator, results rounded to the
 * output type with round-to-nearest-even) and in the register-tiling section of
 * "CUDA GEMM 优化实践笔记" (fp32 SGEMM, same indexing).  The sum is accumulated in
 * fp32 in an order of the library's choosing.  There is no transpose, and C is
 * overwritten; the *_epilogue variants below add alpha, beta, a bias and relu.
 * Bytes of C outside the M x N window (the padding between N and ldc) are never
 * written.
 *
 * Conventions shared by every entry point:
 *   - A, B, C (and the fp8 scales) are DEVICE pointers owned by the caller, on the
 *     current HIP device; the library never allocates, frees or synchronises, keeps
 *     no state between calls and may be called from several host threads.
 *   - 0 <= M, N, K <= 2^31 - 2^16 (else GEMM_ERR_DIM); lda >= K, ldb >= N,
 *     ldc >= N (elements, not bytes).
 *   - Pointers must be aligned to their element size and non-NULL whenever the
 *     region they describe is non-empty.  C must not overlap A, B or the scales.
 *   - M == 0 or N == 0: nothing to do, returns GEMM_OK without a launch.
 *     K == 0: the sums are empty, so the M x N window of C is set to zero.
 *   - Work is enqueued on `stream` (NULL = the default stream) and the call returns
 *     without waiting.  Argument errors are detected synchronously and nothing is
 *     launched.  A fault inside a kernel surfaces at the caller's next
 *     synchronisation, as for any HIP kernel.
 *   - Return value: GEMM_OK (0) or a negative gemm_status; gemm_status_string()
 *     describes it.
 */
#ifndef LIBGEMM_H
#define LIBGEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same definition as in the HIP runtime headers. */
typedef struct ihipStream_t *hipStream_t;

enum gemm_status {
    GEMM_OK = 0,
    GEMM_ERR_NULL = -1,    /* a required pointer is NULL */
    GEMM_ERR_DIM = -2,     /* M, N or K negative, or larger than the library supports */
    GEMM_ERR_LD = -3,      /* lda < K, ldb < N or ldc < N */
    GEMM_ERR_ALIGN = -4,   /* a pointer is not aligned to its element size */
    GEMM_ERR_ALIAS = -5,   /* an output overlaps an input (or another output) */
    GEMM_ERR_DEVICE = -6,  /* the current device is not a gfx950 GPU, or it cannot be queried */
    GEMM_ERR_LAUNCH = -7,  /* the kernel launch was rejected by the runtime */
    GEMM_ERR_ARG = -8,     /* an option (input type, block size, FP8 format, activation, alpha/beta) is not supported */
    GEMM_ERR_WORKSPACE = -9, /* a caller-provided workspace is missing or too small */
    GEMM_ERR_SCRATCH = -10   /* the call needs more than the library's fixed scratch array holds */
};

/* Element types of the convolution entry points. */
enum gemm_dtype { GEMM_DTYPE_F16 = 0, GEMM_DTYPE_BF16 = 1, GEMM_DTYPE_F32 = 2 };

/* FP8 formats (OCP): E4M3 ("E4M3FN": bias 7, largest finite 448, no infinities)
 * and E5M2 (bias 15, largest finite 57344). */
enum gemm_fp8_format { GEMM_FP8_E4M3 = 0, GEMM_FP8_E5M2 = 1 };

/* Element types the FP8 quantiser reads. */
enum gemm_quant_input { GEMM_QUANT_IN_F32 = 0, GEMM_QUANT_IN_BF16 = 1 };

/* Activations of the fused epilogue. */
enum gemm_activation { GEMM_ACT_NONE = 0, GEMM_ACT_RELU = 1 };

/* fp16 (IEEE binary16) A, B and C; fp32 accumulation; C rounded to nearest-even.
 * "[CUDA 优化实战] hgemm - 超越 cuBLAS", sections 1-4 (the half-precision kernels). */
int gemm_f16(const void *A, const void *B, void *C, int64_t M, int64_t N, int64_t K,
             int64_t lda, int64_t ldb, int64_t ldc, hipStream_t stream);

/* bfloat16 A, B and C; fp32 accumulation; C rounded to nearest-even.
 * Same passage as gemm_f16: one kernel design serves both half formats. */
int gemm_bf16(const void *A, const void *B, void *C, int64_t M, int64_t N, int64_t K,
              int64_t lda, int64_t ldb, int64_t ldc, hipStream_t stream);

/* fp32 A, B and C (SGEMM); fp32 accumulation.
 * "CUDA GEMM 优化实践笔记", register-tiling section (BM/BN/BK/TM/TN listing and the
 * zero fill of out-of-range operand elements). */
int gemm_f32(const float *A, const float *B, float *C, int64_t M, int64_t N, int64_t K,
             int64_t lda, int64_t ldb, int64_t ldc, hipStream_t stream);

/* FP8 block-scaled GEMM.  A and B hold OCP E4M3 ("E4M3FN") codes, one byte each.
 * Every 64 x 64 sub-block of A and of B carries one fp32 scale:
 *   a(i,k) = e4m3(A[i*lda + k]) * scale_a[(i/64) * ceil(K/64) + k/64]
 *   b(k,j) = e4m3(B[k*ldb + j]) * scale_b[(k/64) * ceil(N/64) + j/64]
 * i.e. scale_a is the row-major ceil(M/64) x ceil(K/64) grid and scale_b the
 * row-major ceil(K/64) x ceil(N/64) grid (blocks at ragged edges are partial).
 * The products are accumulated in fp32 and C is bfloat16, rounded to nearest-even.
 * "深度学习加速核心：GEMM优化从分块到TensorCore的实战解析", section 4.3 (E4M3
 * operands scaled per 32x32 or 64x64 sub-block; 64x64 here) and section 5.2, third
 * pitfall (the scale factors are kept in 32 bits).  Scales must be finite. */
int gemm_fp8_blockscaled(const uint8_t *A, const uint8_t *B, void *C, int64_t M, int64_t N,
                         int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
                         const float *scale_a, const float *scale_b, hipStream_t stream);

/* Fused epilogue variants of the four GEMMs.  Same operands, layouts, checks
 * and rules as the plain entry points above, except that every entry of the
 * M x N window becomes
 *   C[i*ldc + j] = round_out( act( alpha * s(i,j) + beta * c(i,j) + bias[j] ) )
 * with s(i,j) the fp32-accumulated sum of the plain entry point, c(i,j) the
 * value C[i*ldc + j] held before the call, and the whole expression evaluated
 * in fp32 before the one rounding to C's type.
 *   - A fully connected layer is a product plus one bias per output feature,
 *     "深度学习加速核心：GEMM优化从分块到TensorCore的实战解析" section 1.1: bias
 *     is a device vector of N fp32 values, one per column of C (NULL: no bias).
 *   - activation: GEMM_ACT_NONE, or GEMM_ACT_RELU = max(x, 0) applied last, the
 *     epilogue of the vendor kernel "[CUDA 优化实战] hgemm - 超越 cuBLAS" section 5
 *     compares against.
 *   - alpha, beta: host fp32 scalars (the pages name neither; they are the usual
 *     scales of the product and of the prior C).  When beta == 0, C is not read,
 *     so it may hold anything, NaN included.
 *   - K == 0: every sum is empty, so C becomes act(beta * c + bias[j]).
 * Errors: GEMM_ERR_ARG for an unknown activation or a non-finite alpha or beta
 * (checked before anything else); then those of the plain entry point; then,
 * for a call with work to do, GEMM_ERR_ALIGN for a bias not 4-byte aligned and
 * GEMM_ERR_ALIAS for a bias overlapping C.  The bias is read only, caller-owned
 * and on the device. */
int gemm_f16_epilogue(const void *A, const void *B, void *C, int64_t M, int64_t N, int64_t K,
                      int64_t lda, int64_t ldb, int64_t ldc, float alpha, float beta,
                      const float *bias, int activation, hipStream_t stream);
int gemm_bf16_epilogue(const void *A, const void *B, void *C, int64_t M, int64_t N, int64_t K,
                       int64_t lda, int64_t ldb, int64_t ldc, float alpha, float beta,
                       const float *bias, int activation, hipStream_t stream);
int gemm_f32_epilogue(const float *A, const float *B, float *C, int64_t M, int64_t N, int64_t K,
                      int64_t lda, int64_t ldb, int64_t ldc, float alpha, float beta,
                      const float *bias, int activation, hipStream_t stream);
int gemm_fp8_blockscaled_epilogue(const uint8_t *A, const uint8_t *B, void *C, int64_t M,
                                  int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
                                  const float *scale_a, const float *scale_b, float alpha,
                                  float beta, const float *bias, int activation,
                                  hipStream_t stream);

/* Block-scaled FP8 quantiser: the step that produces gemm_fp8_blockscaled's
 * operands.  X is rows x cols, row-major with leading dimension ldx (elements),
 * fp32 (in_type GEMM_QUANT_IN_F32) or bfloat16 (GEMM_QUANT_IN_BF16).  For every
 * block x block block (block 32 or 64; blocks at ragged edges are partial):
 *   amax = the largest |x| of the block's elements,
 *   s    = amax / F in fp32 (F = 448 for E4M3, 57344 for E5M2); s = 1 if amax = 0,
 *   Q[i*ldq + j] = the FP8 code (fmt) nearest to clamp(x(i,j) / s, -F, F) in fp32,
 *                  ties to the even code, sign kept for results that round to 0,
 *   scales[(i/block) * ceil(cols/block) + j/block] = s   (row-major, contiguous).
 * With block 64 and E4M3, an M x K matrix gives exactly gemm_fp8_blockscaled's A
 * and scale_a, and a K x N matrix its B and scale_b.
 * "深度学习加速核心：GEMM优化从分块到TensorCore的实战解析", section 4.3 (FP8
 * operands with one scale per 32x32 or 64x64 sub-block) and section 5.2, third
 * pitfall (32-bit scales).  The pages only say that each block is scaled into
 * the FP8 range; the amax / F scale and the round-to-nearest-even encoding are
 * the plain reading of that.
 * X must be finite.  X, Q and scales are caller-owned device pointers (X aligned
 * to its element size, scales to 4 bytes); Q and scales must not overlap X or
 * each other.  rows == 0 or cols == 0 is a no-op.  Bytes of Q between cols and
 * ldq are never written.  Errors: GEMM_ERR_ARG for an unknown in_type, block or
 * fmt, else as for the GEMM entry points. */
int gemm_quantize_fp8(const void *X, int in_type, int64_t rows, int64_t cols, int64_t ldx,
                      int block, int fmt, uint8_t *Q, int64_t ldq, float *scales,
                      hipStream_t stream);

/* Rungs of the measured optimisation ladder (gemm_h16_ladder). */
enum gemm_ladder_rung {
    GEMM_LADDER_NAIVE = 0,           /* one thread per entry, operands from global memory */
    GEMM_LADDER_LDS_TILED = 1,       /* 64 x 64 tiles staged in LDS, operands read from LDS */
    GEMM_LADDER_REGISTER_TILED = 2,  /* + 4 x 4 outputs per thread from register-held fragments,
                                        bank-conflict-free LDS layout */
    GEMM_LADDER_MFMA = 3,            /* matrix cores: 128 x 128 tiles, 4 waves, one LDS stage */
    GEMM_LADDER_MFMA_DOUBLE_BUFFER = 4,  /* + two-stage LDS ring (loads overlap the MFMAs) */
    GEMM_LADDER_MFMA_SWIZZLE = 5,    /* + XOR-swizzled 16-byte LDS chunks */
    GEMM_LADDER_LIBRARY = 6,         /* the library's own dispatch (gemm_f16 / gemm_bf16) */
    GEMM_LADDER_MFMA_ONE_WG = 7,     /* rung 3 with LDS reserved so that one workgroup runs per CU */
    GEMM_LADDER_MFMA_DOUBLE_BUFFER_ONE_WG = 8  /* rung 4, likewise: the ring's overlap is no longer
                                                  hidden by other resident workgroups */
};

/* The optimisation ladder, for measurement: the same product as gemm_f16
 * (is_bf16 = 0) or gemm_bf16 (is_bf16 = 1), computed by the kernel of one rung
 * of "深度学习加速核心：GEMM优化从分块到TensorCore的实战解析" section 5.3 (plain
 * triple loop; 64 x 64 shared-memory tiles; register caching with bank
 * conflicts avoided; matrix-core instructions; double buffering; swizzled
 * layout), with the kernel design of sections 3.1-3.2 for the tiled rungs and
 * the last steps of "[CUDA 优化实战] hgemm - 超越 cuBLAS" for the top rung (the
 * library's LDS-direct, coalesced-store kernel).  Rungs 7 and 8 repeat rungs 3
 * and 4 at one workgroup per CU, where double buffering is not hidden by other
 * resident workgroups.  Rungs 0-2 run on the vector
 * ALUs (fp32 FMAs, k ascending); rungs 3-6 on the matrix cores.  Every rung
 * takes every shape and layout gemm_f16 takes, except that rungs 0-2 allow at
 * most 65535 grid rows (M <= 1048560 for rung 0, M <= 4194240 for rungs 1-2;
 * else GEMM_ERR_DIM).  Same checks, errors and ownership as gemm_f16; an
 * unknown rung or is_bf16 gives GEMM_ERR_ARG. */
int gemm_h16_ladder(int rung, int is_bf16, const void *A, const void *B, void *C, int64_t M,
                    int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
                    hipStream_t stream);

/* MFMA-only ceiling of the large-tile fp16 (is_bf16 = 0) or bf16 kernel, for
 * measurement: one workgroup of 4 waves per 256 x 256 tile issues exactly that
 * kernel's matrix-core instructions for an M x N x K product (K/16 steps of 16
 * v_mfma_f32_32x32x16 per wave, in the same order) on operand fragments loaded
 * once from A[:, 0:32] and B[0:32, :] and held in registers, alternating the
 * k = 0..15 and k = 16..31 halves step by step, with no memory traffic in the
 * loop.  Its time is what the matrix cores sustain on these operand values at
 * the clock the chip holds under that load.  It writes
 *   C = round( (K/32) * A[:, 0:32] * B[0:32, :] )    (fp32 accumulation),
 * needs M and N multiples of 256, K a multiple of 32 (else GEMM_ERR_DIM) and
 * 16-byte aligned A, B, C with leading dimensions multiples of 8 (else
 * GEMM_ERR_ALIGN).  Otherwise as gemm_f16. */
int gemm_h16_mfma_ceiling(int is_bf16, const void *A, const void *B, void *C, int64_t M,
                          int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
                          hipStream_t stream);

/* Geometry of a 2-D convolution (all elements, not bytes):
 *   input  X : n x h x w x c_in            (NHWC, dense)
 *   weights Wt: kh x kw x c_in x c_out     ("HWIO", dense)
 *   output Y : n x ho x wo x c_out         (NHWC, dense)
 * with ho = floor((h + 2 pad_h - dil_h (kh - 1) - 1) / stride_h) + 1 and wo
 * likewise (0 when the dilated kernel does not fit).  kh, kw, strides and
 * dilations >= 1; paddings >= 0 (zeros); h, w, kh, kw, strides, paddings and
 * dilations at most 32768; n, c_in, c_out, n*ho*wo and kh*kw*c_in at most
 * 2^31 - 2^16. */
typedef struct gemm_conv2d_shape {
    int64_t n, h, w, c_in, c_out, kh, kw, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w;
} gemm_conv2d_shape;

/* Convolution as a GEMM through im2col, "深度学习加速核心：GEMM优化从分块到
 * TensorCore的实战解析" section 1.1 (each output position's receptive field laid
 * out as one row of a large matrix turns the convolution into a GEMM, for the
 * extra memory that matrix takes):
 *   Y[n][oh][ow][co] = round( act( sum_{kh, kw, ci} X[n][ih][iw][ci] * Wt[kh][kw][ci][co]
 *                                  + bias[co] ) ),
 *   ih = oh*stride_h - pad_h + kh*dil_h,  iw = ow*stride_w - pad_w + kw*dil_w,
 * X read as 0 outside the image.  The im2col matrix (n*ho*wo rows of
 * kh*kw*c_in elements, row (n, oh, ow), column (kh, kw, ci)) is built in the
 * caller's workspace by gemm_im2col_nhwc's kernel and multiplied by Wt, seen as
 * the (kh*kw*c_in) x c_out row-major matrix it already is, by the GEMM of the
 * same type (fp32 accumulation, one rounding), with bias and activation fused
 * as in gemm_*_epilogue (bias: NULL or c_out device fp32 values, one per output
 * channel).  A 1 x 1 convolution with unit strides and no padding uses X
 * directly and needs no workspace.  dtype: GEMM_DTYPE_F16, _BF16 or _F32 for
 * X, Wt and Y alike.  The layouts are a reading: the pages fix none.
 * Work is enqueued on `stream` (im2col, then the GEMM); the workspace is
 * caller-owned device memory of at least gemm_conv2d_workspace_bytes() bytes
 * that must stay untouched until that work is done.  n*ho*wo == 0 or
 * c_out == 0: nothing to do.  c_in == 0: Y = act(bias).
 * Errors: GEMM_ERR_ARG (dtype, activation), GEMM_ERR_NULL (shape or a needed
 * pointer), GEMM_ERR_DIM (geometry), GEMM_ERR_ALIGN (pointers not aligned to the
 * element size, bias to 4 bytes), GEMM_ERR_WORKSPACE, GEMM_ERR_ALIAS (Y, the
 * workspace and the inputs must not overlap), then those of the GEMM. */
int gemm_conv2d_nhwc(int dtype, const void *X, const void *Wt, void *Y, void *workspace,
                     int64_t workspace_bytes, const gemm_conv2d_shape *shape, const float *bias,
                     int activation, hipStream_t stream);

/* Bytes of the device array gemm_conv2d_nhwc_noalloc builds its im2col matrix
 * in: 64 MiB, held by every GPU the library runs on until the process ends. */
#define GEMM_CONV2D_SCRATCH_BYTES (64LL << 20)

/* For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): gemm_conv2d_nhwc with
 * the im2col matrix built in a library-owned device array of
 * GEMM_CONV2D_SCRATCH_BYTES instead of a caller workspace.  Same operation,
 * arguments (less the workspace), layouts, checks, errors and kernels as
 * gemm_conv2d_nhwc; the call allocates and frees nothing.
 *   - A call whose im2col matrix (n*ho*wo * kh*kw*c_in elements, see
 *     gemm_conv2d_workspace_bytes) exceeds GEMM_CONV2D_SCRATCH_BYTES returns
 *     GEMM_ERR_SCRATCH and launches nothing.  The direct 1 x 1 case uses no
 *     scratch.
 *   - There is one array per GPU, shared by every call on that GPU, and it
 *     keeps whatever the last call wrote (every call rewrites all of the matrix
 *     it reads).  Calls that overlap in time on one GPU (two host threads, or
 *     two streams whose work runs concurrently) race on it and must not be
 *     issued; calls on one stream are ordered and safe.
 *   - The array's device address is looked up on the first call on each device
 *     (GEMM_ERR_DEVICE if that fails). */
int gemm_conv2d_nhwc_noalloc(int dtype, const void *X, const void *Wt, void *Y,
                             const gemm_conv2d_shape *shape, const float *bias, int activation,
                             hipStream_t stream);

/* Bytes of workspace gemm_conv2d_nhwc needs for this dtype and geometry (the
 * im2col matrix, n*ho*wo * kh*kw*c_in elements; 0 for the direct 1 x 1 case),
 * or a negative gemm_status for a bad dtype or geometry.  Host only. */
int64_t gemm_conv2d_workspace_bytes(int dtype, const gemm_conv2d_shape *shape);

/* The im2col matrix alone: with KW = shape->kw,
 *   col[((n*ho + oh)*wo + ow) * ldcol + (kh*KW + kw)*c_in + ci] = X[n][ih][iw][ci]
 * (ih, iw as above), or 0 where the tap falls outside the image.
 * Pure data movement, bit for bit.  ldcol >= kh*kw*c_in (else GEMM_ERR_LD);
 * col must not overlap X; bytes of col past each row's kh*kw*c_in elements are
 * not written.  Errors otherwise as gemm_conv2d_nhwc. */
int gemm_im2col_nhwc(int dtype, const void *X, void *col, int64_t ldcol,
                     const gemm_conv2d_shape *shape, hipStream_t stream);

/* Static, NUL-terminated description of a gemm_status value. */
const char *gemm_status_string(int status);

/* Library version as major*10000 + minor*100 + patch. */
int gemm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBGEMM_H */
