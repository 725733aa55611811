// libgemm C ABI: argument checks, device check, dispatch to the kernel launchers.
//
// Every entry point checks its arguments synchronously and launches nothing on
// an error; the work itself is enqueued on the caller's stream.  The library
// allocates nothing and keeps no per-call state (it caches, per device, whether
// the device is a gfx950).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdlib>
#include <cstring>

#include <cmath>

#include "gemm_device.hpp"
#include "gemm_launch.hpp"
#include "libgemm.h"

namespace gemm {

namespace {

// The K == 0 case, every sum empty: the M x N window of C becomes zero, or with
// an epilogue act(beta * c_prior + bias[column]).
template <int OUT, bool EPI>
__global__ void empty_sum_kernel(void *C, int M, int N, int64_t ldc, Epilogue epi)
{
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)M * N) return;
    const int64_t m = idx / N;
    const int n = (int)(idx % N);
    float v = 0.f;
    if constexpr (EPI) {
        const size_t row_bytes = (size_t)m * ldc * (OUT == OUT_F32 ? 4 : 2);
        const void *row = static_cast<const char *>(C) + row_bytes;
        float x = v;
        if (epi.beta != 0.f) x = epi.beta * load_out<OUT>(row, n);
        if (epi.bias) x += epi.bias[n];
        if (epi.relu) x = x > 0.f ? x : 0.f;
        v = x;
    }
    if constexpr (OUT == OUT_F32)
        static_cast<float *>(C)[m * ldc + n] = v;
    else if constexpr (OUT == OUT_BF16)
        static_cast<uint16_t *>(C)[m * ldc + n] = to_bf16_bits(v);
    else
        static_cast<uint16_t *>(C)[m * ldc + n] = to_f16_bits(v);
}

constexpr int MAX_DEVICES = 64;
// Per device: 0 = not looked at yet, -1 = not a gfx950, else its compute-unit
// count (the number of workgroups of the large-tile kernels one round runs).
std::atomic<int> g_device_cus[MAX_DEVICES];

int check_device(int *cus = nullptr)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return GEMM_ERR_DEVICE;
    if (dev >= MAX_DEVICES) return GEMM_ERR_DEVICE;
    int state = g_device_cus[dev].load(std::memory_order_relaxed);
    if (state == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return GEMM_ERR_DEVICE;
        state = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 && prop.multiProcessorCount > 0
                    ? prop.multiProcessorCount
                    : -1;
        g_device_cus[dev].store(state, std::memory_order_relaxed);
    }
    if (cus) *cus = state;
    return state > 0 ? GEMM_OK : GEMM_ERR_DEVICE;
}

bool overlaps(const void *a, int64_t a_bytes, const void *b, int64_t b_bytes)
{
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + (uintptr_t)b_bytes && b0 < a0 + (uintptr_t)a_bytes;
}

// Bytes spanned by a rows x cols row-major window with leading dimension ld.
int64_t span_bytes(int64_t rows, int64_t cols, int64_t ld, int64_t esize)
{
    if (rows == 0 || cols == 0) return 0;
    return ((rows - 1) * ld + cols) * esize;
}

// Largest M, N or K: 2^31 - 2^16.  Kernels round a dimension up to whole tiles
// or K blocks (at most 1024 past it) in 32-bit arithmetic; the headroom keeps
// every such index below 2^31.
constexpr int64_t DIM_LIMIT = 0x7fff0000;

// Checks shared by all dtypes.  On success returns GEMM_OK and, when there is
// work to do, leaves *work = true.
int check_args(const void *A, const void *B, const void *C, int64_t M, int64_t N, int64_t K,
               int64_t lda, int64_t ldb, int64_t ldc, int64_t esize_in, int64_t esize_out,
               bool *work)
{
    *work = false;
    if (M < 0 || N < 0 || K < 0) return GEMM_ERR_DIM;
    if (M > DIM_LIMIT || N > DIM_LIMIT || K > DIM_LIMIT) return GEMM_ERR_DIM;
    if (lda < K || ldb < N || ldc < N) return GEMM_ERR_LD;
    if (lda > (int64_t)1 << 40 || ldb > (int64_t)1 << 40 || ldc > (int64_t)1 << 40)
        return GEMM_ERR_LD;
    if (M == 0 || N == 0) return GEMM_OK;
    if (C == nullptr) return GEMM_ERR_NULL;
    if (K > 0 && (A == nullptr || B == nullptr)) return GEMM_ERR_NULL;
    if ((uintptr_t)C % esize_out) return GEMM_ERR_ALIGN;
    if (K > 0 && ((uintptr_t)A % esize_in || (uintptr_t)B % esize_in)) return GEMM_ERR_ALIGN;
    const int64_t cb = span_bytes(M, N, ldc, esize_out);
    if (K > 0 && (overlaps(C, cb, A, span_bytes(M, K, lda, esize_in)) ||
                  overlaps(C, cb, B, span_bytes(K, N, ldb, esize_in))))
        return GEMM_ERR_ALIAS;
    *work = true;
    return GEMM_OK;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15) == 0; }

int to_status(hipError_t e) { return e == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH; }

// Checks of the epilogue options (before any other check) and, once the call
// has work, of the bias vector against C.  *epi is filled from the options.
int check_epilogue_options(float alpha, float beta, int activation, Epilogue *epi)
{
    if (activation != GEMM_ACT_NONE && activation != GEMM_ACT_RELU) return GEMM_ERR_ARG;
    if (!std::isfinite(alpha) || !std::isfinite(beta)) return GEMM_ERR_ARG;
    *epi = Epilogue{alpha, beta, nullptr, activation == GEMM_ACT_RELU ? 1 : 0};
    return GEMM_OK;
}

int check_bias(const float *bias, const void *C, int64_t M, int64_t N, int64_t ldc,
               int64_t esize_out)
{
    if (bias == nullptr) return GEMM_OK;
    if ((uintptr_t)bias & 3) return GEMM_ERR_ALIGN;
    if (overlaps(C, span_bytes(M, N, ldc, esize_out), bias, N * 4)) return GEMM_ERR_ALIAS;
    return GEMM_OK;
}

int h16_entry(bool is_bf16, const void *A, const void *B, void *C, int64_t M, int64_t N,
              int64_t K, int64_t lda, int64_t ldb, int64_t ldc, const Epilogue *epi,
              hipStream_t stream)
{
    bool work;
    int st = check_args(A, B, C, M, N, K, lda, ldb, ldc, 2, 2, &work);
    if (st != GEMM_OK || !work) return st;
    if (epi && (st = check_bias(epi->bias, C, M, N, ldc, 2)) != GEMM_OK) return st;
    int cus = 0;
    if ((st = check_device(&cus)) != GEMM_OK) return st;
    if (K == 0)
        return to_status(empty_sum_launch(C, (int)M, (int)N, ldc, is_bf16 ? OUT_BF16 : OUT_F16,
                                          epi, stream));
    Problem p{A, B, C, (int)M, (int)N, (int)K, lda, ldb, ldc, false, stream, epi};
    p.aligned = aligned16(A) && aligned16(B) && aligned16(C) && lda % 8 == 0 && ldb % 8 == 0 &&
                ldc % 8 == 0;
    // Tuning / testing override: LIBGEMM_H16_CONFIG=<H16Config id> (the large-tile
    // paths only where they are eligible).
    if (const char *e = std::getenv("LIBGEMM_H16_CONFIG")) {
        const int forced = std::atoi(e);
        if (forced >= 0 && forced < H16_NUM_CONFIGS &&
            (forced != H16_FAST_256x256 || h16_fast_eligible(p)) &&
            (forced != H16_GEN_256x256 || h16_general_eligible(p)) &&
            (forced != H16_NARROW_32x64 || h16_narrow_eligible(p)) &&
            (forced != H16_NARROW_GEN || h16_narrow_general_eligible(p)) &&
            (forced != H16_NARROW64 || h16_narrow64_eligible(p)) &&
            (forced != H16_NARROW64_GEN || h16_narrow_general_eligible(p)) &&
            (forced != H16_ROWS || rows_eligible(p)) &&
            (forced != H16_FAST_128 || h16_fast128_eligible(p)) &&
            (forced != H16_GEN_128 || h16_general_eligible(p)) &&
            (forced != H16_FAST_128x256 || h16_fast128x256_eligible(p)) &&
            (forced != H16_GEN_128x256 || h16_general_eligible(p)) &&
            (forced != H16_FEWROWS || h16_fewrows_eligible(p)))
            return to_status(h16_launch(is_bf16, forced, p));
    }
    // The large-tile kernel with 256 x 256 tiles, when their grid fills more than
    // half the chip (one workgroup per CU); at half or less its 128 x 128 tiles
    // (two workgroups per CU) are faster: 2048 x 4096 x 4096 (128 tiles) 72.2 us
    // against 81.2, but 3072^3 (144 tiles) 65.8 against 73.2.
    const int64_t tiles_n = (p.N + 255) / 256;
    const int64_t big_tiles = (int64_t)((p.M + 255) / 256) * tiles_n;
    const bool big = 2 * big_tiles > cus;
    if (big && h16_fast_eligible(p))
        return to_status(h16_launch(is_bf16, H16_FAST_256x256, p));
    // Tall, narrow products with a long K: 32 x 64 tiles, K split over the waves
    // (8192 x 64 x 4096: 21 us against 47 us on 64 x 64 tiles; with K = 576 the
    // split leaves each wave two blocks and 64 x 64 tiles are twice as fast).
    const int64_t narrow_tiles = (int64_t)((p.M + 31) / 32) * ((p.N + 63) / 64);
    // 64-row tiles when 32-row tiles would need a second round of workgroups
    // (one per CU; 1000^3: 512 tiles of 32 x 64, 256 of 64 x 64).
    const auto narrow = [&]() {
        const int64_t t32 = (int64_t)((p.M + 31) / 32) * ((p.N + 63) / 64);
        if (t32 > cus && p.M >= 64)
            return to_status(h16_launch(
                is_bf16, h16_narrow64_eligible(p) ? H16_NARROW64 : H16_NARROW64_GEN, p));
        return to_status(h16_launch(
            is_bf16, h16_narrow_eligible(p) ? H16_NARROW_32x64 : H16_NARROW_GEN, p));
    };
    if (p.N <= 128 && narrow_tiles >= 128 && p.K >= 2048 && h16_narrow_general_eligible(p))
        return narrow();
    // Large problems with ragged edges or unaligned rows: the guarded large-tile
    // kernel.  A few rows left below the whole 256-row tiles that would cost an
    // extra, mostly idle round of workgroups go to the narrow kernel instead.
    if (p.M >= 256 && p.N >= 256 && big && h16_general_eligible(p)) {
        const int tail = p.M % 256;
        const int64_t main_tiles = (int64_t)(p.M / 256) * tiles_n;
        if (tail > 0 && tail <= 64 && (main_tiles + cus - 1) / cus < (big_tiles + cus - 1) / cus) {
            Problem top = p, bottom = p;
            top.M = p.M - tail;
            bottom.M = tail;
            bottom.A = static_cast<const uint16_t *>(p.A) + (int64_t)top.M * p.lda;
            bottom.C = static_cast<uint16_t *>(p.C) + (int64_t)top.M * p.ldc;
            // Up to four rows: the few-row kernel where it was measured faster
            // (1 x 4095 x 4100: 12.0 us against 17.6 on the narrow kernel's 64
            // workgroups); otherwise the narrow kernel.
            const int tail_cfg = h16_fewrows_preferred(bottom)         ? H16_FEWROWS
                                 : h16_narrow_general_eligible(bottom) ? H16_NARROW_GEN
                                                                       : -1;
            if (tail_cfg >= 0) {
                st = to_status(h16_launch(
                    is_bf16, h16_fast_eligible(top) ? H16_FAST_256x256 : H16_GEN_256x256, top));
                if (st != GEMM_OK) return st;
                return to_status(h16_launch(is_bf16, tail_cfg, bottom));
            }
        }
        return to_status(h16_launch(is_bf16, H16_GEN_256x256, p));
    }
    // At most 32 rows (one row strip of the narrow kernel) with a long K: the
    // narrow kernel, or for up to four rows the few-row kernel where it is faster; the
    // 64 x 64 tiles below would walk all of K in each workgroup
    // (1 x 8192 x 8192: 27.2 us against 80.1; 1 x 16384 x 12288: 79 against 169).
    if (p.M <= 32 && p.K >= 256) {
        if (h16_fewrows_preferred(p)) return to_status(h16_launch(is_bf16, H16_FEWROWS, p));
        if (h16_narrow_general_eligible(p)) return narrow();
    }
    // Small grids: with few tiles and a long K, splitting K over the narrow
    // kernel's waves beats walking all of K in one workgroup per tile.  Measured
    // on MI355X (bf16): 256^3 4.1 us narrow against 5.0 on 64 x 64 tiles;
    // 1 x 4096 x 1000 6.1 against 11.2.  Up to 256 tiles of 64 x 64 it also beats
    // 128 x 128 tiles where its whole-tile form applies (1024^3 6.2 against 8.4,
    // 512 x 2048 x 2048 9.1 against 13.3) or where 128 x 128 tiles would be fewer
    // than 64 (3000 x 200 x 3000: 22.9 against 34.4); its guarded form otherwise
    // ties or loses (2048 x 512 x 1000: 11.1 against 9.9).
    const int64_t small_tiles = (int64_t)((p.M + 63) / 64) * ((p.N + 63) / 64);
    const int64_t tiles128 = (int64_t)((p.M + 127) / 128) * ((p.N + 127) / 128);
    const bool narrow_whole = (int64_t)((p.M + 31) / 32) * ((p.N + 63) / 64) > cus && p.M >= 64
                                  ? h16_narrow64_eligible(p)
                                  : h16_narrow_eligible(p);
    if (p.K >= 256 && h16_narrow_general_eligible(p) &&
        (small_tiles < 64 ||
         (p.K >= 512 && small_tiles <= 256 && (narrow_whole || tiles128 < 64))))
        return narrow();
    // Medium grids: 128 x 128 tiles of the large-tile kernel (LDS-direct ring,
    // two workgroups per CU; whole tiles where they fit, else guarded), ahead of
    // the register-staged and narrow kernels there: 1500^3 22.4 us against 45.3
    // (unaligned rows), 2048^3 22.9 against 40.2, 1000 x 4096 x 4096 41.5
    // against 70.9, 2000 x 3000 x 1000 24.3 against 44.2.
    // When 128 x 256 tiles (one workgroup per CU, 64 x 128 wave tiles) fill more
    // than half the chip they are faster still: 2560^3 37.4 against 43.6,
    // 4096 x 2048 x 4096 63.6 against 74.3; at half or less 128 x 128 tiles keep
    // more CUs busy (2048^3: 22.6 against 27.6).
    if (p.M >= 128 && p.N >= 128 && h16_general_eligible(p)) {
        const int64_t tiles128x256 = (int64_t)((p.M + 127) / 128) * ((p.N + 255) / 256);
        if (p.N >= 256 && 2 * tiles128x256 > cus)
            return to_status(h16_launch(
                is_bf16, h16_fast128x256_eligible(p) ? H16_FAST_128x256 : H16_GEN_128x256, p));
        return to_status(
            h16_launch(is_bf16, h16_fast128_eligible(p) ? H16_FAST_128 : H16_GEN_128, p));
    }
    return to_status(h16_launch(is_bf16, h16_pick_config(p.M, p.N, p.K), p));
}

}  // namespace

template <int OUT>
static void empty_sum_typed(dim3 grid, dim3 block, void *C, int M, int N, int64_t ldc,
                            const Epilogue *epi, hipStream_t stream)
{
    if (epi)
        hipLaunchKernelGGL((empty_sum_kernel<OUT, true>), grid, block, 0, stream, C, M, N, ldc, *epi);
    else
        hipLaunchKernelGGL((empty_sum_kernel<OUT, false>), grid, block, 0, stream, C, M, N, ldc,
                           Epilogue{1.f, 0.f, nullptr, 0});
}

hipError_t empty_sum_launch(void *C, int M, int N, int64_t ldc, int out, const Epilogue *epi,
                            hipStream_t stream)
{
    const int64_t total = (int64_t)M * N;
    const int threads = 256;
    const int64_t blocks = (total + threads - 1) / threads;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid((unsigned)blocks), block(threads);
    if (out == OUT_F32) empty_sum_typed<OUT_F32>(grid, block, C, M, N, ldc, epi, stream);
    else if (out == OUT_BF16) empty_sum_typed<OUT_BF16>(grid, block, C, M, N, ldc, epi, stream);
    else empty_sum_typed<OUT_F16>(grid, block, C, M, N, ldc, epi, stream);
    return hipGetLastError();
}

namespace {

int f32_entry(const float *A, const float *B, float *C, int64_t M, int64_t N, int64_t K,
              int64_t lda, int64_t ldb, int64_t ldc, const Epilogue *epi, hipStream_t stream)
{
    bool work;
    int st = check_args(A, B, C, M, N, K, lda, ldb, ldc, 4, 4, &work);
    if (st != GEMM_OK || !work) return st;
    if (epi && (st = check_bias(epi->bias, C, M, N, ldc, 4)) != GEMM_OK) return st;
    int cus = 0;
    if ((st = check_device(&cus)) != GEMM_OK) return st;
    if (K == 0) return to_status(empty_sum_launch(C, (int)M, (int)N, ldc, OUT_F32, epi, stream));
    Problem p{A, B, C, (int)M, (int)N, (int)K, lda, ldb, ldc, false, stream, epi};
    p.aligned = aligned16(A) && aligned16(B) && aligned16(C) && lda % 4 == 0 && ldb % 4 == 0 &&
                ldc % 4 == 0;
    return to_status(f32_launch(p, cus));
}

int fp8_entry(const uint8_t *A, const uint8_t *B, void *C, int64_t M, int64_t N, int64_t K,
              int64_t lda, int64_t ldb, int64_t ldc, const float *scale_a, const float *scale_b,
              const Epilogue *epi, hipStream_t stream)
{
    bool work;
    int st = check_args(A, B, C, M, N, K, lda, ldb, ldc, 1, 2, &work);
    if (st != GEMM_OK || !work) return st;
    if (K > 0 && (scale_a == nullptr || scale_b == nullptr)) return GEMM_ERR_NULL;
    if (K > 0 && (((uintptr_t)scale_a & 3) || ((uintptr_t)scale_b & 3))) return GEMM_ERR_ALIGN;
    if (K > 0) {
        const int64_t cb = span_bytes(M, N, ldc, 2);
        const int64_t sab = ((M + 63) / 64) * ((K + 63) / 64) * 4;
        const int64_t sbb = ((K + 63) / 64) * ((N + 63) / 64) * 4;
        if (overlaps(C, cb, scale_a, sab) || overlaps(C, cb, scale_b, sbb)) return GEMM_ERR_ALIAS;
    }
    if (epi && (st = check_bias(epi->bias, C, M, N, ldc, 2)) != GEMM_OK) return st;
    int cus = 0;
    if ((st = check_device(&cus)) != GEMM_OK) return st;
    if (K == 0) return to_status(empty_sum_launch(C, (int)M, (int)N, ldc, OUT_BF16, epi, stream));
    Problem p{A, B, C, (int)M, (int)N, (int)K, lda, ldb, ldc, false, stream, epi};
    p.aligned = aligned16(A) && ((uintptr_t)B & 3) == 0 && aligned16(C) && lda % 16 == 0 &&
                ldb % 4 == 0 && ldc % 8 == 0;
    return to_status(fp8_launch(p, scale_a, scale_b, cus));
}

}  // namespace

}  // namespace gemm

using namespace gemm;

extern "C" int gemm_f16(const void *A, const void *B, void *C, int64_t M, int64_t N, int64_t K,
                        int64_t lda, int64_t ldb, int64_t ldc, hipStream_t stream)
{
    return h16_entry(false, A, B, C, M, N, K, lda, ldb, ldc, nullptr, stream);
}

extern "C" int gemm_bf16(const void *A, const void *B, void *C, int64_t M, int64_t N, int64_t K,
                         int64_t lda, int64_t ldb, int64_t ldc, hipStream_t stream)
{
    return h16_entry(true, A, B, C, M, N, K, lda, ldb, ldc, nullptr, stream);
}

extern "C" int gemm_f32(const float *A, const float *B, float *C, int64_t M, int64_t N, int64_t K,
                        int64_t lda, int64_t ldb, int64_t ldc, hipStream_t stream)
{
    return f32_entry(A, B, C, M, N, K, lda, ldb, ldc, nullptr, stream);
}

extern "C" int gemm_fp8_blockscaled(const uint8_t *A, const uint8_t *B, void *C, int64_t M,
                                    int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
                                    const float *scale_a, const float *scale_b, hipStream_t stream)
{
    return fp8_entry(A, B, C, M, N, K, lda, ldb, ldc, scale_a, scale_b, nullptr, stream);
}

extern "C" int gemm_f16_epilogue(const void *A, const void *B, void *C, int64_t M, int64_t N,
                                 int64_t K, int64_t lda, int64_t ldb, int64_t ldc, float alpha,
                                 float beta, const float *bias, int activation, hipStream_t stream)
{
    Epilogue epi;
    const int st = check_epilogue_options(alpha, beta, activation, &epi);
    if (st != GEMM_OK) return st;
    epi.bias = bias;
    return h16_entry(false, A, B, C, M, N, K, lda, ldb, ldc, &epi, stream);
}

extern "C" int gemm_bf16_epilogue(const void *A, const void *B, void *C, int64_t M, int64_t N,
                                  int64_t K, int64_t lda, int64_t ldb, int64_t ldc, float alpha,
                                  float beta, const float *bias, int activation, hipStream_t stream)
{
    Epilogue epi;
    const int st = check_epilogue_options(alpha, beta, activation, &epi);
    if (st != GEMM_OK) return st;
    epi.bias = bias;
    return h16_entry(true, A, B, C, M, N, K, lda, ldb, ldc, &epi, stream);
}

extern "C" int gemm_f32_epilogue(const float *A, const float *B, float *C, int64_t M, int64_t N,
                                 int64_t K, int64_t lda, int64_t ldb, int64_t ldc, float alpha,
                                 float beta, const float *bias, int activation, hipStream_t stream)
{
    Epilogue epi;
    const int st = check_epilogue_options(alpha, beta, activation, &epi);
    if (st != GEMM_OK) return st;
    epi.bias = bias;
    return f32_entry(A, B, C, M, N, K, lda, ldb, ldc, &epi, stream);
}

extern "C" int gemm_fp8_blockscaled_epilogue(const uint8_t *A, const uint8_t *B, void *C,
                                             int64_t M, int64_t N, int64_t K, int64_t lda,
                                             int64_t ldb, int64_t ldc, const float *scale_a,
                                             const float *scale_b, float alpha, float beta,
                                             const float *bias, int activation, hipStream_t stream)
{
    Epilogue epi;
    const int st = check_epilogue_options(alpha, beta, activation, &epi);
    if (st != GEMM_OK) return st;
    epi.bias = bias;
    return fp8_entry(A, B, C, M, N, K, lda, ldb, ldc, scale_a, scale_b, &epi, stream);
}

extern "C" int gemm_h16_ladder(int rung, int is_bf16, const void *A, const void *B, void *C,
                               int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                               int64_t ldc, hipStream_t stream)
{
    if (rung < GEMM_LADDER_NAIVE || rung > GEMM_LADDER_MFMA_DOUBLE_BUFFER_ONE_WG)
        return GEMM_ERR_ARG;
    if (is_bf16 != 0 && is_bf16 != 1) return GEMM_ERR_ARG;
    if (rung == GEMM_LADDER_LIBRARY)
        return h16_entry(is_bf16 == 1, A, B, C, M, N, K, lda, ldb, ldc, nullptr, stream);
    bool work;
    int st = check_args(A, B, C, M, N, K, lda, ldb, ldc, 2, 2, &work);
    if (st != GEMM_OK || !work) return st;
    // one grid row per 16 (naive) or 64 (tiled) rows of C, at most 65535 of them
    if (rung <= GEMM_LADDER_REGISTER_TILED && M > 65535LL * (rung == GEMM_LADDER_NAIVE ? 16 : 64))
        return GEMM_ERR_DIM;
    if ((st = check_device()) != GEMM_OK) return st;
    if (K == 0)
        return to_status(empty_sum_launch(C, (int)M, (int)N, ldc, is_bf16 ? OUT_BF16 : OUT_F16,
                                          nullptr, stream));
    Problem p{A, B, C, (int)M, (int)N, (int)K, lda, ldb, ldc, false, stream, nullptr};
    p.aligned = aligned16(A) && aligned16(B) && aligned16(C) && lda % 8 == 0 && ldb % 8 == 0 &&
                ldc % 8 == 0;
    if (rung <= GEMM_LADDER_REGISTER_TILED) return to_status(ladder_valu_launch(rung, is_bf16, p));
    return to_status(h16_ladder_launch(rung, is_bf16, p));
}

extern "C" int gemm_h16_mfma_ceiling(int is_bf16, const void *A, const void *B, void *C,
                                     int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                                     int64_t ldc, hipStream_t stream)
{
    if (is_bf16 != 0 && is_bf16 != 1) return GEMM_ERR_ARG;
    bool work;
    int st = check_args(A, B, C, M, N, K, lda, ldb, ldc, 2, 2, &work);
    if (st != GEMM_OK || !work) return st;
    if (M % 256 || N % 256 || K % 32) return GEMM_ERR_DIM;
    Problem p{A, B, C, (int)M, (int)N, (int)K, lda, ldb, ldc, false, stream, nullptr};
    p.aligned = aligned16(A) && aligned16(B) && aligned16(C) && lda % 8 == 0 && ldb % 8 == 0 &&
                ldc % 8 == 0;
    if (!p.aligned) return GEMM_ERR_ALIGN;
    if ((st = check_device()) != GEMM_OK) return st;
    if (K == 0)
        return to_status(empty_sum_launch(C, (int)M, (int)N, ldc, is_bf16 ? OUT_BF16 : OUT_F16,
                                          nullptr, stream));
    return to_status(mfma_ceiling_launch(is_bf16, p));
}

namespace {

// Checks of a convolution call's type and geometry; fills the kernel-side shape,
// the output size and the element size.
int conv_check(int dtype, const gemm_conv2d_shape *sp, ConvShape *cs, int64_t *ho, int64_t *wo,
               int64_t *esize)
{
    if (dtype != GEMM_DTYPE_F16 && dtype != GEMM_DTYPE_BF16 && dtype != GEMM_DTYPE_F32)
        return GEMM_ERR_ARG;
    if (sp == nullptr) return GEMM_ERR_NULL;
    const gemm_conv2d_shape &s = *sp;
    const int64_t f[13] = {s.n, s.h, s.w, s.c_in, s.c_out, s.kh, s.kw, s.stride_h, s.stride_w,
                           s.pad_h, s.pad_w, s.dil_h, s.dil_w};
    for (int64_t v : f)
        if (v < 0) return GEMM_ERR_DIM;
    if (s.kh < 1 || s.kw < 1 || s.stride_h < 1 || s.stride_w < 1 || s.dil_h < 1 || s.dil_w < 1)
        return GEMM_ERR_DIM;
    // spatial sizes small enough that every input coordinate fits in int
    constexpr int64_t SPATIAL = 1 << 15;
    for (int i = 1; i < 13; ++i)
        if (i != 3 && i != 4 && f[i] > SPATIAL) return GEMM_ERR_DIM;
    if (s.n > DIM_LIMIT || s.c_in > DIM_LIMIT || s.c_out > DIM_LIMIT) return GEMM_ERR_DIM;
    const int64_t eh = s.h + 2 * s.pad_h - s.dil_h * (s.kh - 1) - 1;
    const int64_t ew = s.w + 2 * s.pad_w - s.dil_w * (s.kw - 1) - 1;
    *ho = eh < 0 ? 0 : eh / s.stride_h + 1;
    *wo = ew < 0 ? 0 : ew / s.stride_w + 1;
    if (s.n * *ho * *wo > DIM_LIMIT || s.kh * s.kw * s.c_in > DIM_LIMIT ||
        s.n * s.h * s.w > ((int64_t)1 << 40) / (s.c_in > 0 ? s.c_in : 1))
        return GEMM_ERR_DIM;
    *cs = ConvShape{(int)s.n, (int)s.h, (int)s.w, (int)s.c_in, (int)s.c_out, (int)s.kh, (int)s.kw,
                    (int)s.stride_h, (int)s.stride_w, (int)s.pad_h, (int)s.pad_w, (int)s.dil_h,
                    (int)s.dil_w};
    *esize = dtype == GEMM_DTYPE_F32 ? 4 : 2;
    return GEMM_OK;
}

// A 1 x 1 convolution with unit stride and no padding needs no im2col matrix:
// the NHWC input already is it.
bool conv_direct(const ConvShape &s)
{
    return s.kh == 1 && s.kw == 1 && s.stride_h == 1 && s.stride_w == 1 && s.pad_h == 0 &&
           s.pad_w == 0;
}

}  // namespace

extern "C" int64_t gemm_conv2d_workspace_bytes(int dtype, const gemm_conv2d_shape *shape)
{
    ConvShape s;
    int64_t ho, wo, esize;
    const int st = conv_check(dtype, shape, &s, &ho, &wo, &esize);
    if (st != GEMM_OK) return st;
    if (conv_direct(s)) return 0;
    return (int64_t)s.n * ho * wo * s.kh * s.kw * s.c_in * esize;
}

extern "C" int gemm_im2col_nhwc(int dtype, const void *X, void *col, int64_t ldcol,
                                const gemm_conv2d_shape *shape, hipStream_t stream)
{
    ConvShape s;
    int64_t ho, wo, esize;
    int st = conv_check(dtype, shape, &s, &ho, &wo, &esize);
    if (st != GEMM_OK) return st;
    const int64_t M = (int64_t)s.n * ho * wo, K = (int64_t)s.kh * s.kw * s.c_in;
    if (ldcol < K || ldcol > (int64_t)1 << 40) return GEMM_ERR_LD;
    if (M == 0 || K == 0) return GEMM_OK;
    if (X == nullptr || col == nullptr) return GEMM_ERR_NULL;
    if ((uintptr_t)X % esize || (uintptr_t)col % esize) return GEMM_ERR_ALIGN;
    if (overlaps(col, span_bytes(M, K, ldcol, esize), X,
                 (int64_t)s.n * s.h * s.w * s.c_in * esize))
        return GEMM_ERR_ALIAS;
    if ((st = check_device()) != GEMM_OK) return st;
    return to_status(im2col_launch((int)esize, X, col, ldcol, s, (int)ho, (int)wo, stream));
}

namespace {

// Scratch for the convolution entry point that allocates nothing: the im2col
// matrix of a call lives here instead of in a caller workspace.  Each GPU the
// library runs on holds its own copy from the moment the code object is loaded
// until the process ends.  In host code `scratch` names a host-side stand-in,
// not device memory: only the address hipGetSymbolAddress returns for the
// current device may be handed to kernels.
constexpr int64_t SCRATCH_BYTES = GEMM_CONV2D_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[SCRATCH_BYTES];

// Per device: the device address of `scratch`, looked up on the first call that
// needs it with that device current (0: not looked up yet).
std::atomic<uintptr_t> g_scratch[MAX_DEVICES];

// The current device's scratch address, or nullptr when it cannot be had.
void *scratch_ptr()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
    uintptr_t p = g_scratch[dev].load(std::memory_order_acquire);
    if (p == 0) {
        void *addr = nullptr;
        if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || addr == nullptr)
            return nullptr;
        p = (uintptr_t)addr;
        g_scratch[dev].store(p, std::memory_order_release);
    }
    return (void *)p;
}

// Both convolution entry points.  use_scratch: the im2col matrix goes to the
// current device's scratch array (workspace and workspace_bytes are ignored)
// and calls that need more than it holds are refused with GEMM_ERR_SCRATCH.
int conv_entry(int dtype, const void *X, const void *Wt, void *Y, void *workspace,
               int64_t workspace_bytes, bool use_scratch, const gemm_conv2d_shape *shape,
               const float *bias, int activation, hipStream_t stream)
{
    if (activation != GEMM_ACT_NONE && activation != GEMM_ACT_RELU) return GEMM_ERR_ARG;
    ConvShape s;
    int64_t ho, wo, esize;
    int st = conv_check(dtype, shape, &s, &ho, &wo, &esize);
    if (st != GEMM_OK) return st;
    const int64_t M = (int64_t)s.n * ho * wo, K = (int64_t)s.kh * s.kw * s.c_in, N = s.c_out;
    if (M == 0 || N == 0) return GEMM_OK;
    const bool direct = conv_direct(s);
    const int64_t need = direct || K == 0 ? 0 : M * K * esize;
    if (Y == nullptr || (K > 0 && (X == nullptr || Wt == nullptr))) return GEMM_ERR_NULL;
    if ((uintptr_t)Y % esize || (K > 0 && ((uintptr_t)X % esize || (uintptr_t)Wt % esize)))
        return GEMM_ERR_ALIGN;
    if (use_scratch) {
        if (need > SCRATCH_BYTES) return GEMM_ERR_SCRATCH;
    } else {
        if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return GEMM_ERR_WORKSPACE;
        if (need > 0 && (uintptr_t)workspace % esize) return GEMM_ERR_ALIGN;
    }
    const int64_t yb = M * N * esize, xb = (int64_t)s.n * s.h * s.w * s.c_in * esize;
    const int64_t wb = K * N * esize;
    if (K > 0 && (overlaps(Y, yb, X, xb) || overlaps(Y, yb, Wt, wb))) return GEMM_ERR_ALIAS;
    if (!use_scratch && need > 0 &&
        (overlaps(workspace, need, X, xb) || overlaps(workspace, need, Wt, wb) ||
         overlaps(workspace, need, Y, yb)))
        return GEMM_ERR_ALIAS;
    if ((st = check_bias(bias, Y, M, N, N, esize)) != GEMM_OK) return st;
    if ((st = check_device()) != GEMM_OK) return st;
    if (use_scratch && need > 0 && (workspace = scratch_ptr()) == nullptr) return GEMM_ERR_DEVICE;
    Epilogue epi{1.f, 0.f, bias, activation == GEMM_ACT_RELU ? 1 : 0};
    const Epilogue *pe = bias || activation == GEMM_ACT_RELU ? &epi : nullptr;
    const int out = dtype == GEMM_DTYPE_F32 ? OUT_F32 : dtype == GEMM_DTYPE_BF16 ? OUT_BF16 : OUT_F16;
    if (K == 0) return to_status(empty_sum_launch(Y, (int)M, (int)N, N, out, pe, stream));
    const void *A = X;
    if (!direct) {
        st = to_status(im2col_launch((int)esize, X, workspace, K, s, (int)ho, (int)wo, stream));
        if (st != GEMM_OK) return st;
        A = workspace;
    }
    if (dtype == GEMM_DTYPE_F32)
        return f32_entry(static_cast<const float *>(A), static_cast<const float *>(Wt),
                         static_cast<float *>(Y), M, N, K, K, N, N, pe, stream);
    return h16_entry(dtype == GEMM_DTYPE_BF16, A, Wt, Y, M, N, K, K, N, N, pe, stream);
}

}  // namespace

extern "C" int gemm_conv2d_nhwc(int dtype, const void *X, const void *Wt, void *Y, void *workspace,
                                int64_t workspace_bytes, const gemm_conv2d_shape *shape,
                                const float *bias, int activation, hipStream_t stream)
{
    return conv_entry(dtype, X, Wt, Y, workspace, workspace_bytes, false, shape, bias, activation,
                      stream);
}

extern "C" int gemm_conv2d_nhwc_noalloc(int dtype, const void *X, const void *Wt, void *Y,
                                        const gemm_conv2d_shape *shape, const float *bias,
                                        int activation, hipStream_t stream)
{
    return conv_entry(dtype, X, Wt, Y, nullptr, 0, true, shape, bias, activation, stream);
}

extern "C" int gemm_quantize_fp8(const void *X, int in_type, int64_t rows, int64_t cols,
                                 int64_t ldx, int block, int fmt, uint8_t *Q, int64_t ldq,
                                 float *scales, hipStream_t stream)
{
    if (in_type != GEMM_QUANT_IN_F32 && in_type != GEMM_QUANT_IN_BF16) return GEMM_ERR_ARG;
    if (block != 32 && block != 64) return GEMM_ERR_ARG;
    if (fmt != GEMM_FP8_E4M3 && fmt != GEMM_FP8_E5M2) return GEMM_ERR_ARG;
    if (rows < 0 || cols < 0 || rows > DIM_LIMIT || cols > DIM_LIMIT) return GEMM_ERR_DIM;
    if (ldx < cols || ldq < cols || ldx > (int64_t)1 << 40 || ldq > (int64_t)1 << 40)
        return GEMM_ERR_LD;
    if (rows == 0 || cols == 0) return GEMM_OK;
    if (X == nullptr || Q == nullptr || scales == nullptr) return GEMM_ERR_NULL;
    const int64_t esize = in_type == GEMM_QUANT_IN_BF16 ? 2 : 4;
    if ((uintptr_t)X % esize || ((uintptr_t)scales & 3)) return GEMM_ERR_ALIGN;
    const int64_t xb = span_bytes(rows, cols, ldx, esize), qb = span_bytes(rows, cols, ldq, 1);
    const int64_t sb = ((rows + block - 1) / block) * ((cols + block - 1) / block) * 4;
    if (overlaps(Q, qb, X, xb) || overlaps(scales, sb, X, xb) || overlaps(scales, sb, Q, qb))
        return GEMM_ERR_ALIAS;
    int st;
    if ((st = check_device()) != GEMM_OK) return st;
    QuantProblem p{X, in_type == GEMM_QUANT_IN_BF16, (int)rows, (int)cols, ldx, block, fmt,
                   Q, ldq, scales, stream};
    return to_status(quant_fp8_launch(p));
}

extern "C" const char *gemm_status_string(int status)
{
    switch (status) {
    case GEMM_OK: return "success";
    case GEMM_ERR_NULL: return "a required pointer is NULL";
    case GEMM_ERR_DIM: return "M, N or K is negative or too large";
    case GEMM_ERR_LD: return "leading dimension smaller than the row (lda < K, ldb < N or ldc < N)";
    case GEMM_ERR_ALIGN: return "pointer not aligned to its element size";
    case GEMM_ERR_ALIAS: return "an output overlaps an input (or the two quantiser outputs overlap)";
    case GEMM_ERR_DEVICE: return "current device is not a gfx950 GPU";
    case GEMM_ERR_LAUNCH: return "kernel launch failed";
    case GEMM_ERR_WORKSPACE: return "workspace missing or smaller than the call needs";
    case GEMM_ERR_SCRATCH:
        return "the call needs more scratch than the library's fixed per-GPU array holds";
    case GEMM_ERR_ARG:
        return "unsupported option (input type, block size, FP8 format, activation, or a "
               "non-finite alpha or beta)";
    default: return "unknown status";
    }
}

extern "C" int gemm_version(void) { return 200; }
