// FP8 (OCP E4M3) block-scaled GEMM on gfx950 matrix cores, bf16 output.
//
//   C[i][j] = bf16( sum_kb  sa(i/64, kb) * sb(kb, j/64) * sum_{k in block kb} qa(i,k) qb(k,j) )
//
// "深度学习加速核心：GEMM优化从分块到TensorCore的实战解析", section 4.3: E4M3
// operands, one scale per 64 x 64 sub-block; section 5.2 (third pitfall): fp32
// scales.  The K step equals the scale block (64), so one
// v_mfma_scale_f32_32x32x64_f8f6f4 (hardware block scales left at 2^0) gives the
// exact-integer-grid partial product of one 32x32 output tile over one scale
// block; the partial is then promoted into the fp32 accumulator with one FMA per
// element by the product of the two fp32 block scales.  Wave tiles are 32-row /
// 32-column aligned, so a 32x32 output tile never straddles two scale blocks.
//
// LDS: A as rows of k (64 bytes per row, 16-byte chunks XOR-swizzled); B is
// transposed on the way in (8 k-rows x 4 columns per thread, bytes shuffled in
// registers) so every lane can read 32 consecutive k of one column.
#include <cstdlib>

#include "gemm_device.hpp"
#include "gemm_launch.hpp"

namespace gemm {

namespace {

constexpr int FP8_BK = 64;

__device__ __forceinline__ u32x4 load16b_guarded(const uint8_t *p, bool row_ok, int cols_left)
{
    uint32_t w[4] = {0, 0, 0, 0};
    if (row_ok) {
#pragma unroll
        for (int e = 0; e < 16; ++e)
            if (e < cols_left) w[e >> 2] |= (uint32_t)p[e] << ((e & 3) * 8);
    }
    return u32x4{w[0], w[1], w[2], w[3]};
}

__device__ __forceinline__ uint32_t load4b_guarded(const uint8_t *p, bool row_ok, int cols_left)
{
    uint32_t w = 0;
    if (row_ok) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (e < cols_left) w |= (uint32_t)p[e] << (e * 8);
    }
    return w;
}

// EPI: the fused epilogue is applied to the fp32 results before rounding, by
// the lane that stores them.
template <int BM, int BN, int WM, int WN, bool ALIGNED, bool EPI>
__global__ void __launch_bounds__(WM * WN * 64)
fp8_gemm_kernel(const uint8_t *__restrict__ A, const uint8_t *__restrict__ B,
                uint16_t *__restrict__ C, int M, int N, int K, int64_t lda, int64_t ldb,
                int64_t ldc, const float *__restrict__ scale_a, const float *__restrict__ scale_b,
                int tiles_m, int tiles_n, int group_m, Epilogue epi)
{
    constexpr int BK = FP8_BK;
    constexpr int NT = WM * WN * 64;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    constexpr int A_ITERS = BM * (BK / 16) / NT;       // 16-byte chunks, 4 per row
    constexpr int B_ITERS = (BK / 8) * (BN / 4) / NT;  // units of 8 k-rows x 4 columns
    static_assert(FM >= 1 && FN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "wave tile");
    static_assert(A_ITERS >= 1 && A_ITERS * NT == BM * (BK / 16), "A loader");
    static_assert(B_ITERS >= 1 && B_ITERS * NT == (BK / 8) * (BN / 4), "B loader");

    __shared__ __attribute__((aligned(16))) uint8_t As[2][BM * BK];
    __shared__ __attribute__((aligned(16))) uint8_t Bs[2][BN * BK];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm0 = (wave / WN) * WTM;
    const int wn0 = (wave % WN) * WTN;
    const int l32 = lane & 31, half = lane >> 5;

    int tm, tn;
    tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    const int kblocks = (K + 63) / 64;                 // columns of the scale_a grid
    const int mblocks = (M + 63) / 64, nblocks = (N + 63) / 64;
    // Scale-grid row (A) / column (B) of every 32-row / 32-column MFMA tile,
    // clamped so tiles hanging past M or N (all-zero operands) still index the grid.
    int64_t sa_row[FM];
    int sb_col[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int mb = (m0 + wm0 + i * 32) / 64;
        sa_row[i] = (int64_t)(mb < mblocks ? mb : mblocks - 1) * kblocks;
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int nb = (n0 + wn0 + j * 32) / 64;
        sb_col[j] = nb < nblocks ? nb : nblocks - 1;
    }

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

    u32x4 areg[A_ITERS];
    uint32_t breg[B_ITERS][8];

    auto load_tile = [&](int k0) {
#pragma unroll
        for (int it = 0; it < A_ITERS; ++it) {
            const int q = tid + it * NT;
            const int row = q >> 2, c = q & 3;
            const int gm = m0 + row, gk = k0 + 16 * c;
            const uint8_t *src = A + (int64_t)gm * lda + gk;
            if (ALIGNED && gm < M && gk + 16 <= K)
                areg[it] = *reinterpret_cast<const u32x4 *>(src);
            else
                areg[it] = load16b_guarded(src, gm < M, K - gk);
        }
#pragma unroll
        for (int it = 0; it < B_ITERS; ++it) {
            const int p = tid + it * NT;
            const int nq = p % (BN / 4), kr = p / (BN / 4);
            const int gn = n0 + 4 * nq;
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const int gk = k0 + 8 * kr + r;
                const uint8_t *src = B + (int64_t)gk * ldb + gn;
                if (ALIGNED && gk < K && gn + 4 <= N)
                    breg[it][r] = *reinterpret_cast<const uint32_t *>(src);
                else
                    breg[it][r] = load4b_guarded(src, gk < K, N - gn);
            }
        }
    };

    auto store_tile = [&](int buf) {
#pragma unroll
        for (int it = 0; it < A_ITERS; ++it) {
            const int q = tid + it * NT;
            const int row = q >> 2, c = q & 3;
            *reinterpret_cast<u32x4 *>(&As[buf][row * BK + ((c ^ swz4(row)) << 4)]) = areg[it];
        }
#pragma unroll
        for (int it = 0; it < B_ITERS; ++it) {
            const int p = tid + it * NT;
            const int nq = p % (BN / 4), kr = p / (BN / 4);
            const int kofs = 8 * kr;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                uint32_t lo = 0, hi = 0;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    lo |= ((breg[it][r] >> (8 * t)) & 0xffu) << (8 * r);
                    hi |= ((breg[it][r + 4] >> (8 * t)) & 0xffu) << (8 * r);
                }
                const int nrow = 4 * nq + t;
                *reinterpret_cast<u32x2 *>(
                    &Bs[buf][nrow * BK + (((kofs >> 4) ^ swz4(nrow)) << 4) + (kofs & 15)]) =
                    u32x2{lo, hi};
            }
        }
    };

    auto compute = [&](int buf, int kb) {
        i32x8 af[FM], bfr[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int row = wm0 + i * 32 + l32;
            const u32x4 x0 = *reinterpret_cast<const u32x4 *>(
                &As[buf][row * BK + (((2 * half) ^ swz4(row)) << 4)]);
            const u32x4 x1 = *reinterpret_cast<const u32x4 *>(
                &As[buf][row * BK + (((2 * half + 1) ^ swz4(row)) << 4)]);
            af[i] = i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                          (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int nrow = wn0 + j * 32 + l32;
            const u32x4 y0 = *reinterpret_cast<const u32x4 *>(
                &Bs[buf][nrow * BK + (((2 * half) ^ swz4(nrow)) << 4)]);
            const u32x4 y1 = *reinterpret_cast<const u32x4 *>(
                &Bs[buf][nrow * BK + (((2 * half + 1) ^ swz4(nrow)) << 4)]);
            bfr[j] = i32x8{(int)y0[0], (int)y0[1], (int)y0[2], (int)y0[3],
                           (int)y1[0], (int)y1[1], (int)y1[2], (int)y1[3]};
        }
        float sa[FM], sb[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) sa[i] = scale_a[sa_row[i] + kb];
#pragma unroll
        for (int j = 0; j < FN; ++j) sb[j] = scale_b[(int64_t)kb * nblocks + sb_col[j]];
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                // format 0 = E4M3 for both operands; block scales 127 = 2^0
                const f32x16 part = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    bfr[j], af[i], f32x16{}, 0, 0, 0, 127, 0, 127);
                const float s = sa[i] * sb[j];
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[i][j][e] = __builtin_fmaf(part[e], s, acc[i][j][e]);
            }
    };

    const int ktiles = kblocks;
    load_tile(0);
    store_tile(0);
    __syncthreads();
    for (int t = 0; t < ktiles; ++t) {
        const int cur = t & 1;
        if (t + 1 < ktiles) load_tile((t + 1) * BK);
        compute(cur, t);
        if (t + 1 < ktiles) store_tile(cur ^ 1);
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int m = m0 + wm0 + i * 32 + l32;
        if (m >= M) continue;
        uint16_t *crow = C + (int64_t)m * ldc;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = n0 + wn0 + j * 32 + 8 * g + 4 * half;
                float ev[4] = {acc[i][j][4 * g + 0], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                               acc[i][j][4 * g + 3]};
                if constexpr (EPI) epilogue_row<OUT_BF16, 4>(epi, ev, crow, n, N - n);
                const float v0 = ev[0], v1 = ev[1], v2 = ev[2], v3 = ev[3];
                if (ALIGNED && n + 4 <= N) {
                    *reinterpret_cast<u32x2 *>(crow + n) =
                        u32x2{pack2<true>(v0, v1), pack2<true>(v2, v3)};
                } else {
                    const float v[4] = {v0, v1, v2, v3};
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        if (n + t < N) crow[n + t] = to_bf16_bits(v[t]);
                }
            }
        }
    }
}

template <int BM, int BN, int WM, int WN, bool EPI>
hipError_t launch_cfg_epi(const Problem &p, const float *sa, const float *sb)
{
    const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
    const int64_t nwg = (int64_t)tiles_m * tiles_n;
    if (nwg > 0x7fffffff) return hipErrorInvalidValue;
    const int group_m = tiles_m < 4 ? tiles_m : 4;
    const dim3 grid((unsigned)nwg), block(WM * WN * 64);
    const uint8_t *A = static_cast<const uint8_t *>(p.A);
    const uint8_t *B = static_cast<const uint8_t *>(p.B);
    uint16_t *C = static_cast<uint16_t *>(p.C);
    const Epilogue epi = p.epi ? *p.epi : Epilogue{1.f, 0.f, nullptr, 0};
    if (p.aligned)
        hipLaunchKernelGGL((fp8_gemm_kernel<BM, BN, WM, WN, true, EPI>), grid, block, 0, p.stream,
                           A, B, C, p.M, p.N, p.K, p.lda, p.ldb, p.ldc, sa, sb, tiles_m, tiles_n,
                           group_m, epi);
    else
        hipLaunchKernelGGL((fp8_gemm_kernel<BM, BN, WM, WN, false, EPI>), grid, block, 0, p.stream,
                           A, B, C, p.M, p.N, p.K, p.lda, p.ldb, p.ldc, sa, sb, tiles_m, tiles_n,
                           group_m, epi);
    return hipGetLastError();
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_cfg(const Problem &p, const float *sa, const float *sb)
{
    return p.epi ? launch_cfg_epi<BM, BN, WM, WN, true>(p, sa, sb)
                 : launch_cfg_epi<BM, BN, WM, WN, false>(p, sa, sb);
}

}  // namespace

hipError_t fp8_launch(const Problem &p, const float *scale_a, const float *scale_b, int cus)
{
    // Testing override LIBGEMM_FP8_SMALL: '1' forces the register-staged kernels
    // below, '2' the guarded large-tile kernel, '3' / '4' the K-split kernel with
    // 32-row tiles (whole-tile where eligible / guarded), '5' / '6' the same with
    // 64-row tiles, '7' the whole-tile large-tile kernel and '8' / '9' its 128 x
    // 128 tiles (whole-tile where eligible / guarded), each where it is eligible.
    const char *e = std::getenv("LIBGEMM_FP8_SMALL");
    const int force = e && e[0] >= '1' && e[0] <= '9' ? e[0] - '0' : 0;
    if (force == 7 && fp8_fast_eligible(p)) return fp8_fast_launch(p, scale_a, scale_b);
    if (force >= 8 && fp8_general_eligible(p))
        return fp8_tiles128_launch(p, scale_a, scale_b, force == 9);
    if (force >= 3 && force <= 6 && fp8_narrow_general_eligible(p))
        return fp8_narrow_launch(p, scale_a, scale_b, force >= 5 ? 64 : 32, force == 4 || force == 6);
    // Narrow products (M < 128 or N <= 128) and small grids with a long K (at most
    // one round of 64 x 64 tiles, K >= 2048): the K-split kernel, with 64-row
    // tiles when that costs no more rounds of one workgroup per CU than 32-row
    // tiles.  Measured (us; K-split / 128 x 128 tiles / 256 x 256 tiles):
    // 8192 x 64 x 4096 11.5 / 25.6 / 62.0, 1 x 4096 x 4096 12.8 / 23.4 / 56.8,
    // 512 x 2048 x 2048 11.4 / 14.6 / 31.9; but 1000^3 15.7 / 11.9 / 26.3.
    const int64_t cu = cus > 0 ? cus : 256;
    const int64_t t32 = (int64_t)((p.M + 31) / 32) * ((p.N + 63) / 64);
    const int64_t t64 = (int64_t)((p.M + 63) / 64) * ((p.N + 63) / 64);
    if (force == 0 && (p.M < 128 || p.N <= 128 || (t64 <= cu && p.K >= 2048)) &&
        fp8_narrow_general_eligible(p)) {
        const bool rows64 = p.M >= 64 && 2 * ((t64 + cu - 1) / cu) <= (t32 + cu - 1) / cu;
        return fp8_narrow_launch(p, scale_a, scale_b, rows64 ? 64 : 32, false);
    }
    // Medium grids, which fill at most half the chip in 256 x 256 tiles: 128 x
    // 128 tiles of the same kernel, two workgroups per CU (2048^3 17.0 us against
    // 33.9, 1500^3 15.4 against 32.7, 2048 x 4096 x 4096 48.7 against 67.1).
    const int64_t big = (int64_t)((p.M + 255) / 256) * ((p.N + 255) / 256);
    if (force == 0 && 2 * big <= cu && p.M >= 128 && p.N >= 128 && fp8_general_eligible(p))
        return fp8_tiles128_launch(p, scale_a, scale_b, false);
    if (force == 0 && fp8_fast_eligible(p)) return fp8_fast_launch(p, scale_a, scale_b);
    // Any other shape with N >= 16 and K > 64: the guarded large-tile kernel
    // (measured: 4097 x 4095 x 4100 145 us against 1772 on the register-staged
    // kernels, 8200^2 x 8192 647 against 1886, 1000^3 26 against 89).
    if (force != 1 && fp8_general_eligible(p)) return fp8_general_launch(p, scale_a, scale_b);
    const int64_t big128 = (int64_t)((p.M + 127) / 128) * ((p.N + 127) / 128);
    if (big128 >= 128) return launch_cfg<128, 128, 2, 2>(p, scale_a, scale_b);
    return launch_cfg<64, 64, 2, 1>(p, scale_a, scale_b);
}

}  // namespace gemm
