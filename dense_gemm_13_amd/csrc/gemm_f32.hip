// fp32 SGEMM on gfx950 matrix cores: C = A * B, all row-major fp32.
//
// The register-tiled SGEMM of "CUDA GEMM 优化实践笔记" (block tile of C in shared
// memory, K walked in BK steps, out-of-range operand elements loaded as zero,
// a per-thread register tile of accumulators) with the per-thread FMA outer
// product replaced by v_mfma_f32_32x32x2_f32 on wave64 tiles.
//
// Accumulation is two-level: every K step of 32 is summed into a fresh fp32
// partial tile, which is then added to the running total.  A single running
// fp32 sum over K = 4096 drifts by ~1e-4 on N(0,1) data, past the 1e-5 relative
// + 1e-4 absolute acceptance bound; the short partial sums keep the error far
// below it.
//
// LDS: A as rows of k with 16-byte chunks XOR-swizzled (the MFMA fragment reads
// walk 32 consecutive rows), B as rows of n exactly as in memory (each lane
// reads single floats of one row, 32 lanes cover 128 contiguous bytes).  Two
// stages ping-pong so the next step's loads are in flight during the MFMAs.
#include <cstdlib>

#include "gemm_device.hpp"
#include "gemm_launch.hpp"

namespace gemm {

namespace {

constexpr int F32_BK = 32;

__device__ __forceinline__ f32x4 load4_guarded(const float *p, bool row_ok, int cols_left)
{
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    if (row_ok) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (e < cols_left) v[e] = p[e];
    }
    return f32x4{v[0], v[1], v[2], v[3]};
}

// EPI: the fused epilogue is applied to the results by the lane that stores them.
template <int BM, int BN, int WM, int WN, bool ALIGNED, bool EPI>
__global__ void __launch_bounds__(WM * WN * 64)
f32_gemm_kernel(const float *__restrict__ A, const float *__restrict__ B, float *__restrict__ C,
                int M, int N, int K, int64_t lda, int64_t ldb, int64_t ldc, int tiles_m,
                int tiles_n, int group_m, Epilogue epi)
{
    constexpr int BK = F32_BK;
    constexpr int NT = WM * WN * 64;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    constexpr int A_ITERS = BM * (BK / 4) / NT;
    constexpr int B_ITERS = BK * (BN / 4) / NT;
    static_assert(FM >= 1 && FN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "wave tile");
    static_assert(A_ITERS >= 1 && A_ITERS * NT == BM * (BK / 4), "A loader");
    static_assert(B_ITERS >= 1 && B_ITERS * NT == BK * (BN / 4), "B loader");

    __shared__ __attribute__((aligned(16))) float As[2][BM * BK];
    __shared__ __attribute__((aligned(16))) float Bs[2][BK * BN];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm0 = (wave / WN) * WTM;
    const int wn0 = (wave % WN) * WTN;
    const int l32 = lane & 31, half = lane >> 5;

    int tm, tn;
    tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    f32x16 total[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) total[i][j] = f32x16{};

    f32x4 areg[A_ITERS], breg[B_ITERS];
    // Chunks are 16-byte loads whatever the rows' alignment (the hardware runs in
    // unaligned-access mode).  !ALIGNED: a chunk at an edge is one 16-byte load
    // from inside the matrix (masked16_load) whose zeros past M, N and K are
    // applied when it is stored to LDS, after the step's MFMAs, so load_tile
    // waits for nothing.  (ALIGNED keeps element loads at the edges, which
    // measured faster there: fewer registers.)
    int loaded_k0 = 0;                                   // K step in the registers
    // Bytes a chunk's masked load shifts out (0 for a chunk wholly inside).
    const auto drop_of = [](int row, int rows, int k, int cols) {
        if (ALIGNED || cols < 4) return 0;               // (element loads instead)
        if (row >= rows || k >= cols) return 16;
        return k + 4 > cols ? 4 * (k + 4 - cols) : 0;
    };

    auto load_tile = [&](int k0) {
        loaded_k0 = k0;
#pragma unroll
        for (int it = 0; it < A_ITERS; ++it) {
            const int q = tid + it * NT;
            const int row = q >> 3, c = q & 7;
            const int gm = m0 + row, gk = k0 + 4 * c;
            const float *src = A + (int64_t)gm * lda + gk;
            if (gm < M && gk + 4 <= K)
                areg[it] = *reinterpret_cast<const f32x4 *>(src);
            else if (!ALIGNED && K >= 4)
                areg[it] = __builtin_bit_cast(f32x4, masked16_load<4>(A, lda, gm, M, gk, K).raw);
            else
                areg[it] = load4_guarded(src, gm < M, K - gk);
        }
#pragma unroll
        for (int it = 0; it < B_ITERS; ++it) {
            const int q = tid + it * NT;
            const int row = q / (BN / 4), c = q % (BN / 4);
            const int gk = k0 + row, gn = n0 + 4 * c;
            const float *src = B + (int64_t)gk * ldb + gn;
            if (gk < K && gn + 4 <= N)
                breg[it] = *reinterpret_cast<const f32x4 *>(src);
            else if (!ALIGNED && N >= 4)
                breg[it] = __builtin_bit_cast(f32x4, masked16_load<4>(B, ldb, gk, K, gn, N).raw);
            else
                breg[it] = load4_guarded(src, gk < K, N - gn);
        }
    };

    auto store_tile = [&](int buf) {
        const int k0 = loaded_k0;
        if (!ALIGNED && (m0 + BM > M || n0 + BN > N || k0 + BK > K)) {
#pragma unroll
            for (int it = 0; it < A_ITERS; ++it) {
                const int q = tid + it * NT;
                areg[it] = __builtin_bit_cast(
                    f32x4, shift_down_bytes(__builtin_bit_cast(u32x4, areg[it]),
                                            drop_of(m0 + (q >> 3), M, k0 + 4 * (q & 7), K)));
            }
#pragma unroll
            for (int it = 0; it < B_ITERS; ++it) {
                const int q = tid + it * NT;
                const int row = q / (BN / 4), c = q % (BN / 4);
                breg[it] = __builtin_bit_cast(
                    f32x4, shift_down_bytes(__builtin_bit_cast(u32x4, breg[it]),
                                            drop_of(k0 + row, K, n0 + 4 * c, N)));
            }
        }
#pragma unroll
        for (int it = 0; it < A_ITERS; ++it) {
            const int q = tid + it * NT;
            const int row = q >> 3, c = q & 7;
            *reinterpret_cast<f32x4 *>(&As[buf][row * BK + ((c ^ swz8(row)) << 2)]) = areg[it];
        }
#pragma unroll
        for (int it = 0; it < B_ITERS; ++it) {
            const int q = tid + it * NT;
            const int row = q / (BN / 4), c = q % (BN / 4);
            *reinterpret_cast<f32x4 *>(&Bs[buf][row * BN + 4 * c]) = breg[it];
        }
    };

    // One K step: lanes of half h supply k = 8s + 4h + e to the e-th MFMA of
    // sub-step s, for both operands, so every MFMA adds two matching k terms.
    auto compute = [&](int buf) {
        f32x16 part[FM][FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) part[i][j] = f32x16{};
#pragma unroll
        for (int s = 0; s < BK / 8; ++s) {
            const int c = 2 * s + half;
            f32x4 af[FM];
            float bv[FN][4];
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int row = wm0 + i * 32 + l32;
                af[i] = *reinterpret_cast<const f32x4 *>(&As[buf][row * BK + ((c ^ swz8(row)) << 2)]);
            }
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    bv[j][e] = Bs[buf][(8 * s + 4 * half + e) * BN + wn0 + j * 32 + l32];
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        part[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(bv[j][e], af[i][e],
                                                                         part[i][j], 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) total[i][j] += part[i][j];
    };

    const int ktiles = (K + BK - 1) / BK;
    load_tile(0);
    store_tile(0);
    __syncthreads();
    for (int t = 0; t < ktiles; ++t) {
        const int cur = t & 1;
        if (t + 1 < ktiles) load_tile((t + 1) * BK);
        compute(cur);
        if (t + 1 < ktiles) store_tile(cur ^ 1);
        __syncthreads();
    }

    // Lane holds C[m][n..n+3], n = 8g + 4*half (+ tile offsets).
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int m = m0 + wm0 + i * 32 + l32;
        if (m >= M) continue;
        float *crow = C + (int64_t)m * ldc;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = n0 + wn0 + j * 32 + 8 * g + 4 * half;
                float ev[4] = {total[i][j][4 * g], total[i][j][4 * g + 1], total[i][j][4 * g + 2],
                               total[i][j][4 * g + 3]};
                if constexpr (EPI) epilogue_row<OUT_F32, 4>(epi, ev, crow, n, N - n);
                const f32x4 v{ev[0], ev[1], ev[2], ev[3]};
                if (ALIGNED && n + 4 <= N) {
                    *reinterpret_cast<f32x4 *>(crow + n) = v;
                } else {
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        if (n + t < N) crow[n + t] = v[t];
                }
            }
        }
    }
}

template <int BM, int BN, int WM, int WN, bool EPI>
hipError_t launch_cfg_epi(const Problem &p)
{
    const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
    const int64_t nwg = (int64_t)tiles_m * tiles_n;
    if (nwg > 0x7fffffff) return hipErrorInvalidValue;
    const int group_m = tiles_m < 4 ? tiles_m : 4;
    const dim3 grid((unsigned)nwg), block(WM * WN * 64);
    const float *A = static_cast<const float *>(p.A);
    const float *B = static_cast<const float *>(p.B);
    float *C = static_cast<float *>(p.C);
    const Epilogue epi = p.epi ? *p.epi : Epilogue{1.f, 0.f, nullptr, 0};
    if (p.aligned)
        hipLaunchKernelGGL((f32_gemm_kernel<BM, BN, WM, WN, true, EPI>), grid, block, 0, p.stream,
                           A, B, C, p.M, p.N, p.K, p.lda, p.ldb, p.ldc, tiles_m, tiles_n, group_m,
                           epi);
    else
        hipLaunchKernelGGL((f32_gemm_kernel<BM, BN, WM, WN, false, EPI>), grid, block, 0, p.stream,
                           A, B, C, p.M, p.N, p.K, p.lda, p.ldb, p.ldc, tiles_m, tiles_n, group_m,
                           epi);
    return hipGetLastError();
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_cfg(const Problem &p)
{
    return p.epi ? launch_cfg_epi<BM, BN, WM, WN, true>(p) : launch_cfg_epi<BM, BN, WM, WN, false>(p);
}

}  // namespace

hipError_t f32_launch(const Problem &p, int cus)
{
    // Testing override LIBGEMM_F32_SMALL: '1' forces the register-staged kernels
    // below, '2' the guarded large-tile kernel, '3' the whole-tile large-tile
    // kernel, '4' / '5' the K-split kernel with 32-row tiles (whole-tile where
    // eligible / guarded), '6' / '7' the same with 64-row tiles and '8' the
    // vector-ALU kernel for at most 4 rows (each where it is eligible).
    const char *e = std::getenv("LIBGEMM_F32_SMALL");
    const int force = e && e[0] >= '1' && e[0] <= '8' ? e[0] - '0' : 0;
    if (force == 3 && f32_fast_eligible(p)) return f32_fast_launch(p, cus);
    if (force == 8 && rows_eligible(p)) return rows_launch(OUT_F32, p);
    if (force >= 4 && force <= 7 && f32_narrow_general_eligible(p))
        return f32_narrow_launch(p, force >= 6 ? 64 : 32, force == 5 || force == 7);
    if (force == 2 && f32_general_eligible(p)) return f32_general_launch(p);
    // At most 4 rows: the vector-ALU stream over B (1 x 4096 x 4096 16.8 us
    // against 44.5 on the K-split kernel, 4 x 16384 x 4096 41.3 against 54.4,
    // 1 x 64 x 16384 44.9 against 153).
    if (force == 0 && rows_eligible(p)) return rows_launch(OUT_F32, p);
    if (force == 0) {
        // Measured on MI355X (us; large-tile / K-split / register-staged):
        //  * from 256 tiles of 128 x 128, or 128 with K < 512, the large-tile
        //    kernels (whole tiles, else guarded): 1000 x 4096 x 4096 291 / 316 /
        //    360, 2048 x 1500 x 256 25.3 / 34.1 / 31.6;
        //  * other grids with K >= 512, and small grids (< 96 tiles) with K >=
        //    128, the K-split kernel: 2048 x 1500 x 4096 295 / 246 / 499,
        //    8192 x 64 x 4096 289 / 50 / 133, 300 x 1500 x 4096 289 / 48 / 195;
        //  * 96 to 127 tiles with K < 512, the register-staged kernels:
        //    300 x 4096 x 256 23.5 / 20.3 / 15.8;
        //  * products at most 64 columns wide never take 128-column tiles, half
        //    of which would be padding.
        const int64_t tiles128 = (int64_t)((p.M + 127) / 128) * ((p.N + 127) / 128);
        const bool large = p.N > 64 && (tiles128 >= 256 || (tiles128 >= 128 && p.K < 512));
        if (large && f32_fast_eligible(p)) return f32_fast_launch(p, cus);
        if (large && f32_general_eligible(p)) return f32_general_launch(p);
        const bool ksplit = p.K >= 512 || (p.K >= 128 && tiles128 < 96);
        if (!large && ksplit && f32_narrow_general_eligible(p)) {
            // 64-row tiles do twice the work per workgroup: take them when that
            // costs no more rounds of one workgroup per CU (1000^3: 28 against 33
            // us; 300 x 4096 x 4096: 159 against 137 the other way).
            const int64_t cu = cus > 0 ? cus : 256;
            const int64_t t32 = (int64_t)((p.M + 31) / 32) * ((p.N + 63) / 64);
            const int64_t t64 = (int64_t)((p.M + 63) / 64) * ((p.N + 63) / 64);
            const bool rows64 = p.M >= 64 && 2 * ((t64 + cu - 1) / cu) <= (t32 + cu - 1) / cu;
            return f32_narrow_launch(p, rows64 ? 64 : 32, false);
        }
    }
    const int64_t big = (int64_t)((p.M + 127) / 128) * ((p.N + 127) / 128);
    if (big >= 128) return launch_cfg<128, 128, 2, 2>(p);
    return launch_cfg<64, 64, 2, 2>(p);
}

}  // namespace gemm
