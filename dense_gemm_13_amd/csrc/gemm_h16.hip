// fp16 / bf16 GEMM on gfx950 matrix cores: C = A * B, A (M x K) and B (K x N)
// row-major, fp32 accumulation, C rounded to nearest-even.
//
// Design (the half-precision kernels of "[CUDA 优化实战] hgemm - 超越 cuBLAS",
// sections 1-4, re-made for CDNA4 wave64 MFMA):
//   * one workgroup per BM x BN tile of C; the grid is remapped XCD-aware;
//   * K is walked in steps of 64; each step's A tile (BM x 64) and B tile
//     (64 x BN) are fetched with 16-byte global loads, out-of-range elements read
//     as zero.  Rows need no alignment beyond the element size: the hardware
//     runs in unaligned-access mode, so 16-byte loads and 8-byte stores at
//     2-byte-aligned addresses are legal; only chunks that straddle the edge of
//     a row are read or written element by element;
//   * LDS holds two stages (ping-pong): while the waves multiply stage t, the
//     loads of stage t+1 are in flight in registers;
//   * A sits in LDS as rows of k (as in memory).  The MFMA needs, in every lane,
//     8 consecutive k of one column of B, so B is transposed on its way into LDS
//     (8 x 8 blocks shuffled in registers) and sits as rows of k per column n;
//   * 16-byte LDS chunks are XOR-swizzled so the fragment reads and the
//     transposed writes are spread over the banks;
//   * every wave owns a (BM/WM) x (BN/WN) sub-tile made of 32x32 MFMA tiles
//     (v_mfma_f32_32x32x16_{bf16,f16}).  B supplies the MFMA's first operand, so
//     each lane ends up holding 4 consecutive columns of one row of C and the
//     epilogue writes 8 bytes per lane.
#include "gemm_device.hpp"
#include "gemm_launch.hpp"

namespace gemm {

namespace {

constexpr int H16_BK = 64;

// Rows of B per transposed load unit (each unit is R rows x 8 columns).
template <int BN, int NT>
constexpr int b_unit_rows()
{
    return ((H16_BK / 8) * (BN / 8)) % NT == 0 ? 8
         : ((H16_BK / 4) * (BN / 8)) % NT == 0 ? 4
         : ((H16_BK / 2) * (BN / 8)) % NT == 0 ? 2 : 0;
}

// 8 consecutive halves at p (row `r` of a matrix with `rows` rows), elements at
// or beyond `cols_left` read as zero.
__device__ __forceinline__ u32x4 load8_guarded(const uint16_t *p, bool row_ok, int cols_left)
{
    uint32_t w[4] = {0, 0, 0, 0};
    if (row_ok) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (e < cols_left) w[e >> 1] |= (uint32_t)p[e] << ((e & 1) * 16);
    }
    return u32x4{w[0], w[1], w[2], w[3]};
}

// EPI: the fused epilogue is applied to the fp32 results before rounding, by
// the lane that stores them.
// DBUF, SWZ (both on for the library's own calls) switch off the two-stage LDS
// ring and the XOR swizzle, for the measured optimisation ladder: without DBUF
// each K step loads, stores to LDS, synchronises and multiplies in turn; without
// SWZ the 16-byte chunks sit in LDS in their natural order.
template <bool IS_BF16, int BM, int BN, int WM, int WN, bool EPI, bool DBUF = true, bool SWZ = true>
__global__ void __launch_bounds__(WM * WN * 64)
h16_gemm_kernel(const uint16_t *__restrict__ A, const uint16_t *__restrict__ B,
                uint16_t *__restrict__ C, int M, int N, int K, int64_t lda, int64_t ldb,
                int64_t ldc, int tiles_m, int tiles_n, int group_m, Epilogue epi)
{
    constexpr int BK = H16_BK;
    constexpr int NT = WM * WN * 64;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    constexpr int A_ITERS = BM * (BK / 8) / NT;
    constexpr int BR = b_unit_rows<BN, NT>();
    constexpr int B_ITERS = (BK / BR) * (BN / 8) / NT;
    static_assert(FM >= 1 && FN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "wave tile");
    static_assert(A_ITERS >= 1 && A_ITERS * NT == BM * (BK / 8), "A loader");
    static_assert(BR != 0 && B_ITERS >= 1, "B loader");

    __shared__ __attribute__((aligned(16))) uint16_t As[DBUF ? 2 : 1][BM * BK];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[DBUF ? 2 : 1][BN * BK];
    auto swz8 = [](int row) { return SWZ ? gemm::swz8(row) : 0; };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm0 = (wave / WN) * WTM;
    const int wn0 = (wave % WN) * WTN;
    const int l32 = lane & 31, half = lane >> 5;

    int tm, tn;
    tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

    u32x4 areg[A_ITERS];
    u32x4 breg[B_ITERS][BR];
    // Chunks at the edges: one 16-byte load from inside the matrix (masked16_load)
    // whose zeros past M, N and K are applied when the chunk is stored to LDS,
    // after the step's MFMAs, so no load is waited for inside load_tile.  The
    // shift of each chunk is worked out again from its indices then.  (Not in
    // the 8-wave 256 x 256 tiles, whose registers are full: element loads there.)
    constexpr bool MASKED = BM * BN <= 128 * 128;
    int loaded_k0 = 0;                                   // K step in the registers
    // Bytes a chunk's masked load shifts out (0 for a chunk wholly inside).
    const auto drop_of = [](int row, int rows, int k, int cols) {
        if (!MASKED || cols < 8) return 0;               // (element loads instead)
        if (row >= rows || k >= cols) return 16;
        return k + 8 > cols ? 2 * (k + 8 - cols) : 0;
    };

    // ---- global -> registers for the K step starting at k0
    auto load_tile = [&](int k0) {
        loaded_k0 = k0;
#pragma unroll
        for (int it = 0; it < A_ITERS; ++it) {
            const int q = tid + it * NT;
            const int row = q >> 3, c = q & 7;
            const int gm = m0 + row, gk = k0 + c * 8;
            const uint16_t *src = A + (int64_t)gm * lda + gk;
            if (gm < M && gk + 8 <= K) {
                areg[it] = *reinterpret_cast<const u32x4 *>(src);
            } else if (MASKED && K >= 8) {
                areg[it] = masked16_load<2>(A, lda, gm, M, gk, K).raw;
            } else {
                areg[it] = load8_guarded(src, gm < M, K - gk);
            }
        }
#pragma unroll
        for (int it = 0; it < B_ITERS; ++it) {
            const int p = tid + it * NT;
            const int nb = p % (BN / 8), kb = p / (BN / 8);
            const int gn = n0 + nb * 8;
#pragma unroll
            for (int r = 0; r < BR; ++r) {
                const int gk = k0 + kb * BR + r;
                const uint16_t *src = B + (int64_t)gk * ldb + gn;
                if (gk < K && gn + 8 <= N) {
                    breg[it][r] = *reinterpret_cast<const u32x4 *>(src);
                } else if (MASKED && N >= 8) {
                    breg[it][r] = masked16_load<2>(B, ldb, gk, K, gn, N).raw;
                } else {
                    breg[it][r] = load8_guarded(src, gk < K, N - gn);
                }
            }
        }
    };

    // ---- registers -> LDS stage `buf` (A as is, B transposed)
    auto store_tile = [&](int buf) {
        const int k0 = loaded_k0;
        if (MASKED && (m0 + BM > M || n0 + BN > N || k0 + BK > K)) {
#pragma unroll
            for (int it = 0; it < A_ITERS; ++it) {
                const int q = tid + it * NT;
                areg[it] = shift_down_bytes(areg[it], drop_of(m0 + (q >> 3), M, k0 + (q & 7) * 8, K));
            }
#pragma unroll
            for (int it = 0; it < B_ITERS; ++it) {
                const int p = tid + it * NT;
                const int gn = n0 + (p % (BN / 8)) * 8, kb = p / (BN / 8);
#pragma unroll
                for (int r = 0; r < BR; ++r)
                    breg[it][r] = shift_down_bytes(breg[it][r], drop_of(k0 + kb * BR + r, K, gn, N));
            }
        }
#pragma unroll
        for (int it = 0; it < A_ITERS; ++it) {
            const int q = tid + it * NT;
            const int row = q >> 3, c = q & 7;
            *reinterpret_cast<u32x4 *>(&As[buf][row * BK + ((c ^ swz8(row)) << 3)]) = areg[it];
        }
#pragma unroll
        for (int it = 0; it < B_ITERS; ++it) {
            const int p = tid + it * NT;
            const int nb = p % (BN / 8), kb = p / (BN / 8);
            const int kofs = kb * BR;
#pragma unroll
            for (int n = 0; n < 8; ++n) {
                const int pw = n >> 1;
                uint32_t w[BR / 2];
#pragma unroll
                for (int j = 0; j < BR / 2; ++j) {
                    const uint32_t lo = breg[it][2 * j][pw], hi = breg[it][2 * j + 1][pw];
                    w[j] = (n & 1) ? ((lo >> 16) | (hi & 0xffff0000u))
                                   : ((lo & 0xffffu) | (hi << 16));
                }
                const int nrow = nb * 8 + n;
                uint16_t *dst = &Bs[buf][nrow * BK + (((kofs >> 3) ^ swz8(nrow)) << 3) + (kofs & 7)];
                if constexpr (BR == 8)
                    *reinterpret_cast<u32x4 *>(dst) = u32x4{w[0], w[1], w[2], w[3]};
                else if constexpr (BR == 4)
                    *reinterpret_cast<u32x2 *>(dst) = u32x2{w[0], w[1]};
                else
                    *reinterpret_cast<uint32_t *>(dst) = w[0];
            }
        }
    };

    // ---- LDS stage `buf` -> MFMA
    auto compute = [&](int buf) {
#pragma unroll
        for (int s = 0; s < BK / 16; ++s) {
            const int c = 2 * s + half;
            u32x4 af[FM], bfr[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int row = wm0 + i * 32 + l32;
                af[i] = *reinterpret_cast<const u32x4 *>(&As[buf][row * BK + ((c ^ swz8(row)) << 3)]);
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int nrow = wn0 + j * 32 + l32;
                bfr[j] = *reinterpret_cast<const u32x4 *>(&Bs[buf][nrow * BK + ((c ^ swz8(nrow)) << 3)]);
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = mfma32x32x16<IS_BF16>(bfr[j], af[i], acc[i][j]);
        }
    };

    const int ktiles = (K + BK - 1) / BK;
    if constexpr (DBUF) {
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
    } else {
        for (int t = 0; t < ktiles; ++t) {
            load_tile(t * BK);
            store_tile(0);
            __syncthreads();
            compute(0);
            __syncthreads();
        }
    }

    // ---- epilogue: lane holds C[m][n..n+3] for n = 8g + 4*half (+ tile offsets)
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
                if constexpr (EPI)
                    epilogue_row<IS_BF16 ? OUT_BF16 : OUT_F16, 4>(epi, ev, crow, n, N - n);
                const float v0 = ev[0], v1 = ev[1], v2 = ev[2], v3 = ev[3];
                if (n + 4 <= N) {
                    *reinterpret_cast<u32x2 *>(crow + n) =
                        u32x2{pack2<IS_BF16>(v0, v1), pack2<IS_BF16>(v2, v3)};
                } else {
                    const float v[4] = {v0, v1, v2, v3};
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        if (n + t < N)
                            crow[n + t] = IS_BF16 ? to_bf16_bits(v[t]) : to_f16_bits(v[t]);
                }
            }
        }
    }
}

template <bool IS_BF16, int BM, int BN, int WM, int WN, bool EPI>
hipError_t launch_cfg_epi(const Problem &p)
{
    const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
    const int64_t nwg = (int64_t)tiles_m * tiles_n;
    if (nwg > 0x7fffffff) return hipErrorInvalidValue;
    const int group_m = tiles_m < 4 ? tiles_m : 4;
    const dim3 grid((unsigned)nwg), block(WM * WN * 64);
    const uint16_t *A = static_cast<const uint16_t *>(p.A);
    const uint16_t *B = static_cast<const uint16_t *>(p.B);
    uint16_t *C = static_cast<uint16_t *>(p.C);
    const Epilogue epi = p.epi ? *p.epi : Epilogue{1.f, 0.f, nullptr, 0};
    hipLaunchKernelGGL((h16_gemm_kernel<IS_BF16, BM, BN, WM, WN, EPI>), grid, block, 0, p.stream,
                       A, B, C, p.M, p.N, p.K, p.lda, p.ldb, p.ldc, tiles_m, tiles_n, group_m,
                       epi);
    return hipGetLastError();
}

template <bool IS_BF16, int BM, int BN, int WM, int WN>
hipError_t launch_cfg(const Problem &p)
{
    return p.epi ? launch_cfg_epi<IS_BF16, BM, BN, WM, WN, true>(p)
                 : launch_cfg_epi<IS_BF16, BM, BN, WM, WN, false>(p);
}

template <bool IS_BF16>
hipError_t launch_typed(int config, const Problem &p)
{
    switch (config) {
    case H16_256x256_W8: return launch_cfg<IS_BF16, 256, 256, 2, 4>(p);
    case H16_128x128_W4: return launch_cfg<IS_BF16, 128, 128, 2, 2>(p);
    case H16_64x64_W4: return launch_cfg<IS_BF16, 64, 64, 2, 2>(p);
    case H16_32x64_W2: return launch_cfg<IS_BF16, 32, 64, 1, 2>(p);
    default: return hipErrorInvalidValue;
    }
}

// Rungs of the measured optimisation ladder that use this kernel: 128 x 128
// tiles of 4 waves, MFMA; rung 3 plain LDS, one stage; rung 4 with the two-stage
// ring; rung 5 with the ring and the swizzle (the library's own 128 x 128 kernel).
// Rungs 7 and 8 are rungs 3 and 4 launched with LADDER_RESERVE_LDS bytes of LDS
// reserved (and unused) per workgroup, so that at most one workgroup fits on a
// CU: with several resident workgroups, one workgroup's loads already overlap
// another's MFMAs, which hides what the two-stage ring adds.
constexpr unsigned LADDER_RESERVE_LDS = 80 * 1024;

template <bool IS_BF16>
hipError_t ladder_typed(int rung, const Problem &p)
{
    constexpr int BM = 128, BN = 128, WM = 2, WN = 2;
    const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
    const int64_t nwg = (int64_t)tiles_m * tiles_n;
    if (nwg > 0x7fffffff) return hipErrorInvalidValue;
    const int group_m = tiles_m < 4 ? tiles_m : 4;
    const dim3 grid((unsigned)nwg), block(WM * WN * 64);
    const uint16_t *A = static_cast<const uint16_t *>(p.A);
    const uint16_t *B = static_cast<const uint16_t *>(p.B);
    uint16_t *C = static_cast<uint16_t *>(p.C);
    const Epilogue none{1.f, 0.f, nullptr, 0};
#define LADDER_LAUNCH(DB, SW, LDS)                                                                 \
    do {                                                                                           \
        auto *kern = h16_gemm_kernel<IS_BF16, BM, BN, WM, WN, false, DB, SW>;                       \
        if ((LDS) > 0) {                                                                           \
            const hipError_t e = hipFuncSetAttribute(                                              \
                reinterpret_cast<const void *>(kern),                                              \
                hipFuncAttributeMaxDynamicSharedMemorySize, (int)(LDS));                           \
            if (e != hipSuccess) return e;                                                         \
        }                                                                                          \
        hipLaunchKernelGGL(kern, grid, block, (LDS), p.stream, A, B, C, p.M, p.N, p.K, p.lda,      \
                           p.ldb, p.ldc, tiles_m, tiles_n, group_m, none);                         \
    } while (0)
    switch (rung) {
    case 3: LADDER_LAUNCH(false, false, 0u); break;
    case 4: LADDER_LAUNCH(true, false, 0u); break;
    case 5: LADDER_LAUNCH(true, true, 0u); break;
    case 7: LADDER_LAUNCH(false, false, LADDER_RESERVE_LDS); break;
    case 8: LADDER_LAUNCH(true, false, LADDER_RESERVE_LDS); break;
    default: return hipErrorInvalidValue;
    }
#undef LADDER_LAUNCH
    return hipGetLastError();
}

}  // namespace

hipError_t h16_ladder_launch(int rung, bool is_bf16, const Problem &p)
{
    return is_bf16 ? ladder_typed<true>(rung, p) : ladder_typed<false>(rung, p);
}

// Register-staged kernels: the largest tile whose padding costs at most a
// quarter more MFMA work than the product and whose grid still gives the chip
// at least half a workgroup per CU; if none reaches that, the one with the most
// workgroups (measured on MI355X: a 100352 x 64 x 576 product takes 24 us on
// 64 x 64 tiles against 75 us on 256 x 256 tiles, three quarters of them empty).
int h16_pick_config(int M, int N, int K)
{
    // Among the register-staged kernels (the large-tile kernels take big grids
    // before this is asked): 256 x 256 when it fills half the chip with little
    // padding; 128 x 128 only from two tiles per CU on; else 64 x 64, which
    // measured faster than 128 x 128 up to ~256 tiles of 128 x 128 and faster
    // than 32 x 64 tiles on every shape tried (e.g. 2048 x 1500 x 1000: 32.5 us
    // on 64 x 64, 48.3 on 128 x 128; 300 x 1500 x 256: 7.9 against 11.3 on
    // 32 x 64).
    (void)K;
    const auto tiles = [&](int bm, int bn) { return (int64_t)((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
    const auto lean = [&](int bm, int bn) { return 4 * tiles(bm, bn) * bm * bn <= 5 * (int64_t)M * N; };
    if (lean(256, 256) && tiles(256, 256) >= 128) return H16_256x256_W8;
    if (lean(128, 128) && tiles(128, 128) >= 512) return H16_128x128_W4;
    return H16_64x64_W4;
}

hipError_t h16_launch(bool is_bf16, int config, const Problem &p)
{
    if (config == H16_FAST_256x256) return h16_fast_launch(is_bf16, p);
    if (config == H16_GEN_256x256) return h16_general_launch(is_bf16, p);
    if (config == H16_NARROW_32x64) return h16_narrow_launch(is_bf16, p);
    if (config == H16_NARROW_GEN) return h16_narrow_general_launch(is_bf16, p);
    if (config == H16_NARROW64) return h16_narrow64_launch(is_bf16, p);
    if (config == H16_NARROW64_GEN) return h16_narrow64_general_launch(is_bf16, p);
    if (config == H16_ROWS) return rows_launch(is_bf16 ? OUT_BF16 : OUT_F16, p);
    if (config == H16_FEWROWS) return h16_fewrows_launch(is_bf16, p);
    if (config == H16_FAST_128) return h16_fast128_launch(is_bf16, p);
    if (config == H16_GEN_128) return h16_general128_launch(is_bf16, p);
    if (config == H16_FAST_128x256) return h16_fast128x256_launch(is_bf16, p);
    if (config == H16_GEN_128x256) return h16_general128x256_launch(is_bf16, p);
    return is_bf16 ? launch_typed<true>(config, p) : launch_typed<false>(config, p);
}

}  // namespace gemm
