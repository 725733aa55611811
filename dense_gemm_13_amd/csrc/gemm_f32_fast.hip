// fp32 SGEMM, large-tile path for gfx950: whole 128 x 128 tiles, K a multiple of
// 64, 16-byte aligned rows.
//
// The register-tiled SGEMM of "CUDA GEMM 优化实践笔记" (block tile of C staged in
// shared memory, K walked in BK steps, per-thread register tile) with the FMA
// outer product replaced by v_mfma_f32_32x32x2_f32 on 64 x 64 wave tiles, and
// the operands moved with global_load_lds_dwordx4 into two LDS stages (one array
// per stage, indexed at compile time; the 16-byte chunk swizzle is applied on
// the global side).  Two-level accumulation as in gemm_f32.hip: each 32-wide K
// step is summed into a fresh partial and then added to the running total.
// 64 KiB of LDS and at most 256 registers per lane (two waves per SIMD) let two
// workgroups share a CU, so one workgroup's MFMAs cover the other's barriers.
//
// LDS: A as rows of k (128 bytes per row, chunk XOR swz8(row)); B as rows of n
// (512 bytes per row), read as single floats: 32 lanes cover 128 contiguous
// bytes of row k while the other 32 read row k+4; rows with bit 2 set have
// their chunks XOR-moved by 128 bytes so the two halves never share banks.
#include <utility>

#include "gemm_device.hpp"
#include "gemm_launch.hpp"

namespace gemm {

namespace {

typedef __attribute__((address_space(3))) void lds_void32_t;

constexpr int SBM = 128, SBN = 128, SBK = 32, SSTAGES = 2;
constexpr int SWM = 2, SWN = 2, SNW = SWM * SWN;
constexpr int SWTM = SBM / SWM, SWTN = SBN / SWN;       // 64 x 64 per wave
constexpr int SFM = SWTM / 32, SFN = SWTN / 32;         // 2 x 2 MFMA tiles
constexpr int SA_STAGE = SBM * SBK;                      // floats per stage (16 KiB)
constexpr int SB_STAGE = SBK * SBN;
constexpr int SA_BLK = SA_STAGE * 4 / 1024 / SNW;        // 1 KiB loads per wave per stage
constexpr int SB_BLK = SB_STAGE * 4 / 1024 / SNW;

template <int TAG>
__shared__ __attribute__((aligned(1024))) float s_stage[4096];

__host__ __device__ __forceinline__ int swz_bf(int k) { return ((k >> 2) & 1) << 3; }

__device__ __forceinline__ void s_barrier_nf() { asm volatile("s_barrier" ::: "memory"); }

// GEN = false: whole 128 x 128 tiles, K a multiple of 64, 16-byte aligned rows.
// GEN = true: any M, N >= 4, K > 32 and any leading dimensions (the hardware
// runs in unaligned-access mode, so 16-byte loads and stores at 4-byte-aligned
// addresses are legal):
//   * the last K block (possibly partial) is step 0, loaded through registers
//     with zero fill past K, M and N; steps 1, 2, ... load blocks 0, 1, ...
//     LDS-direct, whole blocks that never touch B's last row;
//   * A rows past M are clamped to row M-1 and B column chunks starting past N
//     to the chunk at N-4 (their products only reach C entries that are not
//     stored; a chunk straddling N reads a few floats past N inside a row that
//     is not B's last);
//   * an odd number of K steps ends with one more step, and C stores (and the
//     epilogue's reads) are masked to the M x N window.
// EPI: the fused epilogue is applied to the results by the lane that stores them.
template <bool GEN, bool EPI>
__global__ void __launch_bounds__(SNW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
f32_fast_kernel(const float *__restrict__ A, const float *__restrict__ B, float *__restrict__ C,
                int M, int N, int K, int64_t lda, int64_t ldb, int64_t ldc, int tiles_m,
                int tiles_n, int group_m, Epilogue epi)
{
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm0 = (wave / SWN) * SWTM;
    const int wn0 = (wave % SWN) * SWTN;
    const int l32 = lane & 31, half = lane >> 5;

    int tm, tn;
    tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * SBM, n0 = tn * SBN;

    // A block b: 8 rows of 128 bytes, lane -> row 8b + lane/8, slot lane%8
    // (logical chunk slot ^ swz8(row)).  B block b: 2 rows of 512 bytes, lane ->
    // row 2b + lane/32, slot lane%32 (logical chunk slot ^ swz_bf(row)).
    uint32_t a_off[SA_BLK], b_off[SB_BLK];
#pragma unroll
    for (int j = 0; j < SA_BLK; ++j) {
        const int row = 8 * (wave * SA_BLK + j) + (lane >> 3);
        const int lrow = GEN && m0 + row >= M ? M - 1 - m0 : row;
        a_off[j] = (uint32_t)(lrow * lda + 4 * ((lane & 7) ^ swz8(row))) * 4u;
    }
    // (GEN: the column, n0 included, is part of the per-lane offset.)
#pragma unroll
    for (int j = 0; j < SB_BLK; ++j) {
        const int row = 2 * (wave * SB_BLK + j) + (lane >> 5);
        int col = 4 * ((lane & 31) ^ swz_bf(row));
        if (GEN) col = n0 + col >= N ? N - 4 : n0 + col;
        b_off[j] = (uint32_t)(row * ldb + col) * 4u;
    }
    const char *a_base = reinterpret_cast<const char *>(A + (int64_t)m0 * lda);
    const char *b_base = reinterpret_cast<const char *>(GEN ? B : B + n0);
    const int64_t b_step = (int64_t)SBK * ldb * 4;
    // K step s loads K block s (GEN: block s - 1; step 0 is the last block).
    auto issue = [&](float *as, float *bs, int s) {
        const int kt = GEN ? s - 1 : s;
        const char *ab = a_base + (int64_t)kt * SBK * 4;
        const char *bb = b_base + kt * b_step;
#pragma unroll
        for (int j = 0; j < SA_BLK; ++j)
            __builtin_amdgcn_global_load_lds(ab + a_off[j], (lds_void32_t *)(as + (wave * SA_BLK + j) * 256), 16, 0, 0);
#pragma unroll
        for (int j = 0; j < SB_BLK; ++j)
            __builtin_amdgcn_global_load_lds(bb + b_off[j], (lds_void32_t *)(bs + (wave * SB_BLK + j) * 256), 16, 0, 0);
    };

    // Fragments (floats, relative to a stage).  Sub-step s covers k = 8s .. 8s+7;
    // the e-th MFMA of it takes k = 8s + 4*half + e in both operands.
    int a_off_r[SFM], a_swz[SFM];
#pragma unroll
    for (int i = 0; i < SFM; ++i) {
        const int row = wm0 + 32 * i + l32;
        a_off_r[i] = row * SBK;
        a_swz[i] = swz8(row);
    }
    int b_col[SFN];
#pragma unroll
    for (int j = 0; j < SFN; ++j) b_col[j] = wn0 + 32 * j + l32;

    f32x16 total[SFM][SFN];
#pragma unroll
    for (int i = 0; i < SFM; ++i)
#pragma unroll
        for (int j = 0; j < SFN; ++j) total[i][j] = f32x16{};

    auto compute = [&](const float *as, const float *bs) {
        f32x16 part[SFM][SFN];
#pragma unroll
        for (int i = 0; i < SFM; ++i)
#pragma unroll
            for (int j = 0; j < SFN; ++j) part[i][j] = f32x16{};
#pragma unroll
        for (int s = 0; s < SBK / 8; ++s) {
            const int c = 2 * s + half;
            f32x4 af[SFM];
            float bv[SFN][4];
#pragma unroll
            for (int i = 0; i < SFM; ++i)
                af[i] = *reinterpret_cast<const f32x4 *>(as + a_off_r[i] + ((c ^ a_swz[i]) << 2));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int k = 8 * s + 4 * half + e;
#pragma unroll
                for (int j = 0; j < SFN; ++j) {
                    const int n = b_col[j];
                    bv[j][e] = bs[k * SBN + (((n >> 2) ^ swz_bf(k)) << 2) + (n & 3)];
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int i = 0; i < SFM; ++i)
#pragma unroll
                    for (int j = 0; j < SFN; ++j)
                        part[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(bv[j][e], af[i][e],
                                                                         part[i][j], 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < SFM; ++i)
#pragma unroll
            for (int j = 0; j < SFN; ++j) total[i][j] += part[i][j];
    };

    auto step = [&](float *as, float *bs, float *nas, float *nbs, int next_kt, bool dma) {
        __builtin_amdgcn_s_waitcnt(0x0f70);              // vmcnt(0): this stage (own loads)
        s_barrier_nf();                                  // ... everyone's; the other stage is free
        if (dma) issue(nas, nbs, next_kt);
        compute(as, bs);
    };

    const int ktiles = (K + SBK - 1) / SBK;              // !GEN: K / SBK, even
    if constexpr (GEN) {
        // Step 0: the last K block [SBK*(ktiles-1), K) through registers, zero
        // filled, in the swizzled layout the LDS-direct loads produce.
        const int k0 = SBK * (ktiles - 1);
        float *as = s_stage<0>, *bs = s_stage<2>;
        for (int q = tid; q < SBM * SBK / 4; q += SNW * 64) {
            const int r = q >> 3, c = q & 7;
            const int gm = m0 + r, gk = k0 + 4 * c;
            f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
            if (gm < M) {
                const float *src = A + (int64_t)gm * lda + gk;
                if (gk + 4 <= K) {
                    v = *reinterpret_cast<const f32x4 *>(src);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (gk + e < K) v[e] = src[e];
                }
            }
            *reinterpret_cast<f32x4 *>(as + r * SBK + ((c ^ swz8(r)) << 2)) = v;
        }
        for (int q = tid; q < SBK * SBN / 4; q += SNW * 64) {
            const int r = q >> 5, c = q & 31;
            const int gk = k0 + r, gn = n0 + 4 * c;
            f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
            if (gk < K) {
                const float *src = B + (int64_t)gk * ldb + gn;
                if (gn + 4 <= N) {
                    v = *reinterpret_cast<const f32x4 *>(src);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (gn + e < N) v[e] = src[e];
                }
            }
            *reinterpret_cast<f32x4 *>(bs + r * SBN + ((c ^ swz_bf(r)) << 2)) = v;
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);              // lgkmcnt(0): the LDS writes landed
    } else {
        issue(s_stage<0>, s_stage<2>, 0);
    }
    // Pairs of steps over the two stages; GEN: an odd count ends with one more.
    int kt = 0;
    for (; kt + 1 < ktiles; kt += 2) {
        step(s_stage<0>, s_stage<2>, s_stage<1>, s_stage<3>, kt + 1, true);
        step(s_stage<1>, s_stage<3>, s_stage<0>, s_stage<2>, kt + 2, kt + 2 < ktiles);
    }
    if (GEN && kt < ktiles) step(s_stage<0>, s_stage<2>, s_stage<1>, s_stage<3>, kt + 1, false);

    // lane holds C[m][n..n+3], n = 8g + 4*half (+ tile offsets): one 16-byte store
#pragma unroll
    for (int i = 0; i < SFM; ++i) {
        const int gm = m0 + wm0 + 32 * i + l32;
        if (GEN && gm >= M) continue;
        float *const rowp = C + (int64_t)gm * ldc;
#pragma unroll
        for (int j = 0; j < SFN; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int gn = n0 + wn0 + 4 * half + 32 * j + 8 * g;
                const int cnt = GEN ? N - gn : 4;
                float ev[4] = {total[i][j][4 * g], total[i][j][4 * g + 1], total[i][j][4 * g + 2],
                               total[i][j][4 * g + 3]};
                if constexpr (EPI) epilogue_row<OUT_F32, 4>(epi, ev, rowp, gn, cnt);
                if (!GEN || cnt >= 4) {
                    *reinterpret_cast<f32x4 *>(rowp + gn) = f32x4{ev[0], ev[1], ev[2], ev[3]};
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (e < cnt) rowp[gn + e] = ev[e];
                }
            }
    }
}

}  // namespace

bool f32_fast_eligible(const Problem &p)
{
    return p.aligned && p.M % SBM == 0 && p.N % SBN == 0 && p.K % (SBK * SSTAGES) == 0 &&
           p.lda < (1 << 22) && p.ldb < (1 << 22);
}

// The guarded instantiation: any M, N >= 4 (a clamped column chunk starts at
// N - 4), two K blocks at least, and per-lane 32-bit byte offsets that fit.
bool f32_general_eligible(const Problem &p)
{
    return p.M >= 1 && p.N >= 4 && p.K > SBK && p.lda < (1 << 22) &&
           (int64_t)SBK * p.ldb + p.N < ((int64_t)1 << 30);
}

template <bool GEN>
static hipError_t f32_fast_typed(const Problem &p)
{
    const int tiles_m = (p.M + SBM - 1) / SBM, tiles_n = (p.N + SBN - 1) / SBN;
    const int64_t nwg = (int64_t)tiles_m * tiles_n;
    if (nwg > 0x7fffffff) return hipErrorInvalidValue;
    const int group_m = tiles_m < 4 ? tiles_m : 4;
    const float *A = static_cast<const float *>(p.A), *B = static_cast<const float *>(p.B);
    float *C = static_cast<float *>(p.C);
    const Epilogue epi = p.epi ? *p.epi : Epilogue{1.f, 0.f, nullptr, 0};
    if (p.epi)
        hipLaunchKernelGGL((f32_fast_kernel<GEN, true>), dim3((unsigned)nwg), dim3(SNW * 64), 0,
                           p.stream, A, B, C, p.M, p.N, p.K, p.lda, p.ldb, p.ldc, tiles_m, tiles_n,
                           group_m, epi);
    else
        hipLaunchKernelGGL((f32_fast_kernel<GEN, false>), dim3((unsigned)nwg), dim3(SNW * 64), 0,
                           p.stream, A, B, C, p.M, p.N, p.K, p.lda, p.ldb, p.ldc, tiles_m, tiles_n,
                           group_m, epi);
    return hipGetLastError();
}

hipError_t f32_fast_launch(const Problem &p)
{
    if (!f32_fast_eligible(p)) return hipErrorInvalidValue;
    return f32_fast_typed<false>(p);
}

hipError_t f32_general_launch(const Problem &p)
{
    if (!f32_general_eligible(p)) return hipErrorInvalidValue;
    return f32_fast_typed<true>(p);
}

}  // namespace gemm
