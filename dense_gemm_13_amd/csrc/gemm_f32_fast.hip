// fp32 SGEMM, large-tile path for gfx950: 128 x 128 tiles of C, 4 waves of
// 64 x 64 (2 x 2 MFMA tiles of v_mfma_f32_32x32x2_f32).
//
// The register-tiled SGEMM of "CUDA GEMM 优化实践笔记" (block tile of C staged in
// shared memory, K walked in BK steps, per-thread register tile) with the FMA
// outer product replaced by MFMAs on 64 x 64 wave tiles, and the operands moved
// with global_load_lds_dwordx4 into a ring of 4 LDS stages of 16-wide K steps
// (one array per stage, indexed at compile time; the 16-byte chunk swizzle is
// applied on the global side).  Each step waits only for the loads of the
// stage after it, and its workgroup barrier sits before its last sub-step:
// that sub-step's MFMAs cover the reads of the next stage's first fragments and
// the global loads of the step three ahead, and every sub-step multiplies while
// the following one's fragments are read, so no LDS latency is exposed.
// Two-level accumulation: each 64-wide K block (one turn of the ring) is summed
// into a fresh partial that is then added to the running total (with b-wide
// partials the rounding error of a K-term sum grows like b + K/b, least at b
// near sqrt(K): 64 for K = 4096).  64 KiB of LDS and at
// most 256 registers per lane (two waves per SIMD) let two workgroups share a
// CU.
//
// LDS: A as rows of k (64 bytes per row, chunk XOR swz_af(row)); B as rows of n
// (512 bytes per row), read as single floats: 32 lanes cover 128 contiguous
// bytes of row k while the other 32 read row k+4; rows with bit 2 set have
// their chunks XOR-moved by 128 bytes so the two halves never share banks.
#include <utility>

#include "gemm_device.hpp"
#include "gemm_launch.hpp"
#include "gemm_lds_layout.hpp"

namespace gemm {

namespace {

typedef __attribute__((address_space(3))) void lds_void32_t;

constexpr int SBM = 128, SBN = 128, SBK = 16, SSTAGES = 4;
constexpr int SWM = 2, SWN = 2, SNW = SWM * SWN;
constexpr int SWTM = SBM / SWM, SWTN = SBN / SWN;       // 64 x 64 per wave
constexpr int SFM = SWTM / 32, SFN = SWTN / 32;         // 2 x 2 MFMA tiles
constexpr int SA_STAGE = SBM * SBK;                      // floats per stage (8 KiB)
constexpr int SB_STAGE = SBK * SBN;
constexpr int SA_BLK = SA_STAGE * 4 / 1024 / SNW;        // 1 KiB loads per wave per stage
constexpr int SB_BLK = SB_STAGE * 4 / 1024 / SNW;

template <int TAG>
__shared__ __attribute__((aligned(1024))) float s_stage[2048];

// The XOR swizzles of the stages and the lane -> address maps of every LDS
// access below are in gemm_lds_layout.hpp (checked on the host for banks).
using lds::swz_af;
using lds::swz_bf;

__device__ __forceinline__ void s_barrier_nf() { asm volatile("s_barrier" ::: "memory"); }

// s_waitcnt vmcnt(N) (N < 64), leaving expcnt and lgkmcnt alone.
template <int N>
__device__ __forceinline__ void s_wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// One 16-byte global -> LDS load per lane (lane t's bytes land at lds + 16t).
__device__ __forceinline__ void s_dma16(const void *src, float *lds)
{
    __builtin_amdgcn_global_load_lds(src, (lds_void32_t *)lds, 16, 0, 0);
}

template <typename F, int... I>
__device__ __forceinline__ void s_unroll_impl(F &&f, std::integer_sequence<int, I...>)
{
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void s_unroll(F &&f)
{
    s_unroll_impl(f, std::make_integer_sequence<int, N>{});
}

// GEN = false: whole 128 x 128 tiles, K a multiple of 64, 16-byte aligned rows.
// GEN = true: any M, N >= 4, K > 16 and any leading dimensions (the hardware
// runs in unaligned-access mode, so 16-byte loads and stores at 4-byte-aligned
// addresses are legal):
//   * the last K block (possibly partial) is step 0, loaded through registers
//     with zero fill past K, M and N; steps 1, 2, ... load blocks 0, 1, ...
//     LDS-direct, whole blocks that never touch B's last row;
//   * A rows past M are clamped to row M-1 and B column chunks starting past N
//     to the last whole chunk at a multiple of 4 columns (their products only reach C entries that are not
//     stored; a chunk straddling N reads a few floats past N inside a row that
//     is not B's last);
//   * whole turns of the ring are followed by the remaining steps, and C
//     stores (and the epilogue's reads) are masked to the M x N window.
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

    // !GEN: a persistent workgroup walks the tiles blockIdx.x, blockIdx.x +
    // gridDim.x, ... (gridDim.x a multiple of 8, so under the remap they are all
    // tiles of this workgroup's XCD); GEN: one tile per workgroup.
    const int ntiles = tiles_m * tiles_n;
    int tm, tn;
    tile_coords(blockIdx.x, ntiles, tiles_m, tiles_n, group_m, tm, tn);
    int m0 = tm * SBM, n0 = tn * SBN;

    // A block b: 16 rows of 64 bytes, lane -> row 16b + lane/4, slot lane%4
    // (logical chunk slot ^ swz_af(row)).  B block b: 2 rows of 512 bytes, lane
    // -> row 2b + lane/32, slot lane%32 (logical chunk slot ^ swz_bf(row)).
    uint32_t a_off[SA_BLK], b_off[SB_BLK];
#pragma unroll
    for (int j = 0; j < SA_BLK; ++j) {
        int row, chunk;
        lds::f32_a_dma(wave * SA_BLK + j, lane, row, chunk);
        const int lrow = GEN && m0 + row >= M ? M - 1 - m0 : row;
        a_off[j] = (uint32_t)(lrow * lda + 4 * chunk) * 4u;
    }
    // (GEN: the column, n0 included, is part of the per-lane offset.)
#pragma unroll
    for (int j = 0; j < SB_BLK; ++j) {
        int row, chunk;
        lds::f32_b_dma(wave * SB_BLK + j, lane, row, chunk);
        int col = 4 * chunk;
        if (GEN) col = n0 + col >= N ? ((N - 4) & ~3) : n0 + col;
        b_off[j] = (uint32_t)(row * ldb + col) * 4u;
    }
    auto a_tile = [&](int tile_m) {
        return reinterpret_cast<const char *>(A + (int64_t)tile_m * SBM * lda);
    };
    auto b_tile = [&](int tile_n) { return reinterpret_cast<const char *>(GEN ? B : B + tile_n * SBN); };
    const char *a_cur = a_tile(tm), *b_cur = b_tile(tn);
    // The next tile of this workgroup and its bases (!GEN).  Without one they
    // stay the current tile's: loads past its last step then re-fetch that step
    // into a stage nobody reads any more.
    int next_tile = blockIdx.x + gridDim.x;
    bool has_next = !GEN && next_tile < ntiles;
    int ntm = tm, ntn = tn;
    if (has_next) tile_coords(next_tile, ntiles, tiles_m, tiles_n, group_m, ntm, ntn);
    const char *a_nxt = a_tile(ntm), *b_nxt = b_tile(ntn);
    const int64_t b_step = (int64_t)SBK * ldb * 4;
    // K step s of the tile with bases abase, bbase loads its K block s (GEN:
    // block s - 1; step 0 is the last block).
    auto issue = [&](float *as, float *bs, const char *abase, const char *bbase, int s) {
        const int kt = GEN ? s - 1 : s;
        const char *ab = abase + (int64_t)kt * SBK * 4;
        const char *bb = bbase + kt * b_step;
#pragma unroll
        for (int j = 0; j < SA_BLK; ++j) s_dma16(ab + a_off[j], as + (wave * SA_BLK + j) * 256);
#pragma unroll
        for (int j = 0; j < SB_BLK; ++j) s_dma16(bb + b_off[j], bs + (wave * SB_BLK + j) * 256);
    };

    // Fragments (floats, relative to a stage).  Sub-step s covers k = 8s .. 8s+7;
    // the e-th MFMA of it takes k = 8s + 4*half + e in both operands.
    static_assert(SBK == 16 && SBN == 128, "stage rows of 16 and 128 floats");
    int a_row[SFM];
#pragma unroll
    for (int i = 0; i < SFM; ++i) a_row[i] = wm0 + 32 * i + l32;
    int b_col[SFN];
#pragma unroll
    for (int j = 0; j < SFN; ++j) b_col[j] = wn0 + 32 * j + l32;

    f32x16 total[SFM][SFN], part[SFM][SFN];
#pragma unroll
    for (int i = 0; i < SFM; ++i)
#pragma unroll
        for (int j = 0; j < SFN; ++j) total[i][j] = part[i][j] = f32x16{};

    // Fragments of one 8-wide K sub-step: SFM A reads of 16 bytes and 4 B floats
    // per column tile.
    struct Frags {
        f32x4 a[SFM];
        float b[SFN][4];
    };
    auto load_frags = [&](Frags &f, const float *as, const float *bs, int s) {
        const int c = 2 * s + half;
#pragma unroll
        for (int i = 0; i < SFM; ++i)
            f.a[i] = *reinterpret_cast<const f32x4 *>(as + lds::f32_a_frag(a_row[i], c));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int k = 8 * s + 4 * half + e;
#pragma unroll
            for (int j = 0; j < SFN; ++j) {
                const int n = b_col[j];
                f.b[j][e] = bs[lds::f32_b_elem(k, n)];
            }
        }
    };
    auto mfmas = [&](const Frags &f) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int i = 0; i < SFM; ++i)
#pragma unroll
                for (int j = 0; j < SFN; ++j)
                    part[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(f.b[j][e], f.a[i][e],
                                                                     part[i][j], 0, 0, 0);
    };
    // The partial of a 64-wide K block into the total (after every fourth step).
    auto close_part = [&]() {
#pragma unroll
        for (int i = 0; i < SFM; ++i)
#pragma unroll
            for (int j = 0; j < SFN; ++j) {
                total[i][j] += part[i][j];
                part[i][j] = f32x16{};
            }
    };

    // K step t runs on stage t % 4 with the fragments of its first sub-step
    // already in registers: sub-step 0 multiplies while sub-step 1's fragments
    // are read.  Then: wait for this wave's loads of stage t+1, barrier
    // (everyone's loads of stage t+1 have landed, everyone has finished reading
    // stage t-1), read stage t+1's first fragments and issue the loads of K step
    // t+3 into stage t-1 while sub-step 1 multiplies.  A load has two steps to
    // land.
    constexpr int SUB = SBK / 8;                         // sub-steps per K step (2)
    constexpr int NMF = 4 * SFM * SFN;                   // MFMAs per sub-step (16)
    constexpr int DS = SFM + 2 * SFN;                    // LDS reads per sub-step (B pairs merged)
    constexpr int NBLK = SA_BLK + SB_BLK;                // global->LDS loads per step
    static_assert(SUB == 2, "one sub-step before the barrier");
    static_assert(NMF >= DS + NBLK, "MFMAs to interleave with");
    Frags cur, nxt;
    auto step = [&](auto FIRST, const float *as, const float *bs, const float *nas_read,
                    const float *nbs_read, float *nas_dma, float *nbs_dma, const char *abase,
                    const char *bbase, int next_kt, bool close) {
        load_frags(nxt, as, bs, 1);
        mfmas(cur);
        cur = nxt;
#pragma unroll
        for (int x = 0; x < DS; ++x) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, NMF - DS, 0);
        __builtin_amdgcn_sched_barrier(0);
        // (The first step of a tile after another one waits for everything: the
        // previous tile's stores share the counter with the loads, and the two
        // kinds need not complete in order.)
        if constexpr (FIRST) s_wait_vmcnt<0>();
        else s_wait_vmcnt<(SSTAGES - 3) * NBLK>();
        s_barrier_nf();
        __builtin_amdgcn_sched_barrier(0);
        load_frags(nxt, nas_read, nbs_read, 0);
        issue(nas_dma, nbs_dma, abase, bbase, next_kt);
        mfmas(cur);
        cur = nxt;
#pragma unroll
        for (int x = 0; x < DS; ++x) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
#pragma unroll
        for (int x = 0; x < NBLK; ++x) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, NMF - DS - NBLK, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (close) close_part();
    };

    // Prologue: K steps 0 .. 2 in flight (GEN: step 0 through registers), stage
    // 0 published, its first fragments read.  Indices past the end are clamped:
    // the last steps re-fetch the final K step into stages nobody reads any
    // more, and the last step's look-ahead reads a stage whose contents are not
    // used (identical code in every step).  All loads are drained before the
    // stores.
    const int ktiles = (K + SBK - 1) / SBK;              // !GEN: K / SBK, a multiple of 4
    if constexpr (GEN) {
        // Step 0: the last K block [SBK*(ktiles-1), K) through registers, zero
        // filled, in the swizzled layout the LDS-direct loads produce.
        const int k0 = SBK * (ktiles - 1);
        float *as = s_stage<0>, *bs = s_stage<SSTAGES>;
        constexpr int NT = SNW * 64, NQA = SBM * SBK / 4 / NT, NQB = SBK * SBN / 4 / NT;
        static_assert(NQA * NT * 4 == SBM * SBK && NQB * NT * 4 == SBK * SBN, "whole chunks");
        if (K >= 4) {
            // One 16-byte load inside the matrix per chunk, all in flight before
            // the first wait; zeros past M, N and K applied in registers.
            Masked16 va[NQA], vb[NQB];
#pragma unroll
            for (int i = 0; i < NQA; ++i) {
                const int q = tid + NT * i, r = q >> 2, c = q & 3;
                va[i] = masked16_load<4>(A, lda, m0 + r, M, k0 + 4 * c, K);
            }
#pragma unroll
            for (int i = 0; i < NQB; ++i) {
                const int q = tid + NT * i, r = q >> 5, c = q & 31;
                vb[i] = masked16_load<4>(B, ldb, k0 + r, K, n0 + 4 * c, N);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < NQA; ++i) {
                const int q = tid + NT * i, r = q >> 2, c = q & 3;
                *reinterpret_cast<f32x4 *>(as + lds::f32_a_frag(r, c)) =
                    __builtin_bit_cast(f32x4, masked16_value(va[i]));
            }
#pragma unroll
            for (int i = 0; i < NQB; ++i) {
                const int q = tid + NT * i, r = q >> 5, c = q & 31;
                *reinterpret_cast<f32x4 *>(bs + lds::f32_b_elem(r, 4 * c)) =
                    __builtin_bit_cast(f32x4, masked16_value(vb[i]));
            }
        } else {
            // K < 4: element by element.
            for (int q = tid; q < SBM * SBK / 4; q += NT) {
                const int r = q >> 2, c = q & 3;
                const int gm = m0 + r, gk = k0 + 4 * c;
                f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
                if (gm < M) {
                    const float *src = A + (int64_t)gm * lda + gk;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (gk + e < K) v[e] = src[e];
                }
                *reinterpret_cast<f32x4 *>(as + lds::f32_a_frag(r, c)) = v;
            }
            for (int q = tid; q < SBK * SBN / 4; q += NT) {
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
                *reinterpret_cast<f32x4 *>(bs + lds::f32_b_elem(r, 4 * c)) = v;
            }
        }
    }
    // (GEN: steps past the last one re-load the last full block, K > SBK.)
    s_unroll<SSTAGES - 1>([&](auto S) {
        if (!GEN || S > 0)
            issue(s_stage<S>, s_stage<SSTAGES + S>, a_cur, b_cur,
                  !GEN || S < ktiles ? (int)S : ktiles - 1);
    });
    // GEN: stage 0 came through registers (its global loads were waited for
    // before the LDS writes); the writes must land before the barrier.
    if constexpr (GEN) __builtin_amdgcn_s_waitcnt(0xc07f);      // lgkmcnt(0)
    s_wait_vmcnt<(SSTAGES - 2) * NBLK>();
    s_barrier_nf();
    load_frags(cur, s_stage<0>, s_stage<SSTAGES>, 0);
    // Whole turns of the ring without conditions (a step skipped at run time
    // would let the compiler merge the steps' code and lose track of which
    // stage array each LDS read addresses).  Steps past the tile's last one
    // load the next tile's first steps.  GEN: the remaining ktiles % 4 steps
    // follow, once, and their partial is added at the end.
    auto ring_step = [&](auto S, int kt, auto FIRST) {
        constexpr int N1 = (S + 1) % SSTAGES;          // next stage (read ahead)
        constexpr int NS = (S + SSTAGES - 1) % SSTAGES; // stage to refill
        const int next = kt + S + SSTAGES - 1;
        const bool wrap = next >= ktiles;
        const int lkt = !wrap ? next : has_next ? next - ktiles : ktiles - 1;
        step(FIRST, s_stage<S>, s_stage<SSTAGES + S>, s_stage<N1>, s_stage<SSTAGES + N1>,
             s_stage<NS>, s_stage<SSTAGES + NS>, wrap ? a_nxt : a_cur, wrap ? b_nxt : b_cur, lkt,
             S == SSTAGES - 1);
    };
    const std::integral_constant<bool, false> plain{};

    // lane holds C[m][n..n+3], n = 8g + 4*half (+ tile offsets): one 16-byte store
    auto store_tile = [&]() {
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
                    float ev[4] = {total[i][j][4 * g], total[i][j][4 * g + 1],
                                   total[i][j][4 * g + 2], total[i][j][4 * g + 3]};
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
    };

    if constexpr (GEN) {
        const int kwhole = ktiles - ktiles % SSTAGES;
        for (int kt = 0; kt < kwhole; kt += SSTAGES)
            s_unroll<SSTAGES>([&](auto S) { ring_step(S, kt, plain); });
        const int rem = ktiles - kwhole;
        s_unroll<SSTAGES - 1>([&](auto S) {
            if (S < rem) ring_step(S, kwhole, plain);
        });
        if (rem > 0) close_part();
        s_wait_vmcnt<0>();
        store_tile();
    } else {
        for (bool first = true;; first = false) {
            // The first turn of a tile after another one starts with a full wait.
            if (first) {
                s_unroll<SSTAGES>([&](auto S) { ring_step(S, 0, plain); });
            } else {
                s_unroll<SSTAGES>([&](auto S) {
                    ring_step(S, 0, std::integral_constant<bool, S == 0>{});
                });
            }
            for (int kt = SSTAGES; kt < ktiles; kt += SSTAGES)
                s_unroll<SSTAGES>([&](auto S) { ring_step(S, kt, plain); });
            store_tile();
            if (!has_next) break;
#pragma unroll
            for (int i = 0; i < SFM; ++i)
#pragma unroll
                for (int j = 0; j < SFN; ++j) total[i][j] = f32x16{};
            tm = ntm, tn = ntn;
            m0 = tm * SBM, n0 = tn * SBN;
            a_cur = a_nxt, b_cur = b_nxt;
            next_tile += gridDim.x;
            has_next = next_tile < ntiles;
            if (has_next) {
                tile_coords(next_tile, ntiles, tiles_m, tiles_n, group_m, ntm, ntn);
                a_nxt = a_tile(ntm), b_nxt = b_tile(ntn);
            }
        }
        s_wait_vmcnt<0>();
    }
}

}  // namespace

bool f32_fast_eligible(const Problem &p)
{
    return p.aligned && p.M % SBM == 0 && p.N % SBN == 0 && p.K % (SBK * SSTAGES) == 0 &&
           p.lda < (1 << 22) && p.ldb < (1 << 22);
}

// The guarded instantiation: any M, N >= 4 (a clamped column chunk starts at
// N - 4 rounded down to a multiple of 4), two K blocks at least, and per-lane 32-bit byte offsets that fit.
bool f32_general_eligible(const Problem &p)
{
    return p.M >= 1 && p.N >= 4 && p.K > SBK && p.lda < (1 << 22) &&
           (int64_t)SBK * p.ldb + p.N < ((int64_t)1 << 30);
}

// GEN: one workgroup per tile; whole tiles: min(tiles, 2 per CU) persistent
// workgroups (a multiple of 8 when it is the CU bound).
template <bool GEN>
static hipError_t f32_fast_typed(const Problem &p, int cus)
{
    const int tiles_m = (p.M + SBM - 1) / SBM, tiles_n = (p.N + SBN - 1) / SBN;
    const int64_t ntiles = (int64_t)tiles_m * tiles_n;
    if (ntiles > 0x7fffffff) return hipErrorInvalidValue;
    const int64_t slots = (int64_t)2 * (cus > 0 ? cus : 256) / 8 * 8;
    const int64_t nwg = GEN || ntiles <= slots ? ntiles : slots;
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

hipError_t f32_fast_launch(const Problem &p, int cus)
{
    if (!f32_fast_eligible(p)) return hipErrorInvalidValue;
    return f32_fast_typed<false>(p, cus);
}

hipError_t f32_general_launch(const Problem &p)
{
    if (!f32_general_eligible(p)) return hipErrorInvalidValue;
    return f32_fast_typed<true>(p, 0);
}

}  // namespace gemm
