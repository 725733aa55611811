// fp16 / bf16 GEMM, large-tile path for gfx950 (whole 256 x 256 tiles, K a
// multiple of BK * STAGES, 16-byte aligned operands; 128 x 128 tiles of the same
// design for medium grids, two workgroups per CU).
//
// Same product as gemm_h16.hip; what changes is how operands travel:
//   * global -> LDS with global_load_lds_dwordx4: each lane's 16 bytes land at
//     LDS base + 16*lane without passing through registers.  The XOR swizzle of
//     the 16-byte chunks is applied by choosing which global chunk each lane
//     fetches, so the LDS writes stay contiguous;
//   * B stays in LDS as rows of k (n contiguous, exactly as in memory) and the
//     MFMA operand "8 consecutive k of one column" is produced by the LDS
//     transposing read ds_read_b64_tr_b16: within each 16-lane group, lanes
//     4r..4r+3 address 16 consecutive n of row r and lane j receives element j of
//     each of the 4 rows;
//   * 4 waves (one per SIMD), each owning a 128 x 128 sub-tile as 4 x 4 MFMA
//     32x32x16 tiles (256 fp32 accumulators per lane), which halves the LDS
//     bytes read per MFMA compared with 64-column wave tiles (128 x 128 tiles:
//     64 x 64 sub-tiles, and half the LDS, so two workgroups share a CU);
//   * a ring of STAGES LDS stages, one separate array per stage and stage
//     indices known at compile time, so the compiler can tell that loads into
//     one stage do not alias reads of another and does not serialise them.  The
//     loads for K step t + STAGES - 1 are issued at step t: a global load has
//     STAGES - 1 steps to land.  Each wave waits for its own loads of the
//     current stage and a barrier publishes the stage to all waves.
// "[CUDA 优化实战] hgemm - 超越 cuBLAS" sections 1-4 describe the same stages
// (asynchronous 16-byte copies, swizzled shared memory, double buffering,
// transposing fragment loads) for a different machine.
#include <type_traits>
#include <utility>

#include "gemm_device.hpp"
#include "gemm_launch.hpp"
#include "gemm_lds_layout.hpp"

namespace gemm {

namespace {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;

constexpr int FAST_BK = 32, FAST_STAGES = 4;
constexpr int FAST_WM = 2, FAST_WN = 2;                  // waves along M and N

// One LDS array per (stage, operand): distinct objects for alias analysis.
template <int TAG, int HALVES>
__shared__ __attribute__((aligned(1024))) uint16_t lds_stage[HALVES];

// The XOR swizzles of the stages and the lane -> address maps of every LDS
// access below are in gemm_lds_layout.hpp (checked on the host for banks).
using lds::swz_a;
using lds::swz_b;

__device__ __forceinline__ void dma16(const void *src, uint16_t *lds_block)
{
    __builtin_amdgcn_global_load_lds(src, (lds_void_t *)lds_block, 16, 0, 0);
}
// Whole tiles load through buffer descriptors: the step's base in scalar
// registers and the lane's 32-bit offset in a vector register, so the loop
// spends no vector instructions on 64-bit load addresses (4096^3: 103.9 ->
// 102.4 us).  `reach` bounds the bytes a tile may touch from the base (an
// offset past it reads zeros).  The 4th descriptor word 0x00020000 is the raw
// 32-bit data format of gfx9.  The guarded instantiations use them for each
// operand whose rows start on 4-byte boundaries and dma16 otherwise: buffer
// LDS-direct loads at offsets that are not 4-byte aligned were measured to
// return wrong data.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t h_rsrc(const void *base, int reach)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, reach, 0x00020000);
}
__device__ __forceinline__ void bdma16(__amdgpu_buffer_rsrc_t r, uint32_t off, uint16_t *lds_block)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)lds_block, 16, (int)off, 0, 0, 0);
}

// s_waitcnt vmcnt(N) (N < 64), leaving expcnt and lgkmcnt alone.
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier without the release/acquire fences of __syncthreads(): those
// would wait for every outstanding global->LDS load (vmcnt(0)) and collapse the
// ring to one stage in flight.  Callers wait for exactly the loads they need
// first; the "memory" clobber keeps the compiler from moving memory accesses
// across the barrier.  LDS reads issued before it have all been consumed by
// MFMAs already, so no stage is overwritten while still being read.
__device__ __forceinline__ void barrier_no_fence() { asm volatile("s_barrier" ::: "memory"); }

template <typename F, int... I>
__device__ __forceinline__ void unroll_impl(F &&f, std::integer_sequence<int, I...>)
{
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void unroll(F &&f)
{
    unroll_impl(f, std::make_integer_sequence<int, N>{});
}

// The ring array with index idx (stages of A first, then of B).
template <int HALVES>
__device__ __forceinline__ uint16_t *ring_array(int idx)
{
    switch (idx) {
    case 0: return lds_stage<0, HALVES>;
    case 1: return lds_stage<1, HALVES>;
    case 2: return lds_stage<2, HALVES>;
    case 3: return lds_stage<3, HALVES>;
    case 4: return lds_stage<4, HALVES>;
    case 5: return lds_stage<5, HALVES>;
    case 6: return lds_stage<6, HALVES>;
    default: return lds_stage<7, HALVES>;
    }
}

// The B-stage ring array with index idx (B stages follow the STAGES A stages;
// naming only these keeps the A stages of wider tiles at their own size).
template <int HALVES, int STAGES>
__device__ __forceinline__ uint16_t *b_ring_array(int idx)
{
    static_assert(STAGES == 4, "four B stages");
    switch (idx) {
    case 0: return lds_stage<STAGES + 0, HALVES>;
    case 1: return lds_stage<STAGES + 1, HALVES>;
    case 2: return lds_stage<STAGES + 2, HALVES>;
    default: return lds_stage<STAGES + 3, HALVES>;
    }
}

// TBM x TBN: tile rows and columns (256 x 256, 128 x 128 or 128 x 256).
// GEN = false: whole TB x TB tiles, K a multiple of BK * STAGES, 16-byte
// aligned operands.  GEN = true: any M, N >= 8, K > BK and any leading
// dimensions (the hardware runs in unaligned-access mode, so 16-byte loads and
// stores at 2-byte-aligned addresses are legal):
//   * the last K block (possibly partial) is done first, loaded through
//     registers with zero fill, so every LDS-direct block is a full one that
//     never touches B's last row;
//   * A rows past M are clamped to row M-1 and B column chunks starting past N
//     to the last whole chunk at a multiple of 8 columns (their products only
//     reach C entries that are not stored; the clamped loads stay 16-byte
//     aligned when B's rows are); a chunk straddling N reads a few elements
//     past N inside a row
//     that is not B's last, i.e. inside the operand;
//   * steps are guarded when the number of K steps is not a multiple of the
//     ring depth, and C stores are masked to the M x N window.
//
// EPI: the fused epilogue is applied to the fp32 accumulators before they are
// rounded (each lane reads the bias and, for beta != 0, the prior C of the
// entries it holds; it never stores them itself, but the store of an entry
// depends through LDS on the value this read produced).
template <bool IS_BF16, int BK, int STAGES, int WM, int WN, bool GEN, bool EPI, int TBM, int TBN,
          int BUF>
__global__ void __launch_bounds__(WM * WN * 64) __attribute__((amdgpu_waves_per_eu(
    TBM * TBN == 128 * 128 ? 2 : WM * WN / 4, TBM * TBN == 128 * 128 ? 2 : WM * WN / 4)))
h16_fast_kernel(const uint16_t *__restrict__ A, const uint16_t *__restrict__ B,
                uint16_t *__restrict__ C, int M, int N, int K, int64_t lda, int64_t ldb,
                int64_t ldc, int tiles_m, int tiles_n, int group_m, Epilogue epi)
{
    constexpr int FBM = TBM, FBN = TBN;
    constexpr int FNW = WM * WN;
    constexpr int FWTM = FBM / WM, FWTN = FBN / WN;      // wave sub-tile
    constexpr int FFM = FWTM / 32, FFN = FWTN / 32;      // MFMA tiles per wave
    constexpr int A_STAGE = FBM * BK;                    // halves per stage
    constexpr int B_STAGE = BK * FBN;
    constexpr int CPR = BK / 8;                          // 16-byte chunks per A row
    constexpr int A_BLK = A_STAGE * 2 / 1024 / FNW;      // 1 KiB loads per wave per stage
    constexpr int B_BLK = B_STAGE * 2 / 1024 / FNW;
    constexpr int SUB = BK / 16;                         // MFMA K sub-steps per stage
    static_assert(A_BLK >= 1 && B_BLK >= 1 && SUB >= 2, "stage shape");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm0 = (wave / WN) * FWTM;
    const int wn0 = (wave % WN) * FWTN;
    const int l32 = lane & 31, half = lane >> 5;

    int tm, tn;
    tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * FBM, n0 = tn * FBN;

    // ---- per-lane sources of this wave's 1 KiB loads: a wave-uniform base
    // (this tile's first row of A / first column of B at K step kt) plus a
    // 32-bit byte offset per lane and load.
    // A block b: lane -> row (1024 / (2 BK)) b + lane/CPR, slot lane%CPR,
    // which holds logical chunk slot ^ swz_a(row) (lds::h16_a_dma).
    uint32_t a_off[A_BLK];
#pragma unroll
    for (int j = 0; j < A_BLK; ++j) {
        int row, chunk;
        lds::h16_a_dma<BK>(wave * A_BLK + j, lane, row, chunk);
        const int lrow = GEN && m0 + row >= M ? M - 1 - m0 : row;
        a_off[j] = (uint32_t)(lrow * lda + 8 * chunk) * 2u;
    }
    // B block b (rows of FBN halves, BCPR = FBN / 8 chunks each: 2 rows of 512
    // bytes, or 4 of 256): lane -> row (64 / BCPR) b + lane/BCPR, slot
    // lane%BCPR (lds::h16_b_dma).  For GEN the column (including n0) is part of
    // the per-lane offset.
    uint32_t b_off_g[B_BLK];
#pragma unroll
    for (int j = 0; j < B_BLK; ++j) {
        int row, chunk;
        lds::h16_b_dma<FBN>(wave * B_BLK + j, lane, row, chunk);
        int col = 8 * chunk;
        if (GEN) col = n0 + col >= N ? ((N - 8) & ~7) : n0 + col;
        b_off_g[j] = (uint32_t)(row * ldb + col) * 2u;
    }
    const char *a_base = reinterpret_cast<const char *>(A + (int64_t)m0 * lda);
    const char *b_base = reinterpret_cast<const char *>(GEN ? B : B + n0);
    const int64_t a_step = (int64_t)BK * 2, b_step = (int64_t)BK * ldb * 2;

    // Step s loads K block s (GEN: block s-1; step 0 is the last block, below).
    // (below 2^31 under the whole-tile limits lda, ldb < 2^22)
    const int a_reach = (int)(FBM * lda * 2), b_reach = (int)(BK * ldb * 2);
    auto issue = [&](uint16_t *as, uint16_t *bs, int s) {
        const int kb = GEN ? s - 1 : s;
        const char *ab = a_base + kb * a_step;
        const char *bb = b_base + kb * b_step;
        if constexpr (GEN) {
            // Each operand through a buffer descriptor when its rows start on
            // 4-byte boundaries (BUF bit 0: A, bit 1: B), else global loads.
            if constexpr (BUF & 1) {
                const __amdgpu_buffer_rsrc_t ra = h_rsrc(ab, a_reach);
#pragma unroll
                for (int j = 0; j < A_BLK; ++j) bdma16(ra, a_off[j], as + (wave * A_BLK + j) * 512);
            } else {
#pragma unroll
                for (int j = 0; j < A_BLK; ++j) dma16(ab + a_off[j], as + (wave * A_BLK + j) * 512);
            }
            if constexpr (BUF & 2) {
                const __amdgpu_buffer_rsrc_t rb = h_rsrc(bb, b_reach);
#pragma unroll
                for (int j = 0; j < B_BLK; ++j) bdma16(rb, b_off_g[j], bs + (wave * B_BLK + j) * 512);
            } else {
#pragma unroll
                for (int j = 0; j < B_BLK; ++j) dma16(bb + b_off_g[j], bs + (wave * B_BLK + j) * 512);
            }
        } else {
            const __amdgpu_buffer_rsrc_t ra = h_rsrc(ab, a_reach), rb = h_rsrc(bb, b_reach);
#pragma unroll
            for (int j = 0; j < A_BLK; ++j) bdma16(ra, a_off[j], as + (wave * A_BLK + j) * 512);
#pragma unroll
            for (int j = 0; j < B_BLK; ++j) bdma16(rb, b_off_g[j], bs + (wave * B_BLK + j) * 512);
        }
    };

    // ---- fragment addressing (in halves, relative to a stage)
    // A: lane reads row wm0 + 32i + l32, logical chunk 2s + half.
    int a_row[FFM];
#pragma unroll
    for (int i = 0; i < FFM; ++i) a_row[i] = wm0 + 32 * i + l32;
    // B: 16-lane group g, lane w in it: row r = w/4 of the 4 rows read, column
    // piece 4*(w%4); groups 0/1 take columns 0-15 / 16-31 of the 32-wide tile,
    // groups 0,1 / 2,3 take k 0-7 / 8-15 of the 16-wide step.
    const int g = lane >> 4, w16 = lane & 15, r4 = w16 >> 2, c4 = w16 & 3;
    int b_off[FFN];
#pragma unroll
    for (int j = 0; j < FFN; ++j) {
        const int n = wn0 + 32 * j + 16 * (g & 1) + 4 * c4;
        b_off[j] = lds::h16_b_col(r4, n);     // rows 16 s + b_krow (+4) share r4 = k % 4
    }
    const int b_krow = 8 * (g >> 1) + r4;    // + 16 s + 4 q

    f32x16 acc[FFM][FFN];
#pragma unroll
    for (int i = 0; i < FFM; ++i)
#pragma unroll
        for (int j = 0; j < FFN; ++j) acc[i][j] = f32x16{};

    // Fragments of one 16-wide K sub-step: 4 A tiles (ds_read_b128) and 4 B
    // tiles (two transposing reads each).
    struct Frags {
        u32x4 a[FFM], b[FFN];
    };
    auto load_frags = [&](Frags &f, const uint16_t *as, const uint16_t *bs, int s) {
        const int c = 2 * s + half;
#pragma unroll
        for (int i = 0; i < FFM; ++i)
            f.a[i] = *reinterpret_cast<const u32x4 *>(as + lds::h16_a_frag<BK>(a_row[i], c));
#pragma unroll
        for (int j = 0; j < FFN; ++j) {
            const uint16_t *p0 = bs + (16 * s + b_krow) * FBN + b_off[j];
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)p0);
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(p0 + 4 * FBN));
            const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
            f.b[j] = u32x4{l2[0], l2[1], h2[0], h2[1]};
        }
    };
    auto mfmas = [&](const Frags &f) {
#pragma unroll
        for (int i = 0; i < FFM; ++i)
#pragma unroll
            for (int j = 0; j < FFN; ++j)
                acc[i][j] = mfma32x32x16<IS_BF16>(f.b[j], f.a[i], acc[i][j]);
    };

    // K step t runs on stage t % STAGES with the fragments of its first
    // sub-step already in registers.  Sub-steps 0 .. SUB-2 multiply while the
    // following sub-step's fragments are read.  Then, before the last sub-step:
    // wait for this wave's loads of stage t+1, barrier (everyone's loads of stage
    // t+1 have landed, everyone has finished reading stage t-1), read stage
    // t+1's first fragments and issue the global->LDS loads of K step
    // t + STAGES - 1 into stage t-1 while the last sub-step multiplies.  A load
    // therefore has STAGES - 2 steps to land, and the LDS latency of a step's
    // first fragments hides behind the previous step's last MFMAs.
    constexpr int NBLK = A_BLK + B_BLK;
    constexpr int DS = 2 * FFN + FFM;                   // LDS reads per sub-step (12)
    static_assert(STAGES >= 3, "ring depth");
    Frags cur, nxt;
    // WAIT: loads of this wave allowed to stay in flight at the wait (the ones
    // issued after the stage the next step reads).  ISSUE: this step loads K
    // step next_kt.  LAST: the final step, with nothing left to wait for,
    // publish or read ahead.
    auto step = [&](auto wait_c, auto issue_c, auto last_c, const uint16_t *as,
                    const uint16_t *bs, const uint16_t *nas_read, const uint16_t *nbs_read,
                    uint16_t *nas_dma, uint16_t *nbs_dma, int next_kt) {
        constexpr int WAIT = decltype(wait_c)::value;
        constexpr bool ISSUE = decltype(issue_c)::value, LAST = decltype(last_c)::value;
#pragma unroll
        for (int s = 0; s + 1 < SUB; ++s) {
            load_frags(nxt, as, bs, s + 1);
            mfmas(cur);
            cur = nxt;
#pragma unroll
            for (int x = 0; x < DS / 2; ++x) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, FFM * FFN - DS / 2, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (!LAST) {
            wait_vmcnt<WAIT>();
            barrier_no_fence();
            __builtin_amdgcn_sched_barrier(0);
            load_frags(nxt, nas_read, nbs_read, 0);
            if constexpr (ISSUE) issue(nas_dma, nbs_dma, next_kt);
        }
        mfmas(cur);
        constexpr int MF = FFM * FFN;                    // MFMAs per sub-step
        if constexpr (!LAST) cur = nxt;
        if constexpr (!LAST && ISSUE && MF >= DS && MF >= NBLK) {
            // One fragment read after each of the first DS MFMAs and the NBLK
            // loads spread evenly over all of them: issued in a burst, the loads
            // of the four waves overfill the texture unit's address queue and the
            // waves stall on them (SQ_VMEM_TA_CMD_FIFO_FULL 4.7M -> 1.0M,
            // 4096^3 104.5 -> 103.0 us, 4097 x 4095 x 4100 139.0 -> 135.4 us).
#pragma unroll
            for (int x = 0; x < MF; ++x) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (x < DS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                if ((x * NBLK) % MF < NBLK) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            }
        } else {
            if constexpr (!LAST) {
#pragma unroll
                for (int x = 0; x < DS / 2; ++x) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                }
            }
            if constexpr (ISSUE && MF >= DS / 2 + NBLK) {
#pragma unroll
                for (int x = 0; x < NBLK; ++x) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, MF - DS / 2 - NBLK, 0);
            } else if constexpr (ISSUE) {
                // (64 x 64 sub-tiles: too few MFMAs to pair each load with one.)
                static_assert(MF > DS / 2, "MFMAs to interleave with");
                __builtin_amdgcn_sched_group_barrier(0x020, NBLK, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, MF - DS / 2, 0);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    using std::integral_constant;
    using steady_wait = integral_constant<int, (STAGES - 3) * NBLK>;
    using yes = std::true_type;
    using no = std::false_type;

    // Prologue: K steps 0 .. STAGES-2 in flight, stage 0 published, its first
    // fragments read.  Step kt + S issues K step kt + S + STAGES - 1 into the
    // stage step kt + S - 1 used.  Indices past the end are clamped: the last
    // steps re-fetch the final K tile into stages nobody reads any more, and the
    // last step's look-ahead reads a stage whose contents are not used
    // (identical code in every step).  All loads are drained before the epilogue.
    // GEN: step 0 is the last K block [BK*(ktiles-1), K), through registers
    // with zero fill, in the same swizzled layout the LDS-direct loads produce.
    const int ktiles = (K + BK - 1) / BK;   // !GEN: K / BK, a multiple of STAGES
    if constexpr (GEN) {
        const int k0 = BK * (ktiles - 1);
        uint16_t *as = lds_stage<0, A_STAGE>, *bs = lds_stage<STAGES, B_STAGE>;
        constexpr int NT = FNW * 64;
        constexpr int NQA = A_STAGE / 8 / NT, NQB = B_STAGE / 8 / NT;   // chunks per thread
        static_assert(NQA * NT * 8 == A_STAGE && NQB * NT * 8 == B_STAGE, "whole chunks");
        if (K >= 8) {
            // Every chunk one 16-byte load inside the matrix, all issued before
            // the first wait; the zeros past M, N and K applied in registers.
            Masked16 va[NQA], vb[NQB];
#pragma unroll
            for (int i = 0; i < NQA; ++i) {
                const int q = tid + NT * i, r = q / CPR, c = q % CPR;
                va[i] = masked16_load<2>(A, lda, m0 + r, M, k0 + 8 * c, K);
            }
#pragma unroll
            for (int i = 0; i < NQB; ++i) {
                const int q = tid + NT * i, r = q / (FBN / 8), c = q % (FBN / 8);
                vb[i] = masked16_load<2>(B, ldb, k0 + r, K, n0 + 8 * c, N);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < NQA; ++i) {
                const int q = tid + NT * i, r = q / CPR, c = q % CPR;
                *reinterpret_cast<u32x4 *>(as + lds::h16_a_frag<BK>(r, c)) = masked16_value(va[i]);
            }
#pragma unroll
            for (int i = 0; i < NQB; ++i) {
                const int q = tid + NT * i, r = q / (FBN / 8), c = q % (FBN / 8);
                *reinterpret_cast<u32x4 *>(bs + r * FBN + lds::h16_b_col(r, 8 * c)) =
                    masked16_value(vb[i]);
            }
        } else {
            // K < 8: element by element.
#pragma unroll
            for (int q = tid; q < A_STAGE / 8; q += NT) {
                const int r = q / CPR, c = q % CPR;
                const int gm = m0 + r, gk = k0 + 8 * c;
                uint32_t w[4] = {0, 0, 0, 0};
                if (gm < M) {
                    const uint16_t *src = A + (int64_t)gm * lda + gk;
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (gk + e < K) w[e >> 1] |= (uint32_t)src[e] << (16 * (e & 1));
                }
                *reinterpret_cast<u32x4 *>(as + lds::h16_a_frag<BK>(r, c)) = u32x4{w[0], w[1], w[2], w[3]};
            }
#pragma unroll
            for (int q = tid; q < B_STAGE / 8; q += NT) {
                const int r = q / (FBN / 8), c = q % (FBN / 8);
                const int gk = k0 + r, gn = n0 + 8 * c;
                uint32_t w[4] = {0, 0, 0, 0};
                if (gk < K) {
                    const uint16_t *src = B + (int64_t)gk * ldb + gn;
                    if (gn + 8 <= N) {
                        const u32x4 v = *reinterpret_cast<const u32x4 *>(src);
                        w[0] = v[0], w[1] = v[1], w[2] = v[2], w[3] = v[3];
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            if (gn + e < N) w[e >> 1] |= (uint32_t)src[e] << (16 * (e & 1));
                    }
                }
                *reinterpret_cast<u32x4 *>(bs + r * FBN + lds::h16_b_col(r, 8 * c)) =
                    u32x4{w[0], w[1], w[2], w[3]};
            }
        }
    }
    // (GEN: steps past the last one re-load the last full block, K > BK.)
    unroll<STAGES - 1>([&](auto S) {
        if (!GEN || S > 0)
            issue(lds_stage<S, A_STAGE>, lds_stage<STAGES + S, B_STAGE>,
                  !GEN || S < ktiles ? (int)S : ktiles - 1);
    });
    // GEN: stage 0 came through registers (its global loads were waited for
    // before the LDS writes); the writes must land before the barrier.
    if constexpr (GEN) __builtin_amdgcn_s_waitcnt(0xc07f);      // lgkmcnt(0)
    wait_vmcnt<(STAGES - 2) * NBLK>();
    barrier_no_fence();
    load_frags(cur, lds_stage<0, A_STAGE>, lds_stage<STAGES, B_STAGE>, 0);
    // Whole turns of the ring without conditions: a step skipped at run time
    // would let the compiler merge the steps' code, lose track of which stage
    // array each LDS read addresses and wait for every outstanding load before
    // it.  GEN: the remaining ktiles % STAGES steps follow, once.
    auto ring_step = [&](auto S, int kt, auto wait_c, auto issue_c, auto last_c) {
        constexpr int N1 = (S + 1) % STAGES;           // next stage (read ahead)
        constexpr int NS = (S + STAGES - 1) % STAGES;  // stage to refill
        const int next = kt + S + STAGES - 1;
        step(wait_c, issue_c, last_c, lds_stage<S, A_STAGE>, lds_stage<STAGES + S, B_STAGE>,
             lds_stage<N1, A_STAGE>, lds_stage<STAGES + N1, B_STAGE>,
             lds_stage<NS, A_STAGE>, lds_stage<STAGES + NS, B_STAGE>,
             next < ktiles ? next : ktiles - 1);
    };
    if constexpr (!GEN) {
        // Whole turns, then the last turn peeled: only its first step has a K
        // step left to load, the waits shrink to what is still in flight, and
        // the final step neither waits, publishes nor reads ahead, so the
        // epilogue starts as soon as the last MFMAs are issued.
        for (int kt = 0; kt < ktiles - STAGES; kt += STAGES)
            unroll<STAGES>([&](auto S) { ring_step(S, kt, steady_wait{}, yes{}, no{}); });
        const int kt = ktiles - STAGES;
        static_assert(STAGES == 4, "peeled last turn of a 4-stage ring");
        ring_step(integral_constant<int, 0>{}, kt, steady_wait{}, yes{}, no{});
        ring_step(integral_constant<int, 1>{}, kt, integral_constant<int, NBLK>{}, no{}, no{});
        ring_step(integral_constant<int, 2>{}, kt, integral_constant<int, 0>{}, no{}, no{});
        ring_step(integral_constant<int, 3>{}, kt, integral_constant<int, 0>{}, no{}, yes{});
    } else {
        const int kwhole = ktiles - ktiles % STAGES;
        for (int kt = 0; kt < kwhole; kt += STAGES)
            unroll<STAGES>([&](auto S) { ring_step(S, kt, steady_wait{}, yes{}, no{}); });
        const int rem = ktiles - kwhole;
        unroll<STAGES - 1>([&](auto S) {
            if (S < rem) ring_step(S, kwhole, steady_wait{}, yes{}, no{});
        });
    }
    wait_vmcnt<0>();

    // ---- epilogue through LDS (the ring is idle now): each wave converts its
    // sub-tile to 16-bit and writes it to its own ring arrays, then stores
    // whole row segments of the sub-tile with 16 bytes per lane.  Lane l holds
    // C[32i + l%32][32j + 8q + 4*(l/32) .. +3]: 8 bytes in 16-byte chunk 4j + q,
    // half l/32.  Chunks are XORed with the row modulo the chunks per row and the
    // half with row bit 3 (lds::h16_epi_write), so the 16 rows one write cycle
    // touches spread over the banks.  (Flipping it with the row bit above the
    // chunk count, as before, left 256-byte rows with chunks c and c + 8 on
    // the same banks: 256 conflict cycles per wave, all of the kernel's.)
    // Square tiles stage in the A and B arrays alike; wider tiles (B stages
    // larger than A stages) in the B arrays only, one per wave.
    constexpr int SQ = A_STAGE == B_STAGE;
    constexpr int ARR_SZ = SQ ? A_STAGE : B_STAGE;       // halves per staging array
    static_assert(2 * STAGES == 8 && (SQ || (B_STAGE > A_STAGE && FNW <= STAGES)),
                  "epilogue staging");
    constexpr int ARR = FWTM * FWTN / ARR_SZ;            // ring arrays per wave
    constexpr int ROWS_PER_ARR = ARR_SZ / FWTN;
    constexpr int CPRC = FWTN / 8;                       // 16-byte chunks per staged row
    constexpr int RPI = 1024 / (FWTN * 2);               // rows per 1 KiB store
    static_assert(ARR >= 1 && ARR * FNW <= (SQ ? 8 : STAGES), "staging space");
    __builtin_amdgcn_s_waitcnt(0xc07f);                  // lgkmcnt(0): own LDS reads done
    barrier_no_fence();                                  // every wave is done with the ring
    uint16_t *st[ARR];
#pragma unroll
    for (int a = 0; a < ARR; ++a) {
        if constexpr (SQ) st[a] = ring_array<ARR_SZ>(wave * ARR + a);
        else st[a] = b_ring_array<ARR_SZ, STAGES>(wave * ARR + a);
    }
    // EPI, whole tiles: the bias of this lane's columns, loaded once for all
    // its rows.  Column offsets are multiples of 4, so whether the 16-byte bias
    // loads and 8-byte prior loads are aligned is a property of the kernel's
    // arguments, decided once.
    [[maybe_unused]] float ebias[EPI && !GEN ? FFN : 1][4][4];
    [[maybe_unused]] const bool prior_on = EPI && !GEN && epi.beta != 0.f;
    [[maybe_unused]] const bool prior_vec = ((uintptr_t)C & 7) == 0 && (ldc & 3) == 0;
    if constexpr (EPI && !GEN) {
        const bool bias_vec = epi.bias && ((uintptr_t)epi.bias & 15) == 0;
#pragma unroll
        for (int j = 0; j < FFN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                epilogue_bias_whole<4>(epi, n0 + wn0 + 32 * j + 8 * q + 4 * half, bias_vec,
                                       ebias[j][q]);
    }
    // The rows, as one body per combination of the two uniform epilogue
    // switches (prior C read, relu), so that no entry branches on them.
    auto stage_rows = [&](auto PRIOR, auto RELU) {
#pragma unroll
        for (int i = 0; i < FFM; ++i) {
            const int row = 32 * i + l32;
            uint16_t *buf = st[row / ROWS_PER_ARR] + (row % ROWS_PER_ARR) * FWTN;
            [[maybe_unused]] const int gm = m0 + wm0 + row;
            [[maybe_unused]] const uint16_t *crow = C + (int64_t)gm * ldc;
            // EPI, whole tiles: the prior C of half the row's entries first
            // (all their loads in flight at once), then their arithmetic, then
            // the other half (the whole row at once spilled registers in the
            // fp16 instantiation).  The guarded variant, shorter of registers,
            // takes each group of 4 entries on its own.
            constexpr int JH = FFN > 1 ? FFN / 2 : 1;    // column tiles per half
#pragma unroll
            for (int h0 = 0; h0 < FFN; h0 += JH) {
            [[maybe_unused]] float prior[EPI && !GEN && PRIOR ? JH : 1][4][4];
            if constexpr (EPI && !GEN && PRIOR) {
#pragma unroll
                for (int jj = 0; jj < JH; ++jj)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        epilogue_prior_whole<IS_BF16 ? OUT_BF16 : OUT_F16, 4>(
                            crow, n0 + wn0 + 32 * (h0 + jj) + 8 * q + 4 * half, prior_vec,
                            prior[jj][q]);
            }
#pragma unroll
            for (int jj = 0; jj < JH; ++jj)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int j = h0 + jj;
                    float v[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                  acc[i][j][4 * q + 3]};
                    if constexpr (EPI && GEN) {
                        const int gn = n0 + wn0 + 32 * j + 8 * q + 4 * half;
                        if (gm < M)
                            epilogue_row<IS_BF16 ? OUT_BF16 : OUT_F16, 4>(epi, v, crow, gn, N - gn);
                    } else if constexpr (EPI) {
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            if constexpr (PRIOR)
                                v[t] = epilogue_value(epi, v[t], ebias[j][q][t], prior[jj][q][t]);
                            else
                                v[t] = epilogue_value(epi, v[t], ebias[j][q][t]);
                            if constexpr (RELU) v[t] = epilogue_relu(v[t]);
                        }
                    }
                    *reinterpret_cast<u32x2 *>(buf + lds::h16_epi_write<CPRC>(row, 4 * j + q, half)) =
                        u32x2{pack2<IS_BF16>(v[0], v[1]), pack2<IS_BF16>(v[2], v[3])};
                }
            }
        }
    };
    if constexpr (EPI && !GEN) {
        if (prior_on) {
            if (epi.relu) stage_rows(yes{}, yes{});
            else stage_rows(yes{}, no{});
        } else {
            if (epi.relu) stage_rows(no{}, yes{});
            else stage_rows(no{}, no{});
        }
    } else {
        stage_rows(no{}, no{});
    }
    uint16_t *const cbase = C + (int64_t)(m0 + wm0) * ldc + n0 + wn0;
    const int cl = lane % CPRC;
    // Rows of C start on 16-byte boundaries: the chunk stores are aligned and
    // can stream past L2.  (Non-temporal stores at 2-byte-aligned addresses
    // measured slower than plain ones: 4096 x 4095 x 4100 with ldc 4095, 128.1
    // against 130.1 us.)
    [[maybe_unused]] const bool c_rows16 = ((uintptr_t)C & 15) == 0 && (ldc & 7) == 0;
#pragma unroll
    for (int it = 0; it < FWTM / RPI; ++it) {
        const int row = RPI * it + lane / CPRC;
        const uint16_t *buf = st[row / ROWS_PER_ARR] + (row % ROWS_PER_ARR) * FWTN;
        u32x4 v = *reinterpret_cast<const u32x4 *>(buf + lds::h16_epi_read<CPRC>(row, cl));
        if (lds::h16_epi_swap(row)) v = u32x4{v[2], v[3], v[0], v[1]};
        uint16_t *dst = cbase + (int64_t)row * ldc + 8 * cl;
        if (!GEN) {
            // Non-temporal (here and for the guarded kernel's whole chunks in
            // 16-byte-aligned rows): the tile is written once and never read
            // back here, so the stores stream past L2 and little is left for
            // the write-back of dirty lines at the end of the kernel (1.4 us of
            // fixed cost at 4096^3, same loop time).
            __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(dst));
        } else {
            const int gm = m0 + wm0 + row, gn = n0 + wn0 + 8 * cl;
            if (gm < M) {
                if (gn + 8 <= N) {
                    if (c_rows16)
                        __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(dst));
                    else
                        *reinterpret_cast<u32x4 *>(dst) = v;
                }
                // (a chunk straddling N is stored below; chunks past N are not)
            }
        }
    }
    if constexpr (GEN) {
        // The chunk of each row that straddles N, if this wave's columns hold
        // one: taken out of the loop above, where its element-wise stores ran
        // with one lane in 16 active in every iteration, and stored here with
        // every lane on a row of its own (measured: 4096 x 4095 x 4096 cost
        // 6 us more than 4096 x 4088 x 4096 that way).
        static_assert(FWTM % 64 == 0, "one row per lane");
        const int wcols = N - (n0 + wn0);                    // wave-uniform
        if (wcols > 0 && wcols < FWTN && (wcols & 7) != 0) {
            const int cs = wcols >> 3, cnt = wcols & 7;
#pragma unroll
            for (int r0 = 0; r0 < FWTM; r0 += 64) {
                const int row = r0 + lane;
                if (m0 + wm0 + row < M) {
                    const uint16_t *buf = st[row / ROWS_PER_ARR] + (row % ROWS_PER_ARR) * FWTN;
                    u32x4 v = *reinterpret_cast<const u32x4 *>(buf + lds::h16_epi_read<CPRC>(row, cs));
                    if (lds::h16_epi_swap(row)) v = u32x4{v[2], v[3], v[0], v[1]};
                    uint16_t *dst = cbase + (int64_t)row * ldc + 8 * cs;
#pragma unroll
                    for (int e = 0; e < 7; ++e)
                        if (e < cnt) dst[e] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
                }
            }
        }
    }
}

}  // namespace

// Whole tiles, a whole number of stage rings and 16-byte alignment: the
// unguarded instantiation.  The per-lane 32-bit byte offsets (up to 256 rows of
// A or BK rows of B past a base) must fit.
static bool fast_whole(const Problem &p, int tbm, int tbn)
{
    return p.aligned && p.M % tbm == 0 && p.N % tbn == 0 &&
           p.K % (FAST_BK * FAST_STAGES) == 0 && p.lda < (1 << 22) && p.ldb < (1 << 22);
}
bool h16_fast_eligible(const Problem &p) { return fast_whole(p, 256, 256); }
bool h16_fast128_eligible(const Problem &p) { return fast_whole(p, 128, 128); }
bool h16_fast128x256_eligible(const Problem &p) { return fast_whole(p, 128, 256); }

// The guarded instantiation: any leading dimensions, N >= 8, two K steps at
// least, and offsets that fit in 32 bits (A rows are addressed from the tile's
// first row, B from its first column of the current K block).
bool h16_general_eligible(const Problem &p)
{
    return p.M >= 1 && p.N >= 8 && p.K > FAST_BK && p.lda < (1 << 22) && p.ldb < (1 << 22) &&
           (int64_t)FAST_BK * p.ldb + p.N < (int64_t)1 << 30;
}

template <bool GEN, bool EPI, int TBM, int TBN, int BUF>
static hipError_t fast_launch(bool is_bf16, const Problem &p)
{
    const int tiles_m = (p.M + TBM - 1) / TBM, tiles_n = (p.N + TBN - 1) / TBN;
    const int64_t nwg = (int64_t)tiles_m * tiles_n;
    if (nwg > 0x7fffffff) return hipErrorInvalidValue;
    const int group_m = tiles_m < 4 ? tiles_m : 4;
    const uint16_t *A = static_cast<const uint16_t *>(p.A);
    const uint16_t *B = static_cast<const uint16_t *>(p.B);
    uint16_t *C = static_cast<uint16_t *>(p.C);
    const dim3 grid((unsigned)nwg), block(FAST_WM * FAST_WN * 64);
    const Epilogue epi = p.epi ? *p.epi : Epilogue{1.f, 0.f, nullptr, 0};
    if (is_bf16)
        hipLaunchKernelGGL(
            (h16_fast_kernel<true, FAST_BK, FAST_STAGES, FAST_WM, FAST_WN, GEN, EPI, TBM, TBN, BUF>), grid,
            block, 0, p.stream, A, B, C, p.M, p.N, p.K, p.lda, p.ldb, p.ldc, tiles_m, tiles_n,
            group_m, epi);
    else
        hipLaunchKernelGGL(
            (h16_fast_kernel<false, FAST_BK, FAST_STAGES, FAST_WM, FAST_WN, GEN, EPI, TBM, TBN, BUF>), grid,
            block, 0, p.stream, A, B, C, p.M, p.N, p.K, p.lda, p.ldb, p.ldc, tiles_m, tiles_n,
            group_m, epi);
    return hipGetLastError();
}

// Guarded instantiations load an operand through a buffer descriptor when its
// rows start on 4-byte boundaries (base pointer 4-byte aligned, even leading
// dimension); buffer LDS-direct loads at offsets that are not 4-byte aligned
// returned wrong data.  Measured on one box: 4096 x 4000 x 4096 109.1 -> 106.6
// us, 4000^3 107.2 -> 104.5 us with both operands; 4097 x 4095 x 4100 (A rows
// 4-byte aligned, B rows only 2-byte aligned) 132.9 -> 131.2 us.
template <bool GEN, bool EPI, int TBM, int TBN>
static hipError_t fast_buf_dispatch(bool is_bf16, const Problem &p)
{
    if constexpr (!GEN) {
        return fast_launch<false, EPI, TBM, TBN, 3>(is_bf16, p);
    } else {
        const bool a4 = ((uintptr_t)p.A & 3) == 0 && p.lda % 2 == 0;
        const bool b4 = ((uintptr_t)p.B & 3) == 0 && p.ldb % 2 == 0;
        switch ((a4 ? 1 : 0) | (b4 ? 2 : 0)) {
        case 3: return fast_launch<true, EPI, TBM, TBN, 3>(is_bf16, p);
        case 2: return fast_launch<true, EPI, TBM, TBN, 2>(is_bf16, p);
        case 1: return fast_launch<true, EPI, TBM, TBN, 1>(is_bf16, p);
        default: return fast_launch<true, EPI, TBM, TBN, 0>(is_bf16, p);
        }
    }
}

template <int TBM, int TBN>
static hipError_t fast_dispatch(bool is_bf16, bool gen, const Problem &p)
{
    if (gen)
        return p.epi ? fast_buf_dispatch<true, true, TBM, TBN>(is_bf16, p)
                     : fast_buf_dispatch<true, false, TBM, TBN>(is_bf16, p);
    return p.epi ? fast_buf_dispatch<false, true, TBM, TBN>(is_bf16, p)
                 : fast_buf_dispatch<false, false, TBM, TBN>(is_bf16, p);
}

hipError_t h16_fast_launch(bool is_bf16, const Problem &p)
{
    if (!h16_fast_eligible(p)) return hipErrorInvalidValue;
    return fast_dispatch<256, 256>(is_bf16, false, p);
}

hipError_t h16_general_launch(bool is_bf16, const Problem &p)
{
    if (!h16_general_eligible(p)) return hipErrorInvalidValue;
    return fast_dispatch<256, 256>(is_bf16, true, p);
}

hipError_t h16_fast128_launch(bool is_bf16, const Problem &p)
{
    if (!h16_fast128_eligible(p)) return hipErrorInvalidValue;
    return fast_dispatch<128, 128>(is_bf16, false, p);
}

hipError_t h16_general128_launch(bool is_bf16, const Problem &p)
{
    if (!h16_general_eligible(p)) return hipErrorInvalidValue;
    return fast_dispatch<128, 128>(is_bf16, true, p);
}

hipError_t h16_fast128x256_launch(bool is_bf16, const Problem &p)
{
    if (!h16_fast128x256_eligible(p)) return hipErrorInvalidValue;
    return fast_dispatch<128, 256>(is_bf16, false, p);
}

hipError_t h16_general128x256_launch(bool is_bf16, const Problem &p)
{
    if (!h16_general_eligible(p)) return hipErrorInvalidValue;
    return fast_dispatch<128, 256>(is_bf16, true, p);
}

}  // namespace gemm
