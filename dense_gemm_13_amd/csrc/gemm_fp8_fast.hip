// FP8 (OCP E4M3) block-scaled GEMM, large-tile path for gfx950: 256 x 256
// tiles (128 x 128 for medium grids, two workgroups per CU); whole tiles with K
// a multiple of 256 and 16-byte aligned rows, or (the guarded instantiation)
// any shape with N >= 16 and K > 64.
//
//   C[i][j] = bf16( sum_kb  sa(i/64, kb) * sb(kb, j/64) * sum_{k in block kb} qa(i,k) qb(k,j) )
//
// "深度学习加速核心：GEMM优化从分块到TensorCore的实战解析", section 4.3: E4M3
// operands with one scale per 64 x 64 sub-block; section 5.2 (third pitfall):
// 32-bit scales.  Same movement of operands as the half-precision large-tile
// path (gemm_h16_fast.hip): global_load_lds_dwordx4 into a 4-stage LDS ring,
// one array per stage, the XOR chunk swizzle applied on the global side.
//
// One K step is one 64-wide scale block.  Every 32 x 32 output tile of a wave
// gets one v_mfma_scale_f32_32x32x64_f8f6f4 per step (hardware block scales at
// 2^0) into a zeroed partial, which is promoted into the fp32 accumulator with
// one FMA per element by sa * sb of that block.  The promotion runs on the
// vector ALU, so the accumulators live in VGPRs: 8 waves (two per SIMD), each
// with a 128 x 64 sub-tile (128 accumulator VGPRs); one wave's MFMAs overlap the
// other's promotion.  The promotion costs as many vector-ALU cycles as the MFMAs
// take on the matrix core (16 wave64 FMAs of 4 cycles per 64-cycle MFMA), so
// the kernel is bound by how well the two overlap.  The block scales of each K
// step travel into LDS with its operands, and one barrier per step (half-way
// through its MFMAs) lets the next stage's fragments be read while the
// current one is multiplied.
//
// B stays in LDS as rows of k (n contiguous, 256-byte rows) and the MFMA operand
// "32 consecutive k of one column" comes from four ds_read_b64_tr_b8: within a
// 16-lane group, lanes 2r and 2r+1 address the two 8-byte halves of 16
// consecutive columns of row r (8 rows), and lane j receives byte j of each of
// the 8 rows.
#include <utility>

#include "gemm_device.hpp"
#include "gemm_launch.hpp"
#include "gemm_lds_layout.hpp"

namespace gemm {

namespace {

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void8_t;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2_t;

constexpr int QBK = 64, QSTAGES = 4;
constexpr int QNW = 8;                                   // waves

// Tile shapes: TB = 256 (waves 2 x 4 of 128 x 64, 4 x 2 MFMA tiles each) or
// TB = 128 (waves 4 x 2 of 32 x 64, 1 x 2 MFMA tiles each).  Every wave's
// sub-tile is 64 columns wide, so each MFMA pair shares one A tile and the
// step below runs the same way for both.
template <int TB>
struct QShape {
    static constexpr int BM = TB, BN = TB;
    static constexpr int WM = TB == 256 ? 2 : 4, WN = QNW / WM;
    static constexpr int WTM = BM / WM, WTN = BN / WN;   // 128 x 64 or 32 x 64 per wave
    static constexpr int FM = WTM / 32, FN = WTN / 32;   // 4 x 2 or 1 x 2 MFMA tiles
    static constexpr int A_STAGE = BM * QBK;             // bytes per stage (16 or 8 KiB)
    static constexpr int B_STAGE = QBK * BN;
    static constexpr int A_BLK = A_STAGE / 1024 / QNW;   // 1 KiB loads per wave per stage
    static constexpr int B_BLK = B_STAGE / 1024 / QNW;
    static constexpr int NBLK = A_BLK + B_BLK;
    static constexpr int BCPR = BN / 16;                 // 16-byte chunks per B row
    static constexpr int BRPK = 64 / BCPR;               // B rows per 1 KiB load
    static_assert(WTN == 64 && A_BLK >= 1 && B_BLK >= 1, "tile shape");
};

template <int TAG, int BYTES>
__shared__ __attribute__((aligned(1024))) uint8_t q_stage[BYTES];
// The block scales of one stage (4 of A's scale rows, then 4 of B's scale
// columns), 64 copies of each (one per lane of the wave that loads it), one
// array per stage like the operand stages.
template <int TAG>
__shared__ __attribute__((aligned(256))) float q_scale[8 * 64];

template <int BYTES>
__device__ __forceinline__ uint8_t *q_ring(int idx)
{
    switch (idx) {
    case 0: return q_stage<0, BYTES>;
    case 1: return q_stage<1, BYTES>;
    case 2: return q_stage<2, BYTES>;
    case 3: return q_stage<3, BYTES>;
    case 4: return q_stage<4, BYTES>;
    case 5: return q_stage<5, BYTES>;
    case 6: return q_stage<6, BYTES>;
    default: return q_stage<7, BYTES>;
    }
}

// The XOR swizzles of the stages and the lane -> address maps of every LDS
// access below are in gemm_lds_layout.hpp (checked on the host for banks).

// Global -> LDS loads of 16 bytes (operands) and 4 bytes (scales) per lane.
// (Functions of their own: with arguments that depend on the kernel's template
// parameters, the builtin called directly in the kernel's lambdas leaves the
// host-side instantiation of the kernel invalid and its launch stub undefined.)
// Operands go through a buffer descriptor: the base in scalar registers, the
// lane's 32-bit offset in a vector register, so no per-load 64-bit address
// arithmetic runs on the vector ALU that the promotion keeps busy.  `reach` is
// the number of bytes the tile may touch from the base; an offset past it would
// read zeros instead of leaving the operand.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t q_rsrc(const void *base, int reach)
{
    // 4th word 0x00020000: 32-bit data format, the raw-buffer setting for gfx9.
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, reach, 0x00020000);
}
// (Whole tiles only: their rows are 16-byte aligned.  Buffer loads at byte
// offsets that are not were measured to return wrong data, so the guarded
// instantiation, which takes any leading dimension, uses q_gdma16.)
__device__ __forceinline__ void q_dma16(__amdgpu_buffer_rsrc_t r, uint32_t off, uint8_t *lds)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void8_t *)lds, 16, (int)off, 0, 0, 0);
}
__device__ __forceinline__ void q_gdma16(const void *src, uint8_t *lds)
{
    __builtin_amdgcn_global_load_lds(src, (lds_void8_t *)lds, 16, 0, 0);
}
__device__ __forceinline__ void q_dma4(const void *src, float *lds)
{
    __builtin_amdgcn_global_load_lds(src, (lds_void8_t *)lds, 4, 0, 0);
}

template <int N>
__device__ __forceinline__ void q_wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
__device__ __forceinline__ void q_barrier() { asm volatile("s_barrier" ::: "memory"); }

template <typename F, int... I>
__device__ __forceinline__ void q_unroll_impl(F &&f, std::integer_sequence<int, I...>)
{
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void q_unroll(F &&f)
{
    q_unroll_impl(f, std::make_integer_sequence<int, N>{});
}

// GEN = false: whole 256 x 256 tiles, K a multiple of 256, 16-byte aligned
// rows.  GEN = true: any M, N >= 16, K > 64 and any leading dimensions (the
// hardware runs in unaligned-access mode, so 16-byte loads at any address are
// legal), as the guarded half-precision kernel does it:
//   * the last K block (possibly partial) is step 0, loaded through registers
//     with zero fill past K, M and N together with its scales; steps 1, 2, ...
//     load blocks 0, 1, ... LDS-direct, all of them whole blocks that never
//     touch B's last row;
//   * A rows past M are clamped to row M-1 and B column chunks starting past N
//     to the last whole chunk at a multiple of 16 columns (their products only reach C entries that are not
//     stored; a chunk straddling N reads a few bytes past N inside a row that is
//     not B's last), scale rows and columns past the grids to the last ones;
//   * after the whole turns of the ring the remaining steps run once, guarded;
//   * C stores, and the epilogue's reads of bias and prior C, are masked to the
//     M x N window.
// EPI: the fused epilogue is applied to the fp32 accumulators before they are
// rounded; the lane that reads an entry's prior C does not store it, but the
// store depends through LDS on the value that read produced.
template <bool GEN, bool EPI, int TB>
__global__ void __launch_bounds__(QNW * 64) __attribute__((amdgpu_waves_per_eu(
    TB == 256 ? 2 : 4, TB == 256 ? 2 : 4)))
fp8_fast_kernel(const uint8_t *__restrict__ A, const uint8_t *__restrict__ B,
                uint16_t *__restrict__ C, int M, int N, int K, int64_t lda, int64_t ldb,
                int64_t ldc, const float *__restrict__ scale_a, const float *__restrict__ scale_b,
                int mblocks, int kblocks, int nblocks, int tiles_m, int tiles_n, int group_m,
                Epilogue epi)
{
    using Sh = QShape<TB>;
    constexpr int QBM = Sh::BM, QBN = Sh::BN, QWN = Sh::WN, QWTM = Sh::WTM, QWTN = Sh::WTN;
    constexpr int QFM = Sh::FM, QFN = Sh::FN, QA_BLK = Sh::A_BLK, QB_BLK = Sh::B_BLK;
    constexpr int QNBLK = Sh::NBLK, QSTAGE = Sh::A_STAGE;
    static_assert(Sh::A_STAGE == Sh::B_STAGE, "square tiles");
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm0 = (wave / QWN) * QWTM;
    const int wn0 = (wave % QWN) * QWTN;
    const int l32 = lane & 31, half = lane >> 5;

    int tm, tn;
    tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * QBM, n0 = tn * QBN;

    // ---- this wave's 1 KiB loads.  A block b: 16 rows of 64 bytes, lane ->
    // row 16b + lane/4, slot lane%4 holding logical chunk slot ^ qswz_a(row).
    // B block b: BRPK rows of BN bytes (4 of 256 or 8 of 128), lane -> row
    // BRPK*b + lane/BCPR, slot lane%BCPR.
    uint32_t a_off[QA_BLK], b_off[QB_BLK];
#pragma unroll
    for (int j = 0; j < QA_BLK; ++j) {
        int row, chunk;
        lds::fp8_a_dma(wave * QA_BLK + j, lane, row, chunk);
        const int lrow = GEN && m0 + row >= M ? M - 1 - m0 : row;
        a_off[j] = (uint32_t)(lrow * lda + 16 * chunk);
    }
    // (GEN: the column, n0 included, is part of the per-lane offset.)
#pragma unroll
    for (int j = 0; j < QB_BLK; ++j) {
        int row, chunk;
        lds::fp8_b_dma<QBN>(wave * QB_BLK + j, lane, row, chunk);
        int col = 16 * chunk;
        if (GEN) col = n0 + col >= N ? ((N - 16) & ~15) : n0 + col;
        b_off[j] = (uint32_t)(row * ldb + col);
    }
    const uint8_t *a_base = A + (int64_t)m0 * lda;
    const uint8_t *b_base = GEN ? B : B + n0;
    const int64_t b_step = (int64_t)QBK * ldb;
    // (QBM rows of A and QBK rows of B from the step's base: below 2^31 bytes
    // under the eligibility limits lda < 2^23, ldb < 2^24.)
    const int a_reach = (int)(QBM * lda), b_reach = (int)(QBK * ldb);
    auto issue = [&](uint8_t *as, uint8_t *bs, int kt) {
        const uint8_t *ab = a_base + kt * QBK;
        const uint8_t *bb = b_base + kt * b_step;
        if constexpr (GEN) {
#pragma unroll
            for (int j = 0; j < QA_BLK; ++j) q_gdma16(ab + a_off[j], as + (wave * QA_BLK + j) * 1024);
#pragma unroll
            for (int j = 0; j < QB_BLK; ++j) q_gdma16(bb + b_off[j], bs + (wave * QB_BLK + j) * 1024);
        } else {
            const __amdgpu_buffer_rsrc_t ra = q_rsrc(ab, a_reach), rb = q_rsrc(bb, b_reach);
#pragma unroll
            for (int j = 0; j < QA_BLK; ++j) q_dma16(ra, a_off[j], as + (wave * QA_BLK + j) * 1024);
#pragma unroll
            for (int j = 0; j < QB_BLK; ++j) q_dma16(rb, b_off[j], bs + (wave * QB_BLK + j) * 1024);
        }
    };

    // ---- fragment addressing (bytes, relative to a stage)
    // A tile i: lane reads row wm0 + 32i + l32, k bytes 32*half .. +31 (chunks 2h, 2h+1).
    static_assert(QBK == 64, "64-byte A rows");
    int a_off0[QFM], a_off1[QFM];
#pragma unroll
    for (int i = 0; i < QFM; ++i) {
        const int row = wm0 + 32 * i + l32;
        a_off0[i] = lds::fp8_a_frag(row, 2 * half);
        a_off1[i] = lds::fp8_a_frag(row, 2 * half + 1);
    }
    // B tile j, read q: 16-lane group g, lane w: row 32*(g/2) + 8q + w/2, columns
    // wn0 + 32j + 16*(g%2) + 8*(w%2) .. +7.  (k rows with the same k % 8 share a swizzle.)
    const int g = lane >> 4, w16 = lane & 15, r8 = w16 >> 1;
    int b_off_r[QFN];
#pragma unroll
    for (int j = 0; j < QFN; ++j) {
        const int n = wn0 + 32 * j + 16 * (g & 1) + 8 * (w16 & 1);
        // rows 32 (g/2) + 8q + r8 share their swizzle with row r8
        b_off_r[j] = (32 * (g >> 1) + r8) * QBN + lds::fp8_b_col<QBN>(r8, n);
    }

    // ---- block scales.  Every stage also carries the 8 scales of its K block
    // that this tile needs: scale_a of the tile's 4 scale rows and scale_b of
    // its 4 scale columns.  Wave w fetches one of them (w < 4: row w of A's
    // scales, else column w - 4 of B's) with a 4-byte LDS-direct load in which
    // every lane reads the same address (no branch), so the scales travel and
    // are waited for exactly like the operands.
    const int sc_blk = wave < 4 ? m0 / 64 + wave : n0 / 64 + (wave - 4);
    const float *sc_src = wave < 4 ? scale_a + (int64_t)(sc_blk < mblocks ? sc_blk : mblocks - 1) * kblocks
                                   : scale_b + (sc_blk < nblocks ? sc_blk : nblocks - 1);
    const int64_t sc_step = wave < 4 ? 1 : nblocks;
    // This wave's scale row pair (A tiles 0,1 / 2,3) and scale column, in the slot.
    const int sc_row = wm0 / 64, sc_col = 4 + wn0 / 64;

    // K step s loads K block s (GEN: block s - 1; step 0 is the last block).
    auto issue_all = [&](auto S, int s) {
        const int kb = GEN ? s - 1 : s;
        // (B stages take the first array tags and A stages the last: placed
        // that way, every B read's stage base fits the LDS instruction's
        // 16-bit offset field, and only the two A read bases need an add per
        // step: 5 -> 2 vector adds per K step.)
        issue(q_stage<QSTAGES + S, QSTAGE>, q_stage<S, QSTAGE>, kb);
        q_dma4(sc_src + kb * sc_step, &q_scale<S>[64 * wave]);
    };
    constexpr int QLOADS = QNBLK + 1;                    // loads per wave per stage
    const int ktiles = (K + QBK - 1) / QBK;              // !GEN: K / QBK, a multiple of QSTAGES

    f32x16 acc[QFM][QFN];
#pragma unroll
    for (int i = 0; i < QFM; ++i)
#pragma unroll
        for (int j = 0; j < QFN; ++j) acc[i][j] = f32x16{};

    // Fragments of one stage: A tile i (ds_read_b128 x 2), B tile j (four
    // transposing reads), and the two products sa * sb of the wave's scale rows.
    i32x8 af[QFM], bfr[QFN];
    const auto read_a = [&](const uint8_t *as, int i) {
        const u32x4 x0 = *reinterpret_cast<const u32x4 *>(as + a_off0[i]);
        const u32x4 x1 = *reinterpret_cast<const u32x4 *>(as + a_off1[i]);
        af[i] = i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                      (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
    };
    const auto read_b = [&](const uint8_t *bs, int j) {
        i32x2 r[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
            r[q] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (lds_i32x2_t *)(bs + b_off_r[j] + 8 * q * QBN));
        bfr[j] = i32x8{r[0][0], r[0][1], r[1][0], r[1][1], r[2][0], r[2][1], r[3][0], r[3][1]};
    };
    // The raw scales of the next step are read at the end of a step and
    // multiplied in the next step's first slot (not at once, which would wait
    // for the reads just issued).
    float rsa0, rsa1, rsb;
    const auto read_scales = [&](const float *sl) {
        rsb = sl[64 * sc_col];
        rsa0 = sl[64 * sc_row];
        rsa1 = sl[64 * (sc_row + 1)];
    };
    float cs0 = 0.f, cs1 = 0.f;                          // sa * sb of the current step

    // One MFMA per 32 x 32 tile and K block (E4M3 operands, format 0; hardware
    // block scales 127 = 2^0) into a fresh partial, promoted into the fp32
    // accumulator with one FMA per element by that block's sa * sb.  The
    // promotion of tile t runs after the MFMA of tile t + 1 has been issued
    // (two partial register sets), so the vector ALU works on one tile while the
    // matrix core works on the next and no FMA waits for the MFMA that feeds it.
    // Tiles t = 0..3 use B tile 0, t = 4..7 B tile 1; tile t is A tile t % 4.
    constexpr int NT = QFM * QFN;
    f32x16 part[2];
    const auto mma = [&](int t) {
        part[t & 1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            bfr[t / QFM], af[t % QFM], f32x16{}, 0, 0, 0, 127, 0, 127);
    };
    const auto promote = [&](int t, float s0, float s1) {
        const int i = t % QFM, j = t / QFM;
        const float s = i < 2 ? s0 : s1;
#pragma unroll
        for (int e = 0; e < 16; ++e)
            acc[i][j][e] = __builtin_fmaf(part[t & 1][e], s, acc[i][j][e]);
    };

    // K step s runs on stage S = s % QSTAGES with its fragments and scales
    // already in registers:
    //   * tiles 0..3 (B tile 0; the first slot also promotes the previous
    //     step's last tile, with that step's scales);
    //   * wait for this wave's loads of stage s + 1 and for its outstanding LDS
    //     reads, barrier: stage s + 1 is complete, and every wave has read all
    //     of stage s that it will read;
    //   * issue the loads of K step s + QSTAGES into stage S; read B tile 0 of
    //     stage s + 1;
    //   * tiles 4..7 (B tile 1), reading A tile t - 4 of stage s + 1 after each
    //     tile's MFMA (its last use of that A tile), then B tile 1 and the
    //     scales of stage s + 1.
    // A load has QSTAGES - 1 steps to land.  Slots are fenced so the compiler
    // keeps this order.
    float ps0 = 0.f, ps1 = 0.f;                          // scales of the previous step
    const auto step = [&](auto S, int s) {
        constexpr int N1 = (S + 1) % QSTAGES;
#pragma unroll
        for (int t = 0; t < NT / 2; ++t) {
            mma(t);
            if (t == 0) {
                promote(NT - 1, ps0, ps1);
                // Wave-uniform: held in scalar registers, so each promotion FMA
                // reads two vector registers instead of three.
                cs0 = __builtin_bit_cast(
                    float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, rsa0 * rsb)));
                cs1 = __builtin_bit_cast(
                    float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, rsa1 * rsb)));
            } else {
                promote(t - 1, cs0, cs1);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);              // lgkmcnt(0)
        q_wait_vmcnt<(QSTAGES - 2) * QLOADS>();
        q_barrier();
        __builtin_amdgcn_sched_barrier(0);
        const int nxt = s + QSTAGES;
        issue_all(S, nxt < ktiles ? nxt : ktiles - 1);
        read_b(q_stage<N1, QSTAGE>, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = NT / 2; t < NT; ++t) {
            mma(t);
            promote(t - 1, cs0, cs1);
            read_a(q_stage<QSTAGES + N1, QSTAGE>, t - NT / 2);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        read_b(q_stage<N1, QSTAGE>, 1);
        ps0 = cs0;
        ps1 = cs1;
        read_scales(q_scale<N1>);
        __builtin_amdgcn_sched_barrier(0);
    };

    // Prologue: K steps 0 .. QSTAGES-1 in flight, stage 0 published, its
    // fragments and scales read.  The partial set the first slot promotes is
    // zero (with zero scales).  Steps past the end re-load the last K block
    // moved LDS-direct into stages nobody reads any more, and the last step's
    // look-ahead reads a stage whose contents are not used.
    // GEN: step 0 is the last K block [QBK*(ktiles-1), K), through registers
    // with zero fill, in the swizzled layout the LDS-direct loads produce, with
    // its scales (written before any LDS-direct load is issued).
    if constexpr (GEN) {
        const int k0 = QBK * (ktiles - 1);
        uint8_t *as = q_stage<QSTAGES, QSTAGE>, *bs = q_stage<0, QSTAGE>;
        constexpr int NT = QNW * 64, NQA = QBM * QBK / 16 / NT, NQB = QBK * QBN / 16 / NT;
        static_assert(NQA * NT * 16 == QBM * QBK && NQB * NT * 16 == QBK * QBN, "whole chunks");
        if (K >= 16) {
            // One 16-byte load inside the matrix per chunk, all in flight before
            // the first wait; zeros past M, N and K applied in registers.
            Masked16 va[NQA], vb[NQB];
#pragma unroll
            for (int i = 0; i < NQA; ++i) {
                const int q = tid + NT * i, r = q >> 2, c = q & 3;
                va[i] = masked16_load<1>(A, lda, m0 + r, M, k0 + 16 * c, K);
            }
#pragma unroll
            for (int i = 0; i < NQB; ++i) {
                const int q = tid + NT * i, r = q / Sh::BCPR, c = q % Sh::BCPR;
                vb[i] = masked16_load<1>(B, ldb, k0 + r, K, n0 + 16 * c, N);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < NQA; ++i) {
                const int q = tid + NT * i, r = q >> 2, c = q & 3;
                *reinterpret_cast<u32x4 *>(as + lds::fp8_a_frag(r, c)) = masked16_value(va[i]);
            }
#pragma unroll
            for (int i = 0; i < NQB; ++i) {
                const int q = tid + NT * i, r = q / Sh::BCPR, c = q % Sh::BCPR;
                *reinterpret_cast<u32x4 *>(bs + r * QBN + lds::fp8_b_col<QBN>(r, 16 * c)) =
                    masked16_value(vb[i]);
            }
        } else {
            // K < 16: element by element.
            for (int q = tid; q < QBM * QBK / 16; q += NT) {
                const int r = q >> 2, c = q & 3;
                const int gm = m0 + r, gk = k0 + 16 * c;
                uint32_t w[4] = {0, 0, 0, 0};
                if (gm < M) {
                    const uint8_t *src = A + (int64_t)gm * lda + gk;
                    for (int e = 0; e < 16; ++e)
                        if (gk + e < K) w[e >> 2] |= (uint32_t)src[e] << (8 * (e & 3));
                }
                *reinterpret_cast<u32x4 *>(as + lds::fp8_a_frag(r, c)) = u32x4{w[0], w[1], w[2], w[3]};
            }
            for (int q = tid; q < QBK * QBN / 16; q += NT) {
                const int r = q / Sh::BCPR, c = q % Sh::BCPR;
                const int gk = k0 + r, gn = n0 + 16 * c;
                u32x4 v = u32x4{0, 0, 0, 0};
                if (gk < K) {
                    const uint8_t *src = B + (int64_t)gk * ldb + gn;
                    if (gn + 16 <= N) {
                        v = *reinterpret_cast<const u32x4 *>(src);
                    } else {
                        uint32_t w[4] = {0, 0, 0, 0};
                        for (int e = 0; e < 16; ++e)
                            if (gn + e < N) w[e >> 2] |= (uint32_t)src[e] << (8 * (e & 3));
                        v = u32x4{w[0], w[1], w[2], w[3]};
                    }
                }
                *reinterpret_cast<u32x4 *>(bs + r * QBN + lds::fp8_b_col<QBN>(r, 16 * c)) = v;
            }
        }
        q_scale<0>[64 * wave + lane] = sc_src[(int64_t)(ktiles - 1) * sc_step];
        q_unroll<QSTAGES - 1>([&](auto S) {
            constexpr int S1 = S + 1;
            issue_all(std::integral_constant<int, S1>{}, S1 < ktiles ? S1 : ktiles - 1);
        });
        __builtin_amdgcn_s_waitcnt(0xc07f);              // lgkmcnt(0): the LDS writes landed
    } else {
        q_unroll<QSTAGES>([&](auto S) { issue_all(S, (int)S); });
        q_wait_vmcnt<(QSTAGES - 1) * QLOADS>();
    }
    q_barrier();
#pragma unroll
    for (int i = 0; i < QFM; ++i) read_a(q_stage<QSTAGES, QSTAGE>, i);
#pragma unroll
    for (int j = 0; j < QFN; ++j) read_b(q_stage<0, QSTAGE>, j);
    read_scales(q_scale<0>);
    part[(NT - 1) & 1] = f32x16{};
    // Whole turns of the ring without conditions (a step skipped at run time
    // would let the compiler merge the steps' code and lose track of which
    // stage array each LDS read addresses).  GEN: the remaining ktiles % QSTAGES
    // steps follow, once.
    const int kwhole = GEN ? ktiles - ktiles % QSTAGES : ktiles;
    for (int kt = 0; kt < kwhole; kt += QSTAGES)
        q_unroll<QSTAGES>([&](auto S) { step(S, kt + S); });
    if constexpr (GEN) {
        const int rem = ktiles - kwhole;
        q_unroll<QSTAGES - 1>([&](auto S) {
            if (S < rem) step(S, kwhole + S);
        });
    }
    promote(NT - 1, ps0, ps1);
    q_wait_vmcnt<0>();

    // ---- epilogue through LDS: each wave's 128 x 64 bf16 sub-tile (16 KiB) goes
    // to its own ring array (128-byte rows, chunks XORed with row % 8, the 8-byte
    // half with bit 3 of the row), then out as whole 128-byte row segments.
    __builtin_amdgcn_s_waitcnt(0xc07f);                  // lgkmcnt(0)
    q_barrier();
    uint16_t *st = reinterpret_cast<uint16_t *>(q_ring<QSTAGE>(wave));
    // EPI: the bias of this lane's columns, loaded once for all its rows.
    [[maybe_unused]] float ebias[EPI ? QFN : 1][4][4];
    if constexpr (EPI) {
#pragma unroll
        for (int j = 0; j < QFN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int gn = n0 + wn0 + 32 * j + 8 * q + 4 * half;
                epilogue_bias<4>(epi, gn, GEN ? N - gn : 4, ebias[j][q]);
            }
    }
#pragma unroll
    for (int i = 0; i < QFM; ++i) {
        const int row = 32 * i + l32;
        uint16_t *buf = st + row * QWTN;
        if constexpr (EPI) {
            // The prior C of the row's entries first, then the arithmetic.
            const bool row_in = !GEN || m0 + wm0 + row < M;
            const uint16_t *crow = C + (int64_t)(row_in ? m0 + wm0 + row : 0) * ldc;
            float prior[QFN][4][4];
#pragma unroll
            for (int j = 0; j < QFN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int gn = n0 + wn0 + 32 * j + 8 * q + 4 * half;
                    epilogue_prior<OUT_BF16, 4>(epi, crow, gn, !row_in ? 0 : GEN ? N - gn : 4,
                                                prior[j][q]);
                }
#pragma unroll
            for (int j = 0; j < QFN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float v[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                  acc[i][j][4 * q + 3]};
                    epilogue_apply<4>(epi, v, ebias[j][q], prior[j][q], 4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[i][j][4 * q + e] = v[e];
                }
        }
#pragma unroll
        for (int j = 0; j < QFN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                *reinterpret_cast<u32x2 *>(buf + lds::fp8_epi_write(row, 4 * j + q, half)) =
                    u32x2{pack2<true>(acc[i][j][4 * q], acc[i][j][4 * q + 1]),
                          pack2<true>(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3])};
            }
    }
    uint16_t *const cbase = C + (int64_t)(m0 + wm0) * ldc + n0 + wn0;
    const int cl = lane & 7;
#pragma unroll
    for (int it = 0; it < QWTM / 8; ++it) {
        const int row = 8 * it + (lane >> 3);
        u32x4 v = *reinterpret_cast<const u32x4 *>(st + row * QWTN + lds::fp8_epi_read(row, cl));
        if ((row >> 3) & 1) v = u32x4{v[2], v[3], v[0], v[1]};
        uint16_t *dst = cbase + (int64_t)row * ldc + 8 * cl;
        if (!GEN) {
            *reinterpret_cast<u32x4 *>(dst) = v;
        } else {
            const int gm = m0 + wm0 + row, gn = n0 + wn0 + 8 * cl;
            if (gm < M && gn + 8 <= N) *reinterpret_cast<u32x4 *>(dst) = v;
            // (a chunk straddling N is stored below; chunks past N are not)
        }
    }
    if constexpr (GEN) {
        // The chunk of each row that straddles N, with every lane on a row of
        // its own rather than one lane in 8 active per row group of the loop.
        const int wcols = N - (n0 + wn0);                    // wave-uniform
        if (wcols > 0 && wcols < QWTN && (wcols & 7) != 0) {
            const int cs = wcols >> 3, cnt = wcols & 7;
#pragma unroll
            for (int r0 = 0; r0 < QWTM; r0 += 64) {
                const int row = r0 + lane;
                if (row < QWTM && m0 + wm0 + row < M) {
                    u32x4 v = *reinterpret_cast<const u32x4 *>(st + row * QWTN + lds::fp8_epi_read(row, cs));
                    if ((row >> 3) & 1) v = u32x4{v[2], v[3], v[0], v[1]};
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

static bool fp8_whole(const Problem &p, int tb)
{
    return p.M % tb == 0 && p.N % tb == 0 && p.K % (QBK * QSTAGES) == 0 &&
           ((uintptr_t)p.A & 15) == 0 && ((uintptr_t)p.B & 15) == 0 &&
           ((uintptr_t)p.C & 15) == 0 && p.lda % 16 == 0 && p.ldb % 16 == 0 && p.ldc % 8 == 0 &&
           p.lda < (1 << 23) && p.ldb < (1 << 24);
}
bool fp8_fast_eligible(const Problem &p) { return fp8_whole(p, 256); }
bool fp8_fast128_eligible(const Problem &p) { return fp8_whole(p, 128); }

// The guarded instantiation: any M, N >= 16 (a clamped column chunk starts at
// N - 16 rounded down to a multiple of 16), two K blocks at least, and per-lane 32-bit byte offsets that fit (256
// rows of A from the tile's first row; 64 rows of B plus the column).
bool fp8_general_eligible(const Problem &p)
{
    return p.M >= 1 && p.N >= 16 && p.K > QBK && p.lda < (1 << 23) &&
           (int64_t)QBK * p.ldb + p.N < ((int64_t)1 << 31);
}

template <bool GEN, int TB>
static hipError_t fp8_fast_typed(const Problem &p, const float *scale_a, const float *scale_b)
{
    const int tiles_m = (p.M + TB - 1) / TB, tiles_n = (p.N + TB - 1) / TB;
    const int64_t nwg = (int64_t)tiles_m * tiles_n;
    if (nwg > 0x7fffffff) return hipErrorInvalidValue;
    const int group_m = tiles_m < 4 ? tiles_m : 4;
    const uint8_t *A = static_cast<const uint8_t *>(p.A), *B = static_cast<const uint8_t *>(p.B);
    uint16_t *C = static_cast<uint16_t *>(p.C);
    const int mblocks = (p.M + 63) / 64, kblocks = (p.K + 63) / 64, nblocks = (p.N + 63) / 64;
    const Epilogue epi = p.epi ? *p.epi : Epilogue{1.f, 0.f, nullptr, 0};
    if (p.epi)
        hipLaunchKernelGGL((fp8_fast_kernel<GEN, true, TB>), dim3((unsigned)nwg), dim3(QNW * 64), 0,
                           p.stream, A, B, C, p.M, p.N, p.K, p.lda, p.ldb, p.ldc, scale_a, scale_b,
                           mblocks, kblocks, nblocks, tiles_m, tiles_n, group_m, epi);
    else
        hipLaunchKernelGGL((fp8_fast_kernel<GEN, false, TB>), dim3((unsigned)nwg), dim3(QNW * 64), 0,
                           p.stream, A, B, C, p.M, p.N, p.K, p.lda, p.ldb, p.ldc, scale_a, scale_b,
                           mblocks, kblocks, nblocks, tiles_m, tiles_n, group_m, epi);
    return hipGetLastError();
}

hipError_t fp8_fast_launch(const Problem &p, const float *scale_a, const float *scale_b)
{
    if (!fp8_fast_eligible(p)) return hipErrorInvalidValue;
    return fp8_fast_typed<false, 256>(p, scale_a, scale_b);
}

hipError_t fp8_general_launch(const Problem &p, const float *scale_a, const float *scale_b)
{
    if (!fp8_general_eligible(p)) return hipErrorInvalidValue;
    return fp8_fast_typed<true, 256>(p, scale_a, scale_b);
}

// 128 x 128 tiles (whole where eligible, else guarded).
hipError_t fp8_tiles128_launch(const Problem &p, const float *scale_a, const float *scale_b,
                               bool force_general)
{
    if (!force_general && fp8_fast128_eligible(p))
        return fp8_fast_typed<false, 128>(p, scale_a, scale_b);
    if (!fp8_general_eligible(p)) return hipErrorInvalidValue;
    return fp8_fast_typed<true, 128>(p, scale_a, scale_b);
}

}  // namespace gemm
