// FP8 (OCP E4M3) block-scaled GEMM for tall, narrow and small grids:
// C (bf16) = sum over 64-wide K blocks kb of sa(i/64, kb) * sb(kb, j/64) * (qA qB
// over the block), with 32 x 64 or 64 x 64 tiles of C whose K sum is split
// over the workgroup's waves.
//
// The 256 x 256 tiles of the large-tile kernel leave most of the chip idle on
// small or narrow grids (8192 x 64 x 4096: 32 tiles; it is bound by reading A's
// 32 MiB once).  Here a workgroup owns a TBM x 64 tile (TBM = 32 or 64, so the
// tile lies in one 64 x 64 scale block of C) and its 4 waves split K: wave w
// takes the 64-wide K blocks w, w + 4, w + 8, ..., each row strip starting its
// walk at its own block.  A K block is one scale block, so every step of a
// wave uses one product sa * sb; the tile's scale row of A and scale column of
// B are staged in LDS once at the start.  Each wave streams its blocks of A
// (TBM rows of 64 bytes) and B (64 rows of 64 bytes) through a private ring of
// LDS stages with global_load_lds_dwordx4 and waits only for its own loads.
// Per step and 32 x 32 output tile: one v_mfma_scale_f32_32x32x64_f8f6f4
// (hardware block scales at 2^0) into a zeroed partial, promoted into the fp32
// accumulator with one FMA per element by sa * sb.  The four fp32 partial tiles
// are added through LDS at the end, the epilogue applied, and the sum rounded
// to bf16.
//
// GEN = true takes any M, N >= 16, K >= 1 and any leading dimensions: A rows
// past M are clamped to row M-1 and B column chunks starting past N to the
// last whole chunk at a multiple of 16 columns (their products only reach C entries that are not stored; a
// chunk straddling N reads a few bytes past N inside a row that is not B's
// last); the last K block, possibly partial, is loaded through registers with
// zero fill by the wave whose turn it would be, so no LDS-direct load touches
// B's last row; stores are masked to the M x N window.  The hardware runs in
// unaligned-access mode, so 16-byte loads at any address are legal.
//
// The operand formats and the per-block scales are those of
// "深度学习加速核心：GEMM优化从分块到TensorCore的实战解析" section 4.3 (E4M3, one
// scale per 64 x 64 sub-block) and section 5.2 (32-bit scales); the split of the
// K sum into separately accumulated blocks is the "K split" of "CUDA GEMM 优化
// 实践笔记".
#include <type_traits>

#include "gemm_device.hpp"
#include "gemm_launch.hpp"

namespace gemm {

namespace {

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void_g_t;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2_g_t;

constexpr int GBN = 64, GBK = 64;                        // tile columns; K block = scale block
constexpr int GNW = 4;                                   // waves, each its own K blocks
constexpr int GSTG = 4;                                  // LDS stages per wave
constexpr int GB_WAVE = GBK * GBN;                       // bytes of B per wave and stage (4 KiB)
constexpr int GB_BLK = GB_WAVE / 1024;                   // 1 KiB loads per wave and stage
constexpr int GMAX_KBLOCKS = 2048;                       // scale row / column staged in LDS

template <int TAG, int BYTES>
__shared__ __attribute__((aligned(1024))) uint8_t g_stage[BYTES];

// A rows are 64 bytes (4 chunks): the swizzle of the large-tile kernel's A rows.
__host__ __device__ __forceinline__ int gswz_a(int row) { return ((row >> 1) ^ (row >> 2)) & 3; }
// B rows are 64 bytes (4 chunks).  A transposing read of a 16-lane group covers
// 8 consecutive rows x 16 bytes, and the neighbouring group the next 16 bytes of
// the same rows: rows r and r + 4 share banks, so rows with bit 2 set have their
// chunks moved by two.
__host__ __device__ __forceinline__ int gswz_b(int k) { return ((k >> 2) & 1) << 1; }

// s_waitcnt vmcnt(N) lgkmcnt(0): this wave's global->LDS loads but the last N
// have landed, and its LDS reads have all returned (a stage may be refilled).
template <int N>
__device__ __forceinline__ void g_wait()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));
}

// One 16-byte global -> LDS load per lane (lane t's bytes land at lds + 16t).
__device__ __forceinline__ void g_dma16(const void *src, uint8_t *lds)
{
    __builtin_amdgcn_global_load_lds(src, (lds_void_g_t *)lds, 16, 0, 0);
}

// This workgroup's A and B arrays of stage S (A stages first, then B).
template <int S, int TBM>
__device__ __forceinline__ uint8_t *ga_stage() { return g_stage<S, GNW * TBM * GBK>; }
template <int S>
__device__ __forceinline__ uint8_t *gb_stage() { return g_stage<GSTG + S, GNW * GB_WAVE>; }

// EPI: the fused epilogue on the reduced fp32 sums before rounding (the thread
// that reads an entry's prior C is the one that stores it).  TBM: 32 or 64.
template <bool GEN, bool EPI, int TBM>
__global__ void __launch_bounds__(GNW * 64)
fp8_narrow_kernel(const uint8_t *__restrict__ A, const uint8_t *__restrict__ B,
                  uint16_t *__restrict__ C, int M, int N, int K, int64_t lda, int64_t ldb,
                  int64_t ldc, const float *__restrict__ scale_a,
                  const float *__restrict__ scale_b, int kblocks, int nblocks, int tiles_n,
                  Epilogue epi)
{
    static_assert(TBM == 32 || TBM == 64, "tile rows");
    constexpr int GA_WAVE = TBM * GBK;                   // bytes of A per wave and stage
    constexpr int GA_BLK = GA_WAVE / 1024;               // 1 KiB loads per wave and stage
    constexpr int GBLK = GA_BLK + GB_BLK;
    constexpr int FM = TBM / 32;                         // 32-row MFMA tiles
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, half = lane >> 5;
    // Consecutive workgroups take consecutive column tiles of one row strip.
    const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
    const int m0 = tm * TBM, n0 = tn * GBN;

    // The tile's scale row of A (scale block m0/64, all K blocks) and scale
    // column of B (scale block n0/64), staged once.
    __shared__ float s_a[GMAX_KBLOCKS], s_b[GMAX_KBLOCKS];
    {
        const float *ra = scale_a + (int64_t)(m0 / 64) * kblocks;
        const float *cb = scale_b + n0 / 64;
        for (int q = tid; q < kblocks; q += GNW * 64) {
            s_a[q] = ra[q];
            s_b[q] = cb[(int64_t)q * nblocks];
        }
    }

    // Load sources: 1 KiB block j of A is rows 16j .. 16j+15 (lane -> row 16j +
    // lane/4, slot lane%4 holding logical chunk slot ^ gswz_a(row)); block j of
    // B is K rows 16j .. 16j+15 of the 64 columns, slot lane%4 holding logical
    // chunk slot ^ gswz_b(row).
    uint32_t a_off[GA_BLK], b_off_g[GB_BLK];
#pragma unroll
    for (int j = 0; j < GA_BLK; ++j) {
        const int row = 16 * j + (lane >> 2);
        const int lrow = GEN && m0 + row >= M ? M - 1 - m0 : row;
        a_off[j] = (uint32_t)(lrow * lda + 16 * ((lane & 3) ^ gswz_a(row)));
    }
#pragma unroll
    for (int j = 0; j < GB_BLK; ++j) {
        const int row = 16 * j + (lane >> 2);
        int col = 16 * ((lane & 3) ^ gswz_b(row));
        if (GEN) col = n0 + col >= N ? ((N - 16) & ~15) : n0 + col;
        b_off_g[j] = (uint32_t)(row * ldb + col);
    }
    const uint8_t *a_base = A + (int64_t)m0 * lda;
    const uint8_t *b_base = GEN ? B : B + n0;

    // K blocks moved LDS-direct: all of them, or (GEN) all but the last one.
    const int kdma = GEN ? kblocks - 1 : K / GBK;
    const int nsteps = wave < kdma ? (kdma - wave + GNW - 1) / GNW : 0;   // this wave's share
    // Each row strip starts its walk over K at a different block (a rotation of
    // the block order): with all strips in step, the loads in flight would sit
    // at one K offset of rows lda apart, which for power-of-two row strides
    // crowds a few HBM channels.  Workgroups go to the XCDs in turn, so with
    // one column of tiles strip tm runs on XCD tm % 8: the XCDs start 2 GNW blocks
    // apart, the strips of one XCD GNW apart (16384 x 64 x
    // 8192 from cold caches: 45.4 us with start GNW * tm, 35.2 us with this one).
    const int krot = kdma > 0 ? (int)(((int64_t)GNW * (tm / 8 + 2 * (tm % 8))) % kdma) : 0;
    const auto block_of = [&](int t) {
        int kb = wave + GNW * (t < nsteps ? t : nsteps - 1) + krot;
        return kb >= kdma ? kb - kdma : kb;
    };
    auto issue = [&](uint8_t *as, uint8_t *bs, int t) {
        const int kb = block_of(t);
        const uint8_t *ab = a_base + (int64_t)kb * GBK;
        const uint8_t *bb = b_base + (int64_t)kb * GBK * ldb;
#pragma unroll
        for (int j = 0; j < GA_BLK; ++j) g_dma16(ab + a_off[j], as + wave * GA_WAVE + 1024 * j);
#pragma unroll
        for (int j = 0; j < GB_BLK; ++j) g_dma16(bb + b_off_g[j], bs + wave * GB_WAVE + 1024 * j);
    };

    // Fragments (bytes, relative to this wave's part of a stage).  A tile i:
    // lane reads row 32i + l32, k bytes 32*half .. +31 (logical chunks 2h, 2h+1).
    // B tile j, read q: 16-lane group g, lane w: k row 32*(g/2) + 8q + w/2,
    // columns 32j + 16*(g%2) + 8*(w%2) .. +7 (rows of one read share a swizzle,
    // which depends on k % 8 only).
    int a_off0[FM], a_off1[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int row = 32 * i + l32;
        a_off0[i] = row * GBK + (((2 * half) ^ gswz_a(row)) << 4);
        a_off1[i] = row * GBK + (((2 * half + 1) ^ gswz_a(row)) << 4);
    }
    const int g = lane >> 4, w16 = lane & 15, r8 = w16 >> 1;
    int b_off_r[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int n = 32 * j + 16 * (g & 1) + 8 * (w16 & 1);
        b_off_r[j] = (32 * (g >> 1) + r8) * GBN + (((n >> 4) ^ gswz_b(r8)) << 4) + (n & 15);
    }

    f32x16 acc[FM][2];
#pragma unroll
    for (int i = 0; i < FM; ++i) acc[i][0] = acc[i][1] = f32x16{};
    // One step: the fragments of one K block of this wave's part of a stage,
    // one scaled MFMA per 32 x 32 tile into a fresh partial, then the promotion
    // by sa * sb of the block.
    auto compute = [&](const uint8_t *as, const uint8_t *bs, int kb) {
        as += wave * GA_WAVE;
        bs += wave * GB_WAVE;
        const float s = __builtin_bit_cast(
            float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, s_a[kb] * s_b[kb])));
        i32x8 af[FM], bfr[2];
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const u32x4 x0 = *reinterpret_cast<const u32x4 *>(as + a_off0[i]);
            const u32x4 x1 = *reinterpret_cast<const u32x4 *>(as + a_off1[i]);
            af[i] = i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                          (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            i32x2 r[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
                r[q] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                    (lds_i32x2_g_t *)(bs + b_off_r[j] + 8 * q * GBN));
            bfr[j] = i32x8{r[0][0], r[0][1], r[1][0], r[1][1], r[2][0], r[2][1], r[3][0], r[3][1]};
        }
        f32x16 part[FM][2];
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                part[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    bfr[j], af[i], f32x16{}, 0, 0, 0, 127, 0, 127);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    acc[i][j][e] = __builtin_fmaf(part[i][j][e], s, acc[i][j][e]);
    };

    // The staged scales are read by every wave.
    __syncthreads();
    // Step t: this wave's loads of stage t % 4 have landed once at most two
    // later steps' loads are outstanding; the stage refilled now (step t + 3)
    // was read by step t - 1, whose LDS reads have returned.  Steps past nsteps
    // re-load the last block into stages nobody reads and skip the MFMAs.
    if (nsteps > 0) {
        issue(ga_stage<0, TBM>(), gb_stage<0>(), 0);
        issue(ga_stage<1, TBM>(), gb_stage<1>(), 1);
        issue(ga_stage<2, TBM>(), gb_stage<2>(), 2);
    }
    // GEN: the last K block through registers, zero-filled past M, N and K, in
    // the layout the LDS-direct loads produce, into this wave's part of the
    // last stage (refilled only once the loop's first step has waited for these
    // reads).
    if (GEN && wave == kdma % GNW) {
        const int k0 = GBK * kdma;
        uint8_t *as = ga_stage<GSTG - 1, TBM>() + wave * GA_WAVE;
        uint8_t *bs = gb_stage<GSTG - 1>() + wave * GB_WAVE;
        constexpr int NQA = TBM * 4 / 64, NQB = GBK * 4 / 64;     // chunks per lane
        if (K >= 16) {
            // One 16-byte load inside the matrix per chunk, all in flight before
            // the first wait; zeros past M, N and K applied in registers.
            Masked16 va[NQA], vb[NQB];
#pragma unroll
            for (int i = 0; i < NQA; ++i) {
                const int q = lane + 64 * i, r = q >> 2, c = q & 3;
                va[i] = masked16_load<1>(A, lda, m0 + r, M, k0 + 16 * c, K);
            }
#pragma unroll
            for (int i = 0; i < NQB; ++i) {
                const int q = lane + 64 * i, r = q >> 2, c = q & 3;
                vb[i] = masked16_load<1>(B, ldb, k0 + r, K, n0 + 16 * c, N);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < NQA; ++i) {
                const int q = lane + 64 * i, r = q >> 2, c = q & 3;
                *reinterpret_cast<u32x4 *>(as + r * GBK + ((c ^ gswz_a(r)) << 4)) = masked16_value(va[i]);
            }
#pragma unroll
            for (int i = 0; i < NQB; ++i) {
                const int q = lane + 64 * i, r = q >> 2, c = q & 3;
                *reinterpret_cast<u32x4 *>(bs + r * GBN + ((c ^ gswz_b(r)) << 4)) = masked16_value(vb[i]);
            }
        } else {
            // K < 16: element by element.
#pragma unroll
            for (int q = lane; q < TBM * 4; q += 64) {
                const int r = q >> 2, c = q & 3;
                const int gm = m0 + r, gk = k0 + 16 * c;
                u32x4 v = u32x4{0u, 0u, 0u, 0u};
                if (gm < M) {
                    const uint8_t *src = A + (int64_t)gm * lda + gk;
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        if (gk + e < K) v[e >> 2] |= (uint32_t)src[e] << (8 * (e & 3));
                }
                *reinterpret_cast<u32x4 *>(as + r * GBK + ((c ^ gswz_a(r)) << 4)) = v;
            }
#pragma unroll
            for (int q = lane; q < GBK * 4; q += 64) {
                const int r = q >> 2, c = q & 3;
                const int gk = k0 + r, gn = n0 + 16 * c;
                u32x4 v = u32x4{0u, 0u, 0u, 0u};
                if (gk < K) {
                    const uint8_t *src = B + (int64_t)gk * ldb + gn;
                    if (gn + 16 <= N) {
                        v = *reinterpret_cast<const u32x4 *>(src);
                    } else {
#pragma unroll
                        for (int e = 0; e < 16; ++e)
                            if (gn + e < N) v[e >> 2] |= (uint32_t)src[e] << (8 * (e & 3));
                    }
                }
                *reinterpret_cast<u32x4 *>(bs + r * GBN + ((c ^ gswz_b(r)) << 4)) = v;
            }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);              // lgkmcnt(0): the LDS writes landed
        compute(ga_stage<GSTG - 1, TBM>(), gb_stage<GSTG - 1>(), kdma);
    }
    for (int t = 0; t < nsteps; t += GSTG) {
        g_wait<2 * GBLK>();
        issue(ga_stage<3, TBM>(), gb_stage<3>(), t + 3);
        compute(ga_stage<0, TBM>(), gb_stage<0>(), block_of(t));
        g_wait<2 * GBLK>();
        issue(ga_stage<0, TBM>(), gb_stage<0>(), t + 4);
        if (t + 1 < nsteps) compute(ga_stage<1, TBM>(), gb_stage<1>(), block_of(t + 1));
        g_wait<2 * GBLK>();
        issue(ga_stage<1, TBM>(), gb_stage<1>(), t + 5);
        if (t + 2 < nsteps) compute(ga_stage<2, TBM>(), gb_stage<2>(), block_of(t + 2));
        g_wait<2 * GBLK>();
        issue(ga_stage<2, TBM>(), gb_stage<2>(), t + 6);
        if (t + 3 < nsteps) compute(ga_stage<3, TBM>(), gb_stage<3>(), block_of(t + 3));
    }
    g_wait<0>();

    // Partial tiles into LDS: 32-row tile i of this wave goes to the wave's own
    // 4 KiB parts of B stages 2i and 2i + 1 (16 rows of 64 floats each; 16-byte
    // chunk index XOR row, so the rows one store touches spread over the
    // banks).  Lane l holds row l%32 of the tile, columns 32j + 8q + 4*(l/32)
    // .. +3.
    const auto part_row = [&](auto I, int row) -> float * {
        constexpr int S0 = 2 * I;
        uint8_t *base = row < 16 ? gb_stage<S0>() : gb_stage<S0 + 1>();
        return reinterpret_cast<float *>(base + wave * GB_WAVE) + (row & 15) * GBN;
    };
    const auto store_partial = [&](auto I) {
        float *mine = part_row(I, l32);
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int chunk = (8 * j + 2 * q + half) ^ (l32 & 15);
                *reinterpret_cast<f32x4 *>(mine + 4 * chunk) =
                    f32x4{acc[I][j][4 * q], acc[I][j][4 * q + 1], acc[I][j][4 * q + 2],
                          acc[I][j][4 * q + 3]};
            }
    };
    store_partial(std::integral_constant<int, 0>{});
    if constexpr (FM == 2) store_partial(std::integral_constant<int, 1>{});
    __syncthreads();
    // Thread t sums row t/8 of each 32-row tile, columns 8(t%8) .. +7, over the
    // four partials (in wave order), then applies the epilogue, rounds and stores.
    const int rr = tid >> 3, c8 = tid & 7;
    const auto finish = [&](auto I) {
        constexpr int S0 = 2 * I;
        const int row = 32 * I + rr;
        const uint8_t *base = rr < 16 ? gb_stage<S0>() : gb_stage<S0 + 1>();
        float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < GNW; ++w) {
            const float *part = reinterpret_cast<const float *>(base + w * GB_WAVE) + (rr & 15) * GBN;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const f32x4 v = *reinterpret_cast<const f32x4 *>(part + 4 * ((2 * c8 + h) ^ (rr & 15)));
#pragma unroll
                for (int e = 0; e < 4; ++e) s[4 * h + e] += v[e];
            }
        }
        if (GEN && m0 + row >= M) return;
        uint16_t *rowp = C + (int64_t)(m0 + row) * ldc;
        const int gn = n0 + 8 * c8;
        const int cnt = GEN ? N - gn : 8;
        if constexpr (EPI) epilogue_row<OUT_BF16, 8>(epi, s, rowp, gn, cnt);
        const u32x4 out{pack2<true>(s[0], s[1]), pack2<true>(s[2], s[3]), pack2<true>(s[4], s[5]),
                        pack2<true>(s[6], s[7])};
        if (!GEN || cnt >= 8) {
            *reinterpret_cast<u32x4 *>(rowp + gn) = out;
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (e < cnt) rowp[gn + e] = (uint16_t)(out[e >> 1] >> (16 * (e & 1)));
        }
    };
    finish(std::integral_constant<int, 0>{});
    if constexpr (FM == 2) finish(std::integral_constant<int, 1>{});
}

}  // namespace

// Whole tiles (32 or 64 rows x 64), K in whole 64-wide blocks with at least one
// per wave, 16-byte aligned rows, per-lane 32-bit offsets that fit (64 rows of
// A or B past a base), and a scale row that fits the LDS staging.
static bool fp8_narrow_whole(const Problem &p, int tbm)
{
    return p.aligned && p.M % tbm == 0 && p.N % GBN == 0 && p.K % GBK == 0 &&
           p.K >= GBK * GNW && p.K / GBK <= GMAX_KBLOCKS && p.lda < (1 << 25) &&
           p.ldb < (1 << 25);
}

// The guarded instantiation: any M, N >= 16 (a clamped column chunk starts at
// N - 16 rounded down to a multiple of 16), any K >= 1 up to the staged scale row, any leading dimensions with
// 32-bit per-lane offsets.
bool fp8_narrow_general_eligible(const Problem &p)
{
    return p.M >= 1 && p.N >= 16 && p.K >= 1 && (p.K + GBK - 1) / GBK <= GMAX_KBLOCKS &&
           p.lda < (1 << 25) && (int64_t)GBK * p.ldb + p.N < ((int64_t)1 << 32);
}

template <bool GEN, bool EPI, int TBM>
static hipError_t fp8_narrow_typed(const Problem &p, const float *scale_a, const float *scale_b)
{
    const int tiles_n = (p.N + GBN - 1) / GBN;
    const int64_t nwg = (int64_t)((p.M + TBM - 1) / TBM) * tiles_n;
    if (nwg > 0x7fffffff) return hipErrorInvalidValue;
    const int kblocks = (p.K + GBK - 1) / GBK, nblocks = (p.N + 63) / 64;
    const uint8_t *A = static_cast<const uint8_t *>(p.A), *B = static_cast<const uint8_t *>(p.B);
    uint16_t *C = static_cast<uint16_t *>(p.C);
    const Epilogue epi = p.epi ? *p.epi : Epilogue{1.f, 0.f, nullptr, 0};
    hipLaunchKernelGGL((fp8_narrow_kernel<GEN, EPI, TBM>), dim3((unsigned)nwg), dim3(GNW * 64), 0,
                       p.stream, A, B, C, p.M, p.N, p.K, p.lda, p.ldb, p.ldc, scale_a, scale_b,
                       kblocks, nblocks, tiles_n, epi);
    return hipGetLastError();
}

template <int TBM>
static hipError_t fp8_narrow_dispatch(bool gen, const Problem &p, const float *sa, const float *sb)
{
    if (gen)
        return p.epi ? fp8_narrow_typed<true, true, TBM>(p, sa, sb)
                     : fp8_narrow_typed<true, false, TBM>(p, sa, sb);
    return p.epi ? fp8_narrow_typed<false, true, TBM>(p, sa, sb)
                 : fp8_narrow_typed<false, false, TBM>(p, sa, sb);
}

// tbm: 32 or 64 tile rows; force_general: the guarded instantiation even for
// whole tiles.
hipError_t fp8_narrow_launch(const Problem &p, const float *scale_a, const float *scale_b, int tbm,
                             bool force_general)
{
    if (tbm != 32 && tbm != 64) return hipErrorInvalidValue;
    const bool whole = !force_general && fp8_narrow_whole(p, tbm);
    if (!whole && !fp8_narrow_general_eligible(p)) return hipErrorInvalidValue;
    return tbm == 32 ? fp8_narrow_dispatch<32>(!whole, p, scale_a, scale_b)
                     : fp8_narrow_dispatch<64>(!whole, p, scale_a, scale_b);
}

}  // namespace gemm
