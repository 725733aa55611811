// fp32 SGEMM for small and narrow grids: C = A * B with 32 x 64 or 64 x 64 tiles
// of C whose K sum is split over the workgroup's waves.
//
// Below about 128 tiles of 128 x 128 a one-workgroup-per-tile kernel leaves
// most SIMDs without a second wave and walks K serially, so every load latency
// is exposed (8192 x 64 x 4096: 4.3 GFLOP, 27 us at the fp32 MFMA peak).  Here
// a workgroup owns a TBM x 64 tile (TBM = 32 or 64) and its 4 waves split K:
// wave w takes the 32-wide K blocks w, w + 4, w + 8, ... (the four waves together
// read 512 contiguous bytes of every A row per round), each row strip starting
// its walk at its own K block.  Each wave streams its blocks of A (TBM x 32
// floats, 128-byte rows) and B (32 x 64 floats, 256-byte rows) through a private
// ring of LDS stages with global_load_lds_dwordx4 and waits only for its own
// loads: the main loop has no workgroup barrier.  The four fp32 partial tiles
// are added through LDS at the end.
//
// A 32-float K block of fp32 is 128 bytes per row, as a 64-element block of
// fp16/bf16 is, so the stage sizes are those of the half-precision narrow
// kernel: 3 stages per wave with 32-row tiles (144 KiB of LDS), 2 with 64-row
// tiles (128 KiB).  MFMA: v_mfma_f32_32x32x2_f32 as in the large-tile fp32
// kernel (one 16-byte LDS read of A feeds four MFMAs, the lanes of the two
// half-waves taking k and k + 4; B read as single floats), with its two-level
// accumulation: each K block is summed into a fresh partial that is then added
// to the wave's running total.
//
// GEN = true takes any M, N >= 4, K >= 1 and any leading dimensions: A rows past
// M are clamped to row M-1 and B column chunks starting past N to the last whole
// chunk at a multiple of 4 columns (their products only reach C entries that are not stored; a chunk
// straddling N reads a few floats past N inside a row that is not B's last);
// the last K block, possibly partial, is loaded through registers with zero
// fill by the wave whose turn it would be, so no LDS-direct load touches B's
// last row; stores are masked to the M x N window.  The hardware runs in
// unaligned-access mode, so 16-byte loads and stores at 4-byte-aligned
// addresses are legal.
//
// The split of the K sum into separately accumulated blocks that are added at
// the end is the "K split" of the register-tiled GEMM in "CUDA GEMM 优化实践笔记";
// here it runs inside one workgroup.
#include <type_traits>

#include "gemm_device.hpp"
#include "gemm_launch.hpp"

namespace gemm {

namespace {

typedef __attribute__((address_space(3))) void lds_void_f_t;

constexpr int FBN = 64, FBK = 32;
constexpr int FNW = 4;                                   // waves, each its own K blocks
constexpr int FB_WAVE = FBK * FBN;                       // floats of B per wave and stage (8 KiB)
constexpr int FB_BLK = FB_WAVE * 4 / 1024;               // 1 KiB loads per wave and stage

template <int TAG, int FLOATS>
__shared__ __attribute__((aligned(1024))) float fl_stage[FLOATS];

// B rows are 256 bytes (16 chunks).  A single-float read covers 32 columns
// (128 bytes) of row k in one half-wave and of row k + 4 in the other: rows
// with bit 2 set have their chunks moved by 128 bytes, so the halves use
// different banks.
__host__ __device__ __forceinline__ int swz_fb(int k) { return ((k >> 2) & 1) << 3; }

// s_waitcnt vmcnt(N) lgkmcnt(0): this wave's global->LDS loads but the last N
// have landed, and its LDS reads have all returned (a stage may be refilled).
template <int N>
__device__ __forceinline__ void f_wait()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));
}

// One 16-byte global -> LDS load per lane (lane t's bytes land at lds + 16t).
// (A function of its own: called with template-dependent arguments inside the
// kernel's lambdas, the builtin would leave the host-side instantiation of the
// kernel invalid and its launch stub undefined.)
__device__ __forceinline__ void f_dma16(const void *src, float *lds)
{
    __builtin_amdgcn_global_load_lds(src, (lds_void_f_t *)lds, 16, 0, 0);
}

// This workgroup's A and B arrays of stage S (A stages first, then B).
template <int S, int TBM>
__device__ __forceinline__ float *fa_stage() { return fl_stage<S, FNW * TBM * FBK>; }
template <int S, int STG>
__device__ __forceinline__ float *fb_stage() { return fl_stage<STG + S, FNW * FB_WAVE>; }

// EPI: the fused epilogue is applied to the reduced sums by the thread that
// stores them.  TBM: tile rows (32 or 64); STG: LDS stages per wave (3 or 2).
template <bool GEN, bool EPI, int TBM, int STG>
__global__ void __launch_bounds__(FNW * 64)
f32_narrow_kernel(const float *__restrict__ A, const float *__restrict__ B, float *__restrict__ C,
                  int M, int N, int K, int64_t lda, int64_t ldb, int64_t ldc, int tiles_n,
                  Epilogue epi)
{
    static_assert((TBM == 32 && STG == 3) || (TBM == 64 && STG == 2), "narrow shapes");
    constexpr int FA_WAVE = TBM * FBK;                   // floats of A per wave and stage
    constexpr int FA_BLK = FA_WAVE * 4 / 1024;           // 1 KiB loads per wave and stage
    constexpr int FBLK = FA_BLK + FB_BLK;
    constexpr int FM = TBM / 32;                         // 32-row MFMA tiles
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, half = lane >> 5;
    // Consecutive workgroups take consecutive column tiles of one row strip:
    // the strip's A rows are fetched from HBM once and shared through L2.
    const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
    const int m0 = tm * TBM, n0 = tn * FBN;

    // Load sources: 1 KiB block j of A is rows 8j .. 8j+7 (lane -> row 8j +
    // lane/8, slot lane%8 holding logical chunk slot ^ swz8(row)); block j of B
    // is K rows 4j .. 4j+3 of the 64 columns (lane -> row 4j + lane/16, slot
    // lane%16 holding logical chunk slot ^ swz_fb(row)).
    uint32_t a_off[FA_BLK], b_off_g[FB_BLK];
#pragma unroll
    for (int j = 0; j < FA_BLK; ++j) {
        const int row = 8 * j + (lane >> 3);
        const int lrow = GEN && m0 + row >= M ? M - 1 - m0 : row;
        a_off[j] = (uint32_t)(lrow * lda + 4 * ((lane & 7) ^ swz8(row))) * 4u;
    }
#pragma unroll
    for (int j = 0; j < FB_BLK; ++j) {
        const int row = 4 * j + (lane >> 4);
        int col = 4 * ((lane & 15) ^ swz_fb(row));
        if (GEN) col = n0 + col >= N ? ((N - 4) & ~3) : n0 + col;
        b_off_g[j] = (uint32_t)(row * ldb + col) * 4u;
    }
    const char *a_base = reinterpret_cast<const char *>(A + (int64_t)m0 * lda);
    const char *b_base = reinterpret_cast<const char *>(GEN ? B : B + n0);

    // K blocks moved LDS-direct: all of them, or (GEN) all but the last one.
    const int kdma = GEN ? (K + FBK - 1) / FBK - 1 : K / FBK;
    const int nsteps = wave < kdma ? (kdma - wave + FNW - 1) / FNW : 0;   // this wave's share
    // Each row strip starts its walk over K at a different block (a rotation of
    // the block order, so every block is still summed once): with all strips in
    // step, the loads in flight would sit at one K offset of rows lda apart,
    // which for power-of-two row strides crowds a few HBM channels.  Workgroups
    // go to the XCDs in turn, so with one column of tiles strip tm runs on XCD
    // tm % 8: the XCDs start 2 FNW blocks apart, the strips of one XCD FNW apart.
    const int krot = kdma > 0 ? (int)(((int64_t)FNW * (tm / 8 + 2 * (tm % 8))) % kdma) : 0;
    auto issue = [&](float *as, float *bs, int t) {
        int kb = wave + FNW * (t < nsteps ? t : nsteps - 1) + krot;
        if (kb >= kdma) kb -= kdma;
        const char *ab = a_base + (int64_t)kb * FBK * 4;
        const char *bb = b_base + (int64_t)kb * FBK * ldb * 4;
#pragma unroll
        for (int j = 0; j < FA_BLK; ++j)
            f_dma16(ab + a_off[j], as + wave * FA_WAVE + 256 * j);
#pragma unroll
        for (int j = 0; j < FB_BLK; ++j)
            f_dma16(bb + b_off_g[j], bs + wave * FB_WAVE + 256 * j);
    };

    // Fragments (floats, relative to this wave's part of a stage).  Sub-step s
    // covers k = 8s .. 8s+7; the e-th MFMA of it takes k = 8s + 4*half + e in
    // both operands: A as one 16-byte read of row 32i + l32, B as single floats
    // of column 32j + l32.
    int a_row[FM], a_sw[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        a_row[i] = (32 * i + l32) * FBK;
        a_sw[i] = swz8(32 * i + l32);
    }
    f32x16 total[FM][2];
#pragma unroll
    for (int i = 0; i < FM; ++i) total[i][0] = total[i][1] = f32x16{};
    auto compute = [&](const float *as, const float *bs) {
        as += wave * FA_WAVE;
        bs += wave * FB_WAVE;
        f32x4 af[FBK / 8][FM];
        float bv[FBK / 8][2][4];
#pragma unroll
        for (int s = 0; s < FBK / 8; ++s) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
                af[s][i] = *reinterpret_cast<const f32x4 *>(as + a_row[i] + (((2 * s + half) ^ a_sw[i]) << 2));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int k = 8 * s + 4 * half + e;
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int n = 32 * j + l32;
                    bv[s][j][e] = bs[k * FBN + (((n >> 2) ^ swz_fb(k)) << 2) + (n & 3)];
                }
            }
        }
        f32x16 part[FM][2];
#pragma unroll
        for (int i = 0; i < FM; ++i) part[i][0] = part[i][1] = f32x16{};
#pragma unroll
        for (int s = 0; s < FBK / 8; ++s)
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        part[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(bv[s][j][e], af[s][i][e],
                                                                         part[i][j], 0, 0, 0);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) total[i][j] += part[i][j];
    };

    // Step t: this wave's loads of stage t % STG have landed once at most
    // STG - 2 later steps' loads are outstanding; the stage refilled now (step
    // t + STG - 1) was read by step t - 1, whose LDS reads have returned.
    // Steps past nsteps re-load the last block into stages nobody reads and
    // skip the MFMAs.
    if (nsteps > 0) {
        issue(fa_stage<0, TBM>(), fb_stage<0, STG>(), 0);
        if constexpr (STG == 3) issue(fa_stage<1, TBM>(), fb_stage<1, STG>(), 1);
    }
    // GEN: the last K block through registers, zero-filled past M, N and K, in
    // the layout the LDS-direct loads produce, into this wave's part of the
    // last stage (refilled only once the loop's first step has waited for
    // these reads).
    if (GEN && wave == kdma % FNW) {
        const int k0 = FBK * kdma;
        float *as = fa_stage<STG - 1, TBM>() + wave * FA_WAVE;
        float *bs = fb_stage<STG - 1, STG>() + wave * FB_WAVE;
        constexpr int NQA = TBM * FBK / 4 / 64, NQB = FBK * FBN / 4 / 64;   // chunks per lane
        if (K >= 4) {
            // One 16-byte load inside the matrix per chunk, all in flight before
            // the first wait; zeros past M, N and K applied in registers.
            Masked16 va[NQA], vb[NQB];
#pragma unroll
            for (int i = 0; i < NQA; ++i) {
                const int q = lane + 64 * i, r = q >> 3, c = q & 7;
                va[i] = masked16_load<4>(A, lda, m0 + r, M, k0 + 4 * c, K);
            }
#pragma unroll
            for (int i = 0; i < NQB; ++i) {
                const int q = lane + 64 * i, r = q >> 4, c = q & 15;
                vb[i] = masked16_load<4>(B, ldb, k0 + r, K, n0 + 4 * c, N);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < NQA; ++i) {
                const int q = lane + 64 * i, r = q >> 3, c = q & 7;
                *reinterpret_cast<f32x4 *>(as + r * FBK + ((c ^ swz8(r)) << 2)) =
                    __builtin_bit_cast(f32x4, masked16_value(va[i]));
            }
#pragma unroll
            for (int i = 0; i < NQB; ++i) {
                const int q = lane + 64 * i, r = q >> 4, c = q & 15;
                *reinterpret_cast<f32x4 *>(bs + r * FBN + ((c ^ swz_fb(r)) << 2)) =
                    __builtin_bit_cast(f32x4, masked16_value(vb[i]));
            }
        } else {
            // K < 4: element by element.
#pragma unroll
            for (int q = lane; q < TBM * FBK / 4; q += 64) {
                const int r = q >> 3, c = q & 7;
                const int gm = m0 + r, gk = k0 + 4 * c;
                f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
                if (gm < M) {
                    const float *src = A + (int64_t)gm * lda + gk;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (gk + e < K) v[e] = src[e];
                }
                *reinterpret_cast<f32x4 *>(as + r * FBK + ((c ^ swz8(r)) << 2)) = v;
            }
#pragma unroll
            for (int q = lane; q < FBK * FBN / 4; q += 64) {
                const int r = q >> 4, c = q & 15;
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
                *reinterpret_cast<f32x4 *>(bs + r * FBN + ((c ^ swz_fb(r)) << 2)) = v;
            }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);              // lgkmcnt(0): the LDS writes landed
        compute(fa_stage<STG - 1, TBM>(), fb_stage<STG - 1, STG>());
    }
    if constexpr (STG == 3) {
        for (int t = 0; t < nsteps; t += 3) {
            f_wait<FBLK>();
            issue(fa_stage<2, TBM>(), fb_stage<2, STG>(), t + 2);
            compute(fa_stage<0, TBM>(), fb_stage<0, STG>());
            f_wait<FBLK>();
            issue(fa_stage<0, TBM>(), fb_stage<0, STG>(), t + 3);
            if (t + 1 < nsteps) compute(fa_stage<1, TBM>(), fb_stage<1, STG>());
            f_wait<FBLK>();
            issue(fa_stage<1, TBM>(), fb_stage<1, STG>(), t + 4);
            if (t + 2 < nsteps) compute(fa_stage<2, TBM>(), fb_stage<2, STG>());
        }
    } else {
        for (int t = 0; t < nsteps; t += 2) {
            f_wait<0>();
            issue(fa_stage<1, TBM>(), fb_stage<1, STG>(), t + 1);
            compute(fa_stage<0, TBM>(), fb_stage<0, STG>());
            f_wait<0>();
            issue(fa_stage<0, TBM>(), fb_stage<0, STG>(), t + 2);
            if (t + 1 < nsteps) compute(fa_stage<1, TBM>(), fb_stage<1, STG>());
        }
    }
    f_wait<0>();

    // Partial tiles into LDS: 32-row tile i of every wave goes to B stage i
    // (this wave's own 8 KiB of it as 32 rows of 64 floats; 16-byte chunk index
    // XOR row, so the 32 rows one store touches spread over the banks).  Lane l
    // holds row l%32 of the tile, columns 32j + 8q + 4*(l/32) .. +3.
    const auto store_partial = [&](auto I) {
        float *mine = fb_stage<I, STG>() + wave * (32 * FBN);
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int chunk = (8 * j + 2 * q + half) ^ (l32 & 15);
                *reinterpret_cast<f32x4 *>(mine + l32 * FBN + 4 * chunk) =
                    f32x4{total[I][j][4 * q], total[I][j][4 * q + 1], total[I][j][4 * q + 2],
                          total[I][j][4 * q + 3]};
            }
    };
    store_partial(std::integral_constant<int, 0>{});
    if constexpr (FM == 2) store_partial(std::integral_constant<int, 1>{});
    __syncthreads();
    // Thread t sums row t/8 of each 32-row tile, columns 8(t%8) .. +7, over the
    // four partials (in wave order), then applies the epilogue and stores.
    const int rr = tid >> 3, c8 = tid & 7;
    const auto finish = [&](auto I) {
        const int row = 32 * I + rr;
        const float *red = fb_stage<I, STG>();
        float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < FNW; ++w) {
            const float *part = red + w * (32 * FBN) + rr * FBN;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const f32x4 v = *reinterpret_cast<const f32x4 *>(part + 4 * ((2 * c8 + h) ^ (rr & 15)));
#pragma unroll
                for (int e = 0; e < 4; ++e) s[4 * h + e] += v[e];
            }
        }
        if (GEN && m0 + row >= M) return;
        float *rowp = C + (int64_t)(m0 + row) * ldc;
        const int gn = n0 + 8 * c8;
        const int cnt = GEN ? N - gn : 8;
        if constexpr (EPI) epilogue_row<OUT_F32, 8>(epi, s, rowp, gn, cnt);
        if (!GEN || cnt >= 8) {
            *reinterpret_cast<f32x4 *>(rowp + gn) = f32x4{s[0], s[1], s[2], s[3]};
            *reinterpret_cast<f32x4 *>(rowp + gn + 4) = f32x4{s[4], s[5], s[6], s[7]};
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (e < cnt) rowp[gn + e] = s[e];
        }
    };
    finish(std::integral_constant<int, 0>{});
    if constexpr (FM == 2) finish(std::integral_constant<int, 1>{});
}

}  // namespace

// Whole tiles (32 or 64 rows x 64), K in whole 32-wide blocks with at least one
// per wave, 16-byte aligned rows, and per-lane 32-bit byte offsets that fit
// (64 rows of A, 32 rows of B past a base).
static bool f32_narrow_whole(const Problem &p, int tbm)
{
    return p.aligned && p.M % tbm == 0 && p.N % FBN == 0 && p.K % FBK == 0 && p.K >= FBK * FNW &&
           p.lda < (1 << 24) && p.ldb < (1 << 24);
}

// The guarded instantiation: any M, N >= 4 (a clamped column chunk starts at
// N-4 rounded down to a multiple of 4), any K >= 1, any leading dimensions with 32-bit per-lane byte offsets.
bool f32_narrow_general_eligible(const Problem &p)
{
    return p.M >= 1 && p.N >= 4 && p.K >= 1 && p.lda < (1 << 24) &&
           (int64_t)FBK * p.ldb + p.N < ((int64_t)1 << 30);
}

template <bool GEN, bool EPI, int TBM>
static hipError_t f32_narrow_typed(const Problem &p)
{
    constexpr int STG = TBM == 32 ? 3 : 2;
    const int tiles_n = (p.N + FBN - 1) / FBN;
    const int64_t nwg = (int64_t)((p.M + TBM - 1) / TBM) * tiles_n;
    if (nwg > 0x7fffffff) return hipErrorInvalidValue;
    const float *A = static_cast<const float *>(p.A), *B = static_cast<const float *>(p.B);
    float *C = static_cast<float *>(p.C);
    const Epilogue epi = p.epi ? *p.epi : Epilogue{1.f, 0.f, nullptr, 0};
    hipLaunchKernelGGL((f32_narrow_kernel<GEN, EPI, TBM, STG>), dim3((unsigned)nwg),
                       dim3(FNW * 64), 0, p.stream, A, B, C, p.M, p.N, p.K, p.lda, p.ldb, p.ldc,
                       tiles_n, epi);
    return hipGetLastError();
}

template <int TBM>
static hipError_t f32_narrow_dispatch(bool gen, const Problem &p)
{
    if (gen)
        return p.epi ? f32_narrow_typed<true, true, TBM>(p) : f32_narrow_typed<true, false, TBM>(p);
    return p.epi ? f32_narrow_typed<false, true, TBM>(p) : f32_narrow_typed<false, false, TBM>(p);
}

// tbm: 32 or 64 tile rows; force_general: the guarded instantiation even for
// whole tiles.
hipError_t f32_narrow_launch(const Problem &p, int tbm, bool force_general)
{
    if (tbm != 32 && tbm != 64) return hipErrorInvalidValue;
    const bool whole = !force_general && f32_narrow_whole(p, tbm);
    if (!whole && !f32_narrow_general_eligible(p)) return hipErrorInvalidValue;
    return tbm == 32 ? f32_narrow_dispatch<32>(!whole, p) : f32_narrow_dispatch<64>(!whole, p);
}

}  // namespace gemm
