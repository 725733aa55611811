// fp16 / bf16 GEMM for tall, narrow products (N a multiple of 64 up to a few
// hundred, M large): C = A * B with whole 32 x 64 tiles of C, K a multiple of
// 64, 16-byte aligned operands.
//
// With N = 64 a 256 x 256 tiling leaves most of the chip idle and the product is
// bound by reading A once from HBM (8192 x 64 x 4096: 64 MiB of A against
// 4.3 GFLOP).  Here a workgroup owns a 32 x 64 tile of C, so M = 8192 already
// gives 256 workgroups, and its 4 waves split K among themselves: wave w takes
// the 64-wide K blocks w, w + 4, w + 8, ... (the four waves together read 512
// contiguous bytes of every A row per round; each row strip starts at its own
// K block).  Each wave streams its own blocks
// of A (32 x 64) and B (64 x 64) through a private ring of LDS stages with
// global_load_lds_dwordx4 and waits only for its own loads, so the main loop
// has no workgroup barrier at all.  At the end the four fp32 partial tiles are
// added through LDS and the sum is rounded and stored as whole 128-byte rows.
//
// GEN = true takes any M, N >= 8, K >= 1 and any leading dimensions (used for
// the few rows left over below a grid of 256 x 256 tiles): A rows past M are
// clamped to row M-1 and B column chunks starting past N to the last whole
// chunk at a multiple of 8 columns (their products only reach C entries that are not stored); the last K block,
// possibly partial, is loaded through registers with zero fill by the wave whose
// turn it would be, so no LDS-direct load touches B's last row; stores are
// masked to the M x N window.  The hardware runs in unaligned-access mode, so
// the 16-byte loads and stores at 2-byte-aligned addresses are legal.
//
// The split of the K sum into per-wave partials is the "K split" of the
// register-tiled GEMM in "CUDA GEMM 优化实践笔记" (blocks of K accumulated
// separately, then added), here inside one workgroup; operand movement and
// fragment reads are those of the large-tile kernel (gemm_h16_fast.hip).
#include <type_traits>

#include "gemm_device.hpp"
#include "gemm_launch.hpp"

namespace gemm {

namespace {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_n_t;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_n_t;

// Two shapes of the same kernel: 32 x 64 tiles with a 3-stage ring per wave
// (144 KiB of LDS), and 64 x 64 tiles with a 2-stage ring (128 KiB) for grids
// that would need a second round of 32-row tiles (one workgroup per CU either
// way): 1000^3 has 512 tiles of 32 x 64 but 256 of 64 x 64.
constexpr int NBN = 64, NBK = 64;
constexpr int NNW = 4;                                   // waves, each its own K blocks
constexpr int NB_WAVE = NBK * NBN;                       // halves of B per wave and stage (8 KiB)
constexpr int NB_BLK = NB_WAVE * 2 / 1024;               // 1 KiB loads per wave and stage

template <int TAG, int HALVES>
__shared__ __attribute__((aligned(1024))) uint16_t nl_stage[HALVES];

// B rows are 128 bytes (8 chunks).  One transposing read of a 16-lane group
// covers 4 consecutive rows x 32 bytes and two groups read the same rows at
// the next 32 bytes: moving rows with bit 1 set by 64 bytes puts the 4 rows x 64
// bytes of a lane pair-of-groups on distinct banks.
__host__ __device__ __forceinline__ int swz_nb(int k) { return ((k >> 1) & 1) << 2; }

// s_waitcnt vmcnt(N) lgkmcnt(0): this wave's global->LDS loads but the last N
// have landed, and its LDS reads have all returned (a stage may be refilled).
template <int N>
__device__ __forceinline__ void n_wait()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));
}

// One 16-byte global -> LDS load per lane (lane t's bytes land at lds + 16t).
// (A function of its own: with arguments that depend on the kernel's template
// parameters, the builtin called directly in the kernel's lambdas leaves the
// host-side instantiation of the kernel invalid and its launch stub undefined.)
__device__ __forceinline__ void n_dma16(const void *src, uint16_t *lds)
{
    __builtin_amdgcn_global_load_lds(src, (lds_void_n_t *)lds, 16, 0, 0);
}

// This workgroup's A and B arrays of stage S (A stages first, then B).
template <int S, int TBM>
__device__ __forceinline__ uint16_t *a_stage() { return nl_stage<S, NNW * TBM * NBK>; }
template <int S, int STG>
__device__ __forceinline__ uint16_t *b_stage() { return nl_stage<STG + S, NNW * NB_WAVE>; }

// EPI: the fused epilogue is applied to the reduced fp32 sums before rounding
// (the thread that reads an entry's prior C is the one that stores it).
// TBM: tile rows (32 or 64); STG: LDS stages per wave (3 or 2).
template <bool IS_BF16, bool GEN, bool EPI, int TBM, int STG>
__global__ void __launch_bounds__(NNW * 64)
h16_narrow_kernel(const uint16_t *__restrict__ A, const uint16_t *__restrict__ B,
                  uint16_t *__restrict__ C, int M, int N, int K, int64_t lda, int64_t ldb,
                  int64_t ldc, int tiles_n, Epilogue epi)
{
    static_assert((TBM == 32 && STG == 3) || (TBM == 64 && STG == 2), "narrow shapes");
    constexpr int NBM = TBM;
    constexpr int NA_WAVE = NBM * NBK;                   // halves of A per wave and stage
    constexpr int NA_BLK = NA_WAVE * 2 / 1024;           // 1 KiB loads per wave and stage
    constexpr int NBLK_N = NA_BLK + NB_BLK;
    constexpr int FM = NBM / 32;                         // 32-row MFMA tiles
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, half = lane >> 5;
    // Consecutive workgroups take consecutive column tiles of one row strip:
    // the strip's A rows are fetched from HBM once and shared through L2.
    const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
    const int m0 = tm * NBM, n0 = tn * NBN;

    // Load sources: 1 KiB block j of A is rows 8j .. 8j+7 (lane -> row 8j +
    // lane/8, slot lane%8 holding logical chunk slot ^ swz8(row)); block j of B
    // is K rows 8j .. 8j+7 of the 64 columns, slot lane%8 holding logical chunk
    // slot ^ swz_nb(row).
    uint32_t a_off[NA_BLK], b_off_g[NB_BLK];
#pragma unroll
    for (int j = 0; j < NA_BLK; ++j) {
        const int row = 8 * j + (lane >> 3);
        const int lrow = GEN && m0 + row >= M ? M - 1 - m0 : row;
        a_off[j] = (uint32_t)(lrow * lda + 8 * ((lane & 7) ^ swz8(row))) * 2u;
    }
#pragma unroll
    for (int j = 0; j < NB_BLK; ++j) {
        const int row = 8 * j + (lane >> 3);
        int col = 8 * ((lane & 7) ^ swz_nb(row));
        if (GEN) col = n0 + col >= N ? ((N - 8) & ~7) : n0 + col;
        b_off_g[j] = (uint32_t)(row * ldb + col) * 2u;
    }
    const char *a_base = reinterpret_cast<const char *>(A + (int64_t)m0 * lda);
    const char *b_base = reinterpret_cast<const char *>(GEN ? B : B + n0);

    // K blocks moved LDS-direct: all of them, or (GEN) all but the last one.
    const int kdma = GEN ? (K + NBK - 1) / NBK - 1 : K / NBK;
    const int nsteps = wave < kdma ? (kdma - wave + NNW - 1) / NNW : 0;   // this wave's share
    // Each row strip starts its walk over K at a different block (a rotation of
    // the block order, so every block is still summed once): with all strips in
    // step, the loads in flight would sit at one K offset of rows lda apart,
    // which for power-of-two row strides crowds a few HBM channels
    // (8192 x 64 x 4096: 21.1 us in step, 14.1 us rotated).  Workgroups go to
    // the XCDs in turn, so with one column of tiles strip tm runs on XCD tm % 8;
    // the start block mixes both parts of tm: the eight XCDs start 2 NNW blocks
    // apart and the strips within one XCD NNW apart, which
    // keeps the XCDs' L2 misses apart too (16384 x 64 x 8192 from cold caches:
    // 71.5 us with start NNW * tm, 53.7 us with this one).
    const int krot = kdma > 0 ? (int)(((int64_t)NNW * (tm / 8 + 2 * (tm % 8))) % kdma) : 0;
    auto issue = [&](uint16_t *as, uint16_t *bs, int t) {
        int kb = wave + NNW * (t < nsteps ? t : nsteps - 1) + krot;
        if (kb >= kdma) kb -= kdma;
        const char *ab = a_base + (int64_t)kb * NBK * 2;
        const char *bb = b_base + (int64_t)kb * NBK * ldb * 2;
#pragma unroll
        for (int j = 0; j < NA_BLK; ++j)
            n_dma16(ab + a_off[j], as + wave * NA_WAVE + 512 * j);
#pragma unroll
        for (int j = 0; j < NB_BLK; ++j)
            n_dma16(bb + b_off_g[j], bs + wave * NB_WAVE + 512 * j);
    };

    // Fragments (in halves, relative to this wave's part of a stage): A as in
    // the large-tile kernel with 128-byte rows; B from two transposing reads
    // per 32-column tile and 16-wide K sub-step.
    int a_row[FM], a_sw[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        a_row[i] = (32 * i + l32) * NBK;
        a_sw[i] = swz8(32 * i + l32);
    }
    const int g = lane >> 4, w16 = lane & 15, r4 = w16 >> 2, c4 = w16 & 3;
    int b_off[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int n = 32 * j + 16 * (g & 1) + 4 * c4;
        b_off[j] = (((n >> 3) ^ swz_nb(r4)) << 3) + (n & 7);
    }
    const int b_krow = 8 * (g >> 1) + r4;

    f32x16 acc[FM][2];
#pragma unroll
    for (int i = 0; i < FM; ++i) acc[i][0] = acc[i][1] = f32x16{};
    auto compute = [&](const uint16_t *as, const uint16_t *bs) {
        as += wave * NA_WAVE;
        bs += wave * NB_WAVE;
        u32x4 af[NBK / 16][FM], bf[NBK / 16][2];
#pragma unroll
        for (int s = 0; s < NBK / 16; ++s) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
                af[s][i] = *reinterpret_cast<const u32x4 *>(as + a_row[i] + (((2 * s + half) ^ a_sw[i]) << 3));
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const uint16_t *p0 = bs + (16 * s + b_krow) * NBN + b_off[j];
                const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_n_t *)p0);
                const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_n_t *)(p0 + 4 * NBN));
                const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
                bf[s][j] = u32x4{l2[0], l2[1], h2[0], h2[1]};
            }
        }
#pragma unroll
        for (int s = 0; s < NBK / 16; ++s)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = mfma32x32x16<IS_BF16>(bf[s][j], af[s][i], acc[i][j]);
    };

    // Step t: this wave's loads of stage t % STG have landed once at most
    // STG - 2 later steps' loads are outstanding; the stage refilled now (step
    // t + STG - 1) was read by step t - 1, whose LDS reads have returned.
    // Steps past nsteps re-load the last block into stages nobody reads and
    // skip the MFMAs.
    if (nsteps > 0) {
        issue(a_stage<0, TBM>(), b_stage<0, STG>(), 0);
        if constexpr (STG == 3) issue(a_stage<1, TBM>(), b_stage<1, STG>(), 1);
    }
    // GEN: the last K block through registers, zero-filled past M, N and K, in
    // the layout the LDS-direct loads produce, into this wave's part of the
    // last stage (refilled only once the loop's first step has waited for
    // these reads).
    if (GEN && wave == kdma % NNW) {
        const int k0 = NBK * kdma;
        uint16_t *as = a_stage<STG - 1, TBM>() + wave * NA_WAVE;
        uint16_t *bs = b_stage<STG - 1, STG>() + wave * NB_WAVE;
        constexpr int NQA = NBM * NBK / 8 / 64, NQB = NBK * NBN / 8 / 64;   // chunks per lane
        if (K >= 8) {
            // One 16-byte load inside the matrix per chunk, all in flight before
            // the first wait; zeros past M, N and K applied in registers.
            Masked16 va[NQA], vb[NQB];
#pragma unroll
            for (int i = 0; i < NQA; ++i) {
                const int q = lane + 64 * i, r = q >> 3, c = q & 7;
                va[i] = masked16_load<2>(A, lda, m0 + r, M, k0 + 8 * c, K);
            }
#pragma unroll
            for (int i = 0; i < NQB; ++i) {
                const int q = lane + 64 * i, r = q >> 3, c = q & 7;
                vb[i] = masked16_load<2>(B, ldb, k0 + r, K, n0 + 8 * c, N);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < NQA; ++i) {
                const int q = lane + 64 * i, r = q >> 3, c = q & 7;
                *reinterpret_cast<u32x4 *>(as + r * NBK + ((c ^ swz8(r)) << 3)) = masked16_value(va[i]);
            }
#pragma unroll
            for (int i = 0; i < NQB; ++i) {
                const int q = lane + 64 * i, r = q >> 3, c = q & 7;
                *reinterpret_cast<u32x4 *>(bs + r * NBN + ((c ^ swz_nb(r)) << 3)) = masked16_value(vb[i]);
            }
        } else {
            // K < 8: element by element.
#pragma unroll
            for (int q = lane; q < NBM * NBK / 8; q += 64) {
                const int r = q >> 3, c = q & 7;
                const int gm = m0 + r, gk = k0 + 8 * c;
                uint32_t w[4] = {0, 0, 0, 0};
                if (gm < M) {
                    const uint16_t *src = A + (int64_t)gm * lda + gk;
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (gk + e < K) w[e >> 1] |= (uint32_t)src[e] << (16 * (e & 1));
                }
                *reinterpret_cast<u32x4 *>(as + r * NBK + ((c ^ swz8(r)) << 3)) = u32x4{w[0], w[1], w[2], w[3]};
            }
#pragma unroll
            for (int q = lane; q < NBK * NBN / 8; q += 64) {
                const int r = q >> 3, c = q & 7;
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
                *reinterpret_cast<u32x4 *>(bs + r * NBN + ((c ^ swz_nb(r)) << 3)) = u32x4{w[0], w[1], w[2], w[3]};
            }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);              // lgkmcnt(0): the LDS writes landed
        compute(a_stage<STG - 1, TBM>(), b_stage<STG - 1, STG>());
    }
    if constexpr (STG == 3) {
        for (int t = 0; t < nsteps; t += 3) {
            n_wait<NBLK_N>();
            issue(a_stage<2, TBM>(), b_stage<2, STG>(), t + 2);
            compute(a_stage<0, TBM>(), b_stage<0, STG>());
            n_wait<NBLK_N>();
            issue(a_stage<0, TBM>(), b_stage<0, STG>(), t + 3);
            if (t + 1 < nsteps) compute(a_stage<1, TBM>(), b_stage<1, STG>());
            n_wait<NBLK_N>();
            issue(a_stage<1, TBM>(), b_stage<1, STG>(), t + 4);
            if (t + 2 < nsteps) compute(a_stage<2, TBM>(), b_stage<2, STG>());
        }
    } else {
        for (int t = 0; t < nsteps; t += 2) {
            n_wait<0>();
            issue(a_stage<1, TBM>(), b_stage<1, STG>(), t + 1);
            compute(a_stage<0, TBM>(), b_stage<0, STG>());
            n_wait<0>();
            issue(a_stage<0, TBM>(), b_stage<0, STG>(), t + 2);
            if (t + 1 < nsteps) compute(a_stage<1, TBM>(), b_stage<1, STG>());
        }
    }
    n_wait<0>();

    // Partial tiles into LDS: 32-row tile i of every wave goes to B stage i
    // (this wave's own 8 KiB of it as 32 rows of 64 floats; 16-byte chunk index
    // XOR row, so the 32 rows one store touches spread over the banks).  Lane l
    // holds row l%32 of the tile, columns 32j + 8q + 4*(l/32) .. +3.  Each stage
    // array holds exactly the four waves' 32 x 64 fp32 partials.
    const auto store_partial = [&](auto I) {
        float *mine = reinterpret_cast<float *>(b_stage<I, STG>()) + wave * (32 * NBN);
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int chunk = (8 * j + 2 * q + half) ^ (l32 & 15);
                *reinterpret_cast<f32x4 *>(mine + l32 * NBN + 4 * chunk) =
                    f32x4{acc[I][j][4 * q], acc[I][j][4 * q + 1], acc[I][j][4 * q + 2],
                          acc[I][j][4 * q + 3]};
            }
    };
    store_partial(std::integral_constant<int, 0>{});
    if constexpr (FM == 2) store_partial(std::integral_constant<int, 1>{});
    __syncthreads();
    // Thread t sums row t/8 of each 32-row tile, columns 8(t%8) .. +7, over the
    // four partials, then applies the epilogue, rounds and stores.
    const int rr = tid >> 3, c8 = tid & 7;
    const auto finish = [&](auto I) {
        const int row = 32 * I + rr;
        const float *red = reinterpret_cast<const float *>(b_stage<I, STG>());
        float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < NNW; ++w) {
            const float *part = red + w * (32 * NBN) + rr * NBN;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const f32x4 v = *reinterpret_cast<const f32x4 *>(part + 4 * ((2 * c8 + h) ^ (rr & 15)));
#pragma unroll
                for (int e = 0; e < 4; ++e) s[4 * h + e] += v[e];
            }
        }
        if constexpr (EPI) {
            if (!GEN || m0 + row < M)
                epilogue_row<IS_BF16 ? OUT_BF16 : OUT_F16, 8>(epi, s, C + (int64_t)(m0 + row) * ldc,
                                                              n0 + 8 * c8, GEN ? N - n0 - 8 * c8 : 8);
        }
        const u32x4 out{pack2<IS_BF16>(s[0], s[1]), pack2<IS_BF16>(s[2], s[3]),
                        pack2<IS_BF16>(s[4], s[5]), pack2<IS_BF16>(s[6], s[7])};
        uint16_t *dst = C + (int64_t)(m0 + row) * ldc + n0 + 8 * c8;
        if (!GEN) {
            *reinterpret_cast<u32x4 *>(dst) = out;
        } else if (m0 + row < M) {
            const int gn = n0 + 8 * c8;
            if (gn + 8 <= N) {
                *reinterpret_cast<u32x4 *>(dst) = out;
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (gn + e < N) dst[e] = (uint16_t)(out[e >> 1] >> (16 * (e & 1)));
            }
        }
    };
    finish(std::integral_constant<int, 0>{});
    if constexpr (FM == 2) finish(std::integral_constant<int, 1>{});
}


}  // namespace

// Whole tiles (32 or 64 rows x 64), K in whole 64-wide blocks with at least one
// per wave, 16-byte aligned rows, and per-lane 32-bit offsets that fit (64 rows
// of A, 64 rows of B past a base).
static bool narrow_whole(const Problem &p, int tbm)
{
    return p.aligned && p.M % tbm == 0 && p.N % NBN == 0 && p.K % NBK == 0 && p.K >= NBK * NNW &&
           p.lda < (1 << 24) && p.ldb < (1 << 23);
}
bool h16_narrow_eligible(const Problem &p) { return narrow_whole(p, 32); }
bool h16_narrow64_eligible(const Problem &p) { return narrow_whole(p, 64); }

// The guarded instantiation: any M, N >= 8 (a clamped column chunk starts at
// N-8 rounded down to a multiple of 8), any K >= 1, any leading dimensions with 32-bit per-lane offsets.
bool h16_narrow_general_eligible(const Problem &p)
{
    return p.M >= 1 && p.N >= 8 && p.K >= 1 && p.lda < (1 << 24) && p.ldb < (1 << 24) &&
           (int64_t)NBK * p.ldb + p.N < ((int64_t)1 << 31);
}

template <bool GEN, bool EPI, int TBM>
static hipError_t narrow_launch(bool is_bf16, const Problem &p)
{
    constexpr int STG = TBM == 32 ? 3 : 2;
    const int tiles_n = (p.N + NBN - 1) / NBN;
    const int64_t nwg = (int64_t)((p.M + TBM - 1) / TBM) * tiles_n;
    if (nwg > 0x7fffffff) return hipErrorInvalidValue;
    const uint16_t *A = static_cast<const uint16_t *>(p.A);
    const uint16_t *B = static_cast<const uint16_t *>(p.B);
    uint16_t *C = static_cast<uint16_t *>(p.C);
    const Epilogue epi = p.epi ? *p.epi : Epilogue{1.f, 0.f, nullptr, 0};
    if (is_bf16)
        hipLaunchKernelGGL((h16_narrow_kernel<true, GEN, EPI, TBM, STG>), dim3((unsigned)nwg),
                           dim3(NNW * 64), 0, p.stream, A, B, C, p.M, p.N, p.K, p.lda, p.ldb,
                           p.ldc, tiles_n, epi);
    else
        hipLaunchKernelGGL((h16_narrow_kernel<false, GEN, EPI, TBM, STG>), dim3((unsigned)nwg),
                           dim3(NNW * 64), 0, p.stream, A, B, C, p.M, p.N, p.K, p.lda, p.ldb,
                           p.ldc, tiles_n, epi);
    return hipGetLastError();
}

template <int TBM>
static hipError_t narrow_dispatch(bool is_bf16, bool gen, const Problem &p)
{
    if (gen)
        return p.epi ? narrow_launch<true, true, TBM>(is_bf16, p)
                     : narrow_launch<true, false, TBM>(is_bf16, p);
    return p.epi ? narrow_launch<false, true, TBM>(is_bf16, p)
                 : narrow_launch<false, false, TBM>(is_bf16, p);
}

hipError_t h16_narrow_launch(bool is_bf16, const Problem &p)
{
    if (!h16_narrow_eligible(p)) return hipErrorInvalidValue;
    return narrow_dispatch<32>(is_bf16, false, p);
}

hipError_t h16_narrow_general_launch(bool is_bf16, const Problem &p)
{
    if (!h16_narrow_general_eligible(p)) return hipErrorInvalidValue;
    return narrow_dispatch<32>(is_bf16, true, p);
}

hipError_t h16_narrow64_launch(bool is_bf16, const Problem &p)
{
    if (!h16_narrow64_eligible(p)) return hipErrorInvalidValue;
    return narrow_dispatch<64>(is_bf16, false, p);
}

hipError_t h16_narrow64_general_launch(bool is_bf16, const Problem &p)
{
    if (!h16_narrow_general_eligible(p)) return hipErrorInvalidValue;
    return narrow_dispatch<64>(is_bf16, true, p);
}

}  // namespace gemm
