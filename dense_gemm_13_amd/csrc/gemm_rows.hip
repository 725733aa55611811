// GEMM with at most 4 rows of A (a vector or a few vectors times a matrix):
// C (MR x N) = A (MR x K) * B (K x N), fp32 accumulation, on the vector ALUs.
//
// With one to four rows the product is a stream over B: every element of B is
// read once and used for MR multiply-adds, so the bound is HBM (1 x 4095 x 4100
// in bf16: 33.6 MB of B against 33.6 MFLOP).  A matrix-core tile would be at
// most 4 of its 32 rows busy and its workgroups would need whole K blocks in
// LDS before any arithmetic; here each workgroup owns 64 columns of C (one
// 128-byte line of a bf16 B row, two of an fp32 one) and its 16 waves take the
// rows of B in turns of 16 chunks, every lane holding 4 to 8 loads of 16 bytes
// in flight.  The per-lane fp32 sums are added across the lanes of a wave with
// cross-lane shuffles and across the waves through LDS; then the epilogue is
// applied, the result rounded and stored.
//
// Lane l of a wave holds 16 bytes of one B row: column chunk l % CPR (CPR = 8
// chunks of 8 halves, or 16 chunks of 4 floats, per 64 columns) of row
// l / CPR of an RPL-row group (RPL = 64 / CPR).  Rows past K and columns past N
// are read as zeros (a chunk straddling N element by element), so any M <= 4,
// N, K >= 1 and leading dimensions are taken; the hardware runs in
// unaligned-access mode, so 16-byte loads at 2-byte-aligned addresses are
// legal.
//
// The rows of A are the vectors of a matrix-vector product; the split of the K
// sum over waves and lanes with the partial sums added at the end is the "K
// split" of "CUDA GEMM 优化实践笔记".
#include "gemm_device.hpp"
#include "gemm_launch.hpp"

namespace gemm {

namespace {

constexpr int RWAVES = 16;                               // waves per workgroup
constexpr int RCOLS = 64;                                // columns of C per workgroup

// fp32 value of element e of a 16-byte chunk of T (bf16, fp16 or fp32).
template <int OUT>
__device__ __forceinline__ float chunk_elem(const u32x4 &v, int e)
{
    if constexpr (OUT == OUT_F32) {
        return __uint_as_float(v[e]);
    } else {
        const uint16_t bits = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
        if constexpr (OUT == OUT_BF16) return __uint_as_float((uint32_t)bits << 16);
        else return (float)__builtin_bit_cast(_Float16, bits);
    }
}

// OUT: element type of A, B and C (OUT_F16, OUT_BF16 or OUT_F32).  MR: rows.
// EPI: the fused epilogue on the sums before rounding.
template <int OUT, int MR, bool EPI>
__global__ void __launch_bounds__(RWAVES * 64)
rows_kernel(const void *__restrict__ Av, const void *__restrict__ Bv, void *__restrict__ Cv, int N,
            int K, int64_t lda, int64_t ldb, int64_t ldc, Epilogue epi)
{
    constexpr int ES = OUT == OUT_F32 ? 4 : 2;           // element bytes
    constexpr int CW = 16 / ES;                          // columns per lane (8 or 4)
    constexpr int CPR = RCOLS / CW;                      // lanes per 64 columns (8 or 16)
    constexpr int RPL = 64 / CPR;                        // B rows per wave load (8 or 4)
    // 16-byte B loads in flight per lane (fewer with more rows: the 16 waves of
    // a workgroup get 128 registers each).
    constexpr int RUNROLL = MR == 1 ? 8 : MR == 2 ? 6 : 4;
    const char *A = static_cast<const char *>(Av);
    const char *B = static_cast<const char *>(Bv);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int c = lane % CPR, r = lane / CPR;
    const int n = blockIdx.x * RCOLS + CW * c;           // this lane's first column
    const int ncols = N - n;                             // >= CW: whole chunk; <= 0: none

    // A row m at K index k (0 past K).
    auto a_at = [&](int m, int k) -> float {
        if (k >= K) return 0.f;
        const char *p = A + ((int64_t)m * lda + k) * ES;
        if constexpr (OUT == OUT_F32) {
            return *reinterpret_cast<const float *>(p);
        } else {
            const uint16_t bits = *reinterpret_cast<const uint16_t *>(p);
            if constexpr (OUT == OUT_BF16) return __uint_as_float((uint32_t)bits << 16);
            else return (float)__builtin_bit_cast(_Float16, bits);
        }
    };
    // The 16-byte chunk of B row k at this lane's columns (zeros past K or N).
    auto b_at = [&](int k) -> u32x4 {
        u32x4 v = u32x4{0u, 0u, 0u, 0u};
        if (k < K && ncols > 0) {
            const char *p = B + ((int64_t)k * ldb + n) * ES;
            if (ncols >= CW) {
                v = *reinterpret_cast<const u32x4 *>(p);
            } else if constexpr (ES == 4) {
#pragma unroll
                for (int e = 0; e < CW; ++e)
                    if (e < ncols) v[e] = reinterpret_cast<const uint32_t *>(p)[e];
            } else {
#pragma unroll
                for (int e = 0; e < CW; ++e)
                    if (e < ncols)
                        v[e >> 1] |= (uint32_t)reinterpret_cast<const uint16_t *>(p)[e] << (16 * (e & 1));
            }
        }
        return v;
    };

    float acc[MR][CW];
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int e = 0; e < CW; ++e) acc[m][e] = 0.f;

    // Row groups of RPL rows; wave w takes groups w, w + 16, w + 32, ..., and
    // RUNROLL of its groups at a time (all their loads issued before the
    // arithmetic).
    const int ngroups = (K + RPL - 1) / RPL;
    for (int g0 = wave; g0 < ngroups; g0 += RWAVES * RUNROLL) {
        u32x4 bv[RUNROLL];
        float av[RUNROLL][MR];
#pragma unroll
        for (int u = 0; u < RUNROLL; ++u) {
            const int k = group_elem(g0 + RWAVES * u, ngroups, RPL, r, K);
            bv[u] = b_at(k);
#pragma unroll
            for (int m = 0; m < MR; ++m) av[u][m] = a_at(m, k);
        }
#pragma unroll
        for (int u = 0; u < RUNROLL; ++u)
#pragma unroll
            for (int e = 0; e < CW; ++e) {
                const float b = chunk_elem<OUT>(bv[u], e);
#pragma unroll
                for (int m = 0; m < MR; ++m) acc[m][e] = fmaf(av[u][m], b, acc[m][e]);
            }
    }

    // Lanes c, c + CPR, c + 2 CPR, ... hold the same columns: add across them.
#pragma unroll
    for (int off = CPR; off < 64; off *= 2)
#pragma unroll
        for (int m = 0; m < MR; ++m)
#pragma unroll
            for (int e = 0; e < CW; ++e) acc[m][e] += __shfl_xor(acc[m][e], off, 64);

    // Then across the waves: lanes 0 .. CPR-1 of each wave write their sums.
    __shared__ float red[RWAVES][MR][RCOLS];
    if (r == 0) {
#pragma unroll
        for (int m = 0; m < MR; ++m)
#pragma unroll
            for (int e = 0; e < CW; ++e) red[wave][m][CW * c + e] = acc[m][e];
    }
    __syncthreads();
    // Thread t < MR * CPR adds row t / CPR, columns of chunk t % CPR, over the
    // waves (in wave order), applies the epilogue, rounds and stores.
    if (tid < MR * CPR) {
        const int m = tid / CPR, cc = tid % CPR;
        const int gn = blockIdx.x * RCOLS + CW * cc;
        const int cnt = N - gn;
        if (cnt <= 0) return;
        float s[CW];
#pragma unroll
        for (int e = 0; e < CW; ++e) s[e] = 0.f;
        // (At most four waves' values in flight: fully unrolled, all 16 waves'
        // reads would be issued at once and spill.)
#pragma unroll 4
        for (int w = 0; w < RWAVES; ++w)
#pragma unroll
            for (int e = 0; e < CW; ++e) s[e] += red[w][m][CW * cc + e];
        char *rowp = static_cast<char *>(Cv) + (int64_t)m * ldc * ES;
        if constexpr (EPI) epilogue_row<OUT, CW>(epi, s, rowp, gn, cnt);
        if constexpr (OUT == OUT_F32) {
            float *dst = reinterpret_cast<float *>(rowp) + gn;
            if (cnt >= CW) {
                *reinterpret_cast<f32x4 *>(dst) = f32x4{s[0], s[1], s[2], s[3]};
            } else {
#pragma unroll
                for (int e = 0; e < CW; ++e)
                    if (e < cnt) dst[e] = s[e];
            }
        } else {
            constexpr bool BF = OUT == OUT_BF16;
            const u32x4 out{pack2<BF>(s[0], s[1]), pack2<BF>(s[2], s[3]), pack2<BF>(s[4], s[5]),
                            pack2<BF>(s[6], s[7])};
            uint16_t *dst = reinterpret_cast<uint16_t *>(rowp) + gn;
            if (cnt >= CW) {
                *reinterpret_cast<u32x4 *>(dst) = out;
            } else {
#pragma unroll
                for (int e = 0; e < CW; ++e)
                    if (e < cnt) dst[e] = (uint16_t)(out[e >> 1] >> (16 * (e & 1)));
            }
        }
    }
}

template <int OUT, int MR>
static hipError_t rows_typed(const Problem &p)
{
    const int64_t nwg = ((int64_t)p.N + RCOLS - 1) / RCOLS;
    if (nwg > 0x7fffffff) return hipErrorInvalidValue;
    const Epilogue epi = p.epi ? *p.epi : Epilogue{1.f, 0.f, nullptr, 0};
    if (p.epi)
        hipLaunchKernelGGL((rows_kernel<OUT, MR, true>), dim3((unsigned)nwg), dim3(RWAVES * 64), 0,
                           p.stream, p.A, p.B, p.C, p.N, p.K, p.lda, p.ldb, p.ldc, epi);
    else
        hipLaunchKernelGGL((rows_kernel<OUT, MR, false>), dim3((unsigned)nwg), dim3(RWAVES * 64), 0,
                           p.stream, p.A, p.B, p.C, p.N, p.K, p.lda, p.ldb, p.ldc, epi);
    return hipGetLastError();
}

template <int OUT>
static hipError_t rows_by_m(const Problem &p)
{
    switch (p.M) {
    case 1: return rows_typed<OUT, 1>(p);
    case 2: return rows_typed<OUT, 2>(p);
    case 3: return rows_typed<OUT, 3>(p);
    case 4: return rows_typed<OUT, 4>(p);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool rows_eligible(const Problem &p) { return p.M >= 1 && p.M <= 4 && p.N >= 1 && p.K >= 1; }

// out: OUT_F16, OUT_BF16 or OUT_F32 (the element type of A, B and C).
hipError_t rows_launch(int out, const Problem &p)
{
    if (!rows_eligible(p)) return hipErrorInvalidValue;
    if (out == OUT_F32) return rows_by_m<OUT_F32>(p);
    if (out == OUT_BF16) return rows_by_m<OUT_BF16>(p);
    return rows_by_m<OUT_F16>(p);
}

}  // namespace gemm
