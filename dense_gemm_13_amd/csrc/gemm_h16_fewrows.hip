// fp16 / bf16 products with at most 4 rows of A (a vector or a few vectors
// times a matrix), C (MR x N) = A (MR x K) * B (K x N), fp32 accumulation, for
// B rows of any alignment.
//
// Such a product streams B once: 1 x 4095 x 4100 reads 33.6 MB of B for 33.6
// MFLOP, so the bound is memory.  Here a workgroup owns 32 columns of C, 64
// bytes of every B row, so N = 4095 gives 128 workgroups.  Consecutive
// workgroups of one XCD take consecutive column groups, so the 128-byte lines
// of B that two groups share are fetched once into that XCD's L2.  (16-column
// groups, twice the workgroups but four of them to a line, were slower: the
// loads in flight per CU are limited in cache lines, not bytes, and each line
// then brought 32 useful bytes.  1 x 4095 x 4100: 13.3 against 12.0 us;
// 1 x 8192 x 4096: 23.1 against 16.0 us.  64-column groups, whole lines but a
// quarter of the workgroups: 14.7 and 16.2 us.)  The 16 waves of a workgroup
// take the 16-row blocks of B in turns (wave w: blocks w, w + 16, ...), each
// through a private ring of 8 one-KiB LDS slots filled by LDS-direct 16-byte
// loads (lane l: row l/4 of the block, 8 columns at 8*(l%4)), so every lane
// keeps 8 loads in flight and a CU holds 128 KiB of B in flight.  LDS-direct loads keep their rate at 2-byte-aligned addresses,
// where 16-byte loads into registers do not (B rows of 4095 elements).  The
// rows of A are copied into LDS once, zero-padded to whole blocks, so a block
// needs no load of A.  Each lane reads back exactly the 16 bytes it loaded and
// multiplies them by the A value of its row; the sums are added across the
// lanes of a wave with shuffles and across the waves through LDS, then the
// epilogue is applied, the result rounded and stored.
//
// Edges: the ring carries whole 16-row blocks only; the K % 16 rows after them
// come through registers, with zeros past K in both operands.  The last
// workgroup's 32-column window is moved left to end at N (N >= 32), so no load
// leaves B's rows, and it stores only the columns past the previous window.
//
// The rows of A are the vectors of a matrix-vector product; the split of the K
// sum over waves and lanes with partial sums added at the end is the "K split"
// of "CUDA GEMM 优化实践笔记", and the asynchronous copies into a ring of LDS
// stages those of "[CUDA 优化实战] hgemm - 超越 cuBLAS" sections 1-3.
#include <utility>

#include "gemm_device.hpp"
#include "gemm_launch.hpp"

namespace gemm {

namespace {

typedef __attribute__((address_space(3))) void lds_void_f_t;

constexpr int FR_COLS = 32;                              // columns of C per workgroup
constexpr int FR_LPR = FR_COLS / 8;                      // lanes per B row (16 bytes each)
constexpr int FR_WAVES = 16;                             // waves per workgroup
constexpr int FR_SLOTS = 8;                              // ring slots per wave
constexpr int FR_ROWS = 64 / FR_LPR;                     // B rows per block (one 1 KiB load)
constexpr int FR_A_HALVES = 12288;                       // LDS for the rows of A (24 KiB)

// One LDS array per ring slot (each wave its own KiB in it): distinct objects,
// so the compiler can tell that a load into one slot does not alias reads of
// another and does not wait for it.  (It tells apart at most 8 such targets of
// LDS-direct loads; with more, it waits for every load in flight before each
// LDS read at the head of the loop.)
template <int S>
__shared__ __attribute__((aligned(1024))) uint16_t fr_slot[FR_WAVES * 512];
__shared__ __attribute__((aligned(16))) uint16_t fr_a[FR_A_HALVES];

// One 16-byte global -> LDS load per lane (lane t's bytes land at lds + 16t).
__device__ __forceinline__ void fr_dma16(const void *src, uint16_t *lds)
{
    __builtin_amdgcn_global_load_lds(src, (lds_void_f_t *)lds, 16, 0, 0);
}

// s_waitcnt vmcnt(N) lgkmcnt(0).
template <int N>
__device__ __forceinline__ void fr_wait()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));
}

template <typename F, int... I>
__device__ __forceinline__ void fr_unroll_impl(F &&f, std::integer_sequence<int, I...>)
{
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void fr_unroll(F &&f)
{
    fr_unroll_impl(f, std::make_integer_sequence<int, N>{});
}

template <bool IS_BF16>
__device__ __forceinline__ float fr_half(uint16_t bits)
{
    if constexpr (IS_BF16) return __uint_as_float((uint32_t)bits << 16);
    else return (float)__builtin_bit_cast(_Float16, bits);
}

// MR: rows of A and C (1 to 4).  EPI: the fused epilogue on the sums before
// rounding.  Requires N >= 32 and MR * (K rounded up to 16) <= FR_A_HALVES.
template <bool IS_BF16, int MR, bool EPI>
__global__ void __launch_bounds__(FR_WAVES * 64)
h16_fewrows_kernel(const uint16_t *__restrict__ A, const uint16_t *__restrict__ B,
                   uint16_t *__restrict__ C, int N, int K, int64_t lda, int64_t ldb, int64_t ldc,
                   Epilogue epi)
{
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int tm, tn;
    tile_coords(blockIdx.x, gridDim.x, 1, gridDim.x, 1, tm, tn);
    const int c0 = tn * FR_COLS;                         // first column this workgroup stores
    const int wstart = c0 + FR_COLS <= N ? c0 : N - FR_COLS;   // loaded window

    const int nb = K / FR_ROWS;                          // whole blocks of B rows
    const int kp = (K + FR_ROWS - 1) / FR_ROWS * FR_ROWS;   // K padded to whole blocks
    const int nbw = wave < nb ? (nb - wave + FR_WAVES - 1) / FR_WAVES : 0;   // this wave's

    // Lane -> row r of each block, 8 columns from wstart + 8c.
    const int r = lane / FR_LPR, c = lane % FR_LPR;
    const uint16_t *bsrc = B + wstart + 8 * c;
    // First K row of this wave's t-th block.
    auto blk_k = [&](int t) { return (wave + FR_WAVES * t) * FR_ROWS; };
    // (Rows are clamped to K - 1 only for the first slots of waves with fewer
    // blocks than slots: those loads fill slots nobody reads, so that the loads
    // in flight do not depend on the wave.)
    auto issue = [&](uint16_t *slot, int t) {
        const int k = blk_k(t) + r;
        fr_dma16(bsrc + (int64_t)(k < K ? k : K - 1) * ldb, slot + wave * 512);
    };

    // Loads: this wave's first ring slots, then the rows of the partial last
    // block of B (K % 16 rows, through registers; used by the wave whose turn
    // that block is), then the rows of A (zero past K; up to FR_A_HALVES / 1024
    // per thread).  Loads complete in issue order, so waiting for A waits for
    // the first slots too; with K up to 16 * FR_WAVES * FR_SLOTS (2048) those
    // are all of the blocks.
    fr_unroll<FR_SLOTS>([&](auto S) { issue(fr_slot<S>, S); });
    const bool tail_wave = wave == nb % FR_WAVES && nb * FR_ROWS < K;
    const int ktail = nb * FR_ROWS + r;                  // this lane's row of the partial block
    const u32x4 btail =
        *reinterpret_cast<const u32x4 *>(bsrc + (int64_t)(ktail < K ? ktail : K - 1) * ldb);
    // (Row m of A at fr_a[m * kp], k = tid + 1024 u: no division by kp.)
    constexpr int KU = FR_A_HALVES / (FR_WAVES * 64 * MR);
    uint16_t av[MR][KU];
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int u = 0; u < KU; ++u) {
            const int k = tid + FR_WAVES * 64 * u;
            av[m][u] = k < K ? A[(int64_t)m * lda + k] : (uint16_t)0;   // (waves past K skip)
        }
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int u = 0; u < KU; ++u) {
            const int k = tid + FR_WAVES * 64 * u;
            if (k < kp) fr_a[m * kp + k] = av[m][u];
        }
    __builtin_amdgcn_s_waitcnt(0xc07f);                  // lgkmcnt(0): A is in LDS
    asm volatile("s_barrier" ::: "memory");              // (no fence: B loads stay in flight)

    float acc[MR][8];
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[m][e] = 0.f;
    // acc += a(k) * b for the 8 columns of one B row chunk.
    auto fma_row = [&](const u32x4 &b, int k) {
        float bf[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) bf[e] = fr_half<IS_BF16>((uint16_t)(b[e >> 1] >> (16 * (e & 1))));
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            const float a = fr_half<IS_BF16>(fr_a[m * kp + k]);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[m][e] = fmaf(a, bf[e], acc[m][e]);
        }
    };
    // (Rows of the partial block past K carry zeros in both operands.)
    if (tail_wave) fma_row(ktail < K ? btail : u32x4{0u, 0u, 0u, 0u}, ktail);

    // Block t is in slot t % FR_SLOTS.  While blocks are left to load, the
    // FR_SLOTS - 1 blocks after block t are still in flight at its turn; the
    // last FR_SLOTS blocks wait for everything left.
    for (int t0 = 0; t0 < nbw; t0 += FR_SLOTS) {
        fr_unroll<FR_SLOTS>([&](auto S) {
            const int t = t0 + S;
            if (t + FR_SLOTS <= nbw) fr_wait<FR_SLOTS - 1>();
            else fr_wait<0>();
            if (t < nbw)
                fma_row(*reinterpret_cast<const u32x4 *>(fr_slot<S> + wave * 512 + 8 * lane),
                        blk_k(t) + r);
            if (t + FR_SLOTS < nbw) {
                __builtin_amdgcn_s_waitcnt(0xc07f);      // this slot's reads are done
                issue(fr_slot<S>, t + FR_SLOTS);
            }
        });
    }
    fr_wait<0>();

    // Lanes with the same c hold the same columns: add across the 16 rows.
#pragma unroll
    for (int off = FR_LPR; off < 64; off *= 2)
#pragma unroll
        for (int m = 0; m < MR; ++m)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[m][e] += __shfl_xor(acc[m][e], off, 64);

    // Then across the waves (in wave order), through each wave's own KiB of
    // ring slot 0, which it no longer reads.
    float *red = reinterpret_cast<float *>(fr_slot<0>);  // [wave][m][column], 256 floats a wave
    static_assert(MR * FR_COLS <= 256, "reduction space");
    if (r == 0) {
#pragma unroll
        for (int m = 0; m < MR; ++m)
#pragma unroll
            for (int e = 0; e < 8; ++e) red[wave * 256 + m * FR_COLS + 8 * c + e] = acc[m][e];
    }
    __syncthreads();
    if (tid < FR_LPR * MR) {
        const int m = tid / FR_LPR, cc = tid % FR_LPR;
        const int n = wstart + 8 * cc;                   // first of 8 columns, all < N
        float s[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) s[e] = 0.f;
        // (Four waves' values in flight at a time: all 16 at once would spill.)
#pragma unroll 4
        for (int w = 0; w < FR_WAVES; ++w)
#pragma unroll
            for (int e = 0; e < 8; ++e) s[e] += red[w * 256 + m * FR_COLS + 8 * cc + e];
        uint16_t *rowp = C + (int64_t)m * ldc;
        constexpr int OUT = IS_BF16 ? OUT_BF16 : OUT_F16;
        if constexpr (EPI) {
            if (n >= c0) {
                epilogue_row<OUT, 8>(epi, s, rowp, n, 8);
            } else {
                // The moved window's chunk that starts left of c0: only the
                // columns this workgroup stores read their bias and prior C
                // (the others belong to the previous workgroup, which may be
                // writing them).
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    if (n + e < c0) continue;
                    const float bias = epi.bias ? epi.bias[n + e] : 0.f;
                    float x = epi.beta != 0.f
                                  ? epilogue_value(epi, s[e], bias, load_out<OUT>(rowp, n + e))
                                  : epilogue_value(epi, s[e], bias);
                    if (epi.relu) x = epilogue_relu(x);
                    s[e] = x;
                }
            }
        }
        uint16_t *dst = rowp + n;
        if (n >= c0 && ((uintptr_t)dst & 15) == 0) {
            *reinterpret_cast<u32x4 *>(dst) = u32x4{pack2<IS_BF16>(s[0], s[1]), pack2<IS_BF16>(s[2], s[3]),
                                                    pack2<IS_BF16>(s[4], s[5]), pack2<IS_BF16>(s[6], s[7])};
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (n + e >= c0) dst[e] = IS_BF16 ? to_bf16_bits(s[e]) : to_f16_bits(s[e]);
        }
    }
}

template <bool IS_BF16, int MR>
static hipError_t fewrows_typed(const Problem &p)
{
    const int64_t nwg = ((int64_t)p.N + FR_COLS - 1) / FR_COLS;
    const Epilogue epi = p.epi ? *p.epi : Epilogue{1.f, 0.f, nullptr, 0};
    const auto *A = static_cast<const uint16_t *>(p.A);
    const auto *B = static_cast<const uint16_t *>(p.B);
    auto *C = static_cast<uint16_t *>(p.C);
    if (p.epi)
        hipLaunchKernelGGL((h16_fewrows_kernel<IS_BF16, MR, true>), dim3((unsigned)nwg),
                           dim3(FR_WAVES * 64), 0, p.stream, A, B, C, p.N, p.K, p.lda, p.ldb,
                           p.ldc, epi);
    else
        hipLaunchKernelGGL((h16_fewrows_kernel<IS_BF16, MR, false>), dim3((unsigned)nwg),
                           dim3(FR_WAVES * 64), 0, p.stream, A, B, C, p.N, p.K, p.lda, p.ldb,
                           p.ldc, epi);
    return hipGetLastError();
}

template <bool IS_BF16>
static hipError_t fewrows_by_m(const Problem &p)
{
    switch (p.M) {
    case 1: return fewrows_typed<IS_BF16, 1>(p);
    case 2: return fewrows_typed<IS_BF16, 2>(p);
    case 3: return fewrows_typed<IS_BF16, 3>(p);
    case 4: return fewrows_typed<IS_BF16, 4>(p);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool h16_fewrows_eligible(const Problem &p)
{
    if (p.M < 1 || p.M > 4 || p.N < FR_COLS || p.K < 1) return false;
    const int64_t kp = ((int64_t)p.K + FR_ROWS - 1) / FR_ROWS * FR_ROWS;
    return p.M * kp <= FR_A_HALVES;
}

// Where it was measured ahead of the narrow K-split kernel (guarded form), over
// M = 1..4, N = 256..16384, K = 256..12288, B rows 16-byte aligned or not:
//  * one row with K >= 2048, when B's rows are not 16-byte aligned (the narrow
//    kernel's LDS-direct loads slow down there: 1 x 4096 x 4100 with ldb =
//    4097 12.1 against 17.2 us), when N <= 2048 (64 or fewer workgroups either
//    way: 1 x 1024 x 12288 13.4 against 21.3 us) or while N * K <= 17 M
//    (1 x 4096 x 4100 10.9 against 12.1 us; 1 x 8192 x 4100 16.8 against 15.3);
//  * two rows with K >= 2048 and unaligned B rows up to N = 8192, or K >= 4096
//    with unaligned rows or N <= 2048.
// Elsewhere, and always with short K or from N = 16384 with aligned rows, the
// narrow kernel wins (4 x 16384 x 512: 5.6 against 20.0 us; 1 x 4095 x 1024:
// 7.2 against 8.3).
bool h16_fewrows_preferred(const Problem &p)
{
    if (!h16_fewrows_eligible(p)) return false;
    const bool unaligned = p.ldb % 8 != 0 || (reinterpret_cast<uintptr_t>(p.B) & 15) != 0;
    const int64_t nk = (int64_t)p.N * p.K;
    if (p.M == 1 && p.K >= 2048 && (unaligned || p.N <= 2048 || nk <= 17000000)) return true;
    if (p.M <= 2 && p.K >= 2048 && unaligned && p.N <= 8192) return true;
    if (p.M <= 2 && p.K >= 4096 && (unaligned || p.N <= 2048)) return true;
    return false;
}

hipError_t h16_fewrows_launch(bool is_bf16, const Problem &p)
{
    if (!h16_fewrows_eligible(p)) return hipErrorInvalidValue;
    return is_bf16 ? fewrows_by_m<true>(p) : fewrows_by_m<false>(p);
}

}  // namespace gemm
