// The optimisation ladder, measured on gfx950: the steps by which the pages
// take a half-precision GEMM from a triple loop to a tuned kernel, each one a
// kernel of its own so that its effect can be timed.
//
// "深度学习加速核心：GEMM优化从分块到TensorCore的实战解析" section 5.3 lists the
// rungs for a 4096 x 4096 FP16 GEMM: a plain triple loop; 64 x 64 tiles in
// shared memory; register caching of a small per-thread block with bank
// conflicts avoided; matrix-core instructions; double buffering; a swizzled
// layout.  Sections 3.1-3.2 describe the first two tiled kernels (64 x 64 tiles,
// 4 x 4 outputs per thread from register-held fragments).  "[CUDA 优化实战]
// hgemm - 超越 cuBLAS" takes the matrix-core kernel through the same last steps
// (swizzle, double buffer, coalesced C writes).
//
// Rungs 0-2 live here and run on the vector ALUs (fp32 FMAs on fp16/bf16
// values, fp32 accumulation).  Rungs 3-5 are the library's 128 x 128 MFMA
// kernel with its two-stage ring and its swizzle switched off and on
// (gemm_h16.hip); rung 6 is the library's own dispatch; rungs 7-8 repeat rungs
// 3-4 with one workgroup per CU.  Also here: the
// MFMA-only ceiling, which issues the large-tile kernel's MFMA sequence with
// register-resident operands and no memory traffic, i.e. what the matrix cores
// sustain on these operand values at the clock the chip holds under that load.
#include "gemm_device.hpp"
#include "gemm_launch.hpp"

namespace gemm {

namespace {

template <bool IS_BF16>
__device__ __forceinline__ float h2f(uint16_t bits)
{
    if constexpr (IS_BF16) return __uint_as_float((uint32_t)bits << 16);
    else return (float)__builtin_bit_cast(_Float16, bits);
}

template <bool IS_BF16>
__device__ __forceinline__ uint16_t f2h(float v)
{
    return IS_BF16 ? to_bf16_bits(v) : to_f16_bits(v);
}

// ---- rung 0: one thread per entry of C, operands straight from global memory
// (threads of a row of the 16 x 16 block read consecutive columns of B).
template <bool IS_BF16>
__global__ void __launch_bounds__(256)
ladder_naive_kernel(const uint16_t *__restrict__ A, const uint16_t *__restrict__ B,
                    uint16_t *__restrict__ C, int M, int N, int K, int64_t lda, int64_t ldb,
                    int64_t ldc)
{
    const int col = blockIdx.x * 16 + (threadIdx.x & 15);
    const int row = blockIdx.y * 16 + (threadIdx.x >> 4);
    if (row >= M || col >= N) return;
    const uint16_t *a = A + (int64_t)row * lda;
    const uint16_t *b = B + col;
    float acc = 0.f;
    for (int k = 0; k < K; ++k) acc = fmaf(h2f<IS_BF16>(a[k]), h2f<IS_BF16>(b[(int64_t)k * ldb]), acc);
    C[(int64_t)row * ldc + col] = f2h<IS_BF16>(acc);
}

// Both tiled VALU rungs: 64 x 64 tiles of C, K in steps of 16, 256 threads.
constexpr int LT = 64, LBK = 16;

// ---- rung 1: 64 x 64 tiles staged in LDS as they are in memory (16-bit).
// Thread (ty, tx) of the 16 x 16 block owns entries (ty + 16i, tx + 16j), i,
// j < 4, and each of its multiply-adds reads both operands from LDS: every
// entry runs its own loop over the step's k, so no operand fetched for one
// entry is reused for another.  That per-entry LDS traffic is what the register
// caching of the next rung removes (the pages put it at 4-8x fewer LDS reads).
template <bool IS_BF16>
__global__ void __launch_bounds__(256)
ladder_lds_kernel(const uint16_t *__restrict__ A, const uint16_t *__restrict__ B,
                  uint16_t *__restrict__ C, int M, int N, int K, int64_t lda, int64_t ldb,
                  int64_t ldc)
{
    __shared__ uint16_t As[LT * LBK], Bs[LBK * LT];
    const int t = threadIdx.x, ty = t >> 4, tx = t & 15;
    const int m0 = blockIdx.y * LT, n0 = blockIdx.x * LT;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < K; k0 += LBK) {
        {   // A: thread t -> row t / 4, k 4*(t % 4) .. +3; B: row k t / 16, columns 4*(t % 16) ..
            const int r = t >> 2, c = 4 * (t & 3), gm = m0 + r;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int gk = k0 + c + e;
                As[r * LBK + c + e] = gm < M && gk < K ? A[(int64_t)gm * lda + gk] : 0;
            }
            const int rb = t >> 4, cb = 4 * (t & 15), gk = k0 + rb;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int gn = n0 + cb + e;
                Bs[rb * LT + cb + e] = gk < K && gn < N ? B[(int64_t)gk * ldb + gn] : 0;
            }
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint16_t *ar = As + (ty + 16 * i) * LBK;
                const uint16_t *bc = Bs + tx + 16 * j;
                float v = acc[i][j];
#pragma unroll 1
                for (int k = 0; k < LBK; ++k)
                    v = fmaf(h2f<IS_BF16>(ar[k]), h2f<IS_BF16>(bc[k * LT]), v);
                acc[i][j] = v;
            }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int gm = m0 + ty + 16 * i, gn = n0 + tx + 16 * j;
            if (gm < M && gn < N) C[(int64_t)gm * ldc + gn] = f2h<IS_BF16>(acc[i][j]);
        }
}

// ---- rung 2: register caching and bank-conflict avoidance.  Thread (ty, tx)
// owns the contiguous 4 x 4 block at rows 4ty, columns 4tx.  Operands are
// widened to fp32 once, as they are staged, and A is held transposed (rows of
// m, padded by 4 floats, so the transposing writes of a wave cover 64 distinct
// banks).  For each k the thread then reads its 4 A values and its 4 B values
// with one 16-byte LDS read each and runs the 16 multiply-adds from registers:
// 2 LDS reads per 16 products instead of rung 1's 32.
template <bool IS_BF16>
__global__ void __launch_bounds__(256)
ladder_reg_kernel(const uint16_t *__restrict__ A, const uint16_t *__restrict__ B,
                  uint16_t *__restrict__ C, int M, int N, int K, int64_t lda, int64_t ldb,
                  int64_t ldc)
{
    constexpr int A_LD = LT + 4;
    __shared__ __attribute__((aligned(16))) float As[LBK * A_LD];
    __shared__ __attribute__((aligned(16))) float Bs[LBK * LT];
    const int t = threadIdx.x, ty = t >> 4, tx = t & 15;
    const int m0 = blockIdx.y * LT, n0 = blockIdx.x * LT;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < K; k0 += LBK) {
        {   // A: thread t -> row t / 4, k 4*(t % 4) .. +3, written transposed
            const int r = t >> 2, c = 4 * (t & 3), gm = m0 + r;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int gk = k0 + c + e;
                As[(c + e) * A_LD + r] =
                    gm < M && gk < K ? h2f<IS_BF16>(A[(int64_t)gm * lda + gk]) : 0.f;
            }
        }
        {   // B: thread t -> row k t / 16, columns 4*(t % 16) .. +3, one 16-byte write
            const int r = t >> 4, c = 4 * (t & 15), gk = k0 + r;
            f32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int gn = n0 + c + e;
                v[e] = gk < K && gn < N ? h2f<IS_BF16>(B[(int64_t)gk * ldb + gn]) : 0.f;
            }
            *reinterpret_cast<f32x4 *>(Bs + r * LT + c) = v;
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < LBK; ++k) {
            const f32x4 a = *reinterpret_cast<const f32x4 *>(As + k * A_LD + 4 * ty);
            const f32x4 b = *reinterpret_cast<const f32x4 *>(Bs + k * LT + 4 * tx);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int gm = m0 + 4 * ty + i;
        if (gm >= M) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int gn = n0 + 4 * tx + j;
            if (gn < N) C[(int64_t)gm * ldc + gn] = f2h<IS_BF16>(acc[i][j]);
        }
    }
}

// ---- the MFMA-only ceiling.  One workgroup of 4 waves per 256 x 256 tile, each
// wave a 128 x 128 sub-tile of 4 x 4 v_mfma_f32_32x32x16 tiles, K/16 sub-steps:
// exactly the MFMA instructions of the large-tile kernel, in its order (B
// fragment first).  The operand fragments are loaded once, from the tile's
// rows of A and columns of B at k = 0..31 (two sets, k 0..15 and 16..31), and
// the sub-steps alternate between the two sets, so consecutive MFMAs see
// operands changing as in the real product while no memory is touched.  The
// result, written as C, is therefore (K/32) * A[:, 0:32] * B[0:32, :].
template <bool IS_BF16>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
mfma_ceiling_kernel(const uint16_t *__restrict__ A, const uint16_t *__restrict__ B,
                    uint16_t *__restrict__ C, int K, int64_t lda, int64_t ldb, int64_t ldc,
                    int tiles_m, int tiles_n)
{
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int l32 = lane & 31, half = lane >> 5;
    int tm, tn;
    tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, tiles_m < 4 ? tiles_m : 4, tm, tn);
    const int m0 = tm * 256 + (wave >> 1) * 128, n0 = tn * 256 + (wave & 1) * 128;
    u32x4 af[2][4], bf[2][4];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // A: row m0 + 32i + l32, k = 16s + 8*half .. +7 (one 16-byte load)
            af[s][i] = *reinterpret_cast<const u32x4 *>(A + (int64_t)(m0 + 32 * i + l32) * lda +
                                                        16 * s + 8 * half);
            // B: column n0 + 32i + l32, the same 8 k
            uint32_t w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int k = 16 * s + 8 * half + 2 * e;
                const uint16_t *p = B + (int64_t)k * ldb + n0 + 32 * i + l32;
                w[e] = (uint32_t)p[0] | ((uint32_t)p[ldb] << 16);
            }
            bf[s][i] = u32x4{w[0], w[1], w[2], w[3]};
        }
    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
    for (int s = 0; s < K / 32; ++s) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = mfma32x32x16<IS_BF16>(bf[h][j], af[h][i], acc[i][j]);
    }
    // lane holds C[32i + l32][32j + 8q + 4*half .. +3]
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint16_t *crow = C + (int64_t)(m0 + 32 * i + l32) * ldc + n0 + 4 * half;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *reinterpret_cast<u32x2 *>(crow + 32 * j + 8 * q) =
                    u32x2{pack2<IS_BF16>(acc[i][j][4 * q], acc[i][j][4 * q + 1]),
                          pack2<IS_BF16>(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3])};
    }
}

template <bool IS_BF16>
hipError_t valu_typed(int rung, const Problem &p)
{
    const uint16_t *A = static_cast<const uint16_t *>(p.A);
    const uint16_t *B = static_cast<const uint16_t *>(p.B);
    uint16_t *C = static_cast<uint16_t *>(p.C);
    const int tile = rung == 0 ? 16 : LT;
    const int64_t gx = (p.N + tile - 1) / tile, gy = (p.M + tile - 1) / tile;
    if (gx > 0x7fffffff || gy > 65535) return hipErrorInvalidValue;
    const dim3 grid((unsigned)gx, (unsigned)gy), block(256);
    switch (rung) {
    case 0:
        hipLaunchKernelGGL(ladder_naive_kernel<IS_BF16>, grid, block, 0, p.stream, A, B, C, p.M,
                           p.N, p.K, p.lda, p.ldb, p.ldc);
        break;
    case 1:
        hipLaunchKernelGGL(ladder_lds_kernel<IS_BF16>, grid, block, 0, p.stream, A, B, C, p.M,
                           p.N, p.K, p.lda, p.ldb, p.ldc);
        break;
    case 2:
        hipLaunchKernelGGL(ladder_reg_kernel<IS_BF16>, grid, block, 0, p.stream, A, B, C, p.M,
                           p.N, p.K, p.lda, p.ldb, p.ldc);
        break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

// Rungs 0-2 for fp16 (is_bf16 false) or bf16.  Any shape with at most 65535
// row blocks (M <= 1048560 for rung 0, 4194240 for rungs 1-2).
hipError_t ladder_valu_launch(int rung, bool is_bf16, const Problem &p)
{
    return is_bf16 ? valu_typed<true>(rung, p) : valu_typed<false>(rung, p);
}

// The MFMA-only ceiling: M and N multiples of 256, K a multiple of 32, 16-byte
// aligned A and C rows.
bool mfma_ceiling_eligible(const Problem &p)
{
    return p.aligned && p.M % 256 == 0 && p.N % 256 == 0 && p.K % 32 == 0;
}

hipError_t mfma_ceiling_launch(bool is_bf16, const Problem &p)
{
    if (!mfma_ceiling_eligible(p)) return hipErrorInvalidValue;
    const int tiles_m = p.M / 256, tiles_n = p.N / 256;
    const int64_t nwg = (int64_t)tiles_m * tiles_n;
    if (nwg > 0x7fffffff) return hipErrorInvalidValue;
    const uint16_t *A = static_cast<const uint16_t *>(p.A);
    const uint16_t *B = static_cast<const uint16_t *>(p.B);
    uint16_t *C = static_cast<uint16_t *>(p.C);
    if (is_bf16)
        hipLaunchKernelGGL(mfma_ceiling_kernel<true>, dim3((unsigned)nwg), dim3(256), 0, p.stream,
                           A, B, C, p.K, p.lda, p.ldb, p.ldc, tiles_m, tiles_n);
    else
        hipLaunchKernelGGL(mfma_ceiling_kernel<false>, dim3((unsigned)nwg), dim3(256), 0, p.stream,
                           A, B, C, p.K, p.lda, p.ldb, p.ldc, tiles_m, tiles_n);
    return hipGetLastError();
}

}  // namespace gemm
