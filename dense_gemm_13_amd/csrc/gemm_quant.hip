// Block-scaled FP8 quantiser on gfx950: X (fp32 or bf16, rows x cols, row-major)
// -> Q (FP8 codes, E4M3 or E5M2) plus one fp32 scale per BLOCK x BLOCK block.
//
// "深度学习加速核心：GEMM优化从分块到TensorCore的实战解析", section 4.3 (FP8
// operands with one scale per 32x32 or 64x64 sub-block) and section 5.2, third
// pitfall (the scales are 32-bit floats).  Per block:
//   amax = max |x| over the block's elements inside the matrix,
//   s    = amax / F, one IEEE fp32 division (F = 448 for E4M3, 57344 for E5M2;
//          s = 1 for an all-zero block),
//   q    = the FP8 value nearest to clamp(x / s, -F, F), ties to even, where
//          x / s is again one IEEE fp32 division.
// This is the quantiser the FP8 GEMM's operands come from: its scale grid is
// the ceil(rows/BLOCK) x ceil(cols/BLOCK) row-major grid gemm_fp8_blockscaled
// reads (BLOCK = 64).
//
// One wave per block.  The wave reads its block once into registers (16-byte
// loads, one block row spread over BLOCK*esize/16 lanes), takes the amax with a
// butterfly of lane shuffles, then divides, converts (v_cvt_pk_fp8_f32 /
// v_cvt_pk_bf8_f32, round to nearest-even) and stores from the same registers.
// No LDS and no barrier.  The four waves of a workgroup take four horizontally
// adjacent blocks, so each row of a workgroup's strip is 4*BLOCK*esize
// contiguous bytes.  The kernel is HBM-bound: every input byte is read once and
// every code written once.
#include "gemm_device.hpp"
#include "gemm_launch.hpp"

namespace gemm {

namespace {

constexpr int QUANT_WAVES = 4;

template <int FMT>
struct Fp8Max;
template <>
struct Fp8Max<0> { static constexpr float value = 448.0f; };
template <>
struct Fp8Max<1> { static constexpr float value = 57344.0f; };

// Two FP8 codes (y0 in the low byte) packed into half of `old`.
template <int FMT, bool HIGH>
__device__ __forceinline__ uint32_t cvt2(float y0, float y1, uint32_t old)
{
    if constexpr (FMT == 0)
        return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, (int)old, HIGH);
    else
        return (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(y0, y1, (int)old, HIGH);
}

// Input element types: fp32 as its value, bf16 as its 16 bits (exact widening).
template <typename T>
__device__ __forceinline__ float widen(T v);
template <>
__device__ __forceinline__ float widen<float>(float v) { return v; }
template <>
__device__ __forceinline__ float widen<uint16_t>(uint16_t v)
{
    return __uint_as_float((uint32_t)v << 16);
}

// IN_BF16: X holds bf16 bits, else fp32.  ALIGNED: X, ldx, Q and ldq allow
// whole 16-byte input vectors and whole EPV-byte code stores.
template <bool IN_BF16, int BLOCK, int FMT, bool ALIGNED>
__global__ void __launch_bounds__(QUANT_WAVES * 64)
quant_fp8_kernel(const void *__restrict__ Xv, int rows, int cols, int64_t ldx,
                 uint8_t *__restrict__ Q, int64_t ldq, float *__restrict__ scales,
                 int block_cols, int groups)
{
    using T = typename std::conditional<IN_BF16, uint16_t, float>::type;
    constexpr int EPV = 16 / (int)sizeof(T);   // elements per 16-byte vector
    constexpr int LPR = BLOCK / EPV;           // lanes per block row
    constexpr int RPL = 64 / LPR;              // block rows per wave load
    constexpr int NLOAD = BLOCK / RPL;         // loads per lane
    static_assert(LPR * EPV == BLOCK && RPL * LPR == 64 && NLOAD * RPL == BLOCK, "lane map");
    constexpr float FMAX = Fp8Max<FMT>::value;

    const T *__restrict__ X = static_cast<const T *>(Xv);
    const int lane = threadIdx.x & 63;
    const int br = blockIdx.x / groups;
    const int bc = (blockIdx.x % groups) * QUANT_WAVES + (threadIdx.x >> 6);
    if (bc >= block_cols) return;
    const int r_lane = lane / LPR;
    const int c0 = bc * BLOCK + (lane % LPR) * EPV;
    const int64_t row0 = (int64_t)br * BLOCK + r_lane;

    float v[NLOAD][EPV];
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < NLOAD; ++j) {
        const int64_t r = row0 + j * RPL;
        const T *src = X + r * ldx + c0;
        if (ALIGNED && r < rows && c0 + EPV <= cols) {
            const u32x4 w = *reinterpret_cast<const u32x4 *>(src);
            if constexpr (IN_BF16) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[j][2 * e] = __uint_as_float(w[e] << 16);
                    v[j][2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) v[j][e] = __uint_as_float(w[e]);
            }
        } else {
#pragma unroll
            for (int e = 0; e < EPV; ++e)
                v[j][e] = (r < rows && c0 + e < cols) ? widen<T>(src[e]) : 0.0f;
        }
#pragma unroll
        for (int e = 0; e < EPV; ++e) amax = fmaxf(amax, fabsf(v[j][e]));
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));

    const float s = amax > 0.0f ? amax / FMAX : 1.0f;
    if (lane == 0) scales[(int64_t)br * block_cols + bc] = s;

#pragma unroll
    for (int j = 0; j < NLOAD; ++j) {
        const int64_t r = row0 + j * RPL;
        uint32_t w[EPV / 4];
#pragma unroll
        for (int e = 0; e < EPV / 4; ++e) {
            float y[4];
#pragma unroll
            for (int t = 0; t < 4; ++t)
                y[t] = fminf(fmaxf(v[j][4 * e + t] / s, -FMAX), FMAX);
            w[e] = cvt2<FMT, true>(y[2], y[3], cvt2<FMT, false>(y[0], y[1], 0u));
        }
        if (r >= rows) continue;
        uint8_t *dst = Q + r * ldq + c0;
        if (ALIGNED && c0 + EPV <= cols) {
            if constexpr (EPV == 4)
                *reinterpret_cast<uint32_t *>(dst) = w[0];
            else
                *reinterpret_cast<u32x2 *>(dst) = u32x2{w[0], w[1]};
        } else {
#pragma unroll
            for (int e = 0; e < EPV; ++e)
                if (c0 + e < cols) dst[e] = (uint8_t)(w[e >> 2] >> ((e & 3) * 8));
        }
    }
}

template <bool IN_BF16, int BLOCK, int FMT>
hipError_t quant_launch3(const QuantProblem &p)
{
    const int block_rows = (p.rows + BLOCK - 1) / BLOCK;
    const int block_cols = (p.cols + BLOCK - 1) / BLOCK;
    const int groups = (block_cols + QUANT_WAVES - 1) / QUANT_WAVES;
    const int64_t nwg = (int64_t)groups * block_rows;
    if (nwg > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid((unsigned)nwg);
    const int esize = IN_BF16 ? 2 : 4;
    const int epv = 16 / esize;
    const bool aligned = ((uintptr_t)p.X & 15) == 0 && (p.ldx % epv) == 0 &&
                         ((uintptr_t)p.Q % epv) == 0 && (p.ldq % epv) == 0;
    if (aligned)
        hipLaunchKernelGGL((quant_fp8_kernel<IN_BF16, BLOCK, FMT, true>), grid,
                           dim3(QUANT_WAVES * 64), 0, p.stream, p.X, p.rows, p.cols, p.ldx, p.Q,
                           p.ldq, p.scales, block_cols, groups);
    else
        hipLaunchKernelGGL((quant_fp8_kernel<IN_BF16, BLOCK, FMT, false>), grid,
                           dim3(QUANT_WAVES * 64), 0, p.stream, p.X, p.rows, p.cols, p.ldx, p.Q,
                           p.ldq, p.scales, block_cols, groups);
    return hipGetLastError();
}

template <bool IN_BF16, int BLOCK>
hipError_t quant_launch2(const QuantProblem &p)
{
    return p.fmt == 0 ? quant_launch3<IN_BF16, BLOCK, 0>(p) : quant_launch3<IN_BF16, BLOCK, 1>(p);
}

template <bool IN_BF16>
hipError_t quant_launch1(const QuantProblem &p)
{
    return p.block == 32 ? quant_launch2<IN_BF16, 32>(p) : quant_launch2<IN_BF16, 64>(p);
}

}  // namespace

hipError_t quant_fp8_launch(const QuantProblem &p)
{
    return p.in_bf16 ? quant_launch1<true>(p) : quant_launch1<false>(p);
}

}  // namespace gemm
