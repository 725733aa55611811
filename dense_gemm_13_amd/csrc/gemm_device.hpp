// Device-side building blocks shared by the libgemm kernels (gfx950 only).
//
// Vector types for MFMA operands, LDS helpers, the XOR swizzle of 16-byte LDS
// chunks, the workgroup -> output-tile remap, and fp32 -> fp16/bf16 rounding.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_launch.hpp"

namespace gemm {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// 16-byte chunk index XOR pattern for tiles whose rows are 8 chunks (128 bytes)
// long.  Rows r..r+7 (r a multiple of 8) map a given logical chunk to 8 distinct
// physical chunks, and so do rows r, r+8, ..., r+56: both the column-of-rows
// fragment reads and the strided transposed writes spread over all banks.  It is
// the half-precision XOR swizzle of "[CUDA 优化实战] hgemm - 超越 cuBLAS" section 2
// (XOR row bits into the 16-byte chunk index, leave the bytes inside a chunk
// alone), with the row bits chosen for the access patterns of these kernels.
__host__ __device__ __forceinline__ int swz8(int row) { return (row ^ (row >> 3)) & 7; }

// Same idea for rows of 4 chunks (64 bytes, two rows per 128-byte line).
__host__ __device__ __forceinline__ int swz4(int row) { return (row >> 1) & 3; }

// ---------------------------------------------------------------- tile remap
//
// Workgroups of a 1-D grid are handed to the 8 XCDs of the chip round-robin
// (workgroup b runs on XCD b % 8), and each XCD has its own L2.  The remap first
// gives each XCD a contiguous range of logical tile ids, then walks tile ids in
// strips of `group_m` tile-rows so that the tiles one XCD holds at a time share
// A row-panels and B column-panels in its L2 (the grid swizzle of
// "[CUDA 优化实战] hgemm - 超越 cuBLAS" section 1, made XCD-aware and correct for
// grids that are not multiples of the strip width or of 8).
__host__ __device__ __forceinline__ void tile_coords(int bid, int nwg, int tiles_m, int tiles_n,
                                            int group_m, int &tm, int &tn)
{
    constexpr int XCDS = 8;
    int q = nwg / XCDS, r = nwg % XCDS;
    int xcd = bid % XCDS, pos = bid / XCDS;
    int id = (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + pos;
    int per_group = group_m * tiles_n;
    int g = id / per_group;
    int first_m = g * group_m;
    int rows = tiles_m - first_m < group_m ? tiles_m - first_m : group_m;
    int in_g = id - g * per_group;
    tm = first_m + in_g % rows;
    tn = in_g / rows;
}

// ----------------------------------------------------------- strided K walks
//
// Element index of lane offset r in group g of a walk over `ngroups` groups of
// `per` consecutive elements, or `limit` (one past the last element, read as
// zero by the caller) when g lies past the last group.  The group index is
// compared before it is multiplied, so a wave that steps past the end never
// forms g * per: with ngroups = ceil(limit / per), every index formed is below
// limit + per, which stays in 32-bit range for limit <= 2^31 - 2^16.
__host__ __device__ __forceinline__ int group_elem(int g, int ngroups, int per, int r, int limit)
{
    return g < ngroups ? g * per + r : limit;
}

// ------------------------------------------------------------ output rounding

// Round to nearest, ties to even (hardware conversions on gfx950).
__device__ __forceinline__ uint16_t to_bf16_bits(float f)
{
    __bf16 h = static_cast<__bf16>(f);
    return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ uint16_t to_f16_bits(float f)
{
    _Float16 h = static_cast<_Float16>(f);
    return __builtin_bit_cast(uint16_t, h);
}

template <bool IS_BF16>
__device__ __forceinline__ uint32_t pack2(float lo, float hi)
{
    if constexpr (IS_BF16)
        return (uint32_t)to_bf16_bits(lo) | ((uint32_t)to_bf16_bits(hi) << 16);
    else
        return (uint32_t)to_f16_bits(lo) | ((uint32_t)to_f16_bits(hi) << 16);
}

// ------------------------------------------------------------ fused epilogue

enum OutType { OUT_F16 = 0, OUT_BF16 = 1, OUT_F32 = 2 };

// fp32 value of element n of a C row of type OUT.
template <int OUT>
__device__ __forceinline__ float load_out(const void *row, int n)
{
    if constexpr (OUT == OUT_F32) {
        return static_cast<const float *>(row)[n];
    } else {
        const uint16_t bits = static_cast<const uint16_t *>(row)[n];
        if constexpr (OUT == OUT_BF16) return __uint_as_float((uint32_t)bits << 16);
        else return (float)__builtin_bit_cast(_Float16, bits);
    }
}

// The fused epilogue on W consecutive fp32 results v[0..W) of one row of C,
// columns n .. n+W-1, of which the first `cnt` are inside the matrix (cnt <= 0:
// none).  Those become
//   act(alpha * v + beta * c_prior + bias[column])
// with the prior C read only when beta != 0 and only inside the matrix.  A
// fully connected layer is a product plus one bias per output feature
// ("深度学习加速核心：GEMM优化从分块到TensorCore的实战解析" section 1.1); the relu
// is the epilogue of the vendor kernel "[CUDA 优化实战] hgemm - 超越 cuBLAS"
// compares against (section 5).  The three steps are separate so that a kernel
// can load the bias once per column and the prior C of a whole row block ahead
// of the arithmetic.

// bias[n .. n+W) (0 past cnt or without a bias); one vector load when all W are
// inside and aligned.
template <int W>
__device__ __forceinline__ void epilogue_bias(const Epilogue &e, int n, int cnt, float *b)
{
    static_assert(W == 4 || W == 8, "epilogue width");
    if (e.bias && cnt >= W && ((uintptr_t)(e.bias + n) & 15) == 0) {
#pragma unroll
        for (int h = 0; h < W / 4; ++h) {
            const f32x4 x = *reinterpret_cast<const f32x4 *>(e.bias + n + 4 * h);
#pragma unroll
            for (int t = 0; t < 4; ++t) b[4 * h + t] = x[t];
        }
    } else {
#pragma unroll
        for (int t = 0; t < W; ++t) b[t] = e.bias && t < cnt ? e.bias[n + t] : 0.f;
    }
}

// The prior C at row[n .. n+W) as fp32 (0 past cnt or when beta == 0); 16-bit
// types are read W at a time when all are inside and the address is aligned.
template <int OUT, int W>
__device__ __forceinline__ void epilogue_prior(const Epilogue &e, const void *row, int n, int cnt,
                                               float *c)
{
    static_assert(W == 4 || W == 8, "epilogue width");
    if (e.beta == 0.f) {
#pragma unroll
        for (int t = 0; t < W; ++t) c[t] = 0.f;
        return;
    }
    if constexpr (OUT != OUT_F32) {
        const uint16_t *p = static_cast<const uint16_t *>(row) + n;
        if (cnt >= W && ((uintptr_t)p & (2 * W - 1)) == 0) {
            uint32_t w[W / 2];
            if constexpr (W == 4) {
                const u32x2 x = *reinterpret_cast<const u32x2 *>(p);
                w[0] = x[0]; w[1] = x[1];
            } else {
                const u32x4 x = *reinterpret_cast<const u32x4 *>(p);
                w[0] = x[0]; w[1] = x[1]; w[2] = x[2]; w[3] = x[3];
            }
#pragma unroll
            for (int t = 0; t < W; ++t) {
                const uint16_t bits = (uint16_t)(w[t >> 1] >> (16 * (t & 1)));
                if constexpr (OUT == OUT_BF16) c[t] = __uint_as_float((uint32_t)bits << 16);
                else c[t] = (float)__builtin_bit_cast(_Float16, bits);
            }
            return;
        }
    } else {
        const float *p = static_cast<const float *>(row) + n;
        if (cnt >= W && ((uintptr_t)p & 15) == 0) {
#pragma unroll
            for (int h = 0; h < W / 4; ++h) {
                const f32x4 x = *reinterpret_cast<const f32x4 *>(p + 4 * h);
#pragma unroll
                for (int t = 0; t < 4; ++t) c[4 * h + t] = x[t];
            }
            return;
        }
    }
#pragma unroll
    for (int t = 0; t < W; ++t) c[t] = t < cnt ? load_out<OUT>(row, n + t) : 0.f;
}

// The bias and prior-C loads for whole groups of W columns at offsets that are
// multiples of W, as in a whole tile.  Whether the vector loads apply then
// depends only on the base pointers and ldc, so the caller decides it once per
// kernel (`vec`, a uniform branch) instead of from each lane's own address,
// which made every group a divergent branch with an element-wise fallback.
template <int W>
__device__ __forceinline__ void epilogue_bias_whole(const Epilogue &e, int n, bool vec, float *b)
{
    static_assert(W == 4 || W == 8, "epilogue width");
    if (vec) {
#pragma unroll
        for (int h = 0; h < W / 4; ++h) {
            const f32x4 x = *reinterpret_cast<const f32x4 *>(e.bias + n + 4 * h);
#pragma unroll
            for (int t = 0; t < 4; ++t) b[4 * h + t] = x[t];
        }
    } else if (e.bias) {
#pragma unroll
        for (int t = 0; t < W; ++t) b[t] = e.bias[n + t];
    } else {
#pragma unroll
        for (int t = 0; t < W; ++t) b[t] = 0.f;
    }
}
// Prior C of W whole 16-bit columns; `vec`: row + n is 2W-byte aligned for
// every row and group.  The caller reads nothing when beta == 0.
template <int OUT, int W>
__device__ __forceinline__ void epilogue_prior_whole(const void *row, int n, bool vec, float *c)
{
    static_assert(OUT != OUT_F32 && W == 4, "16-bit groups of 4");
    const uint16_t *p = static_cast<const uint16_t *>(row) + n;
    if (vec) {
        const u32x2 x = *reinterpret_cast<const u32x2 *>(p);
#pragma unroll
        for (int t = 0; t < W; ++t) {
            const uint16_t bits = (uint16_t)(x[t >> 1] >> (16 * (t & 1)));
            if constexpr (OUT == OUT_BF16) c[t] = __uint_as_float((uint32_t)bits << 16);
            else c[t] = (float)__builtin_bit_cast(_Float16, bits);
        }
    } else {
#pragma unroll
        for (int t = 0; t < W; ++t) c[t] = load_out<OUT>(row, n + t);
    }
}

// One entry before the activation: alpha * v + b in one fused multiply-add,
// then + beta * c (a second one) when the prior C is read.  Every kernel's
// epilogue evaluates it this way.
__device__ __forceinline__ float epilogue_value(const Epilogue &e, float v, float b)
{
    return fmaf(e.alpha, v, b);
}
__device__ __forceinline__ float epilogue_value(const Epilogue &e, float v, float b, float c)
{
    return fmaf(e.beta, c, fmaf(e.alpha, v, b));
}
// relu; NaN and -0 become +0, as with x > 0 ? x : 0.
__device__ __forceinline__ float epilogue_relu(float x) { return x > 0.f ? x : 0.f; }

// v = act(alpha * v + beta * c + b) for the first cnt entries.
template <int W>
__device__ __forceinline__ void epilogue_apply(const Epilogue &e, float *v, const float *b,
                                               const float *c, int cnt)
{
#pragma unroll
    for (int t = 0; t < W; ++t) {
        if (t < cnt) {
            float x = e.beta != 0.f ? epilogue_value(e, v[t], b[t], c[t]) : epilogue_value(e, v[t], b[t]);
            if (e.relu) x = epilogue_relu(x);
            v[t] = x;
        }
    }
}

// All three steps for one group of W entries (`row` points at column 0).
template <int OUT, int W>
__device__ __forceinline__ void epilogue_row(const Epilogue &e, float *v, const void *row, int n,
                                             int cnt)
{
    float b[W], c[W];
    epilogue_bias<W>(e, n, cnt, b);
    epilogue_prior<OUT, W>(e, row, n, cnt, c);
    epilogue_apply<W>(e, v, b, c, cnt);
}

// -------------------------------------------------------------- masked loads

// v shifted down by `bytes` (0..16): byte i of the result is byte i + bytes of
// v, zero past the end.  Selects, no branches: a caller's loads can all be in
// flight before the first value is used.
__device__ __forceinline__ u32x4 shift_down_bytes(u32x4 v, int bytes)
{
    const uint64_t lo = (uint64_t)v[0] | ((uint64_t)v[1] << 32);
    const uint64_t hi = (uint64_t)v[2] | ((uint64_t)v[3] << 32);
    const int s = 8 * bytes, a = s & 63;
    const uint64_t hi_a = hi >> a;
    const uint64_t lo_small = (lo >> a) | ((hi << 1) << (63 - a));   // s < 64
    const uint64_t nlo = s >= 128 ? 0 : s >= 64 ? hi_a : lo_small;
    const uint64_t nhi = s >= 64 ? 0 : hi_a;
    return u32x4{(uint32_t)nlo, (uint32_t)(nlo >> 32), (uint32_t)nhi, (uint32_t)(nhi >> 32)};
}

// The 16 bytes of elements [k, k + 16/ESZ) of row `row` of a row-major matrix
// (leading dimension ld elements, rows x cols valid), with zeros for a row
// past `rows` and for columns past `cols`, in two halves: masked16_load issues
// one 16-byte load at an address inside the matrix, masked16_value applies the
// zeros to what it returned.  A chunk that straddles `cols` is loaded as the
// row's last 16 bytes and shifted down; a chunk wholly outside reads the
// matrix's first element and is zeroed.  A caller issues all its loads before
// taking the first value, so they are in flight together.  Requires
// cols * ESZ >= 16.  The address may be only ESZ-aligned (the hardware runs in
// unaligned-access mode).
struct Masked16 {
    u32x4 raw;
    int drop;                                          // bytes to shift out
};
template <int ESZ>
__device__ __forceinline__ Masked16 masked16_load(const void *base, int64_t ld, int row, int rows,
                                                  int k, int cols)
{
    constexpr int EPV = 16 / ESZ;
    const bool inside = row < rows && k < cols;
    int kk = k, drop = 0;
    if (k + EPV > cols) kk = cols - EPV, drop = (k - kk) * ESZ;
    if (!inside) kk = 0, drop = 16;
    const char *src = static_cast<const char *>(base) +
                      ((int64_t)(inside ? row : 0) * ld + kk) * ESZ;
    return Masked16{*reinterpret_cast<const u32x4 *>(src), drop};
}
__device__ __forceinline__ u32x4 masked16_value(const Masked16 &m)
{
    return shift_down_bytes(m.raw, m.drop);
}

// -------------------------------------------------------------- MFMA wrappers

// D(32x32, fp32) += X(32x16) * Y(16x32) with X taken from `x` (row = lane%32,
// k = 8*(lane/32) + 0..7) and Y from `y` (column = lane%32, same k).
template <bool IS_BF16>
__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 x, u32x4 y, f32x16 acc)
{
    if constexpr (IS_BF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, x),
                                                       __builtin_bit_cast(bf16x8, y), acc, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, x),
                                                      __builtin_bit_cast(f16x8, y), acc, 0, 0, 0);
}

}  // namespace gemm
