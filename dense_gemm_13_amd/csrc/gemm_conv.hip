// Convolution as a GEMM through im2col, on gfx950.
//
// "深度学习加速核心：GEMM优化从分块到TensorCore的实战解析" section 1.1: laying out
// each output position's receptive field as one row of a large matrix turns a
// convolution into a GEMM, at the price of the extra memory that matrix takes.
// Channels-last layouts make that matrix cheap to build: with X in NHWC, the row
// of output position (n, oh, ow) is, for each tap (kh, kw), the C_in contiguous
// channels of one input pixel (or zeros where the tap falls in the padding),
// and with the weights in HWIO order (KH x KW x C_in x C_out) they already are
// the GEMM's K x C_out operand, rows in the same (kh, kw, ci) order.
//
// The pack kernel is pure data movement and HBM/L2-bound.  A thread owns one
// 16-byte chunk (8 half-precision or 4 fp32 channels; one element when the
// channel count or the pointers do not allow 16 bytes) of one output position
// and walks the kh x kw taps, so the position's coordinates are derived once
// (three integer divisions, which the GPU does in software) and each tap costs a
// few additions.  The threads of a workgroup cover consecutive chunks of
// consecutive output rows: for every tap a wave reads whole runs of adjacent
// input pixels and writes whole row segments of the matrix.
#include <type_traits>

#include "gemm_device.hpp"
#include "gemm_launch.hpp"

namespace gemm {

namespace {

// VEC elements (of ESIZE bytes) per chunk, 16 bytes when VEC * ESIZE == 16.
// Workgroup b packs output rows [b * rows_per_block, (b + 1) * rows_per_block).
template <int ESIZE, int VEC>
__global__ void __launch_bounds__(256)
im2col_kernel(const void *__restrict__ X, void *__restrict__ col, int64_t ldcol, ConvShape s,
              int ho, int wo, int rows, int rows_per_block)
{
    using T = typename std::conditional<ESIZE == 2, uint16_t, uint32_t>::type;
    const int cv = s.c_in / VEC;                      // chunks per pixel
    const int per_block = rows_per_block * cv;
    const int hw = ho * wo;
    for (int q = threadIdx.x; q < per_block; q += blockDim.x) {
        const int dm = q / cv;
        const int m = blockIdx.x * rows_per_block + dm;
        if (m >= rows) break;
        const int c = (q - dm * cv) * VEC;
        const int img = m / hw, pix = m - img * hw;
        const int oh = pix / wo, ow = pix - oh * wo;
        const int ih0 = oh * s.stride_h - s.pad_h, iw0 = ow * s.stride_w - s.pad_w;
        const T *xim = static_cast<const T *>(X) + (int64_t)img * s.h * s.w * s.c_in + c;
        T *dst = static_cast<T *>(col) + (int64_t)m * ldcol + c;
        for (int kh = 0; kh < s.kh; ++kh) {
            const int ih = ih0 + kh * s.dil_h;
            const bool row_in = ih >= 0 && ih < s.h;
            for (int kw = 0; kw < s.kw; ++kw, dst += s.c_in) {
                const int iw = iw0 + kw * s.dil_w;
                const bool inside = row_in && iw >= 0 && iw < s.w;
                if constexpr (VEC * ESIZE == 16) {
                    u32x4 v = u32x4{0, 0, 0, 0};
                    if (inside)
                        v = *reinterpret_cast<const u32x4 *>(xim + ((int64_t)ih * s.w + iw) * s.c_in);
                    *reinterpret_cast<u32x4 *>(dst) = v;
                } else {
                    *dst = inside ? xim[((int64_t)ih * s.w + iw) * s.c_in] : T(0);
                }
            }
        }
    }
}

template <int ESIZE>
hipError_t im2col_typed(const void *X, void *col, int64_t ldcol, const ConvShape &s, int ho,
                        int wo, hipStream_t stream)
{
    constexpr int V = 16 / ESIZE;
    const bool vec = s.c_in % V == 0 && ((uintptr_t)X & 15) == 0 && ((uintptr_t)col & 15) == 0 &&
                     ldcol % V == 0;
    const int64_t rows = (int64_t)s.n * ho * wo;
    if (rows == 0 || s.c_in == 0) return hipSuccess;
    if (rows > 0x7fffffff) return hipErrorInvalidValue;
    const int cv = vec ? s.c_in / V : s.c_in;
    const int rows_per_block = cv >= 256 ? 1 : 256 / cv;
    const int64_t blocks = (rows + rows_per_block - 1) / rows_per_block;
    if (vec)
        hipLaunchKernelGGL((im2col_kernel<ESIZE, V>), dim3((unsigned)blocks), dim3(256), 0, stream,
                           X, col, ldcol, s, ho, wo, (int)rows, rows_per_block);
    else
        hipLaunchKernelGGL((im2col_kernel<ESIZE, 1>), dim3((unsigned)blocks), dim3(256), 0, stream,
                           X, col, ldcol, s, ho, wo, (int)rows, rows_per_block);
    return hipGetLastError();
}

}  // namespace

hipError_t im2col_launch(int esize, const void *X, void *col, int64_t ldcol, const ConvShape &s,
                         int ho, int wo, hipStream_t stream)
{
    return esize == 2 ? im2col_typed<2>(X, col, ldcol, s, ho, wo, stream)
                      : im2col_typed<4>(X, col, ldcol, s, ho, wo, stream);
}

}  // namespace gemm
