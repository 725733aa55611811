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
// The pack kernel is pure data movement and HBM/L2-bound: one thread per
// 16-byte chunk (8 half-precision or 4 fp32 channels) when the channel count
// and the pointers allow it, else one thread per element.  Consecutive threads
// write consecutive chunks of a row (coalesced) and read consecutive channels
// of one pixel.
#include <type_traits>

#include "gemm_device.hpp"
#include "gemm_launch.hpp"

namespace gemm {

namespace {

// VEC elements (of ESIZE bytes) per thread, 16 bytes when VEC * ESIZE == 16.
template <int ESIZE, int VEC>
__global__ void __launch_bounds__(256)
im2col_kernel(const void *__restrict__ X, void *__restrict__ col, int64_t ldcol, ConvShape s,
              int ho, int wo, int64_t total)
{
    using T = typename std::conditional<ESIZE == 2, uint16_t, uint32_t>::type;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= total) return;
    const int cv = s.c_in / VEC;                      // vectors per pixel
    const int64_t per_row = (int64_t)s.kh * s.kw * cv;
    const int64_t m = t / per_row;
    const int r = (int)(t - m * per_row);
    const int tap = r / cv, c = (r - tap * cv) * VEC;
    const int kh = tap / s.kw, kw = tap - kh * s.kw;
    const int64_t img = m / ((int64_t)ho * wo);
    const int pix = (int)(m - img * ho * wo);
    const int oh = pix / wo, ow = pix - oh * wo;
    const int ih = oh * s.stride_h - s.pad_h + kh * s.dil_h;
    const int iw = ow * s.stride_w - s.pad_w + kw * s.dil_w;
    const bool inside = ih >= 0 && ih < s.h && iw >= 0 && iw < s.w;
    T *dst = static_cast<T *>(col) + m * ldcol + (int64_t)tap * s.c_in + c;
    const T *src = static_cast<const T *>(X) + ((img * s.h + ih) * s.w + iw) * s.c_in + c;
    if constexpr (VEC * ESIZE == 16) {
        *reinterpret_cast<u32x4 *>(dst) =
            inside ? *reinterpret_cast<const u32x4 *>(src) : u32x4{0, 0, 0, 0};
    } else {
        *dst = inside ? *src : T(0);
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
    const int64_t total = rows * s.kh * s.kw * (vec ? s.c_in / V : s.c_in);
    const int64_t blocks = (total + 255) / 256;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    if (vec)
        hipLaunchKernelGGL((im2col_kernel<ESIZE, V>), dim3((unsigned)blocks), dim3(256), 0, stream,
                           X, col, ldcol, s, ho, wo, total);
    else
        hipLaunchKernelGGL((im2col_kernel<ESIZE, 1>), dim3((unsigned)blocks), dim3(256), 0, stream,
                           X, col, ldcol, s, ho, wo, total);
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
