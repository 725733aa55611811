// Host-side interface between the C-ABI entry points and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gemm {

// Fused epilogue of one call: every output value v becomes
//   act(alpha * v + beta * c_prior + bias[column])
// in fp32 before it is rounded to C's type; c_prior (C before the call) is read
// only when beta != 0, bias is nullptr for none, relu is 0 or 1.
struct Epilogue {
    float alpha, beta;
    const float *bias;
    int relu;
};

// One GEMM call after argument checking: every size fits in int, K >= 1,
// M >= 1, N >= 1.  `aligned` says the 16-byte vector paths are legal for this
// call (pointer and leading-dimension alignment as required by the dtype).
struct Problem {
    const void *A;
    const void *B;
    void *C;
    int M, N, K;
    int64_t lda, ldb, ldc;
    bool aligned;
    hipStream_t stream;
    const Epilogue *epi;   // nullptr: plain C = A*B
};

// Half-precision tile configurations (rows x cols of C per workgroup, waves).
enum H16Config {
    H16_256x256_W8 = 0,   // 256x256 tile, 8 waves (2 x 4), wave tile 128x64
    H16_128x128_W4 = 1,   // 128x128 tile, 4 waves (2 x 2), wave tile 64x64
    H16_64x64_W4 = 2,     // 64x64 tile, 4 waves (2 x 2), wave tile 32x32
    H16_32x64_W2 = 3,     // 32x64 tile, 2 waves (1 x 2), wave tile 32x32
    H16_FAST_256x256 = 4, // whole 256x256 tiles, LDS-direct loads, 4 waves of 128x128
    H16_GEN_256x256 = 5,  // same kernel, guarded: ragged M/N/K, any leading dimensions
    H16_NARROW_32x64 = 6, // whole 32x64 tiles, 4 waves splitting K (tall, narrow products)
    H16_NARROW_GEN = 7,   // same kernel, guarded: any M, N >= 8, K, leading dimensions
    H16_NARROW64 = 8,     // whole 64x64 tiles, 4 waves splitting K, 2 LDS stages per wave
    H16_NARROW64_GEN = 9, // same kernel, guarded
    H16_ROWS = 10,        // at most 4 rows: vector-ALU stream over B, 64 columns per workgroup
    H16_FAST_128 = 11,    // whole 128x128 tiles of the large-tile kernel, two workgroups per CU
    H16_GEN_128 = 12,     // same kernel, guarded
    H16_FAST_128x256 = 13, // whole 128x256 tiles of the large-tile kernel, one workgroup per CU
    H16_GEN_128x256 = 14, // same kernel, guarded
    H16_FEWROWS = 15,     // at most 4 rows: B streamed through per-wave LDS rings, 32 columns per workgroup
    H16_NUM_CONFIGS = 16
};

int h16_pick_config(int M, int N, int K);
hipError_t h16_launch(bool is_bf16, int config, const Problem &p);
bool h16_fast_eligible(const Problem &p);
hipError_t h16_fast_launch(bool is_bf16, const Problem &p);
bool h16_general_eligible(const Problem &p);
hipError_t h16_general_launch(bool is_bf16, const Problem &p);
bool h16_fast128_eligible(const Problem &p);
hipError_t h16_fast128_launch(bool is_bf16, const Problem &p);
hipError_t h16_general128_launch(bool is_bf16, const Problem &p);
bool h16_fast128x256_eligible(const Problem &p);
hipError_t h16_fast128x256_launch(bool is_bf16, const Problem &p);
hipError_t h16_general128x256_launch(bool is_bf16, const Problem &p);
bool h16_narrow_eligible(const Problem &p);
hipError_t h16_narrow_launch(bool is_bf16, const Problem &p);
bool h16_narrow_general_eligible(const Problem &p);
hipError_t h16_narrow_general_launch(bool is_bf16, const Problem &p);
bool h16_narrow64_eligible(const Problem &p);
hipError_t h16_narrow64_launch(bool is_bf16, const Problem &p);
hipError_t h16_narrow64_general_launch(bool is_bf16, const Problem &p);
// At most 4 rows of A (N >= 16, the rows of A fit in 32 KiB of LDS).
bool h16_fewrows_eligible(const Problem &p);
bool h16_fewrows_preferred(const Problem &p);
hipError_t h16_fewrows_launch(bool is_bf16, const Problem &p);
// The measured optimisation ladder (fp16 or bf16): rungs 0-2 on the vector
// ALUs, rungs 3-5 the 128 x 128 MFMA kernel with its ring / swizzle switched,
// and the MFMA-only ceiling of the large-tile kernel.
hipError_t ladder_valu_launch(int rung, bool is_bf16, const Problem &p);
hipError_t h16_ladder_launch(int rung, bool is_bf16, const Problem &p);
bool mfma_ceiling_eligible(const Problem &p);
hipError_t mfma_ceiling_launch(bool is_bf16, const Problem &p);
hipError_t f32_launch(const Problem &p, int cus);
// At most 4 rows of A; out: the element type (OUT_F16, OUT_BF16 or OUT_F32).
bool rows_eligible(const Problem &p);
hipError_t rows_launch(int out, const Problem &p);
bool f32_fast_eligible(const Problem &p);
hipError_t f32_fast_launch(const Problem &p, int cus);
bool f32_general_eligible(const Problem &p);
hipError_t f32_general_launch(const Problem &p);
bool f32_narrow_general_eligible(const Problem &p);
hipError_t f32_narrow_launch(const Problem &p, int tbm, bool force_general);
hipError_t fp8_launch(const Problem &p, const float *scale_a, const float *scale_b, int cus);
bool fp8_narrow_general_eligible(const Problem &p);
hipError_t fp8_narrow_launch(const Problem &p, const float *scale_a, const float *scale_b, int tbm,
                             bool force_general);
bool fp8_fast_eligible(const Problem &p);
hipError_t fp8_fast_launch(const Problem &p, const float *scale_a, const float *scale_b);
bool fp8_general_eligible(const Problem &p);
hipError_t fp8_general_launch(const Problem &p, const float *scale_a, const float *scale_b);
bool fp8_fast128_eligible(const Problem &p);
hipError_t fp8_tiles128_launch(const Problem &p, const float *scale_a, const float *scale_b,
                               bool force_general);
// One quantiser call after argument checking: rows, cols >= 1, block 32 or 64,
// fmt 0 (E4M3) or 1 (E5M2).
struct QuantProblem {
    const void *X;
    bool in_bf16;
    int rows, cols;
    int64_t ldx;
    int block, fmt;
    uint8_t *Q;
    int64_t ldq;
    float *scales;
    hipStream_t stream;
};
hipError_t quant_fp8_launch(const QuantProblem &p);
// Convolution geometry after argument checking (every field fits in int; the
// products that index memory are formed in 64 bits).
struct ConvShape {
    int n, h, w, c_in, c_out, kh, kw, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w;
};
// The im2col matrix of an NHWC tensor X (element size esize 2 or 4) into col,
// (n*ho*wo) rows of kh*kw*c_in elements at leading dimension ldcol.
hipError_t im2col_launch(int esize, const void *X, void *col, int64_t ldcol, const ConvShape &s,
                         int ho, int wo, hipStream_t stream);
// K == 0: every sum is empty.  Sets the M x N window of C (out: 0 fp16, 1 bf16,
// 2 fp32; leading dimension ldc) to zero, or with an epilogue to
// act(beta * c_prior + bias[column]).
hipError_t empty_sum_launch(void *C, int M, int N, int64_t ldc, int out, const Epilogue *epi,
                            hipStream_t stream);

}  // namespace gemm
