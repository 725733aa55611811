// LDS layouts of the large-tile kernels (gfx950): the XOR swizzles of their
// 16-byte chunks and the lane -> address map of every LDS access in their main
// loops and staged epilogues.  The kernels compute their addresses with these
// functions, and the host-side bank check includes this file, so what is checked
// is what the kernels do.
//
// The swizzles follow the half-precision XOR swizzle of "[CUDA 优化实战] hgemm -
// 超越 cuBLAS" section 2 (XOR row bits into the 16-byte chunk index, never split
// a chunk), with the row bits chosen for gfx950's LDS: reads are served 256
// bytes per clock (64 banks of 4 bytes: 16 lanes of a 16-byte read, 32 lanes
// of an 8-byte read, per cycle) and writes 128 bytes per clock (16 lanes of an
// 8-byte write per cycle).  Offsets are in elements of the stage's type unless
// a name says bytes.
#pragma once

#include "gemm_device.hpp"

namespace gemm {
namespace lds {

// ------------------------------------------------ bf16 / fp16 (BK = 32 or 64)
//
// A stage: TBM rows of BK halves (64 or 128 bytes).  B stage: BK rows (k) of
// TBN halves (512 bytes for 256 columns).

// 64-byte A rows (4 chunks): rows r..r+15 at one logical chunk land in 16
// distinct banks groups (four rows share a 256-byte bank window, and rows 4
// apart take distinct chunks).
__host__ __device__ __forceinline__ int swz_a4(int row) { return ((row >> 1) ^ (row >> 2)) & 3; }
// 128-byte rows (8 chunks): swz8 of gemm_device.hpp.
template <int BK>
__host__ __device__ __forceinline__ int swz_a(int row)
{
    if constexpr (BK == 64) return swz8(row);
    else return swz_a4(row);
}
// 512-byte B rows: the 4 rows one transposing read touches get their pieces
// XOR-moved by 64 bytes per row, so a 16-lane group covers distinct banks.
__host__ __device__ __forceinline__ int swz_b(int k) { return (k & 3) << 2; }

// A fragment read (ds_read_b128): row `row`, logical 16-byte chunk c.
template <int BK>
__host__ __device__ __forceinline__ int h16_a_frag(int row, int c)
{
    return row * BK + ((c ^ swz_a<BK>(row)) << 3);
}
// The offset of column n (a multiple of 4) inside B row k of a stage, for the
// transposing read ds_read_b64_tr_b16 (4 halves at column n of row k).
__host__ __device__ __forceinline__ int h16_b_col(int k, int n)
{
    return (((n >> 3) ^ swz_b(k)) << 3) + (n & 7);
}
// LDS-direct loads write lane t's 16 bytes at block + 16 t: the logical chunk
// lane t of A block `blk` carries (rows of BK halves) and of B block `blk`.
template <int BK>
__host__ __device__ __forceinline__ void h16_a_dma(int blk, int lane, int &row, int &chunk)
{
    constexpr int CPR = BK / 8, ROWS_PER_KB = 1024 / (BK * 2);
    row = ROWS_PER_KB * blk + lane / CPR;
    chunk = (lane % CPR) ^ swz_a<BK>(row);
}
template <int TBN>
__host__ __device__ __forceinline__ void h16_b_dma(int blk, int lane, int &row, int &chunk)
{
    constexpr int BCPR = TBN / 8, BRPK = 64 / BCPR;
    row = BRPK * blk + lane / BCPR;
    chunk = (lane % BCPR) ^ swz_b(row);
}

// Staged epilogue: a wave's tile of rows of CPRC 16-byte chunks.  Lane (row,
// half) writes 8 bytes of logical chunk L; a whole chunk is read back by one
// lane, which swaps its two 8-byte halves when h16_epi_swap(row).  The half is
// flipped on row bit 3, so the 16 rows of one write cycle (16 lanes, rows
// r..r+15) cover 16 distinct 8-byte bank pairs of a 128-byte window (with 256-
// byte rows, chunks c and c + 8 share banks).
__host__ __device__ __forceinline__ int h16_epi_swap(int row) { return (row >> 3) & 1; }
template <int CPRC>
__host__ __device__ __forceinline__ int h16_epi_write(int row, int L, int half)
{
    return ((L ^ (row % CPRC)) << 3) + ((half ^ h16_epi_swap(row)) << 2);
}
template <int CPRC>
__host__ __device__ __forceinline__ int h16_epi_read(int row, int cl)
{
    return (cl ^ (row % CPRC)) << 3;
}

// ----------------------------------------------------------- fp8 (bytes)
//
// A stage: TBM rows of 64 bytes (one 64-wide K block).  B stage: 64 rows of
// QBN bytes (256 or 128).

// A rows: 64 bytes (4 chunks), the same pattern as 64-byte half-precision rows.
__host__ __device__ __forceinline__ int qswz_a(int row) { return ((row >> 1) ^ (row >> 2)) & 3; }
// B rows of 256 bytes (16 chunks): the 8 rows of one transposing read land in 8
// distinct even chunks (the neighbouring 16-column group in the odd ones).
// Rows of 128 bytes (8 chunks): rows two apart share banks, so the 4 rows of
// each parity take 4 distinct even chunks.
template <int QBN>
__host__ __device__ __forceinline__ int qswz_b(int k)
{
    if constexpr (QBN == 256) return (k & 7) << 1;
    else return ((k >> 1) & 3) << 1;
}
// A fragment read (ds_read_b128): row `row`, logical 16-byte chunk c.
__host__ __device__ __forceinline__ int fp8_a_frag(int row, int c)
{
    return row * 64 + ((c ^ qswz_a(row)) << 4);
}
// Column n (a multiple of 8) of B row k, for ds_read_b64_tr_b8.
template <int QBN>
__host__ __device__ __forceinline__ int fp8_b_col(int k, int n)
{
    return (((n >> 4) ^ qswz_b<QBN>(k)) << 4) + (n & 15);
}
__host__ __device__ __forceinline__ void fp8_a_dma(int blk, int lane, int &row, int &chunk)
{
    row = 16 * blk + (lane >> 2);
    chunk = (lane & 3) ^ qswz_a(row);
}
template <int QBN>
__host__ __device__ __forceinline__ void fp8_b_dma(int blk, int lane, int &row, int &chunk)
{
    constexpr int BCPR = QBN / 16, BRPK = 64 / BCPR;
    row = BRPK * blk + lane / BCPR;
    chunk = (lane % BCPR) ^ qswz_b<QBN>(row);
}
// Staged epilogue (bf16 C, wave tiles 64 columns wide: 8 chunks per row).
__host__ __device__ __forceinline__ int fp8_epi_write(int row, int L, int half)
{
    return ((L ^ (row & 7)) << 3) + ((half ^ ((row >> 3) & 1)) << 2);
}
__host__ __device__ __forceinline__ int fp8_epi_read(int row, int cl) { return (cl ^ (row & 7)) << 3; }

// ------------------------------------------------------- fp32 (floats)
//
// A stage: 128 rows of 16 floats (64 bytes).  B stage: 16 rows of 128 floats.

// A 16-byte read by 16 lanes covers 16 consecutive rows: moving the chunks of
// rows 4a .. 4a+3 by a puts all 16 reads on distinct banks.
__host__ __device__ __forceinline__ int swz_af(int row) { return (row >> 2) & 3; }
// B is read as single floats, 32 lanes over 128 contiguous bytes of row k and
// the other 32 over row k+4: rows with bit 2 set move by 128 bytes.
__host__ __device__ __forceinline__ int swz_bf(int k) { return ((k >> 2) & 1) << 3; }
__host__ __device__ __forceinline__ int f32_a_frag(int row, int c)
{
    return row * 16 + ((c ^ swz_af(row)) << 2);
}
__host__ __device__ __forceinline__ int f32_b_elem(int k, int n)
{
    return k * 128 + (((n >> 2) ^ swz_bf(k)) << 2) + (n & 3);
}
__host__ __device__ __forceinline__ void f32_a_dma(int blk, int lane, int &row, int &chunk)
{
    row = 16 * blk + (lane >> 2);
    chunk = (lane & 3) ^ swz_af(row);
}
__host__ __device__ __forceinline__ void f32_b_dma(int blk, int lane, int &row, int &chunk)
{
    row = 2 * blk + (lane >> 5);
    chunk = (lane & 31) ^ swz_bf(row);
}

}  // namespace lds
}  // namespace gemm
