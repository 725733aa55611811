"""Seeded synthetic operands for the dense GEMM workloads.

This module only draws random numbers and rounds them to the storage format;
it holds none of the product's arithmetic.  Both the GPU tests/bench and the
CPU oracle consume what it returns, so the two sides see identical bits.

Recipe (the pages use synthetic square matrices and fix no distribution, so
this is the plain reading):
* numpy ``default_rng(seed)`` (PCG64);
* fp16/bf16 workloads: ``random(dtype=float32)*2 - 1`` i.e. uniform[-1, 1) in
  fp32, then rounded to nearest-even to the storage type;
* fp32 workload: ``standard_normal(dtype=float32)``;
* fp8 workload ("深度学习加速核心：GEMM优化从分块到TensorCore的实战解析",
  section 4.3: E4M3 operands with one scale per 64x64 sub-block; section 5.2:
  32-bit scales): N(0, 1) fp32 values, per 64x64 block s = amax/448 in fp32
  (s = 1 for an all-zero block), q = E4M3 round-to-nearest-even of
  clamp(x/s, -448, 448).  Blocks at ragged edges cover what is left.
"""
from __future__ import annotations

import numpy as np
import torch

E4M3_MAX = 448.0
SCALE_BLOCK = 64

# Seeds: A = 1000 + workload id, B = 2000 + workload id.
SEED_A_BASE = 1000
SEED_B_BASE = 2000


def _rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def uniform_f32(rows: int, cols: int, seed: int) -> np.ndarray:
    """uniform[-1, 1) float32 matrix."""
    u = _rng(seed).random((rows, cols), dtype=np.float32)
    return u * np.float32(2.0) - np.float32(1.0)


def normal_f32(rows: int, cols: int, seed: int) -> np.ndarray:
    """N(0, 1) float32 matrix."""
    return _rng(seed).standard_normal((rows, cols), dtype=np.float32)


def to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to IEEE binary16 (nearest-even); returns the uint16 bits."""
    return np.ascontiguousarray(x).astype(np.float16).view(np.uint16)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest-even, torch CPU cast); returns uint16 bits."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 already inside [-448, 448] to OCP E4M3 (nearest-even); uint8 bits."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


def uniform_h16(rows: int, cols: int, seed: int, dtype: str) -> np.ndarray:
    """uniform[-1,1) values rounded to 'f16' or 'bf16'; uint16 bit matrix."""
    x = uniform_f32(rows, cols, seed)
    if dtype == "f16":
        return to_f16_bits(x)
    if dtype == "bf16":
        return to_bf16_bits(x)
    raise ValueError(dtype)


def blockscale_e4m3(x: np.ndarray, block: int = SCALE_BLOCK):
    """Quantise a float32 matrix to E4M3 with one fp32 scale per block x block tile.

    Returns (q uint8 of x.shape, scales float32 of (ceil(rows/block), ceil(cols/block))).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, cols = x.shape
    br, bc = -(-rows // block), -(-cols // block)
    # x padded with zeros to whole blocks: padding never raises a block's amax.
    padded = np.zeros((br * block, bc * block), dtype=np.float32)
    padded[:rows, :cols] = x
    tiles = padded.reshape(br, block, bc, block)
    amax = np.abs(tiles).max(axis=(1, 3))
    scales = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    np.divide(tiles, scales[:, None, :, None], out=tiles)          # fp32 x / s per block
    np.clip(tiles, -E4M3_MAX, E4M3_MAX, out=tiles)
    return to_e4m3_bits(padded[:rows, :cols]), scales


def normal_fp8_blockscaled(rows: int, cols: int, seed: int, block: int = SCALE_BLOCK):
    """N(0,1) float32 matrix quantised per block to E4M3 + fp32 scales."""
    return blockscale_e4m3(normal_f32(rows, cols, seed), block)


# ----------------------------------------------------------------- workloads

# The five workloads, by name.  Shapes are (M, N, K); A is M x K, B is K x N,
# row-major and contiguous.
WORKLOADS = {
    "f16_256": dict(id=1, dtype="f16", shapes=[(256, 256, 256)]),
    "h16_4096": dict(id=2, dtype=("bf16", "f16"), shapes=[(4096, 4096, 4096)]),
    "bf16_ragged": dict(id=3, dtype="bf16",
                        shapes=[(1000, 1000, 1000), (4097, 4095, 4100), (8192, 64, 4096)]),
    "f32_4096": dict(id=4, dtype="f32", shapes=[(4096, 4096, 4096)]),
    "fp8_8192": dict(id=5, dtype="fp8", shapes=[(8192, 8192, 8192)]),
}


def operands(dtype: str, M: int, N: int, K: int, wid: int):
    """Raw operands for one GEMM: returns dict(A=..., B=..., scale_a=..., scale_b=...).

    fp16/bf16: uniform[-1,1) rounded; f32: N(0,1); fp8: N(0,1) block-quantised.
    """
    sa, sb = SEED_A_BASE + wid, SEED_B_BASE + wid
    if dtype in ("f16", "bf16"):
        return dict(A=uniform_h16(M, K, sa, dtype), B=uniform_h16(K, N, sb, dtype))
    if dtype == "f32":
        return dict(A=normal_f32(M, K, sa), B=normal_f32(K, N, sb))
    if dtype == "fp8":
        qa, scale_a = normal_fp8_blockscaled(M, K, sa)
        qb, scale_b = normal_fp8_blockscaled(K, N, sb)
        return dict(A=qa, B=qb, scale_a=scale_a, scale_b=scale_b)
    raise ValueError(dtype)
