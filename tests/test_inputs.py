"""Seeded generators: reproducible bits, the stated distributions, and the fp8
block quantiser's properties (|q| <= 448, scale = amax/448, dequantised values
close to the originals)."""
import numpy as np
import torch

import gemm_inputs as gi
import oracle_pins as pins


def test_seeds_reproduce_bits():
    for dtype in ("f16", "bf16"):
        a = gi.uniform_h16(33, 17, 1234, dtype)
        b = gi.uniform_h16(33, 17, 1234, dtype)
        assert a.dtype == np.uint16 and np.array_equal(a, b)
        assert not np.array_equal(a, gi.uniform_h16(33, 17, 1235, dtype))
    q1, s1 = gi.normal_fp8_blockscaled(70, 130, 9)
    q2, s2 = gi.normal_fp8_blockscaled(70, 130, 9)
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)


def test_uniform_range_and_rounding():
    x = gi.uniform_f32(200, 300, 7)
    assert x.dtype == np.float32 and x.min() >= -1.0 and x.max() < 1.0
    assert abs(float(x.mean())) < 0.02
    bf = pins.lib_decode(gi.to_bf16_bits(x), "bf16")
    # round to nearest: error at most half an ulp of bf16 (2^-8 relative)
    assert np.all(np.abs(bf - x) <= np.abs(x) * 2.0 ** -8 + 1e-45)
    f16 = pins.lib_decode(gi.to_f16_bits(x), "f16")
    assert np.all(np.abs(f16 - x) <= np.maximum(np.abs(x) * 2.0 ** -11, 2.0 ** -25))


def test_bf16_rounding_is_nearest_even():
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: nearest-even picks 1.
    # 1 + 3*2^-8 ties between 1+2^-7 and 1+2^-6: even mantissa is 1+2^-6.
    x = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8], dtype=np.float32)
    assert list(pins.lib_decode(gi.to_bf16_bits(x), "bf16")) == [1.0, 1 + 2.0 ** -6]


def test_fp8_quantiser_properties():
    x = gi.normal_f32(130, 200, 11)
    q, s = gi.blockscale_e4m3(x)
    assert q.shape == x.shape and s.shape == (3, 4) and s.dtype == np.float32
    vals = pins.lib_decode(q, "fp8")
    assert not np.isnan(vals).any() and np.abs(vals).max() <= 448.0
    for i in range(3):
        for j in range(4):
            blk = x[64 * i:64 * (i + 1), 64 * j:64 * (j + 1)]
            assert s[i, j] == np.float32(np.abs(blk).max()) / np.float32(448.0)
            # the block's largest magnitude lands on (or rounds to) 448
            qb = vals[64 * i:64 * (i + 1), 64 * j:64 * (j + 1)]
            assert np.abs(qb).max() == 448.0
    deq = vals * np.repeat(np.repeat(s, 64, 0), 64, 1)[:130, :200]
    rel = np.sqrt(np.mean((deq - x) ** 2) / np.mean(x ** 2))
    assert rel < 0.04   # E4M3 keeps 3 mantissa bits: a few percent rms


def test_fp8_quantiser_saturates_and_handles_zero_blocks():
    x = np.zeros((64, 128), np.float32)
    x[0, 64] = 1000.0
    x[1, 64] = -3.0
    q, s = gi.blockscale_e4m3(x)
    assert s[0, 0] == 1.0                  # all-zero block -> unit scale
    vals = pins.lib_decode(q, "fp8")
    assert vals[0, 64] == 448.0 and not np.isnan(vals).any()


def test_workload_operands():
    ops = gi.operands("fp8", 65, 66, 67, 5)
    assert ops["A"].shape == (65, 67) and ops["scale_a"].shape == (2, 2)
    assert ops["B"].shape == (67, 66) and ops["scale_b"].shape == (2, 2)
    ops = gi.operands("f32", 5, 6, 7, 4)
    assert ops["A"].dtype == np.float32 and ops["B"].shape == (7, 6)
    assert torch.is_tensor(torch.from_numpy(ops["A"]))
