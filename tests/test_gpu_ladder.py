"""GPU parity of the measured optimisation ladder (gemm_h16_ladder, every rung,
fp16 and bf16) and of the MFMA-only ceiling kernel (gemm_h16_mfma_ceiling)
against the CPU oracle.

The ceiling kernel's result has a closed form: (K/32) * A[:, :32] * B[:32, :],
which all-ones inputs turn into K exactly, and which the oracle gives for
random inputs (its product over the first 32 columns / rows, times K/32).
"""
import functools

import numpy as np
import pytest
import torch

import gemm_inputs as gi
import oracle
from gpu_helpers import TOL, c_bits, reference, say, to_device

pytestmark = pytest.mark.gpu

RUNGS = range(9)


def run_ladder(rung, dtype, ops, M, N, K, lda=None, ldb=None, ldc=None, offset=0):
    import dense_gemm_13_amd as dg
    A = to_device(ops["A"][:M, :K], dtype, lda, offset)
    B = to_device(ops["B"][:K, :N], dtype, ldb, offset)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    ldc = N if ldc is None else ldc
    buf = torch.full((M, ldc), float("nan"), dtype=tdt, device="cuda")
    dg.gemm_h16_ladder(rung, A, B, buf[:, :N])
    torch.cuda.synchronize()
    pad = c_bits(buf[:, N:], dtype) if ldc > N else None
    return c_bits(buf[:, :N], dtype), pad


def assert_close(dtype, bits, ref, what):
    got = oracle.decode(bits, dtype)
    ok, nfail, worst, idx = oracle.within_tolerance(got, ref, *TOL[dtype])
    assert ok, (f"{what}: {nfail} of {ref.size} entries out of tolerance, worst err/tol "
                f"{worst:.3g} at {idx} (gpu {got[idx]!r}, ref {ref[idx]!r})")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("rung", RUNGS)
@pytest.mark.parametrize("shape,lds", [
    ((256, 256, 256), None),
    ((300, 520, 203), (206, 521, 525)),     # ragged, unaligned rows, offset pointers
    ((1, 70, 33), None),
])
def test_rung_parity(rung, dtype, shape, lds):
    M, N, K = shape
    kw = {} if lds is None else dict(lda=lds[0], ldb=lds[1], ldc=lds[2], offset=1)
    say(f"[ladder] rung {rung} {dtype} {M}x{N}x{K} {kw}")
    ops = gi.operands(dtype, M, N, K, 70 + rung)
    got, pad = run_ladder(rung, dtype, ops, M, N, K, **kw)
    assert_close(dtype, got, reference(dtype, ops, M, N, K), f"rung {rung} {dtype} {shape}")
    if pad is not None:
        assert np.isnan(oracle.decode(pad, dtype)).all(), "C written between N and ldc"


@functools.lru_cache(maxsize=1)
def _full_case():
    ops = gi.operands("f16", 4096, 4096, 4096, 2)
    return ops, reference("f16", ops, 4096, 4096, 4096)


@pytest.mark.parametrize("rung", RUNGS)
def test_rung_full_size(rung):
    """The ladder workload itself: fp16 M = N = K = 4096, every entry."""
    ops, ref = _full_case()
    say(f"[ladder] rung {rung} f16 4096^3")
    got, _ = run_ladder(rung, "f16", ops, 4096, 4096, 4096)
    assert_close("f16", got, ref, f"rung {rung} 4096^3")


def run_ceiling(dtype, A_bits, B_bits, M, N, K):
    import dense_gemm_13_amd as dg
    A, B = to_device(A_bits, dtype), to_device(B_bits, dtype)
    C = dg.gemm_h16_mfma_ceiling(A, B)
    torch.cuda.synchronize()
    return c_bits(C, dtype)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_ceiling_all_ones_gives_k(dtype):
    M, N, K = 512, 256, 1024
    enc = gi.to_f16_bits if dtype == "f16" else gi.to_bf16_bits
    got = run_ceiling(dtype, enc(np.ones((M, K), np.float32)), enc(np.ones((K, N), np.float32)),
                      M, N, K)
    vals = oracle.decode(got, dtype)
    assert (vals == K).all(), f"ceiling all-ones: {np.unique(vals)[:5]}"


@pytest.mark.parametrize("dtype,shape", [("f16", (512, 768, 256)), ("bf16", (4096, 4096, 4096))])
def test_ceiling_matches_closed_form(dtype, shape):
    M, N, K = shape
    say(f"[ceiling] {dtype} {M}x{N}x{K}")
    ops = gi.operands(dtype, M, N, K, 2)
    got = run_ceiling(dtype, ops["A"], ops["B"], M, N, K)
    ref = (K // 32) * oracle.gemm(dtype, ops["A"][:, :32], ops["B"][:32, :], M, N, 32)
    assert_close(dtype, got, ref, f"ceiling {dtype} {shape}")
