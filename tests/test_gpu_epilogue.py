"""GPU parity of the fused epilogue entry points (gemm_*_epilogue): every kernel
path, forced where the dispatcher would not pick it, against the CPU oracle's
act(alpha * A*B + beta * C_prior + bias[column]) entry by entry.

Inputs: the workloads' seeded operands; the prior C is seeded uniform[-1, 1)
(N(0,1) for fp32) rounded to C's type; the bias is seeded uniform[-1, 1) fp32.
The padding of C between N and ldc holds NaN and must come back untouched.
"""
import os

import numpy as np
import pytest
import torch

import gemm_inputs as gi
import oracle
from gpu_helpers import OUT_DTYPE, TOL, TORCH_DT, c_bits, reference, say, to_device

pytestmark = pytest.mark.gpu

FAST, GENERAL, NARROW, NARROW_GEN, NARROW64, NARROW64_GEN = 4, 5, 6, 7, 8, 9


@pytest.fixture(autouse=True)
def _clear_overrides():
    for v in ("LIBGEMM_H16_CONFIG", "LIBGEMM_F32_SMALL", "LIBGEMM_FP8_SMALL"):
        os.environ.pop(v, None)
    yield
    for v in ("LIBGEMM_H16_CONFIG", "LIBGEMM_F32_SMALL", "LIBGEMM_FP8_SMALL"):
        os.environ.pop(v, None)


def prior_bits(dtype: str, M: int, N: int, seed: int) -> np.ndarray:
    out = OUT_DTYPE[dtype]
    if out == "f32":
        return gi.normal_f32(M, N, seed)
    return gi.uniform_h16(M, N, seed, out)


def run_epilogue(dtype, ops, M, N, K, alpha, beta, bias, act, prior, lda=None, ldb=None,
                 ldc=None, offset=0):
    """Run gemm_<dtype>_epilogue with C preloaded with `prior` (bits) inside a
    NaN-padded buffer of leading dimension ldc; returns (C bits, padding bits)."""
    import dense_gemm_13_amd as dg
    A = to_device(ops["A"][:M, :K], dtype, lda, offset)
    B = to_device(ops["B"][:K, :N], dtype, ldb, offset)
    out = OUT_DTYPE[dtype]
    ldc = N if ldc is None else ldc
    buf = torch.full((M, ldc), float("nan"), dtype=TORCH_DT[out], device="cuda")
    C = buf[:, :N]
    if prior is not None:
        C.copy_(to_device(prior, out))
    b = None if bias is None else torch.from_numpy(bias).cuda()
    if dtype == "fp8":
        sa = torch.from_numpy(ops["scale_a"]).cuda()
        sb = torch.from_numpy(ops["scale_b"]).cuda()
        dg.gemm_fp8_blockscaled_epilogue(A, B, sa, sb, C, alpha=alpha, beta=beta, bias=b,
                                         activation=act)
    else:
        getattr(dg, f"gemm_{dtype}_epilogue")(A, B, C, alpha=alpha, beta=beta, bias=b,
                                              activation=act)
    torch.cuda.synchronize()
    pad = c_bits(buf[:, N:], out) if ldc > N else None
    return c_bits(C, out), pad


def check(dtype, ops, M, N, K, alpha, beta, use_bias, act, seed, what, prior_nan=False, **kw):
    bias = gi.uniform_f32(1, N, 7000 + seed)[0] if use_bias else None
    prior = prior_bits(dtype, M, N, 6000 + seed)
    if prior_nan:               # beta = 0 must not read C at all
        prior = np.full_like(prior, np.nan) if prior.dtype == np.float32 else \
            np.full_like(prior, 0x7FC0 if OUT_DTYPE[dtype] == "bf16" else 0x7E00)
    say(f"[epilogue] {what}: {dtype} {M}x{N}x{K} alpha={alpha} beta={beta} "
        f"bias={use_bias} act={act} {kw}")
    got, pad = run_epilogue(dtype, ops, M, N, K, alpha, beta, bias, act, prior, **kw)
    prod = reference(dtype, ops, M, N, K) if K > 0 else np.zeros((M, N))
    ref = oracle.epilogue(OUT_DTYPE[dtype], prod, alpha, beta, prior if beta != 0 else None,
                          bias, act)
    gotv = oracle.decode(got, OUT_DTYPE[dtype])
    rtol, atol = TOL[dtype]
    ok, nfail, worst, idx = oracle.within_tolerance(gotv, ref, rtol, atol)
    assert ok, (f"{what} {dtype}: {nfail} of {ref.size} entries out of tolerance, worst "
                f"err/tol {worst:.3g} at {idx} (gpu {gotv[idx]!r}, ref {ref[idx]!r})")
    if pad is not None:
        padv = oracle.decode(pad, OUT_DTYPE[dtype])
        assert np.isnan(padv).all(), f"{what}: C written between N and ldc"


H16_CASES = [
    # (config, (M, N, K), leading dimensions or None)
    (0, (300, 520, 203), (206, 521, 525)),
    (1, (300, 520, 200), None),
    (2, (130, 70, 96), (99, 73, 75)),
    (3, (45, 100, 64), None),
    (FAST, (512, 768, 384), None),
    (GENERAL, (300, 264, 200), None),
    (GENERAL, (257, 9, 96), (101, 11, 13)),
    (NARROW, (256, 128, 512), None),
    (NARROW_GEN, (40, 100, 1000), (1001, 101, 103)),
    (NARROW64, (128, 128, 512), None),
    (NARROW64_GEN, (100, 150, 700), (701, 151, 153)),
    (10, (3, 200, 300), (301, 203, 205)),   # the vector-ALU kernel for at most 4 rows
    (11, (256, 384, 256), None),             # 128 x 128 tiles of the large-tile kernel
    (12, (300, 264, 200), (203, 267, 269)),  # the same, guarded
    (13, (256, 512, 256), None),             # 128 x 256 tiles of the large-tile kernel
    (14, (300, 520, 200), (203, 523, 525)),  # the same, guarded
    (15, (3, 200, 300), (301, 203, 205)),    # the few-row kernel (B through LDS rings)
    (15, (1, 4095, 4100), (4100, 4095, 4095)),   # the same on the ragged workload's tail row
]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("case", range(len(H16_CASES)))
def test_h16_paths(dtype, case):
    config, (M, N, K), lds = H16_CASES[case]
    os.environ["LIBGEMM_H16_CONFIG"] = str(config)
    kw = {} if lds is None else dict(lda=lds[0], ldb=lds[1], ldc=lds[2], offset=1)
    ops = gi.operands(dtype, M, N, K, 50 + case)
    act = "relu" if case % 2 == 0 else "none"
    check(dtype, ops, M, N, K, 0.75, -0.5, True, act, case, f"config {config}", **kw)


F32_PATHS = {   # override, shape, leading dimensions (None: packed), seed
    "large": ("3", (256, 384, 256), None, 60),
    "small": ("1", (200, 136, 77), (80, 139, 141), 61),
    "guarded": ("2", (300, 270, 200), (203, 275, 277), 64),
    "ksplit32": ("4", (96, 192, 320), None, 65),
    "ksplit32_guarded": ("5", (100, 150, 333), (337, 151, 155), 66),
    "ksplit64": ("6", (128, 128, 256), None, 67),
    "ksplit64_guarded": ("7", (130, 70, 200), (203, 75, 77), 68),
    "rows": ("8", (4, 150, 333), (337, 151, 155), 69),
}


@pytest.mark.parametrize("path", list(F32_PATHS))
def test_f32_paths(path):
    """The whole-tile large-tile kernel ('3'), the register-staged kernels ('1'),
    the guarded large-tile kernel ('2'), the K-split kernel with 32-row ('4',
    '5') and 64-row tiles ('6', '7'), whole-tile and guarded, and the vector-ALU
    kernel for at most 4 rows ('8') (ragged shapes, unaligned leading
    dimensions)."""
    force, (M, N, K), lds, seed = F32_PATHS[path]
    os.environ["LIBGEMM_F32_SMALL"] = force
    kw = {} if lds is None else dict(lda=lds[0], ldb=lds[1], ldc=lds[2], offset=1)
    ops = gi.operands("f32", M, N, K, 60)
    check("f32", ops, M, N, K, 1.5, 0.25, True, "relu", seed, "f32 " + path, **kw)


FP8_PATHS = {   # override, shape, leading dimensions, seed
    "large": ("7", (512, 512, 512), {}, 61),
    "small": ("1", (200, 136, 320), dict(ldc=139), 62),
    "guarded": ("2", (300, 270, 200), dict(lda=203, ldb=275, ldc=277, offset=1), 63),
    "ksplit32": ("3", (96, 192, 320), {}, 64),
    "ksplit64_guarded": ("6", (130, 70, 200), dict(lda=203, ldb=75, ldc=77, offset=1), 65),
    "tiles128": ("8", (256, 384, 512), {}, 66),
    "tiles128_guarded": ("9", (300, 270, 200), dict(lda=203, ldb=275, ldc=277, offset=1), 67),
}


@pytest.mark.parametrize("path", list(FP8_PATHS))
def test_fp8_paths(path):
    """The whole-tile large-tile kernel ('7'), the register-staged kernels ('1'),
    the guarded large-tile kernel ('2') and the K-split kernel ('3': 32-row
    whole tiles, '6': 64-row guarded) on ragged shapes with unaligned leading
    dimensions."""
    force, (M, N, K), kw, seed = FP8_PATHS[path]
    os.environ["LIBGEMM_FP8_SMALL"] = force
    ops = gi.operands("fp8", M, N, K, 61)
    check("fp8", ops, M, N, K, 0.5, 1.0, True, "relu", seed, "fp8 " + path, **kw)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32", "fp8"])
def test_beta_zero_never_reads_c(dtype):
    M, N, K = 256, 256, 256
    ops = gi.operands(dtype, M, N, K, 62)
    check(dtype, ops, M, N, K, 2.0, 0.0, True, "none", 62, "beta 0, NaN prior", prior_nan=True)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32", "fp8"])
def test_relu_without_bias(dtype):
    M, N, K = 128, 192, 160
    ops = gi.operands(dtype, M, N, K, 63)
    check(dtype, ops, M, N, K, -1.0, 0.0, False, "relu", 63, "relu, no bias")


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32", "fp8"])
def test_empty_sum(dtype):
    """K = 0: C becomes act(beta * C + bias)."""
    M, N = 70, 130
    ops = gi.operands(dtype, M, N, 1, 64)
    ops["A"], ops["B"] = ops["A"][:, :0], ops["B"][:0, :]
    if dtype == "fp8":
        ops["scale_a"] = np.ones((2, 0), np.float32)
        ops["scale_b"] = np.ones((0, 3), np.float32)
    check(dtype, ops, M, N, 0, 3.0, -2.0, True, "relu", 64, "K = 0", ldc=N + 2)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_headline_size(dtype):
    """The 4096^3 workload with a full epilogue, in the benchmark's launch
    configuration (large-tile kernel)."""
    M = N = K = 4096
    ops = gi.operands(dtype, M, N, K, 2)
    check(dtype, ops, M, N, K, 0.5, -1.0, True, "relu", 65, "4096^3")


def test_tall_skinny_size():
    """8192 x 64 x 4096 (narrow kernel) with an epilogue."""
    M, N, K = 8192, 64, 4096
    ops = gi.operands("bf16", M, N, K, 3)
    check("bf16", ops, M, N, K, 1.0, 1.0, True, "relu", 66, "8192x64x4096")
