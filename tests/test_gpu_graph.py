"""Every kind of library call captured in a HIP graph (torch.cuda.CUDAGraph)
and replayed: each replay, with other work on the stream between replays, must
give the eager call's output bit for bit.  The kernels are deterministic, the
library allocates nothing during a call and enqueues no memset, so a captured
call is an ordinary kernel sequence."""
import os

import pytest
import torch

import dense_gemm_13_amd as dg
from gpu_helpers import say

pytestmark = pytest.mark.gpu

DT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


@pytest.fixture(autouse=True)
def _no_override():
    for v in ("LIBGEMM_H16_CONFIG", "LIBGEMM_FP8_SMALL", "LIBGEMM_F32_SMALL"):
        os.environ.pop(v, None)
    yield


def _rand(shape, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    return (torch.rand(shape, generator=g) * 2 - 1).to(dtype).cuda()


def _replays_match(call, outs, reset=None, replays=3):
    """Eager call, then the same call captured; every replay must equal the
    eager outputs bit for bit.  `reset` restores inputs the call also reads
    (the prior C of beta != 0) before each run."""
    if reset:
        reset()
    call()
    torch.cuda.synchronize()
    refs = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    if reset:
        reset()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for r in range(replays):
        for o in outs:                                   # other work between replays
            o.view(torch.uint8).fill_(0xA5)
        if reset:
            reset()
        g.replay()
        torch.cuda.synchronize()
        for o, ref in zip(outs, refs):
            assert torch.equal(o.view(torch.uint8), ref.view(torch.uint8)), f"replay {r} differs"


@pytest.mark.parametrize("dtype,M,N,K", [
    ("bf16", 4096, 4096, 4096),   # whole 256 x 256 tiles
    ("bf16", 4097, 4095, 4100),   # guarded tiles, then the row below them (two launches)
    ("f16", 1000, 1000, 1000),    # K split, 64-row tiles
    ("bf16", 8192, 64, 4096),     # tall and narrow
    ("bf16", 2, 1000, 2048),      # few rows
    ("f16", 2048, 2048, 2048),    # 128 x 128 tiles
    ("bf16", 64, 64, 0),          # K = 0: the empty sum
    ("f32", 2048, 2048, 512),     # fp32 large tiles
    ("f32", 300, 1500, 4096),     # fp32 K split
    ("f32", 3, 4096, 1000),       # fp32 rows
])
def test_gemm_in_graph(dtype, M, N, K):
    say(f"[graph] {dtype} {M}x{N}x{K}")
    A, B = _rand((M, K), DT[dtype], 1), _rand((K, N), DT[dtype], 2)
    C = torch.empty((M, N), dtype=DT[dtype], device="cuda")
    fn = getattr(dg, f"gemm_{dtype}")
    _replays_match(lambda: fn(A, B, C), [C])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_epilogue_with_prior_c_in_graph(dtype):
    M, N, K = 1000, 768, 512
    say(f"[graph] {dtype} epilogue {M}x{N}x{K} beta=0.5 bias relu")
    A, B = _rand((M, K), DT[dtype], 3), _rand((K, N), DT[dtype], 4)
    prior = _rand((M, N), DT[dtype], 5)
    bias = _rand((N,), torch.float32, 6)
    C = torch.empty_like(prior)
    fn = getattr(dg, f"gemm_{dtype}_epilogue")
    _replays_match(lambda: fn(A, B, C, alpha=0.75, beta=0.5, bias=bias, activation="relu"), [C],
                   reset=lambda: C.copy_(prior))


def test_quantize_and_fp8_gemm_in_graph():
    M, N, K = 1000, 1024, 1536
    say(f"[graph] fp8 quantise + GEMM {M}x{N}x{K}")
    Xa, Xb = _rand((M, K), torch.float32, 7), _rand((K, N), torch.float32, 8)
    Qa = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    Qb = torch.empty((K, N), dtype=torch.uint8, device="cuda")
    Sa = torch.empty((-(-M // 64), -(-K // 64)), dtype=torch.float32, device="cuda")
    Sb = torch.empty((-(-K // 64), -(-N // 64)), dtype=torch.float32, device="cuda")
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def call():
        dg.gemm_quantize_fp8(Xa, Q=Qa, scales=Sa)
        dg.gemm_quantize_fp8(Xb, Q=Qb, scales=Sb)
        dg.gemm_fp8_blockscaled(Qa, Qb, Sa, Sb, C)
    _replays_match(call, [Qa, Qb, Sa, Sb, C])


@pytest.mark.parametrize("noalloc", [False, True])
def test_conv_in_graph(noalloc):
    n, hw, ci, co = 4, 28, 64, 96
    say(f"[graph] conv 3x3 {n}x{hw}x{hw}x{ci} -> {co} noalloc={noalloc}")
    X = _rand((n, hw, hw, ci), torch.bfloat16, 9)
    Wt = _rand((3, 3, ci, co), torch.bfloat16, 10)
    bias = _rand((co,), torch.float32, 11)
    Y = torch.empty((n, hw, hw, co), dtype=torch.bfloat16, device="cuda")
    if noalloc:
        call = lambda: dg.gemm_conv2d_nhwc_noalloc(X, Wt, Y, padding=1, bias=bias,
                                                   activation="relu")
        _replays_match(call, [Y])
    else:
        shape = dg.conv2d_shape(X, Wt, padding=1)
        import ctypes
        need = dg.lib.gemm_conv2d_workspace_bytes(dg.DTYPES["bf16"], ctypes.byref(shape))
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        call = lambda: dg.gemm_conv2d_nhwc(X, Wt, padding=1, bias=bias, activation="relu", Y=Y,
                                           workspace=ws)
        _replays_match(call, [Y])


def test_calls_on_concurrent_streams():
    """GEMMs of different kernel families issued on two streams at once (the
    GEMM kernels keep no state between calls): each output equals the same
    call run alone, bit for bit."""
    say("[streams] six products on two streams")
    shapes = [("bf16", 4097, 4095, 4100), ("f16", 1000, 1000, 1000), ("bf16", 8192, 64, 4096),
              ("f32", 300, 1500, 4096), ("bf16", 2, 1000, 2048), ("f16", 2048, 2048, 2048)]
    ops = []
    for i, (dt, M, N, K) in enumerate(shapes):
        A, B = _rand((M, K), DT[dt], 20 + i), _rand((K, N), DT[dt], 40 + i)
        ops.append((getattr(dg, f"gemm_{dt}"), A, B, torch.empty((M, N), dtype=DT[dt], device="cuda")))
    refs = []
    for fn, A, B, C in ops:
        fn(A, B, C)
        torch.cuda.synchronize()
        refs.append(C.clone())
        C.view(torch.uint8).fill_(0xA5)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(3):
        for i, (fn, A, B, C) in enumerate(ops):
            fn(A, B, C, stream=streams[i % 2])
        torch.cuda.synchronize()
        for i, (_, _, _, C) in enumerate(ops):
            assert torch.equal(C.view(torch.uint8), refs[i].view(torch.uint8)), f"call {i}, round {rep}"
            C.view(torch.uint8).fill_(0xA5)
        torch.cuda.synchronize()
