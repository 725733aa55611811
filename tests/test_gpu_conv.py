"""GPU parity of the convolution entry points: the im2col pack kernel bit for
bit against the oracle's im2col matrix, and the whole convolution (im2col +
GEMM, with the fused bias + relu) against the oracle's direct convolution.

Inputs: NHWC activations uniform[-1, 1) (fp16/bf16) or N(0, 1) (fp32) from the
seeded generators; HWIO weights the same; bias uniform[-1, 1) fp32.  The
geometries are those of small CNN layers: 3x3 padded, strided, dilated, a 7x7
stem on 3 channels (a K of 147, not a tile multiple), 1x1 direct and strided.
"""
import numpy as np
import pytest
import torch

import gemm_inputs as gi
import oracle
from gpu_helpers import TOL, TORCH_DT, say

pytestmark = pytest.mark.gpu

CASES = [
    # n, h, w, c_in, c_out, kh, kw, stride, pad, dil
    dict(n=2, h=14, w=14, c_in=64, c_out=64, kh=3, kw=3, stride=1, pad=1, dil=1),
    dict(n=2, h=15, w=13, c_in=32, c_out=48, kh=3, kw=3, stride=2, pad=1, dil=1),
    dict(n=1, h=12, w=12, c_in=16, c_out=40, kh=3, kw=3, stride=1, pad=2, dil=2),
    dict(n=2, h=23, w=23, c_in=3, c_out=64, kh=7, kw=7, stride=2, pad=3, dil=1),
    dict(n=3, h=9, w=10, c_in=24, c_out=72, kh=1, kw=1, stride=1, pad=0, dil=1),
    dict(n=2, h=9, w=10, c_in=40, c_out=24, kh=1, kw=1, stride=2, pad=0, dil=1),
    dict(n=1, h=6, w=5, c_in=5, c_out=7, kh=2, kw=3, stride=1, pad=1, dil=1),
]


def geom(c):
    return oracle.conv_geom(n=c["n"], h=c["h"], w=c["w"], c_in=c["c_in"], c_out=c["c_out"],
                            kh=c["kh"], kw=c["kw"], stride_h=c["stride"], stride_w=c["stride"],
                            pad_h=c["pad"], pad_w=c["pad"], dil_h=c["dil"], dil_w=c["dil"])


def operand(dtype, rows, cols, seed):
    if dtype == "f32":
        return gi.normal_f32(rows, cols, seed)
    return gi.uniform_h16(rows, cols, seed, dtype)


def to_dev(bits, dtype, shape):
    if dtype == "f32":
        t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.float32))
    else:
        t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(TORCH_DT[dtype])
    return t.reshape(shape).cuda()


def host_bits(t, dtype):
    t = t.detach().cpu().contiguous()
    return t.numpy() if dtype == "f32" else t.view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_im2col_bit_exact(dtype, case):
    import dense_gemm_13_amd as dg
    c = CASES[case]
    say(f"[im2col] {dtype} {c}")
    X = operand(dtype, c["n"] * c["h"] * c["w"], c["c_in"], 800 + case)
    col = dg.gemm_im2col_nhwc(to_dev(X, dtype, (c["n"], c["h"], c["w"], c["c_in"])),
                              (c["kh"], c["kw"]), c["stride"], c["pad"], c["dil"])
    torch.cuda.synchronize()
    want = oracle.im2col_nhwc(X, geom(c))
    got = host_bits(col, dtype)
    assert got.shape == want.shape
    assert np.array_equal(got.view(np.uint32 if dtype == "f32" else np.uint16),
                          want.view(np.uint32 if dtype == "f32" else np.uint16))


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_conv2d_parity(dtype, case):
    import dense_gemm_13_amd as dg
    c = CASES[case]
    g = geom(c)
    ho, wo = oracle.conv2d_output_size(g)
    X = operand(dtype, c["n"] * c["h"] * c["w"], c["c_in"], 810 + case)
    W = operand(dtype, c["kh"] * c["kw"] * c["c_in"], c["c_out"], 820 + case)
    bias = gi.uniform_f32(1, c["c_out"], 830 + case)[0] if case % 2 == 0 else None
    act = "relu" if case % 3 != 1 else "none"
    say(f"[conv2d] {dtype} {c} bias={bias is not None} act={act}")
    Y = dg.gemm_conv2d_nhwc(to_dev(X, dtype, (c["n"], c["h"], c["w"], c["c_in"])),
                            to_dev(W, dtype, (c["kh"], c["kw"], c["c_in"], c["c_out"])),
                            c["stride"], c["pad"], c["dil"],
                            None if bias is None else torch.from_numpy(bias).cuda(), act)
    torch.cuda.synchronize()
    assert tuple(Y.shape) == (c["n"], ho, wo, c["c_out"])
    prod = oracle.conv2d_nhwc(dtype, X, W, g).reshape(-1, c["c_out"])
    ref = oracle.epilogue(dtype, prod, bias=bias, act=act)
    got = oracle.decode(host_bits(Y, dtype).reshape(-1, c["c_out"]), dtype)
    ok, nfail, worst, idx = oracle.within_tolerance(got, ref, *TOL[dtype])
    assert ok, f"{nfail} entries out of tolerance, worst err/tol {worst:.3g} at {idx}"


def test_resnet_layer_sampled_images():
    """A ResNet-style 3x3 layer at its real size (32 x 56 x 56 x 64 -> 64, bf16,
    bias + relu): images 0 and 31 checked in full against the oracle (the
    convolution treats every image independently)."""
    import dense_gemm_13_amd as dg
    n, h, w, ci, co = 32, 56, 56, 64, 64
    X = operand("bf16", n * h * w, ci, 840)
    W = operand("bf16", 9 * ci, co, 841)
    bias = gi.uniform_f32(1, co, 842)[0]
    Y = dg.gemm_conv2d_nhwc(to_dev(X, "bf16", (n, h, w, ci)), to_dev(W, "bf16", (3, 3, ci, co)),
                            1, 1, 1, torch.from_numpy(bias).cuda(), "relu")
    torch.cuda.synchronize()
    got_all = host_bits(Y, "bf16")
    Xr = X.reshape(n, h * w, ci)
    for img in (0, n - 1):
        g = oracle.conv_geom(n=1, h=h, w=w, c_in=ci, c_out=co, kh=3, kw=3, pad_h=1, pad_w=1)
        prod = oracle.conv2d_nhwc("bf16", Xr[img], W, g).reshape(-1, co)
        ref = oracle.epilogue("bf16", prod, bias=bias, act="relu")
        got = oracle.decode(got_all[img].reshape(-1, co), "bf16")
        ok, nfail, worst, idx = oracle.within_tolerance(got, ref, *TOL["bf16"])
        assert ok, f"image {img}: {nfail} out of tolerance, worst {worst:.3g} at {idx}"


def test_empty_channels_give_bias():
    """c_in = 0: every sum is empty, so Y = relu(bias)."""
    import dense_gemm_13_amd as dg
    X = torch.empty((2, 4, 4, 0), dtype=torch.bfloat16, device="cuda")
    W = torch.empty((3, 3, 0, 5), dtype=torch.bfloat16, device="cuda")
    bias = gi.uniform_f32(1, 5, 850)[0]
    Y = dg.gemm_conv2d_nhwc(X, W, 1, 1, 1, torch.from_numpy(bias).cuda(), "relu")
    torch.cuda.synchronize()
    got = oracle.decode(host_bits(Y, "bf16").reshape(-1, 5), "bf16")
    ref = oracle.epilogue("bf16", np.zeros((32, 5)), bias=bias, act="relu")
    ok, nfail, worst, idx = oracle.within_tolerance(got, ref, *TOL["bf16"])
    assert ok
