"""The convolution entry point that allocates nothing, gemm_conv2d_nhwc_noalloc,
against the one that takes a caller workspace, gemm_conv2d_nhwc, called through
the C ABI on raw device pointers.

Both build the same im2col matrix with the same kernel and hand it to the same
GEMM dispatch (the scratch array and a torch allocation are both 256-byte
aligned), so the outputs must agree bit for bit; each is also checked against
the oracle's direct convolution within the GEMM tolerances.  Two calls in a row
(the second with a smaller matrix, so the array still holds the first call's
larger one) show that a call depends only on what it writes itself; the largest
matrix the array holds, one past it (refused, output untouched) and the direct
1 x 1 case (no scratch) cover the limits.
"""
import ctypes

import numpy as np
import pytest
import torch

import gemm_inputs as gi
import oracle
from gpu_helpers import TOL, TORCH_DT, say

pytestmark = pytest.mark.gpu

GEMM_ERR_SCRATCH = -10


def _bits(dtype, rows, cols, seed):
    if dtype == "f32":
        return gi.normal_f32(rows, cols, seed)
    return gi.uniform_h16(rows, cols, seed, dtype)


def _dev(bits, dtype, shape):
    if dtype == "f32":
        t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.float32))
    else:
        t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(TORCH_DT[dtype])
    return t.reshape(shape).cuda()


def _host(t, dtype):
    t = t.detach().cpu().contiguous()
    return t.numpy().view(np.uint32) if dtype == "f32" else t.view(torch.int16).numpy().view(np.uint16)


class Case:
    def __init__(self, dtype, n, h, w, ci, co, k, stride, pad, seed, act="relu", with_bias=True):
        import dense_gemm_13_amd as dg
        self.dtype, self.seed, self.act = dtype, seed, act
        self.shape = dg.Conv2dShape(n, h, w, ci, co, k, k, stride, stride, pad, pad, 1, 1)
        self.ho, self.wo = dg.conv2d_output_hw(self.shape)
        self.X = _bits(dtype, n * h * w, ci, seed)
        self.W = _bits(dtype, k * k * ci, co, seed + 1)
        self.bias = gi.uniform_f32(1, co, seed + 2)[0] if with_bias else None
        self.Xd = _dev(self.X, dtype, (n, h, w, ci))
        self.Wd = _dev(self.W, dtype, (k, k, ci, co))
        self.bd = None if self.bias is None else torch.from_numpy(self.bias).cuda()
        self.need = dg.lib.gemm_conv2d_workspace_bytes(dg.DTYPES[dtype], ctypes.byref(self.shape))
        self.out_shape = (n, self.ho, self.wo, co)

    def y(self):
        return torch.full(self.out_shape, float("nan"), dtype=TORCH_DT[self.dtype], device="cuda")

    def _args(self, Y):
        import dense_gemm_13_amd as dg
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        return (dg.DTYPES[self.dtype], self.Xd.data_ptr(), self.Wd.data_ptr(), Y.data_ptr(),
                ctypes.byref(self.shape), None if self.bd is None else self.bd.data_ptr(),
                dg.ACTIVATIONS[self.act], stream)

    def noalloc(self, Y):
        import dense_gemm_13_amd as dg
        return dg.lib.gemm_conv2d_nhwc_noalloc(*self._args(Y))

    def with_workspace(self, Y):
        import dense_gemm_13_amd as dg
        ws = torch.empty(max(self.need, 1), dtype=torch.uint8, device="cuda")
        dt, x, w, y, sp, b, act, st = self._args(Y)
        rc = dg.lib.gemm_conv2d_nhwc(dt, x, w, y, ws.data_ptr() if self.need else None,
                                     self.need, sp, b, act, st)
        torch.cuda.synchronize()
        return rc

    def reference(self):
        g = oracle.conv_geom(n=self.shape.n, h=self.shape.h, w=self.shape.w,
                             c_in=self.shape.c_in, c_out=self.shape.c_out, kh=self.shape.kh,
                             kw=self.shape.kw, stride_h=self.shape.stride_h,
                             stride_w=self.shape.stride_w, pad_h=self.shape.pad_h,
                             pad_w=self.shape.pad_w)
        prod = oracle.conv2d_nhwc(self.dtype, self.X, self.W, g).reshape(-1, self.shape.c_out)
        return oracle.epilogue(self.dtype, prod, bias=self.bias, act=self.act)

    def check(self, got_bits, what):
        out = "f32" if self.dtype == "f32" else self.dtype
        got = oracle.decode(got_bits.view(np.float32) if self.dtype == "f32" else got_bits, out)
        ok, nfail, worst, idx = oracle.within_tolerance(got.reshape(-1, self.shape.c_out),
                                                        self.reference(), *TOL[self.dtype])
        assert ok, f"{what}: {nfail} entries out of tolerance, worst err/tol {worst:.3g} at {idx}"


def _same_as_workspace_entry(case, what):
    say(f"[noalloc] {what}: {case.dtype} out {case.out_shape}, im2col {case.need} bytes")
    Yn = case.y()
    rc = case.noalloc(Yn)
    torch.cuda.synchronize()
    assert rc == 0, f"{what}: gemm_conv2d_nhwc_noalloc returned {rc}"
    Yw = case.y()
    assert case.with_workspace(Yw) == 0
    got_n, got_w = _host(Yn, case.dtype), _host(Yw, case.dtype)
    assert np.array_equal(got_n, got_w), \
        f"{what}: {(got_n != got_w).sum()} entries differ from gemm_conv2d_nhwc"
    case.check(got_n, what)
    return got_n


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_two_calls_in_a_row_second_smaller(dtype):
    big = Case(dtype, 4, 28, 28, 64, 64, 3, 1, 1, 900)
    small = Case(dtype, 2, 15, 13, 32, 48, 3, 2, 1, 910, act="none")
    assert 0 < small.need < big.need
    _same_as_workspace_entry(big, "first call")
    _same_as_workspace_entry(small, "second call (smaller matrix)")


def test_largest_matrix_the_scratch_holds():
    """A 1 x 1 convolution with stride 2 over 2 x 256 x 256 x 1024 bf16 builds a
    32768 x 1024 matrix: exactly GEMM_CONV2D_SCRATCH_BYTES."""
    import dense_gemm_13_amd as dg
    case = Case("bf16", 2, 256, 256, 1024, 64, 1, 2, 0, 920)
    assert case.need == dg.CONV2D_SCRATCH_BYTES
    _same_as_workspace_entry(case, "64 MiB matrix")


def test_one_past_the_limit_is_refused_and_writes_nothing():
    import dense_gemm_13_amd as dg
    case = Case("bf16", 2, 256, 256, 1032, 16, 1, 2, 0, 930)
    assert case.need > dg.CONV2D_SCRATCH_BYTES
    say(f"[noalloc] refused: im2col {case.need} bytes")
    Y = case.y()
    assert case.noalloc(Y) == GEMM_ERR_SCRATCH
    torch.cuda.synchronize()
    assert torch.isnan(Y.float()).all()


def test_direct_1x1_uses_no_scratch():
    case = Case("f16", 3, 9, 10, 24, 72, 1, 1, 0, 940, act="none", with_bias=False)
    assert case.need == 0
    _same_as_workspace_entry(case, "direct 1x1")


def test_binding_name_matches():
    """The Python binding of the entry point (argument marshalling only) gives
    the same bits as the raw C call."""
    import dense_gemm_13_amd as dg
    case = Case("bf16", 2, 14, 14, 64, 64, 3, 1, 1, 950)
    got_c = _same_as_workspace_entry(case, "C call")
    Y = case.y()
    dg.gemm_conv2d_nhwc_noalloc(case.Xd, case.Wd, Y, 1, 1, 1, case.bd, case.act)
    torch.cuda.synchronize()
    assert np.array_equal(_host(Y, "bf16"), got_c)
