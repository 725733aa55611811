"""The Python binding refuses, before any library call, tensors the kernels
would dereference as wild device addresses: host tensors, tensors whose rows
overlap (a broadcast row has stride 0), and a stream of another device.  `lib`
is replaced by a recorder, so these run on the CPU and prove that no call
reaches the C ABI."""
import pytest
import torch

import dense_gemm_13_amd as dg


class Recorder:
    def __init__(self):
        self.calls = []

    def __getattr__(self, name):
        def fn(*args):
            self.calls.append(name)
            return 0
        return fn


@pytest.fixture
def rec(monkeypatch):
    r = Recorder()
    monkeypatch.setattr(dg, "lib", r)
    return r


def h16(M, N, K, dt=torch.bfloat16):
    return torch.zeros(M, K, dtype=dt), torch.zeros(K, N, dtype=dt)


@pytest.mark.parametrize("name,dt", [("gemm_bf16", torch.bfloat16), ("gemm_f16", torch.float16),
                                     ("gemm_f32", torch.float32)])
def test_host_tensors_rejected(rec, name, dt):
    A, B = h16(8, 8, 8, dt)
    with pytest.raises(ValueError, match="GPU tensor"):
        getattr(dg, name)(A, B)
    assert rec.calls == []


def test_host_tensors_rejected_epilogue(rec):
    A, B = h16(8, 8, 8)
    with pytest.raises(ValueError, match="GPU tensor"):
        dg.gemm_bf16_epilogue(A, B, bias=torch.zeros(8))
    assert rec.calls == []


def test_host_scales_rejected(rec):
    A = torch.zeros(64, 64, dtype=torch.uint8)
    B = torch.zeros(64, 64, dtype=torch.uint8)
    sa, sb = torch.ones(1, 1), torch.ones(1, 1)
    with pytest.raises(ValueError, match="GPU tensor"):
        dg.gemm_fp8_blockscaled(A, B, sa, sb)
    assert rec.calls == []


@pytest.mark.parametrize("which", ["A", "B", "C"])
def test_overlapping_rows_rejected(rec, which):
    """A row-broadcast view (stride(0) == 0) or any row stride below the row
    length would make the kernel address rows past the allocation."""
    A, B = h16(16, 16, 16)
    C = torch.zeros(16, 16, dtype=torch.bfloat16)
    row = torch.zeros(1, 16, dtype=torch.bfloat16)
    if which == "A":
        A = row.expand(16, 16)
    elif which == "B":
        B = row.expand(16, 16)
    else:
        C = row.expand(16, 16)
    with pytest.raises(ValueError, match="rows overlap"):
        dg.gemm_bf16(A, B, C)
    # a stride just below the row length (rows overlap by one element)
    base = torch.zeros(16 * 15 + 1, dtype=torch.bfloat16)
    A2 = base.as_strided((16, 16), (15, 1))
    with pytest.raises(ValueError, match="rows overlap"):
        dg.gemm_bf16(A2, h16(16, 16, 16)[1])
    assert rec.calls == []


def test_padded_rows_accepted_as_leading_dimension():
    """A padded row stride is a leading dimension, not an error."""
    base = torch.zeros(16, 24, dtype=torch.bfloat16)
    assert dg._ld(base[:, :16]) == 24
    assert dg._ld(torch.zeros(1, 16, dtype=torch.bfloat16).expand(1, 16)) == 16


def test_quantiser_and_conv_host_tensors_rejected(rec):
    with pytest.raises(ValueError, match="GPU tensor"):
        dg.gemm_quantize_fp8(torch.zeros(64, 64))
    X = torch.zeros(1, 8, 8, 4, dtype=torch.bfloat16)
    Wt = torch.zeros(3, 3, 4, 4, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        dg.gemm_conv2d_nhwc(X, Wt, padding=1)
    with pytest.raises(ValueError, match="GPU tensor"):
        dg.gemm_im2col_nhwc(X, 3, padding=1)
    # only the workspace-size query (pure host arithmetic) may have run
    assert set(rec.calls) <= {"gemm_conv2d_workspace_bytes"}


def test_bias_on_host_rejected(rec):
    A, B = h16(8, 8, 8)
    with pytest.raises(ValueError):
        dg.gemm_bf16_epilogue(A, B, bias=torch.zeros(8, dtype=torch.float64))
    assert rec.calls == []
