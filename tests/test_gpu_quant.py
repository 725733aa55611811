"""GPU parity for the block-scaled FP8 quantiser (gemm_quantize_fp8): codes and
scales must equal the CPU oracle's bit for bit (the quantiser's output is a set
of integers decided by fp32 arithmetic that both sides do in the same IEEE fp32
operations).

* the fp8 GEMM workload's operand at full size (8192 x 8192 fp32 N(0,1) ->
  E4M3 with 64 x 64 blocks), in the launch configuration the benchmark times;
* every input type x block x format on ragged shapes, aligned and unaligned
  leading dimensions and offset pointers;
* special values: all-zero blocks, negative zeros, exact rounding midpoints,
  results in the FP8 subnormal range and results that round to zero;
* the padding of Q beyond its columns and memory beyond the scale grid stay
  untouched;
* end to end: quantise A and B on the GPU, multiply with gemm_fp8_blockscaled,
  compare with the oracle's product of the oracle's quantisation.
"""
import numpy as np
import pytest
import torch

import gemm_inputs as gi
import oracle
from gpu_helpers import compare, say

pytestmark = pytest.mark.gpu

FMAX = {"e4m3": 448.0, "e5m2": 57344.0}


def _device_input(x: np.ndarray, in_type: str, ld=None, offset=0):
    """fp32 values (or bf16 bits) -> device tensor view with leading dim ld."""
    rows, cols = x.shape
    ld = cols if ld is None else ld
    if in_type == "bf16":
        host = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    else:
        host = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    buf = torch.full((offset + rows * ld + 16,), float("nan"), dtype=host.dtype, device="cuda")
    view = buf[offset:offset + rows * ld].view(rows, ld)[:, :cols]
    view.copy_(host.cuda())
    return view


def _run(x, in_type, block, fmt, ldx=None, ldq=None, offx=0, offq=0):
    """GPU quantiser with guard bytes around Q and after the scale grid."""
    import dense_gemm_13_amd as dg
    rows, cols = x.shape
    X = _device_input(x, in_type, ldx, offx)
    ldq = cols if ldq is None else ldq
    qbuf = torch.full((offq + rows * ldq + 64,), 0xA5, dtype=torch.uint8, device="cuda")
    Q = qbuf[offq:offq + rows * ldq].view(rows, ldq)[:, :cols]
    br, bc = -(-rows // block), -(-cols // block)
    sbuf = torch.full((br * bc + 16,), -7.0, dtype=torch.float32, device="cuda")
    S = sbuf[:br * bc].view(br, bc)
    dg.gemm_quantize_fp8(X, block, fmt, Q, S)
    torch.cuda.synchronize()
    q = Q.cpu().numpy().copy()
    s = S.cpu().numpy().copy()
    qall = qbuf.cpu().numpy()
    # nothing outside the rows x cols window of Q, nor past the scale grid, changed
    mask = np.ones(qall.size, bool)
    for r in range(rows):
        mask[offq + r * ldq: offq + r * ldq + cols] = False
    assert np.all(qall[mask] == 0xA5), "quantiser wrote outside Q's window"
    assert np.all(sbuf[br * bc:].cpu().numpy() == -7.0), "quantiser wrote past the scale grid"
    return q, s


def _check(x, in_type, block, fmt, what, **kw):
    q, s = _run(x, in_type, block, fmt, **kw)
    q_ref, s_ref = oracle.quantize_fp8(x, in_type, block, fmt)
    bad_s = np.argwhere(s.view(np.uint32) != s_ref.view(np.uint32))
    assert bad_s.size == 0, (f"{what}: scale {tuple(bad_s[0])} gpu {s[tuple(bad_s[0])]!r} "
                             f"oracle {s_ref[tuple(bad_s[0])]!r}")
    bad = np.argwhere(q != q_ref)
    if bad.size:
        i, j = bad[0]
        xv = oracle.decode(x[i:i + 1, j:j + 1], "bf16")[0, 0] if in_type == "bf16" else x[i, j]
        raise AssertionError(f"{what}: {len(bad)} codes differ; first at ({i},{j}) x={xv!r} "
                             f"gpu {q[i, j]:#04x} oracle {q_ref[i, j]:#04x}")


def _values(rows, cols, seed, in_type, scale=1.0):
    x = (gi.normal_f32(rows, cols, seed) * np.float32(scale)).astype(np.float32)
    return gi.to_bf16_bits(x) if in_type == "bf16" else x


def test_workload_8192_e4m3_64():
    """The fp8 GEMM workload's A operand: 8192 x 8192 N(0,1) fp32, E4M3, 64 x 64 blocks."""
    say("[quant] 8192x8192 f32 e4m3/64")
    x = gi.normal_f32(8192, 8192, gi.SEED_A_BASE + 5)
    _check(x, "f32", 64, "e4m3", "8192^2")
    # the same codes and scales as the fp8 GEMM workload's operand recipe
    q, s = _run(x, "f32", 64, "e4m3")
    q2, s2 = gi.blockscale_e4m3(x)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)


SHAPES = [(1, 1), (64, 64), (100, 130), (257, 1000), (33, 7), (1000, 1), (3, 513)]


@pytest.mark.parametrize("in_type", ["f32", "bf16"])
@pytest.mark.parametrize("block", [32, 64])
@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_shapes(in_type, block, fmt):
    for n, (rows, cols) in enumerate(SHAPES):
        say(f"[quant] {in_type} block={block} {fmt} {rows}x{cols}")
        scale = 1000.0 if fmt == "e5m2" else 1.0
        x = _values(rows, cols, 300 + n, in_type, scale)
        _check(x, in_type, block, fmt, f"{rows}x{cols}")


@pytest.mark.parametrize("in_type", ["f32", "bf16"])
@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_unaligned_and_offset(in_type, fmt):
    """Leading dimensions that break 16-byte rows, and pointers off 16 bytes."""
    for ldx, ldq, offx, offq, shape in ((131, 133, 0, 0, (70, 130)), (130, 130, 1, 3, (70, 130)),
                                        (1024, 1027, 2, 1, (130, 1000)), (64, 64, 0, 0, (96, 64))):
        say(f"[quant] {in_type} {fmt} ldx={ldx} ldq={ldq} offx={offx} offq={offq} {shape}")
        x = _values(*shape, 17, in_type)
        for block in (32, 64):
            _check(x, in_type, block, fmt, f"ld {ldx}/{ldq} off {offx}/{offq}", ldx=ldx, ldq=ldq,
                   offx=offx, offq=offq)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_special_values(fmt):
    """Zero blocks, negative zeros, exact midpoints, FP8 subnormals, round-to-zero."""
    F = FMAX[fmt]
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle.decode(codes, fmt)
    pos = np.unique(vals[np.isfinite(vals) & (vals > 0)])
    mids = (pos[:-1] + pos[1:]) / 2
    x = np.zeros((128, 192), np.float32)
    # block (0,0): amax = F exactly so s = 1 and x / s = x: midpoints tie to even
    row = np.concatenate([[F], mids, -mids, pos[:8] / 2, -pos[:8] / 2, pos[:4] / 3])
    row = row[: 64 * 64].astype(np.float32)
    x[:64, :64].flat[: row.size] = row
    # block (0,1): all zeros, some negative -> scale 1, codes 0x00 / 0x80
    x[:64, 64:128] = 0.0
    x[10:20, 64:128] = -0.0
    # block (0,2): one large value, the rest tiny -> results in the subnormal range / zero
    x[:64, 128:192] = np.float32(1e-3) * gi.normal_f32(64, 64, 5)
    x[0, 128] = 1.0e3
    # block (1,0): values already at +-F and beyond the scale's rounding
    x[64:128, :64] = np.float32(F) * np.sign(gi.normal_f32(64, 64, 6))
    # block (1,1): a single non-zero element
    x[100, 100] = -3.0
    # block (1,2): fp32 subnormal inputs
    x[64:128, 128:192] = gi.normal_f32(64, 64, 7) * np.float32(1e-39)
    x[64, 128] = np.float32(1e-38)
    for block in (32, 64):
        say(f"[quant] special {fmt} block={block}")
        _check(x, "f32", block, fmt, f"special/{block}")


def test_end_to_end_quantise_then_multiply():
    """GPU quantiser -> GPU fp8 GEMM against the oracle's quantiser -> oracle GEMM."""
    import dense_gemm_13_amd as dg
    M, N, K = 320, 448, 576
    say(f"[quant] end to end {M}x{N}x{K}")
    a = gi.normal_f32(M, K, 41)
    b = gi.normal_f32(K, N, 42)
    qa, sa = dg.gemm_quantize_fp8(torch.from_numpy(a).cuda())
    qb, sb = dg.gemm_quantize_fp8(torch.from_numpy(b).cuda())
    C = dg.gemm_fp8_blockscaled(qa, qb, sa, sb)
    torch.cuda.synchronize()
    bits = C.cpu().view(torch.int16).numpy().view(np.uint16)
    oqa, osa = oracle.quantize_fp8(a, "f32", 64, "e4m3")
    oqb, osb = oracle.quantize_fp8(b, "f32", 64, "e4m3")
    assert np.array_equal(qa.cpu().numpy(), oqa) and np.array_equal(qb.cpu().numpy(), oqb)
    ref = oracle.gemm("fp8", oqa, oqb, M, N, K, osa, osb)
    ok, msg, _ = compare("fp8", bits, ref, "quantise+gemm")
    assert ok, msg


def test_bf16_matches_fp32_of_same_values():
    """bf16 input is widened exactly: same codes as fp32 input of the same values."""
    import dense_gemm_13_amd as dg
    xb = gi.uniform_h16(200, 300, 9, "bf16")
    xf = oracle.decode(xb, "bf16").astype(np.float32)
    tb = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).cuda()
    qb, sb = dg.gemm_quantize_fp8(tb, 32, "e5m2")
    qf, sf = dg.gemm_quantize_fp8(torch.from_numpy(xf).cuda(), 32, "e5m2")
    torch.cuda.synchronize()
    assert torch.equal(qb, qf) and torch.equal(sb, sf)


def test_empty_is_a_no_op():
    import dense_gemm_13_amd as dg
    x = torch.zeros((0, 5), dtype=torch.float32, device="cuda")
    q, s = dg.gemm_quantize_fp8(x)
    assert q.shape == (0, 5) and s.shape == (0, 1)
