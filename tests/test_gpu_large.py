"""GPU parity at sizes whose element offsets pass 2^31: a C with 2^32 entries on
the large-tile paths, and an A with more than 2^31 entries on the narrow,
small-tile and guarded paths.

Products this large cannot go through the CPU oracle in full, so each case is
an exact probe that holds at any size: B is a selection matrix (column j holds
a single 1, in row sel[j]), so C[i][j] = A[i][sel[j]] exactly: one product
by 1 plus zeros, no rounding for a value that is already representable in the
output type.  Every entry of C is compared with that gather of A, as values, so
that an exact zero may come out with either sign.  An offset computed in 32
bits would wrap by a multiple of 2^31 elements and land on other data:
the large A is tiled from 1021 seeded rows (a prime count, so a wrapped row
index falls on a different bank row) and its entries are random.

FP8 codes are turned into expected bf16 values through the oracle's E4M3
decoder (a 256-entry table; the values are exact in bf16)."""
import os

import numpy as np
import pytest
import torch

import gemm_inputs as gi
import oracle
from gpu_helpers import say

pytestmark = pytest.mark.gpu

ONE_BITS = {"bf16": 0x3F80, "f16": 0x3C00, "fp8": 0x38}   # 1.0 in each encoding
TORCH_IN = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32, "fp8": torch.uint8}
TORCH_OUT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32, "fp8": torch.bfloat16}


@pytest.fixture(autouse=True)
def _clear_config_override():
    for v in ("LIBGEMM_H16_CONFIG", "LIBGEMM_F32_SMALL", "LIBGEMM_FP8_SMALL"):
        os.environ.pop(v, None)
    yield
    for v in ("LIBGEMM_H16_CONFIG", "LIBGEMM_F32_SMALL", "LIBGEMM_FP8_SMALL"):
        os.environ.pop(v, None)
    torch.cuda.empty_cache()


def _device(bits: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype in ("bf16", "f16"):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(TORCH_IN[dtype])
    return torch.from_numpy(np.ascontiguousarray(bits)).cuda()


def _selection(dtype: str, K: int, N: int, seed: int):
    """K x N selection matrix on the device and its row indices sel (on the device)."""
    sel = np.random.default_rng(seed).integers(0, K, N)
    if dtype == "f32":
        B = np.zeros((K, N), np.float32)
        B[sel, np.arange(N)] = 1.0
    else:
        B = np.zeros((K, N), np.uint8 if dtype == "fp8" else np.uint16)
        B[sel, np.arange(N)] = ONE_BITS[dtype]
    return _device(B, dtype), torch.from_numpy(sel).cuda()


def _as_values(A: torch.Tensor, dtype: str) -> torch.Tensor:
    """Operand entries as float32 values (fp8 through the oracle's decoder)."""
    if dtype != "fp8":
        return A.float()
    table = oracle.decode(np.arange(256, dtype=np.uint8), "fp8").astype(np.float32)
    return torch.from_numpy(table).cuda()[A.long()]


def _run(dtype: str, A, B, C, M, K):
    import dense_gemm_13_amd as dg
    if dtype == "fp8":
        sa = torch.ones(-(-M // 64), -(-K // 64), device="cuda")
        sb = torch.ones(-(-K // 64), -(-B.shape[1] // 64), device="cuda")
        dg.gemm_fp8_blockscaled(A, B, sa, sb, C)
    else:
        getattr(dg, "gemm_" + dtype)(A, B, C)
    torch.cuda.synchronize()


def _check_rows(C, rows_of_A, sel, dtype, what, chunk=4096):
    """C[i][j] == value of A-row i at column sel[j], for all i, j; rows_of_A(r0, r1)
    gives the operand rows r0..r1-1."""
    M = C.shape[0]
    for r0 in range(0, M, chunk):
        r1 = min(M, r0 + chunk)
        want = _as_values(rows_of_A(r0, r1), dtype)[:, sel]
        got = C[r0:r1].float()
        if not torch.equal(got, want):
            bad = (got != want).nonzero()[0].tolist()
            i, j = r0 + bad[0], bad[1]
            raise AssertionError(f"{what}: C[{i}][{j}] = {got[bad[0], j].item()}, "
                                 f"want {want[bad[0], j].item()}")


@pytest.mark.parametrize("dtype,K", [("bf16", 128), ("f16", 128), ("fp8", 256), ("f32", 64)])
def test_output_with_2_32_entries_exact(dtype, K):
    M = N = 65536                                  # C: 2^32 entries, whole 256 x 256 tiles
    say(f"[large-C] {dtype} M=N={M} K={K}: generating")
    A = _device(gi.operands(dtype, M, 8, K, 500)["A"], dtype)
    B, sel = _selection(dtype, K, N, 501)
    C = torch.full((M, N), float("nan"), dtype=TORCH_OUT[dtype], device="cuda")
    say(f"[large-C] {dtype}: gpu")
    _run(dtype, A, B, C, M, K)
    say(f"[large-C] {dtype}: checking all {M * N} entries")
    _check_rows(C, lambda r0, r1: A[r0:r1], sel, dtype, f"large-C {dtype}")
    del A, B, C


BANK_ROWS = 1021


@pytest.mark.parametrize("dtype,config", [("bf16", None), ("bf16", 2), ("bf16", 5),
                                          ("fp8", None), ("fp8", 2), ("f32", None), ("f32", 2)])
def test_operand_past_2_31_entries_exact(dtype, config):
    """A holds more than 2^31 entries; N = 64.  Every dtype with the default
    dispatch takes its K-split kernel; bf16 configs 2 and 5 force the 64 x 64
    register-staged kernel and the guarded large-tile kernel, and fp8 / f32
    override 2 their guarded large-tile kernels."""
    if config is not None:
        var = {"f32": "LIBGEMM_F32_SMALL", "fp8": "LIBGEMM_FP8_SMALL"}.get(dtype, "LIBGEMM_H16_CONFIG")
        os.environ[var] = str(config)
    K, N = 2048, 64
    M = (1 << 31) // K + 64                        # M*K = 2^31 + 64K
    say(f"[large-A] {dtype} config={config} M={M} N={N} K={K}: generating")
    bank = _device(gi.operands(dtype, BANK_ROWS, 8, K, 502)["A"], dtype)
    rows = torch.arange(M, device="cuda") % BANK_ROWS
    A = bank[rows]                                 # M x K, row i = bank row i % 1021
    assert A.numel() > 2 ** 31
    B, sel = _selection(dtype, K, N, 503)
    C = torch.full((M, N), float("nan"), dtype=TORCH_OUT[dtype], device="cuda")
    say(f"[large-A] {dtype} config={config}: gpu")
    _run(dtype, A, B, C, M, K)
    say(f"[large-A] {dtype} config={config}: checking all {M * N} entries")
    del A
    _check_rows(C, lambda r0, r1: bank[rows[r0:r1]], sel, dtype,
                f"large-A {dtype} config={config}", chunk=65536)
    del bank, B, C


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rows_operand_B_past_2_31_entries_exact(dtype):
    """The vector-ALU kernel for at most 4 rows (forced) with a B of more than
    2^31 entries (K = 2^20 rows of 2112 columns): C[i][j] = A[i][sel[j]]."""
    M, K, N = 3, 1 << 20, 2112
    os.environ["LIBGEMM_F32_SMALL" if dtype == "f32" else "LIBGEMM_H16_CONFIG"] = (
        "8" if dtype == "f32" else "10")
    say(f"[large-B rows] {dtype} M={M} N={N} K={K}: generating")
    A = _device(gi.operands(dtype, M, 8, K, 504)["A"], dtype)
    sel = torch.from_numpy(np.random.default_rng(505).integers(0, K, N)).cuda()
    B = torch.zeros((K, N), dtype=TORCH_IN[dtype], device="cuda")
    B[sel, torch.arange(N, device="cuda")] = 1
    assert B.numel() > 2 ** 31
    C = torch.full((M, N), float("nan"), dtype=TORCH_OUT[dtype], device="cuda")
    say(f"[large-B rows] {dtype}: gpu")
    _run(dtype, A, B, C, M, K)
    _check_rows(C, lambda r0, r1: A[r0:r1], sel, dtype, f"large-B rows {dtype}")
    del A, B, C


@pytest.mark.parametrize("N", [540000, 540001])
def test_one_row_operand_B_past_2_31_entries_exact(N):
    """One row of A times a B of more than 2^31 entries (K = 4096 rows), through
    the automatic dispatch: with N = 540000 (16-byte-aligned rows) the narrow
    K-split kernel, its 64-bit block offsets and 8438 column tiles; with
    N = 540001 (rows 2-byte aligned) the few-row kernel, its 64-bit row offsets,
    16876 workgroups and the window of the last one moved left."""
    M, K = 1, 4096
    say(f"[large-B fewrows] bf16 M={M} N={N} K={K}: generating")
    A = _device(gi.operands("bf16", M, 8, K, 506)["A"], "bf16")
    sel = torch.from_numpy(np.random.default_rng(507).integers(0, K, N)).cuda()
    B = torch.zeros((K, N), dtype=torch.bfloat16, device="cuda")
    B[sel, torch.arange(N, device="cuda")] = 1
    assert B.numel() > 2 ** 31
    C = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    say("[large-B fewrows] bf16: gpu")
    _run("bf16", A, B, C, M, K)
    _check_rows(C, lambda r0, r1: A[r0:r1], sel, "bf16", "large-B fewrows bf16")
    del A, B, C
