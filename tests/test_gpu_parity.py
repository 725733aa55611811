"""GPU parity: libgemm (through its C ABI via the binding) against the CPU
oracle, entry by entry, on seeded inputs.

* exact probes: permutation matrices and all-ones inputs give results that are
  exactly representable, so they must match bit for bit (this pins the MFMA
  operand/accumulator layouts, LDS swizzles, tile remap and epilogue);
* the five workloads at full size, every entry, in the launch configuration
  the benchmark times;
* every half-precision tile configuration forced on ragged shapes, with
  aligned and unaligned leading dimensions and offset pointers;
* random small and medium shapes through the automatic dispatch, K = 0,
  degenerate sizes, and a guard band around C.
"""
import os

import numpy as np
import pytest
import torch

import gemm_inputs as gi
import oracle
from gpu_helpers import TOL, OUT_DTYPE, compare, reference, run_gemm, say, to_device

pytestmark = pytest.mark.gpu

H16_CONFIGS = (0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 11, 12, 13, 14)
FAST = 4          # whole 256x256 tiles, K % 128 == 0, aligned
GENERAL = 5       # the same kernel, guarded: ragged M/N/K, any leading dimensions
NARROW = 6        # whole 32x64 tiles, K % 64 == 0, K >= 256, aligned; waves split K
NARROW_GEN = 7    # the same kernel, guarded: any M, N >= 8, K >= 1, any leading dimensions
NARROW64 = 8      # whole 64x64 tiles, K % 64 == 0, K >= 256, aligned; waves split K, 2 stages
NARROW64_GEN = 9  # the same kernel, guarded
FAST128 = 11      # whole 128x128 tiles of the large-tile kernel, two workgroups per CU
GEN128 = 12       # the same kernel, guarded
FAST128x256 = 13  # whole 128x256 tiles of the large-tile kernel, one workgroup per CU
GEN128x256 = 14   # the same kernel, guarded
FEWROWS = 15      # at most 4 rows: B streamed through per-wave LDS rings, 32 columns per workgroup


@pytest.fixture(autouse=True)
def _clear_config_override():
    for v in ("LIBGEMM_H16_CONFIG", "LIBGEMM_FP8_SMALL", "LIBGEMM_F32_SMALL"):
        os.environ.pop(v, None)
    yield
    for v in ("LIBGEMM_H16_CONFIG", "LIBGEMM_FP8_SMALL", "LIBGEMM_F32_SMALL"):
        os.environ.pop(v, None)


def _encode(x, dtype):
    x = np.asarray(x, dtype=np.float32)
    return {"f16": gi.to_f16_bits, "bf16": gi.to_bf16_bits, "fp8": gi.to_e4m3_bits,
            "f32": lambda v: np.ascontiguousarray(v, dtype=np.float32)}[dtype](x)


def _unit_scales(r, c):
    return np.ones((-(-r // 64), -(-c // 64)), dtype=np.float32)


def _perm_case(dtype, M, K, seed):
    """A random (M x K), P a K x K permutation: A*P permutes the columns of A."""
    ops = gi.operands(dtype, M, K, K, 90 + seed)
    perm = np.random.default_rng(seed).permutation(K)
    P = np.zeros((K, K), np.float32)
    P[np.arange(K), perm] = 1.0
    ops["B"] = _encode(P, dtype)
    if dtype == "fp8":
        ops["scale_a"], ops["scale_b"] = _unit_scales(M, K), _unit_scales(K, K)
    return ops, perm


@pytest.mark.parametrize("dtype,config", [(d, c) for d in ("bf16", "f16") for c in H16_CONFIGS]
                         + [("f32", None), ("fp8", None)])
def test_permutation_probe_exact(dtype, config):
    if config is not None:
        os.environ["LIBGEMM_H16_CONFIG"] = str(config)
    M, K = (512, 512) if config in (FAST, FAST128, FAST128x256) else (320, 384)
    say(f"[probe] A*P {dtype} config={config} M={M} N=K={K}")
    ops, perm = _perm_case(dtype, M, K, 7)
    _, got = run_gemm(dtype, ops, M, K, K)
    vals = oracle.decode(ops["A"], dtype) if dtype != "fp8" else oracle.decode(ops["A"], "fp8")
    want = np.empty((M, K))
    want[:, perm] = vals
    gotv = oracle.decode(got, OUT_DTYPE[dtype])
    bad = np.argwhere(gotv != want)
    assert bad.size == 0, f"first mismatch at {bad[0]}: gpu {gotv[tuple(bad[0])]}, want {want[tuple(bad[0])]}"
    # P * B permutes the rows of B
    say(f"[probe] P*B {dtype} config={config}")
    opsb = gi.operands(dtype, K, M, K, 95)
    Pm = np.zeros((K, K), np.float32)
    Pm[np.arange(K), perm] = 1.0
    opsb["A"] = _encode(Pm, dtype)
    if dtype == "fp8":
        opsb["scale_a"], opsb["scale_b"] = _unit_scales(K, K), _unit_scales(K, M)
    _, got = run_gemm(dtype, opsb, K, M, K)
    want = oracle.decode(opsb["B"], dtype)[perm]
    gotv = oracle.decode(got, OUT_DTYPE[dtype])
    bad = np.argwhere(gotv != want)
    assert bad.size == 0, f"first mismatch at {bad[0]}"


@pytest.mark.parametrize("dtype,K,want", [("bf16", 4100, 4096.0), ("f16", 256, 256.0),
                                          ("f32", 4100, 4100.0), ("fp8", 4100, 4096.0)])
def test_all_ones_round_to_nearest_even(dtype, K, want):
    M, N = 300, 200
    say(f"[ones] {dtype} K={K}")
    ops = {"A": _encode(np.ones((M, K)), dtype), "B": _encode(np.ones((K, N)), dtype)}
    if dtype == "fp8":
        ops["scale_a"], ops["scale_b"] = _unit_scales(M, K), _unit_scales(K, N)
    _, got = run_gemm(dtype, ops, M, N, K)
    vals = oracle.decode(got, OUT_DTYPE[dtype])
    assert np.all(vals == want), f"values {np.unique(vals)[:5]}"


def _full_check(dtype, M, N, K, wid, what):
    say(f"[{what}] {dtype} M={M} N={N} K={K}: generating")
    ops = gi.operands(dtype, M, N, K, wid)
    say(f"[{what}] {dtype} M={M} N={N} K={K}: gpu")
    _, got = run_gemm(dtype, ops, M, N, K)
    say(f"[{what}] {dtype}: oracle")
    ref = reference(dtype, ops, M, N, K)
    ok, msg, worst = compare(dtype, got, ref, what)
    say(f"[{what}] {msg}")
    assert ok, msg


def test_workload_f16_256():
    _full_check("f16", 256, 256, 256, 1, "f16_256")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_workload_h16_4096(dtype):
    _full_check(dtype, 4096, 4096, 4096, 2, "h16_4096")


@pytest.mark.parametrize("shape", [(1000, 1000, 1000), (4097, 4095, 4100), (8192, 64, 4096)])
def test_workload_bf16_ragged(shape):
    _full_check("bf16", *shape, 3, "bf16_ragged")


def test_workload_f32_4096():
    _full_check("f32", 4096, 4096, 4096, 4, "f32_4096")


@pytest.mark.timeout(900)
def test_workload_fp8_8192_every_entry():
    """The fp8 workload (E4M3, 64x64 block scales, M = N = K = 8192, bf16 C) in
    the launch configuration the benchmark times, checked on all 67,108,864
    entries against the oracle.  A sampled pre-check (random entries, whole
    rows and columns, tile and scale-block edges) runs first so that a layout
    mistake fails fast with a pointed message; then the oracle forms the whole
    product in row blocks of 1024 on the host's cores."""
    M = N = K = 8192
    say("[fp8_8192] generating")
    ops = gi.operands("fp8", M, N, K, 5)
    say("[fp8_8192] gpu")
    _, got = run_gemm("fp8", ops, M, N, K)
    rng = np.random.default_rng(55)
    rows = [rng.integers(0, M, 3000)]
    cols = [rng.integers(0, N, 3000)]
    for r in (0, 4095, M - 1):                # whole rows
        rows.append(np.full(N // 8, r)); cols.append(np.arange(0, N, 8) + (r % 8))
    for c in (0, 4097, N - 1):                # whole columns (strided)
        rows.append(np.arange(0, M, 8) + (c % 8)); cols.append(np.full(M // 8, c))
    edges = np.array([0, 31, 32, 63, 64, 127, 128, 255, 256, M - 129, M - 128, M - 1])
    rr, cc = np.meshgrid(edges, edges)
    rows.append(rr.ravel()); cols.append(cc.ravel())
    rows, cols = np.concatenate(rows), np.concatenate(cols)
    say(f"[fp8_8192] sampled pre-check: oracle on {rows.size} entries")
    ref = oracle.gemm_entries("fp8", ops["A"], ops["B"], M, N, K, rows, cols,
                              ops["scale_a"], ops["scale_b"])
    ok, msg, _ = compare("fp8", got[rows, cols], ref, "fp8_8192 sampled")
    say(msg)
    assert ok, msg
    threads = min(16, len(os.sched_getaffinity(0)))
    rtol, atol = TOL["fp8"]
    nfail, worst, worst_at = 0, 0.0, None
    for r0 in range(0, M, 1024):
        say(f"[fp8_8192] oracle rows {r0}..{r0 + 1023} on {threads} threads")
        sa = ops["scale_a"][r0 // 64:(r0 + 1024) // 64]
        ref = oracle.gemm("fp8", ops["A"][r0:r0 + 1024], ops["B"], 1024, N, K, sa,
                          ops["scale_b"], nthreads=threads)
        blk_ok, blk_fail, blk_worst, idx = oracle.within_tolerance(
            oracle.decode(got[r0:r0 + 1024], "bf16"), ref, rtol, atol)
        nfail += blk_fail
        if blk_worst > worst:
            worst, worst_at = blk_worst, (idx[0] + r0, idx[1]) if idx is not None else None
    msg = (f"fp8_8192 every entry: {nfail} of {M * N} entries outside "
           f"|d| <= {rtol}|ref|+{atol}; worst err/tol {worst:.3g} at {worst_at}")
    say(msg)
    assert nfail == 0, msg


@pytest.mark.parametrize("shape", [(1000, 900, 700), (512, 512, 512), (130, 70, 200)])
def test_fp8_full_ragged(shape):
    _full_check("fp8", *shape, 5, "fp8_small")


@pytest.mark.parametrize("shape", [(256, 256, 256), (768, 512, 1024), (512, 1280, 768)])
def test_fp8_large_tile_path(shape):
    """Whole 256x256 tiles and K % 256 == 0: the large-tile fp8 kernel (forced
    with the testing override '7': by default grids this small take the K-split
    kernel)."""
    os.environ["LIBGEMM_FP8_SMALL"] = "7"
    _full_check("fp8", *shape, 6, "fp8_large")


@pytest.mark.parametrize("shape,lds", [
    ((300, 500, 320), None),                  # ragged M and N; 5 K blocks: one turn of the ring + 1
    ((257, 300, 129), None),                  # one row past a tile; partial last K block
    ((33, 17, 65), None),                     # partial tiles both ways, two K blocks, N barely >= 16
    ((520, 270, 1000), (1003, 277, 281)),     # unaligned leading dimensions, offset pointers
    ((256, 256, 448), None),                  # whole tiles, 7 K blocks: a guarded remainder of 3 steps
    ((600, 700, 832), (840, 704, 712)),       # several tiles each way, 13 K blocks
])
def test_fp8_guarded_large_tile_path(shape, lds):
    """The guarded large-tile fp8 kernel (testing override '2'): clamped rows and
    column chunks, the partial last K block through registers, masked stores."""
    os.environ["LIBGEMM_FP8_SMALL"] = "2"
    M, N, K = shape
    kw = {} if lds is None else dict(lda=lds[0], ldb=lds[1], ldc=lds[2], offset=1)
    say(f"[fp8-guarded] {M}x{N}x{K} {kw}")
    ops = gi.operands("fp8", M, N, K, 64)
    _, got = run_gemm("fp8", ops, M, N, K, **kw)
    ok, msg, _ = compare("fp8", got, reference("fp8", ops, M, N, K), "fp8-guarded")
    assert ok, msg


@pytest.mark.parametrize("force,shape", [
    ("3", (32, 64, 256)),       # 32-row tiles: one tile, one K block per wave
    ("3", (96, 128, 320)),      # 5 K blocks: wave 0 takes two
    ("3", (160, 192, 832)),     # 13 blocks: wave 0 goes round the 4-stage ring and more
    ("3", (2048, 64, 1088)),    # 17 blocks, 64 row strips (rotated K walks)
    ("5", (64, 64, 256)),       # 64-row tiles: one tile
    ("5", (192, 128, 448)),     # 7 blocks: 2,2,2,1 per wave
    ("5", (320, 256, 1088)),    # 17 blocks, several row strips
])
def test_fp8_ksplit_path(force, shape):
    """The fp8 K-split kernel on whole tiles (testing overrides '3': 32-row
    tiles, '5': 64-row tiles): one scale product per wave step, LDS reduction."""
    os.environ["LIBGEMM_FP8_SMALL"] = force
    M, N, K = shape
    say(f"[fp8-ksplit {force}] {M}x{N}x{K}")
    ops = gi.operands("fp8", M, N, K, 52)
    _, got = run_gemm("fp8", ops, M, N, K)
    ok, msg, _ = compare("fp8", got, reference("fp8", ops, M, N, K), "fp8-ksplit")
    assert ok, msg


@pytest.mark.parametrize("force", ["4", "6"])
@pytest.mark.parametrize("shape,lds", [
    ((1, 16, 1), None),                    # one row, sixteen columns, one k
    ((5, 200, 64), None),                  # one K block: the register-loaded block only
    ((33, 65, 65), None),                  # partial tiles both ways, partial K block
    ((31, 64, 300), (303, 67, 71)),        # unaligned leading dimensions, offset pointers
    ((64, 70, 129), None),                 # 3 K blocks: two waves without LDS-direct blocks
    ((100, 300, 1000), (1001, 301, 303)),  # 16 blocks incl. the partial one
    ((1000, 1000, 1000), None),            # the 1000^3 shape
])
def test_fp8_ksplit_general_edges(force, shape, lds):
    """The guarded fp8 K-split kernel (testing overrides '4': 32-row tiles, '6':
    64-row tiles): clamped rows and column chunks, the last K block through
    registers with zero fill, masked stores."""
    os.environ["LIBGEMM_FP8_SMALL"] = force
    M, N, K = shape
    kw = {} if lds is None else dict(lda=lds[0], ldb=lds[1], ldc=lds[2], offset=1)
    say(f"[fp8-ksplit-general {force}] {M}x{N}x{K} {kw}")
    ops = gi.operands("fp8", M, N, K, 53)
    _, got = run_gemm("fp8", ops, M, N, K, **kw)
    ok, msg, _ = compare("fp8", got, reference("fp8", ops, M, N, K), "fp8-ksplit-general")
    assert ok, msg


@pytest.mark.parametrize("force", ["3", "6"])
def test_fp8_ksplit_permutation_exact(force):
    """A * P with unit scales: every output is one product by 1 plus zeros."""
    M, K = 320, 256
    os.environ["LIBGEMM_FP8_SMALL"] = force
    say(f"[probe] fp8 K-split {force} A*P")
    ops, perm = _perm_case("fp8", M, K, 19)
    _, got = run_gemm("fp8", ops, M, K, K)
    want = np.empty((M, K))
    want[:, perm] = oracle.decode(ops["A"], "fp8")
    bad = np.argwhere(oracle.decode(got, "bf16") != want)
    assert bad.size == 0, f"first mismatch at {bad[0]}"


@pytest.mark.parametrize("force,shape,lds", [
    ("8", (128, 128, 256), None),             # one 128 x 128 tile, one turn of the ring
    ("8", (384, 256, 512), None),             # 6 tiles, two turns
    ("8", (640, 896, 1024), None),            # 35 tiles
    ("9", (129, 130, 129), None),             # a row and two columns past a tile, partial K block
    ("9", (300, 520, 333), (337, 521, 525)),  # unaligned leading dimensions, offset pointers
    ("9", (1000, 1000, 1000), None),          # the 1000^3 shape
])
def test_fp8_tiles128_path(force, shape, lds):
    """128 x 128 tiles of the large-tile fp8 kernel (testing overrides '8': whole
    tiles, '9': guarded): 8 waves of 32 x 64, B rows of 128 bytes."""
    os.environ["LIBGEMM_FP8_SMALL"] = force
    M, N, K = shape
    kw = {} if lds is None else dict(lda=lds[0], ldb=lds[1], ldc=lds[2], offset=1)
    say(f"[fp8-tiles128 {force}] {M}x{N}x{K} {kw}")
    ops = gi.operands("fp8", M, N, K, 54)
    _, got = run_gemm("fp8", ops, M, N, K, **kw)
    ok, msg, _ = compare("fp8", got, reference("fp8", ops, M, N, K), "fp8-tiles128")
    assert ok, msg


@pytest.mark.parametrize("force", ["8", "9"])
def test_fp8_tiles128_permutation_exact(force):
    M, K = 384, 512
    os.environ["LIBGEMM_FP8_SMALL"] = force
    say(f"[probe] fp8 128x128 tiles {force} A*P")
    ops, perm = _perm_case("fp8", M, K, 20)
    _, got = run_gemm("fp8", ops, M, K, K)
    want = np.empty((M, K))
    want[:, perm] = oracle.decode(ops["A"], "fp8")
    bad = np.argwhere(oracle.decode(got, "bf16") != want)
    assert bad.size == 0, f"first mismatch at {bad[0]}"


def test_fp8_guarded_permutation_exact():
    M, K = 300, 320
    os.environ["LIBGEMM_FP8_SMALL"] = "2"
    say("[probe] fp8 guarded large-tile A*P")
    ops, perm = _perm_case("fp8", M, K, 13)
    _, got = run_gemm("fp8", ops, M, K, K)
    want = np.empty((M, K))
    want[:, perm] = oracle.decode(ops["A"], "fp8")
    bad = np.argwhere(oracle.decode(got, "bf16") != want)
    assert bad.size == 0, f"first mismatch at {bad[0]}"


@pytest.mark.parametrize("shape,lds", [
    ((300, 500, 320), None),                  # ragged M and N; 10 K blocks
    ((129, 130, 97), None),                   # one row / two columns past a tile; partial last K block
    ((33, 5, 33), None),                      # partial tiles both ways, two K blocks, N barely >= 4
    ((520, 270, 1000), (1003, 277, 281)),     # unaligned leading dimensions, offset pointers
    ((256, 256, 96), None),                   # whole tiles, 3 K blocks: an odd count of steps
])
def test_f32_guarded_large_tile_path(shape, lds):
    """The guarded large-tile fp32 kernel (testing override '2'): clamped rows and
    column chunks, the partial last K block through registers, masked stores."""
    os.environ["LIBGEMM_F32_SMALL"] = "2"
    M, N, K = shape
    kw = {} if lds is None else dict(lda=lds[0], ldb=lds[1], ldc=lds[2], offset=1)
    say(f"[f32-guarded] {M}x{N}x{K} {kw}")
    ops = gi.operands("f32", M, N, K, 65)
    _, got = run_gemm("f32", ops, M, N, K, **kw)
    ok, msg, _ = compare("f32", got, reference("f32", ops, M, N, K), "f32-guarded")
    assert ok, msg


def test_f32_guarded_permutation_exact():
    M, K = 300, 160
    os.environ["LIBGEMM_F32_SMALL"] = "2"
    say("[probe] f32 guarded large-tile A*P")
    ops, perm = _perm_case("f32", M, K, 15)
    _, got = run_gemm("f32", ops, M, K, K)
    want = np.empty((M, K))
    want[:, perm] = oracle.decode(ops["A"], "f32")
    bad = np.argwhere(oracle.decode(got, "f32") != want)
    assert bad.size == 0, f"first mismatch at {bad[0]}"


@pytest.mark.parametrize("shape", [(128, 128, 64), (384, 256, 320), (1024, 640, 2048)])
def test_f32_large_tile_path(shape):
    """Whole 128x128 tiles and K % 64 == 0: the large-tile fp32 kernel (forced
    with the testing override '3': by default grids this small take the
    register-staged kernels)."""
    os.environ["LIBGEMM_F32_SMALL"] = "3"
    _full_check("f32", *shape, 7, "f32_large")


@pytest.mark.parametrize("shape", [(3072, 3072, 64), (5120, 4096, 64), (4096, 4096, 192)])
def test_f32_large_tile_persistent(shape):
    """More tiles than two workgroups per CU (576, 1280 and 1024 tiles of
    128 x 128): each persistent workgroup walks several tiles on one ring, the
    next tile's first steps loading during the current tile's last ones."""
    os.environ["LIBGEMM_F32_SMALL"] = "3"
    _full_check("f32", *shape, 8, "f32_persistent")


def test_f32_large_tile_persistent_permutation_exact():
    M, K = 5120, 2048                       # 640 tiles: 128 workgroups take two
    os.environ["LIBGEMM_F32_SMALL"] = "3"
    say("[probe] f32 persistent large-tile A*P")
    ops, perm = _perm_case("f32", M, K, 17)
    _, got = run_gemm("f32", ops, M, K, K)
    want = np.empty((M, K))
    want[:, perm] = oracle.decode(ops["A"], "f32")
    bad = np.argwhere(oracle.decode(got, "f32") != want)
    assert bad.size == 0, f"first mismatch at {bad[0]}"


def test_f32_large_tile_permutation_exact():
    M, K = 384, 512
    os.environ["LIBGEMM_F32_SMALL"] = "3"
    say("[probe] f32 large-tile A*P")
    ops, perm = _perm_case("f32", M, K, 11)
    _, got = run_gemm("f32", ops, M, K, K)
    want = np.empty((M, K))
    want[:, perm] = oracle.decode(ops["A"], "f32")
    bad = np.argwhere(oracle.decode(got, "f32") != want)
    assert bad.size == 0, f"first mismatch at {bad[0]}"


@pytest.mark.parametrize("force,shape", [
    ("4", (32, 64, 128)),       # 32-row tiles: one tile, one K block per wave
    ("4", (96, 128, 160)),      # 5 K blocks: wave 0 takes two, the others one
    ("4", (160, 192, 416)),     # 13 blocks: a second trip through the 3-stage ring for wave 0
    ("4", (2048, 64, 544)),     # 17 blocks, 64 row strips (rotated K walks)
    ("6", (64, 64, 128)),       # 64-row tiles: one tile, one K block per wave
    ("6", (192, 128, 160)),     # 5 K blocks
    ("6", (128, 192, 224)),     # 7 blocks: 2,2,2,1 per wave (the last step of a pair skipped)
    ("6", (320, 256, 544)),     # 17 blocks, several row strips
])
def test_f32_ksplit_path(force, shape):
    """The fp32 K-split kernel on whole tiles (testing overrides '4': 32-row
    tiles, '6': 64-row tiles)."""
    os.environ["LIBGEMM_F32_SMALL"] = force
    M, N, K = shape
    say(f"[f32-ksplit {force}] {M}x{N}x{K}")
    ops = gi.operands("f32", M, N, K, 48)
    _, got = run_gemm("f32", ops, M, N, K)
    ok, msg, _ = compare("f32", got, reference("f32", ops, M, N, K), "f32-ksplit")
    assert ok, msg


@pytest.mark.parametrize("force", ["5", "7"])
@pytest.mark.parametrize("shape,lds", [
    ((1, 4, 1), None),                     # one row, four columns, one k
    ((5, 200, 32), None),                  # one K block: the register-loaded block only
    ((33, 65, 33), None),                  # partial tiles both ways, partial K block
    ((31, 64, 300), (303, 67, 71)),        # unaligned leading dimensions, offset pointers
    ((64, 70, 65), None),                  # 3 K blocks: two waves without LDS-direct blocks
    ((100, 300, 1000), (1001, 301, 303)),  # 32 blocks incl. the partial one
    ((1000, 1000, 1000), None),            # the 1000^3 workload's shape
])
def test_f32_ksplit_general_edges(force, shape, lds):
    """The guarded fp32 K-split kernel (testing overrides '5': 32-row tiles,
    '7': 64-row tiles): clamped rows and column chunks, the last K block through
    registers, masked stores."""
    os.environ["LIBGEMM_F32_SMALL"] = force
    M, N, K = shape
    kw = {} if lds is None else dict(lda=lds[0], ldb=lds[1], ldc=lds[2], offset=1)
    say(f"[f32-ksplit-general {force}] {M}x{N}x{K} {kw}")
    ops = gi.operands("f32", M, N, K, 49)
    _, got = run_gemm("f32", ops, M, N, K, **kw)
    ok, msg, _ = compare("f32", got, reference("f32", ops, M, N, K), "f32-ksplit-general")
    assert ok, msg


@pytest.mark.parametrize("force", ["4", "7"])
def test_f32_ksplit_permutation_exact(force):
    """A * P with P a permutation: every output is one product by 1 plus zeros,
    so it is exact whatever the order of the K split."""
    M, K = 320, 256
    os.environ["LIBGEMM_F32_SMALL"] = force
    say(f"[probe] f32 K-split {force} A*P")
    ops, perm = _perm_case("f32", M, K, 16)
    _, got = run_gemm("f32", ops, M, K, K)
    want = np.empty((M, K))
    want[:, perm] = oracle.decode(ops["A"], "f32")
    bad = np.argwhere(oracle.decode(got, "f32") != want)
    assert bad.size == 0, f"first mismatch at {bad[0]}"


ROWS_ENV = {"bf16": ("LIBGEMM_H16_CONFIG", "10"), "f16": ("LIBGEMM_H16_CONFIG", "10"),
            "f32": ("LIBGEMM_F32_SMALL", "8")}


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("shape,lds", [
    ((1, 1, 1), None),                      # one element
    ((1, 64, 4100), None),                  # one workgroup; K not a multiple of the row groups
    ((2, 100, 333), (337, 101, 103)),       # partial column chunk, unaligned ld, offset pointers
    ((3, 4095, 517), None),                 # 64 workgroups, the last one ragged
    ((4, 130, 2048), (2051, 131, 133)),     # four rows, unaligned leading dimensions
    ((1, 4095, 4100), (4100, 4095, 4095)),  # the tail row of 4097 x 4095 x 4100
    ((2, 16500, 300), (301, 16501, 16503)), # 258 workgroups, unaligned ld, offset pointers
    ((4, 17, 70), (71, 17, 19)),            # one chunk whole, the next straddling N
])
def test_rows_path(dtype, shape, lds):
    """The vector-ALU kernel for at most 4 rows (testing overrides: half-precision
    config 10, fp32 '8'): zeros past K and N, a chunk straddling N element by
    element, sums across lanes and waves."""
    var, val = ROWS_ENV[dtype]
    os.environ[var] = val
    M, N, K = shape
    kw = {} if lds is None else dict(lda=lds[0], ldb=lds[1], ldc=lds[2], offset=1)
    say(f"[rows] {dtype} {M}x{N}x{K} {kw}")
    ops = gi.operands(dtype, M, N, K, 51)
    _, got = run_gemm(dtype, ops, M, N, K, **kw)
    ok, msg, _ = compare(dtype, got, reference(dtype, ops, M, N, K), "rows")
    assert ok, msg


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_rows_permutation_exact(dtype):
    M, K = 4, 520
    var, val = ROWS_ENV[dtype]
    os.environ[var] = val
    say(f"[probe] rows {dtype} A*P")
    ops, perm = _perm_case(dtype, M, K, 18)
    _, got = run_gemm(dtype, ops, M, K, K)
    want = np.empty((M, K))
    want[:, perm] = oracle.decode(ops["A"], dtype)
    bad = np.argwhere(oracle.decode(got, OUT_DTYPE[dtype]) != want)
    assert bad.size == 0, f"first mismatch at {bad[0]}"


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("shape,lds", [
    ((1, 32, 1), None),                      # one workgroup, K below one block: registers only
    ((1, 4095, 4100), (4100, 4095, 4095)),   # the tail row of 4097 x 4095 x 4100
    ((1, 4096, 4096), None),                 # whole blocks only, every wave 16 blocks (two turns)
    ((2, 100, 333), (337, 101, 103)),        # window of the last workgroup moved left, offsets
    ((3, 4095, 200), None),                  # waves with no block; the partial block to one of them
    ((4, 130, 2048), (2051, 131, 133)),      # four rows, unaligned leading dimensions
    ((1, 16500, 300), (301, 16501, 16503)),  # 516 workgroups, several rounds
    ((4, 33, 3072), (3075, 35, 37)),         # the largest K four rows fit, window straddling
    ((1, 40, 12288), None),                  # the largest K one row fits: six turns of the ring
    ((2, 64, 4650), (4653, 67, 69)),         # two turns and more, partial block
])
def test_fewrows_path(dtype, shape, lds):
    """The few-row kernel (half-precision config 15): B streamed through per-wave
    LDS rings; the partial last block through registers; the last workgroup's
    window moved to end at N."""
    os.environ["LIBGEMM_H16_CONFIG"] = str(FEWROWS)
    M, N, K = shape
    kw = {} if lds is None else dict(lda=lds[0], ldb=lds[1], ldc=lds[2], offset=1)
    say(f"[fewrows] {dtype} {M}x{N}x{K} {kw}")
    ops = gi.operands(dtype, M, N, K, 52)
    C, got = run_gemm(dtype, ops, M, N, K, **kw)
    if lds is not None:
        pad = C.as_strided((M, lds[2] - N), (lds[2], 1), C.storage_offset() + N)
        padv = oracle.decode(pad.cpu().contiguous().view(torch.int16).numpy().view(np.uint16),
                             OUT_DTYPE[dtype])
        assert np.isnan(padv).all(), "C written between N and ldc"
    ok, msg, _ = compare(dtype, got, reference(dtype, ops, M, N, K), "fewrows")
    assert ok, msg


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("shape,lds", [
    ((1, 8192, 8192), None),                 # one row, long K and wide: the narrow kernel
    ((1, 4096, 4096), None),                 # one row, N * K <= 17 M: the few-row kernel
    ((1, 4095, 4100), (4100, 4095, 4095)),   # the same with 2-byte-aligned rows
    ((3, 5000, 2000), (2003, 5001, 5003)),   # three rows, K < 2048: the narrow kernel, guarded
    ((4, 4095, 2048), (2048, 4095, 4095)),   # four rows: the narrow kernel, guarded
    ((2, 1000, 2048), (2048, 1001, 1003)),   # two rows, unaligned B rows, K >= 2048: few-row
    ((2, 16384, 1024), None),                # two rows, wide, short K: the narrow kernel
    ((32, 4100, 1000), None),                # one full row strip of the narrow kernel
])
def test_few_rows_dispatch(dtype, shape, lds):
    """Products of at most 32 rows through the automatic dispatch (no override)."""
    M, N, K = shape
    kw = {} if lds is None else dict(lda=lds[0], ldb=lds[1], ldc=lds[2], offset=1)
    say(f"[few rows, auto] {dtype} {M}x{N}x{K} {kw}")
    ops = gi.operands(dtype, M, N, K, 53)
    _, got = run_gemm(dtype, ops, M, N, K, **kw)
    ok, msg, _ = compare(dtype, got, reference(dtype, ops, M, N, K), "few rows")
    assert ok, msg


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("M,K", [(4, 520), (1, 4100)])
def test_fewrows_permutation_exact(dtype, M, K):
    """A*P on the few-row kernel must equal a column permutation of A bit for bit
    (a row of B moved to another lane, slot or wave shows as a moved entry)."""
    os.environ["LIBGEMM_H16_CONFIG"] = str(FEWROWS)
    say(f"[probe] fewrows {dtype} {M}x{K} A*P")
    ops, perm = _perm_case(dtype, M, K, 19)
    _, got = run_gemm(dtype, ops, M, K, K)
    want = np.empty((M, K))
    want[:, perm] = oracle.decode(ops["A"], dtype)
    bad = np.argwhere(oracle.decode(got, OUT_DTYPE[dtype]) != want)
    assert bad.size == 0, f"first mismatch at {bad[0]}"


def test_fp8_large_tile_permutation_exact():
    M = K = 512
    os.environ["LIBGEMM_FP8_SMALL"] = "7"
    say("[probe] fp8 large-tile A*P")
    ops, perm = _perm_case("fp8", M, K, 9)
    _, got = run_gemm("fp8", ops, M, K, K)
    want = np.empty((M, K))
    want[:, perm] = oracle.decode(ops["A"], "fp8")
    gotv = oracle.decode(got, "bf16")
    bad = np.argwhere(gotv != want)
    assert bad.size == 0, f"first mismatch at {bad[0]}"


@pytest.mark.parametrize("dtype,config,aligned",
                         [(d, c, a) for d in ("bf16", "f16") for c in H16_CONFIGS
                          for a in (True, False)])
def test_forced_config_ragged(dtype, config, aligned):
    os.environ["LIBGEMM_H16_CONFIG"] = str(config)
    M, N, K = 300, 520, 200 if aligned else 203
    kw = {} if aligned else dict(lda=K + 3, ldb=N + 1, ldc=N + 5, offset=1)
    say(f"[forced] {dtype} config={config} aligned={aligned} {M}x{N}x{K} {kw}")
    ops = gi.operands(dtype, M, N, K, 30 + config)
    _, got = run_gemm(dtype, ops, M, N, K, **kw)
    ok, msg, _ = compare(dtype, got, reference(dtype, ops, M, N, K), "forced")
    assert ok, msg


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("config", [GENERAL, GEN128, GEN128x256])
@pytest.mark.parametrize("a_pad,a_off,b_pad,b_off", [
    (0, 0, 0, 0),   # both operands' rows 4-byte aligned: both through buffer descriptors
    (0, 0, 1, 0),   # B's leading dimension odd: A buffer, B global
    (1, 0, 0, 0),   # A's leading dimension odd: A global, B buffer
    (0, 1, 0, 0),   # A's base 2-byte aligned, even leading dimension: A global
    (0, 0, 0, 1),   # B's base 2-byte aligned: B global
    (1, 1, 1, 1),   # neither
])
def test_guarded_operand_alignment(dtype, config, a_pad, a_off, b_pad, b_off):
    """The guarded large-tile kernels load each operand through a buffer
    descriptor when its rows start on 4-byte boundaries and through global loads
    otherwise; every combination against the oracle, with a K tail."""
    os.environ["LIBGEMM_H16_CONFIG"] = str(config)
    M, N, K = 300, 520, 202
    lda, ldb = K + a_pad, N + b_pad
    say(f"[guarded align] {dtype} config={config} lda={lda}+{a_off} ldb={ldb}+{b_off}")
    import dense_gemm_13_amd as dg
    ops = gi.operands(dtype, M, N, K, 54)
    A = to_device(ops["A"][:M, :K], dtype, lda, a_off)
    B = to_device(ops["B"][:K, :N], dtype, ldb, b_off)
    C = torch.full((M, N), float("nan"), dtype=A.dtype, device="cuda")
    getattr(dg, "gemm_" + dtype)(A, B, C)
    torch.cuda.synchronize()
    got = C.cpu().view(torch.int16).numpy().view(np.uint16)
    ok, msg, _ = compare(dtype, got, reference(dtype, ops, M, N, K), "guarded align")
    assert ok, msg


@pytest.mark.parametrize("dtype,var,force,K", [
    ("bf16", "LIBGEMM_H16_CONFIG", "5", 100),    # guarded 256 x 256 tiles
    ("f16", "LIBGEMM_H16_CONFIG", "12", 100),    # guarded 128 x 128 tiles
    ("bf16", "LIBGEMM_H16_CONFIG", "14", 100),   # guarded 128 x 256 tiles
    ("bf16", "LIBGEMM_H16_CONFIG", "7", 100),    # narrow kernel, guarded
    ("f16", "LIBGEMM_H16_CONFIG", "9", 100),     # narrow 64-row kernel, guarded
    ("bf16", "LIBGEMM_H16_CONFIG", "7", 7),      # K below one 16-byte chunk: element loads
    ("f32", "LIBGEMM_F32_SMALL", "2", 101),      # fp32 guarded large tiles
    ("f32", "LIBGEMM_F32_SMALL", "5", 101),      # fp32 K-split, guarded
    ("f32", "LIBGEMM_F32_SMALL", "7", 3),        # fp32 K-split 64-row, K below one chunk
    ("fp8", "LIBGEMM_FP8_SMALL", "2", 130),      # fp8 guarded large tiles
    ("fp8", "LIBGEMM_FP8_SMALL", "4", 130),      # fp8 K-split, guarded
    ("fp8", "LIBGEMM_FP8_SMALL", "6", 9),        # fp8 K-split 64-row, K below one chunk
])
def test_guarded_last_block_at_buffer_end(dtype, var, force, K):
    """The last K block of the guarded kernels goes through registers: one 16-byte
    load per chunk from inside the matrix, a chunk that straddles K or N taken
    from the row's last 16 bytes and shifted.  Leading dimensions equal to the
    row lengths and offset base pointers put those chunks at the very end of A's
    and B's buffers (A's last row straddles K, B's last row straddles N)."""
    os.environ[var] = force
    M, N = 290, 300
    say(f"[last block] {dtype} {var}={force} {M}x{N}x{K}")
    ops = gi.operands(dtype, M, N, K, 56)
    _, got = run_gemm(dtype, ops, M, N, K, lda=K, ldb=N, ldc=N, offset=1)
    ok, msg, _ = compare(dtype, got, reference(dtype, ops, M, N, K), "last block")
    assert ok, msg


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("shape", [(256, 256, 128), (512, 768, 384), (1024, 512, 2048),
                                   (768, 256, 1152)])
def test_fast_path_whole_tiles(dtype, shape):
    os.environ["LIBGEMM_H16_CONFIG"] = str(FAST)
    M, N, K = shape
    say(f"[fast] {dtype} {M}x{N}x{K}")
    ops = gi.operands(dtype, M, N, K, 40)
    _, got = run_gemm(dtype, ops, M, N, K)
    ok, msg, _ = compare(dtype, got, reference(dtype, ops, M, N, K), "fast")
    assert ok, msg


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("shape", [(128, 128, 128), (384, 256, 256), (640, 896, 1152),
                                   (1024, 1024, 2048)])
def test_fast128_whole_tiles(dtype, shape):
    """128 x 128 tiles of the large-tile kernel (config 11): one tile to 64
    tiles, one to four turns of the ring per tile."""
    os.environ["LIBGEMM_H16_CONFIG"] = str(FAST128)
    M, N, K = shape
    say(f"[fast128] {dtype} {M}x{N}x{K}")
    ops = gi.operands(dtype, M, N, K, 44)
    _, got = run_gemm(dtype, ops, M, N, K)
    ok, msg, _ = compare(dtype, got, reference(dtype, ops, M, N, K), "fast128")
    assert ok, msg


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("shape", [(128, 256, 128), (256, 512, 384), (512, 768, 1152),
                                   (1024, 1024, 2048)])
def test_fast128x256_whole_tiles(dtype, shape):
    """128 x 256 tiles of the large-tile kernel (config 13): wave tiles of
    64 x 128, the epilogue staged in the B stage arrays."""
    os.environ["LIBGEMM_H16_CONFIG"] = str(FAST128x256)
    M, N, K = shape
    say(f"[fast128x256] {dtype} {M}x{N}x{K}")
    ops = gi.operands(dtype, M, N, K, 46)
    _, got = run_gemm(dtype, ops, M, N, K)
    ok, msg, _ = compare(dtype, got, reference(dtype, ops, M, N, K), "fast128x256")
    assert ok, msg


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("shape,lds", [
    ((1, 8, 33), None),                      # one row, eight columns, a partial second K block
    ((129, 257, 97), None),                  # a row and a column past a tile
    ((300, 520, 203), (206, 521, 525)),      # unaligned leading dimensions, offset pointers
    ((1000, 1000, 1000), None),              # the 1000^3 workload's shape
])
def test_general128x256_edges(dtype, shape, lds):
    """The guarded 128 x 256 instantiation (config 14)."""
    os.environ["LIBGEMM_H16_CONFIG"] = str(GEN128x256)
    M, N, K = shape
    kw = {} if lds is None else dict(lda=lds[0], ldb=lds[1], ldc=lds[2], offset=1)
    say(f"[general128x256] {dtype} {M}x{N}x{K} {kw}")
    ops = gi.operands(dtype, M, N, K, 47)
    _, got = run_gemm(dtype, ops, M, N, K, **kw)
    ok, msg, _ = compare(dtype, got, reference(dtype, ops, M, N, K), "general128x256")
    assert ok, msg


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("shape,lds", [
    ((1, 8, 33), None),                      # one row, eight columns, a partial second K block
    ((129, 130, 97), None),                  # a row and two columns past a tile
    ((300, 520, 203), (206, 521, 525)),      # unaligned leading dimensions, offset pointers
    ((1000, 1000, 1000), None),              # the 1000^3 workload's shape
    ((1500, 1500, 1500), (1501, 1503, 1505)),  # 144 tiles, unaligned rows
])
def test_general128_edges(dtype, shape, lds):
    """The guarded 128 x 128 instantiation (config 12)."""
    os.environ["LIBGEMM_H16_CONFIG"] = str(GEN128)
    M, N, K = shape
    kw = {} if lds is None else dict(lda=lds[0], ldb=lds[1], ldc=lds[2], offset=1)
    say(f"[general128] {dtype} {M}x{N}x{K} {kw}")
    ops = gi.operands(dtype, M, N, K, 45)
    _, got = run_gemm(dtype, ops, M, N, K, **kw)
    ok, msg, _ = compare(dtype, got, reference(dtype, ops, M, N, K), "general128")
    assert ok, msg


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("shape", [
    (32, 64, 256),        # one tile, one K block per wave
    (96, 64, 320),        # 5 K blocks: wave 0 takes two, the others one
    (64, 128, 448),       # 7 blocks: 2,2,2,1 per wave (last ring step skipped)
    (160, 192, 832),      # 13 blocks: a second trip through the ring for wave 0 only
    (2048, 64, 1088),     # 17 blocks, 64 row strips
])
def test_narrow_path(dtype, shape):
    os.environ["LIBGEMM_H16_CONFIG"] = str(NARROW)
    M, N, K = shape
    say(f"[narrow] {dtype} {M}x{N}x{K}")
    ops = gi.operands(dtype, M, N, K, 42)
    _, got = run_gemm(dtype, ops, M, N, K)
    ok, msg, _ = compare(dtype, got, reference(dtype, ops, M, N, K), "narrow")
    assert ok, msg


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("shape", [
    (64, 64, 256),        # one tile, one K block per wave
    (192, 128, 320),      # 5 K blocks: wave 0 takes two, the others one
    (128, 192, 448),      # 7 blocks: 2,2,2,1 per wave (the last step of a pair skipped)
    (320, 256, 1088),     # 17 blocks, several row strips (rotated K walks)
])
def test_narrow64_path(dtype, shape):
    os.environ["LIBGEMM_H16_CONFIG"] = str(NARROW64)
    M, N, K = shape
    say(f"[narrow64] {dtype} {M}x{N}x{K}")
    ops = gi.operands(dtype, M, N, K, 46)
    _, got = run_gemm(dtype, ops, M, N, K)
    ok, msg, _ = compare(dtype, got, reference(dtype, ops, M, N, K), "narrow64")
    assert ok, msg


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("shape,lds", [
    ((1, 8, 1), None),                     # one row, eight columns, one k
    ((65, 65, 65), None),                  # a row and a column past a tile, partial K block
    ((1000, 1000, 1000), None),            # the 1000^3 workload's shape
    ((100, 300, 1000), (1001, 301, 303)),  # unaligned leading dimensions, offset pointers
    ((64, 70, 129), None),                 # 3 K blocks: two waves without LDS-direct blocks
])
def test_narrow64_general_path_edges(dtype, shape, lds):
    os.environ["LIBGEMM_H16_CONFIG"] = str(NARROW64_GEN)
    M, N, K = shape
    kw = {} if lds is None else dict(lda=lds[0], ldb=lds[1], ldc=lds[2], offset=1)
    say(f"[narrow64-general] {dtype} {M}x{N}x{K} {kw}")
    ops = gi.operands(dtype, M, N, K, 47)
    _, got = run_gemm(dtype, ops, M, N, K, **kw)
    ok, msg, _ = compare(dtype, got, reference(dtype, ops, M, N, K), "narrow64-general")
    assert ok, msg


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("shape,lds", [
    ((1, 8, 1), None),                     # one row, eight columns, one k
    ((5, 200, 64), None),                  # one K block: the register-loaded block only
    ((33, 65, 65), None),                  # two row tiles, two column tiles, partial K block
    ((31, 64, 300), (303, 67, 71)),        # unaligned leading dimensions
    ((64, 70, 129), None),                 # 3 K blocks: two waves without LDS-direct blocks
    ((40, 100, 1000), (1001, 101, 103)),   # 16 blocks: 4 per wave incl. the partial one
    ((1, 4095, 4100), (4100, 4095, 4095)),  # the tail row of the ragged workload
])
def test_narrow_general_path_edges(dtype, shape, lds):
    os.environ["LIBGEMM_H16_CONFIG"] = str(NARROW_GEN)
    M, N, K = shape
    kw = {} if lds is None else dict(lda=lds[0], ldb=lds[1], ldc=lds[2], offset=1)
    say(f"[narrow-general] {dtype} {M}x{N}x{K} {kw}")
    ops = gi.operands(dtype, M, N, K, 43)
    _, got = run_gemm(dtype, ops, M, N, K, **kw)
    ok, msg, _ = compare(dtype, got, reference(dtype, ops, M, N, K), "narrow-general")
    assert ok, msg


@pytest.mark.parametrize("shape,lds", [
    ((4160, 4096, 256), None),                 # 64-row tail below whole tiles (large-tile path)
    ((4127, 4000, 300), (301, 4003, 4001)),    # 31-row tail below guarded tiles, unaligned
])
def test_row_tail_split(shape, lds):
    """A few rows below a grid of 256-row tiles whose extra tile row would need
    a second round of workgroups: those rows are computed by the narrow kernel."""
    M, N, K = shape
    kw = {} if lds is None else dict(lda=lds[0], ldb=lds[1], ldc=lds[2], offset=1)
    say(f"[tail-split] bf16 {M}x{N}x{K} {kw}")
    ops = gi.operands("bf16", M, N, K, 44)
    _, got = run_gemm("bf16", ops, M, N, K, **kw)
    ok, msg, _ = compare("bf16", got, reference("bf16", ops, M, N, K), "tail-split")
    assert ok, msg


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("shape,lds", [
    ((256, 256, 33), None),            # two K steps, the last one partial
    ((256, 256, 64), None),            # two full K steps
    ((300, 264, 200), None),           # 7 K steps: not a multiple of the ring depth
    ((1, 8, 65), None),                # one row, eight columns
    ((257, 9, 96), (101, 11, 13)),     # unaligned leading dimensions
    ((520, 777, 1000), (1003, 779, 781)),
    ((4097, 4095, 4100), None),        # the ragged workload on this path alone (272 tiles)
])
def test_general_path_edges(dtype, shape, lds):
    os.environ["LIBGEMM_H16_CONFIG"] = str(GENERAL)
    M, N, K = shape
    kw = {} if lds is None else dict(lda=lds[0], ldb=lds[1], ldc=lds[2], offset=1)
    say(f"[general] {dtype} {M}x{N}x{K} {kw}")
    ops = gi.operands(dtype, M, N, K, 41)
    _, got = run_gemm(dtype, ops, M, N, K, **kw)
    ok, msg, _ = compare(dtype, got, reference(dtype, ops, M, N, K), "general")
    assert ok, msg


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32", "fp8"])
def test_fuzz_small_shapes(dtype):
    rng = np.random.default_rng({"f16": 1, "bf16": 2, "f32": 3, "fp8": 4}[dtype])
    for case in range(12):
        M, N, K = (int(x) for x in rng.integers(1, 301, 3))
        kw = {}
        if case % 2:
            kw = dict(lda=K + int(rng.integers(0, 9)), ldb=N + int(rng.integers(0, 9)),
                      ldc=N + int(rng.integers(0, 9)), offset=int(rng.integers(0, 4)))
        say(f"[fuzz] {dtype} case {case}: {M}x{N}x{K} {kw}")
        ops = gi.operands(dtype, M, N, K, 60 + case)
        _, got = run_gemm(dtype, ops, M, N, K, **kw)
        ok, msg, _ = compare(dtype, got, reference(dtype, ops, M, N, K), f"fuzz {M}x{N}x{K}")
        assert ok, msg


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32", "fp8"])
def test_fuzz_medium_shapes(dtype):
    """Random medium shapes through the automatic dispatch (the range where it
    picks between the K-split, 128 x 128, 128 x 256, 256 x 256 and register-staged
    kernels), every entry against the oracle; odd cases with padded leading
    dimensions and an offset pointer, whose padding must stay unwritten."""
    rng = np.random.default_rng({"f16": 11, "bf16": 12, "f32": 13, "fp8": 14}[dtype])
    for case in range(8):
        M, N = (int(x) for x in rng.integers(64, 2601, 2))
        K = int(rng.integers(32, 3001))
        kw = {}
        if case % 2:
            kw = dict(lda=K + int(rng.integers(1, 9)), ldb=N + int(rng.integers(1, 9)),
                      ldc=N + int(rng.integers(1, 9)), offset=int(rng.integers(1, 4)))
        say(f"[fuzz-medium] {dtype} case {case}: {M}x{N}x{K} {kw}")
        ops = gi.operands(dtype, M, N, K, 200 + case)
        C, got = run_gemm(dtype, ops, M, N, K, **kw)
        ok, msg, _ = compare(dtype, got, reference(dtype, ops, M, N, K), f"fuzz {M}x{N}x{K}")
        assert ok, msg
        if "ldc" in kw:
            pad = kw["ldc"] - N
            band = C.as_strided((M, pad), (kw["ldc"], 1), C.storage_offset() + N).float().cpu()
            assert torch.isnan(band).all(), "padding between N and ldc was written"


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32", "fp8"])
def test_degenerate_sizes(dtype):
    for (M, N, K) in [(1, 1, 1), (1, 257, 33), (257, 1, 65), (3, 5, 1), (64, 64, 1)]:
        say(f"[degenerate] {dtype} {M}x{N}x{K}")
        ops = gi.operands(dtype, M, N, K, 70)
        _, got = run_gemm(dtype, ops, M, N, K)
        ok, msg, _ = compare(dtype, got, reference(dtype, ops, M, N, K), "degenerate")
        assert ok, msg


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32", "fp8"])
def test_k_zero_sets_window_to_zero(dtype):
    M, N = 70, 90
    say(f"[k0] {dtype}")
    ops = gi.operands(dtype, M, N, 0, 71)
    C, got = run_gemm(dtype, ops, M, N, 0, ldc=N + 6)
    assert np.all(oracle.decode(got, OUT_DTYPE[dtype]) == 0.0)
    pad = C.as_strided((M, 6), (N + 6, 1), C.storage_offset() + N).float().cpu()
    assert torch.isnan(pad).all(), "padding between N and ldc was written"


@pytest.mark.parametrize("dtype", ["bf16", "f32", "fp8"])
def test_guard_band_untouched(dtype):
    M, N, K = 200, 150, 130
    odt = {"bf16": torch.bfloat16, "f32": torch.float32, "fp8": torch.bfloat16}[dtype]
    say(f"[guard] {dtype}")
    ldc = N + 13
    buf = torch.full((M + 2, ldc), float("nan"), dtype=odt, device="cuda")
    C = buf[1:M + 1, :N]
    ops = gi.operands(dtype, M, N, K, 72)
    run_gemm(dtype, ops, M, N, K, C=C)
    host = buf.float().cpu()
    assert torch.isnan(host[0]).all() and torch.isnan(host[M + 1]).all()
    assert torch.isnan(host[1:M + 1, N:]).all()
    assert not torch.isnan(host[1:M + 1, :N]).any()


def test_stream_argument_is_used():
    import dense_gemm_13_amd as dg
    M = N = K = 512
    ops = gi.operands("bf16", M, N, K, 73)
    A, B = to_device(ops["A"], "bf16"), to_device(ops["B"], "bf16")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        C = dg.gemm_bf16(A, B)
    s.synchronize()
    got = C.cpu().view(torch.int16).numpy().view(np.uint16)
    ok, msg, _ = compare("bf16", got, reference("bf16", ops, M, N, K), "side stream")
    assert ok, msg
