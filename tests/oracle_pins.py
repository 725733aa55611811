"""Pins for the CPU oracle: facts fixed by the number formats and by mathematics,
not by the oracle itself.

Each ``pin_*`` function returns a list of failure descriptions (empty = pass),
so the same checks serve the ordinary tests and the mutation tests, which plant
a mistake in a copy of oracle.c and require at least one pin to fail.

Independent sources used here:
* library decoders: numpy float16, torch bfloat16 / float8_e4m3fn, numpy float32;
* closed forms: A*I = A, I*B = B, P*B = row-permuted B, all-ones -> K,
  rank-1 (u 1^T)(1 z^T) = K u z^T, K = 1 outer product, K = 0 -> 0;
* exact rational brute force (fractions.Fraction) on tiny inputs;
* for the FP8 quantiser: torch's float8_e4m3fn / float8_e5m2 casts and decodings,
  brute-force nearest-value search over every FP8 code, exact-midpoint quotients,
  power-of-two block patterns and the independent input recipe in gemm_inputs;
* for the fused epilogue: hand-derived closed forms on all-ones products with a
  per-column bias, a row- and column-dependent prior C in a NaN-padded buffer,
  relu thresholds and a NaN-filled prior that beta = 0 must leave unread;
* for the convolution and im2col: torch's float64 conv2d and unfold, delta and
  shift kernels, tap counts of an all-ones input, and the 1x1 case = the GEMM.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import torch

import gemm_inputs as gi

DTYPES = ("f16", "bf16", "f32", "fp8")


# ------------------------------------------------------------ independent decoding

def lib_decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Decode raw bits with numpy/torch casts (not the oracle's decoders)."""
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float64)
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
        return t.to(torch.float64).numpy()
    if dtype == "fp8":
        t = torch.from_numpy(np.ascontiguousarray(bits)).view(torch.float8_e4m3fn)
        return t.to(torch.float64).numpy()
    if dtype == "f32":
        return np.ascontiguousarray(bits).view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def encode(x: np.ndarray, dtype: str) -> np.ndarray:
    """Float values (exactly representable) -> raw operand bits of dtype."""
    x = np.asarray(x, dtype=np.float32)
    if dtype == "f16":
        return gi.to_f16_bits(x)
    if dtype == "bf16":
        return gi.to_bf16_bits(x)
    if dtype == "f32":
        return np.ascontiguousarray(x)
    if dtype == "fp8":
        return gi.to_e4m3_bits(x)
    raise ValueError(dtype)


def unit_scales(rows: int, cols: int) -> np.ndarray:
    return np.ones((-(-rows // 64), -(-cols // 64)), dtype=np.float32)


def random_operand(rows: int, cols: int, dtype: str, seed: int):
    """(bits, scales-or-None) with the workloads' value distributions."""
    if dtype in ("f16", "bf16"):
        return gi.uniform_h16(rows, cols, seed, dtype), None
    if dtype == "f32":
        return gi.normal_f32(rows, cols, seed), None
    return gi.normal_fp8_blockscaled(rows, cols, seed)


def exact_values(bits: np.ndarray, dtype: str, scales) -> list:
    """Exact rational value of every element (Fraction), from library decoding."""
    vals = lib_decode(bits, dtype)
    rows, cols = vals.shape
    out = [[Fraction(float(vals[r, c])) for c in range(cols)] for r in range(rows)]
    if dtype == "fp8":
        for r in range(rows):
            for c in range(cols):
                out[r][c] *= Fraction(float(scales[r // 64, c // 64]))
    return out


# ------------------------------------------------------------------ the pins

def pin_decoders(orc) -> list:
    fails = []
    all16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    all8 = np.arange(256, dtype=np.uint32).astype(np.uint8)
    for dtype, bits in (("f16", all16), ("bf16", all16), ("fp8", all8)):
        got, want = orc.decode(bits, dtype), lib_decode(bits, dtype)
        same = (got == want) | (np.isnan(got) & np.isnan(want))
        if not same.all():
            i = int(np.argmin(same))
            fails.append(f"decode {dtype}: pattern {int(bits[i]):#x} -> {got[i]!r}, library {want[i]!r}")
    rng = np.random.default_rng(5)
    f32 = np.concatenate([rng.integers(0, 2**32, 200000, dtype=np.uint64).astype(np.uint32),
                          np.array([0, 1, 0x7fffff, 0x800000, 0x7f7fffff, 0x7f800000,
                                    0xff800000, 0x80000001, 0x3f800000], dtype=np.uint32)])
    got = orc.decode(f32.view(np.float32), "f32")
    want = lib_decode(f32.view(np.float32), "f32")
    same = (got == want) | (np.isnan(got) & np.isnan(want))
    if not same.all():
        fails.append("decode f32 mismatch")
    return fails


def _exact(orc, name, dtype, A, B, M, N, K, want, sa=None, sb=None) -> list:
    got = orc.gemm(dtype, A, B, M, N, K, sa, sb, nthreads=2)
    if got.shape != want.shape or not np.array_equal(got, want):
        bad = np.argwhere(~(got == want)) if got.shape == want.shape else [None]
        return [f"{name} {dtype} (M,N,K)=({M},{N},{K}): first mismatch at {bad[0]}"]
    return []


def pin_closed_forms(orc) -> list:
    fails = []
    for dtype in DTYPES:
        M, N, K = 37, 29, 70
        A, sa = random_operand(M, K, dtype, 11)
        B, sb = random_operand(K, N, dtype, 12)
        a, b = lib_decode(A, dtype), lib_decode(B, dtype)
        if dtype == "fp8":
            # unit scales: the operand values are the decoded E4M3 codes themselves
            sa, sb = unit_scales(M, K), unit_scales(K, N)
        eye = encode(np.eye(K), dtype)
        unit_kk = unit_scales(K, K) if dtype == "fp8" else None
        # A * I = A (I is K x K)
        fails += _exact(orc, "A*I", dtype, A, eye, M, K, K, a, sa, unit_kk)
        # I * B = B
        fails += _exact(orc, "I*B", dtype, eye, B, K, N, K, b, unit_kk, sb)
        # P * B = row-permuted B (P is K x K)
        perm = np.random.default_rng(3).permutation(K)
        P = np.zeros((K, K), dtype=np.float32)
        P[np.arange(K), perm] = 1.0
        fails += _exact(orc, "P*B", dtype, encode(P, dtype), B, K, N, K, b[perm],
                        unit_scales(K, K) if dtype == "fp8" else None, sb)
        # all ones -> every entry equals K
        ones_a, ones_b = encode(np.ones((M, K)), dtype), encode(np.ones((K, N)), dtype)
        fails += _exact(orc, "ones", dtype, ones_a, ones_b, M, N, K, np.full((M, N), float(K)),
                        unit_scales(M, K) if dtype == "fp8" else None,
                        unit_scales(K, N) if dtype == "fp8" else None)
        # rank-1: A[i][k] = u_i, B[k][j] = z_j -> C = K u_i z_j (dyadic, exact)
        u = np.array([((i % 9) - 4) / 8.0 for i in range(M)])
        z = np.array([((j % 7) - 3) / 4.0 for j in range(N)])
        fails += _exact(orc, "rank1", dtype, encode(np.repeat(u[:, None], K, 1), dtype),
                        encode(np.repeat(z[None, :], K, 0), dtype), M, N, K, K * np.outer(u, z),
                        unit_scales(M, K) if dtype == "fp8" else None,
                        unit_scales(K, N) if dtype == "fp8" else None)
        # K = 1: outer product of a column and a row (each product exact in fp64)
        A1, sa1 = random_operand(M, 1, dtype, 21)
        B1, sb1 = random_operand(1, N, dtype, 22)
        a1 = lib_decode(A1, dtype) * (sa1[0, 0] if dtype == "fp8" else 1.0)
        b1 = lib_decode(B1, dtype)
        if dtype == "fp8":
            b1 = b1 * np.repeat(sb1, 64, axis=1)[:, :N].astype(np.float64)
            a1 = lib_decode(A1, dtype) * np.repeat(sa1, 64, axis=0)[:M].astype(np.float64)
        fails += _exact(orc, "K=1", dtype, A1, B1, M, N, 1, a1 * b1, sa1, sb1)
        # K = 0: the empty sum
        fails += _exact(orc, "K=0", dtype, A[:, :0], B[:0], M, N, 0, np.zeros((M, N)),
                        np.zeros((-(-M // 64), 0), np.float32), np.zeros((0, -(-N // 64)), np.float32))
        # leading dimensions larger than the row: padding (NaN) is never read
        padA = np.full((M, K + 5), encode(np.array([np.nan]), dtype)[0], dtype=A.dtype)
        padA[:, :K] = A
        padB = np.full((K, N + 3), encode(np.array([np.nan]), dtype)[0], dtype=B.dtype)
        padB[:, :N] = B
        ref = orc.gemm(dtype, A, B, M, N, K, sa, sb, nthreads=1)
        got = orc.gemm(dtype, padA[:, :K], padB[:, :N], M, N, K, sa, sb, nthreads=3)
        if not np.array_equal(ref, got):
            fails.append(f"leading-dimension padding changed the result ({dtype})")
    return fails


def _bruteforce(A, B, M, N, K, dtype, sa=None, sb=None):
    a = exact_values(A, dtype, sa)
    b = exact_values(B, dtype, sb)
    return [[sum((a[i][k] * b[k][j] for k in range(K)), Fraction(0)) for j in range(N)]
            for i in range(M)], a, b


def _check_bound(name, got, exact, a, b, K) -> list:
    """|oracle - exact| <= 2 K eps64 sum|a b| (recursive-summation bound)."""
    fails = []
    eps = 2.0 ** -53
    for i in range(len(exact)):
        for j in range(len(exact[0])):
            mag = sum(abs(float(a[i][k] * b[k][j])) for k in range(K))
            err = abs(Fraction(float(got[i][j])) - exact[i][j])
            if err > Fraction(2 * K * eps * mag + 1e-300):
                fails.append(f"{name}: entry ({i},{j}) off by {float(err)!r}")
                return fails
    return fails


def pin_bruteforce(orc) -> list:
    fails = []
    shapes = [(1, 1, 1), (2, 3, 4), (5, 7, 3), (8, 8, 8), (3, 1, 6), (7, 4, 1)]
    for dtype in DTYPES:
        for t, (M, N, K) in enumerate(shapes):
            A, sa = random_operand(M, K, dtype, 100 + t)
            B, sb = random_operand(K, N, dtype, 200 + t)
            exact, a, b = _bruteforce(A, B, M, N, K, dtype, sa, sb)
            got = orc.gemm(dtype, A, B, M, N, K, sa, sb, nthreads=2)
            fails += _check_bound(f"brute {dtype} {M}x{N}x{K}", got, exact, a, b, K)
    return fails


def pin_scale_blocks(orc) -> list:
    """Several 64x64 scale blocks in every direction, distinct scales: sampled
    entries against exact rationals (which block scales which element)."""
    fails = []
    M, N, K = 150, 140, 200
    A, sa = random_operand(M, K, "fp8", 31)
    B, sb = random_operand(K, N, "fp8", 32)
    rng = np.random.default_rng(4)
    rows = rng.integers(0, M, 12)
    cols = rng.integers(0, N, 12)
    rows[:3], cols[:3] = [0, M - 1, 64], [N - 1, 0, 128]
    a = exact_values(A, "fp8", sa)
    b = exact_values(B, "fp8", sb)
    full = orc.gemm("fp8", A, B, M, N, K, sa, sb, nthreads=4)
    ent = orc.gemm_entries("fp8", A, B, M, N, K, rows, cols, sa, sb)
    for t, (i, j) in enumerate(zip(rows, cols)):
        exact = sum((a[i][k] * b[k][j] for k in range(K)), Fraction(0))
        mag = sum(abs(float(a[i][k] * b[k][j])) for k in range(K))
        tol = Fraction(2 * K * 2.0 ** -53 * mag)
        for name, val in (("gemm", full[i, j]), ("entries", ent[t])):
            if abs(Fraction(float(val)) - exact) > tol:
                fails.append(f"fp8 scale blocks {name}: entry ({i},{j})")
    return fails


def pin_entries(orc) -> list:
    """The per-entry path against exact rationals, every dtype, with ld > row."""
    fails = []
    for t, dtype in enumerate(("f16", "bf16", "f32")):
        M, N, K = 9, 11, 13
        A, _ = random_operand(M, K + 3, dtype, 300 + t)
        B, _ = random_operand(K, N + 2, dtype, 400 + t)
        A, B = A[:, :K], B[:, :N]
        a = exact_values(np.ascontiguousarray(A), dtype, None)
        b = exact_values(np.ascontiguousarray(B), dtype, None)
        rows = np.array([0, 8, 3, 5]); cols = np.array([10, 0, 7, 2])
        got = orc.gemm_entries(dtype, A, B, M, N, K, rows, cols)
        for s, (i, j) in enumerate(zip(rows, cols)):
            exact = sum((a[i][k] * b[k][j] for k in range(K)), Fraction(0))
            mag = sum(abs(float(a[i][k] * b[k][j])) for k in range(K))
            if abs(Fraction(float(got[s])) - exact) > Fraction(2 * K * 2.0 ** -53 * mag):
                fails.append(f"entries {dtype} ({i},{j})")
    return fails


def pin_tolerance_checker(orc) -> list:
    fails = []
    ref = np.array([0.0, 1.0, -2.0, 100.0])
    inside = 0.999 * np.array([1e-3, 1e-3 + 1e-3, -(2e-3 + 1e-3), 0.1 + 1e-3])
    ok, n, _, _ = orc.within_tolerance(ref + inside, ref, 1e-3, 1e-3)
    if not ok or n:
        fails.append("tolerance: boundary values rejected")
    ok, n, _, _ = orc.within_tolerance(ref + np.array([0, 0, 0, 0.1 + 2e-3]), ref, 1e-3, 1e-3)
    if ok or n != 1:
        fails.append("tolerance: out-of-bound value accepted")
    for bad in (np.nan, np.inf, -np.inf):
        ok, n, _, _ = orc.within_tolerance(np.array([0.0, bad, 1.0, 100.0]), ref, 1.0, 1.0)
        if ok:
            fails.append(f"tolerance: {bad} accepted")
    return fails


# ------------------------------------------------------------- FP8 quantiser

FP8_TORCH = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}
FP8_MAX = {"e4m3": 448.0, "e5m2": 57344.0}


def torch_fp8_table(fmt: str):
    """(codes, values) of every finite code, decoded by torch."""
    codes = np.arange(256, dtype=np.uint8)
    vals = torch.from_numpy(codes).view(FP8_TORCH[fmt]).to(torch.float64).numpy()
    fin = np.isfinite(vals)
    return codes[fin], vals[fin]


def brute_nearest(y: np.ndarray, fmt: str) -> np.ndarray:
    """Nearest finite FP8 code by exhaustive search, ties to the even code, the
    sign of y kept for zero results."""
    codes, vals = torch_fp8_table(fmt)
    out = np.empty(y.shape, dtype=np.uint8)
    for t, v in enumerate(np.asarray(y, dtype=np.float64).ravel()):
        d = np.abs(vals - v)
        best = d.min()
        cand = codes[d == best]
        cand = cand[[bool(np.signbit(vals[codes.tolist().index(c)]) == np.signbit(v)) or
                     vals[codes.tolist().index(c)] != 0 for c in cand]]
        even = [c for c in cand if c % 2 == 0]
        out.flat[t] = (even or list(cand))[0]
    return out


def pin_fp8_encode(orc) -> list:
    fails = []
    rng = np.random.default_rng(11)
    for fmt in ("e4m3", "e5m2"):
        codes, vals = torch_fp8_table(fmt)
        # every finite code decodes like torch and encodes back to itself
        d = orc.decode(np.arange(256, dtype=np.uint8), fmt)
        t = torch.from_numpy(np.arange(256, dtype=np.uint8)).view(FP8_TORCH[fmt]).to(torch.float64).numpy()
        if not np.all((d == t) | (np.isnan(d) & np.isnan(t))):
            fails.append(f"{fmt}: decoder differs from torch")
        if not np.array_equal(orc.fp8_encode(vals.astype(np.float32), fmt), codes):
            fails.append(f"{fmt}: a finite value does not encode to its own code")
        # midpoints between neighbouring values and their fp32 neighbours
        pos = np.unique(vals[vals >= 0])
        mids = (pos[:-1] + pos[1:]) / 2
        y = np.concatenate([mids, np.nextafter(mids.astype(np.float32), np.float32(0)),
                            np.nextafter(mids.astype(np.float32), np.float32(np.inf)).astype(np.float64)])
        y = np.concatenate([y, -y, [pos[1] / 4, -pos[1] / 4, -0.0]]).astype(np.float32)
        want = brute_nearest(y, fmt)
        got = orc.fp8_encode(y, fmt)
        bad = np.nonzero(got != want)[0]
        if bad.size:
            fails.append(f"{fmt}: midpoint rounding of {y[bad[0]]!r} gave {got[bad[0]]:#x}, want {want[bad[0]]:#x}")
        # random values within range agree with torch's cast (round to nearest even)
        r = (rng.standard_normal(20000) * rng.choice([1e-3, 1.0, 30.0], 20000)).astype(np.float32)
        r = np.clip(r, -FP8_MAX[fmt], FP8_MAX[fmt]).astype(np.float32)
        tc = torch.from_numpy(r).to(FP8_TORCH[fmt]).view(torch.uint8).numpy()
        if not np.array_equal(orc.fp8_encode(r, fmt), tc):
            fails.append(f"{fmt}: random values differ from torch's cast")
    return fails


def _lib_quantize(x: np.ndarray, block: int, fmt: str):
    """Block quantiser from library pieces: numpy amax / fp32 divide / clip and
    torch's FP8 cast for the rounding."""
    rows, cols = x.shape
    br, bc = -(-rows // block), -(-cols // block)
    S = np.empty((br, bc), np.float32)
    y = np.empty_like(x)
    F = np.float32(FP8_MAX[fmt])
    for i in range(br):
        for j in range(bc):
            blk = x[i * block:(i + 1) * block, j * block:(j + 1) * block]
            amax = np.abs(blk).max()
            s = np.float32(amax / F) if amax > 0 else np.float32(1.0)
            S[i, j] = s
            y[i * block:(i + 1) * block, j * block:(j + 1) * block] = np.clip(blk / s, -F, F)
    q = torch.from_numpy(np.ascontiguousarray(y)).to(FP8_TORCH[fmt]).view(torch.uint8).numpy()
    return q, S


def pin_quantize_fp8(orc) -> list:
    fails = []
    rng = np.random.default_rng(12)
    # 1. the independent input recipe (E4M3) and the library-piece quantiser
    for (rows, cols), block in (((100, 130), 64), ((70, 33), 32), ((64, 64), 64), ((1, 1), 32)):
        x = rng.standard_normal((rows, cols)).astype(np.float32)
        q, S = orc.quantize_fp8(x, "f32", block, "e4m3")
        q2, S2 = gi.blockscale_e4m3(x, block)
        if not (np.array_equal(q, q2) and np.array_equal(S, S2)):
            fails.append(f"quantize e4m3 {rows}x{cols}/{block}: differs from the input recipe")
        for fmt in ("e4m3", "e5m2"):
            q, S = orc.quantize_fp8(x * np.float32(1000.0), "f32", block, fmt)
            q3, S3 = _lib_quantize(x * np.float32(1000.0), block, fmt)
            if not (np.array_equal(q, q3) and np.array_equal(S, S3)):
                fails.append(f"quantize {fmt} {rows}x{cols}/{block}: differs from library pieces")
    # 2. block position: block (i, j) = base * 2^(i + 3j) on a 3 x 5 grid
    for block in (32, 64):
        base = rng.standard_normal((block, block)).astype(np.float32)
        x = np.block([[base * np.float32(2.0 ** (i + 3 * j)) for j in range(5)] for i in range(3)])
        x = np.ascontiguousarray(x[: 3 * block - 5, : 5 * block - 7])   # ragged last blocks
        q, S = orc.quantize_fp8(x, "f32", block, "e4m3")
        want = S[0, 0] * np.array([[2.0 ** (i + 3 * j) for j in range(5)] for i in range(3)])
        if not np.array_equal(S[:2, :4].astype(np.float64), want[:2, :4]):
            fails.append(f"block {block}: scales do not follow the block positions")
        if not np.array_equal(q[:block, :block], q[block:2 * block, 3 * block:4 * block]):
            fails.append(f"block {block}: equal blocks quantised differently")
    # 3. exact-midpoint quotients: x = s * m with m halfway between two FP8 values
    #    and s = amax / 448 exact, so x / s = m exactly and must round to the even code
    for sc in (3.0, 5.0, 7.0, 11.0):
        codes, vals = torch_fp8_table("e4m3")
        pos = np.unique(vals[vals > 0])
        mids = ((pos[:-1] + pos[1:]) / 2)[8:60]
        m = np.stack([np.concatenate([[448.0], mids]), np.concatenate([[-448.0], -mids])])
        x = np.ascontiguousarray((m * sc).astype(np.float32))    # 2 x 53: one 64x64 block
        q, S = orc.quantize_fp8(x, "f32", 64, "e4m3")
        if S.shape != (1, 1) or S[0, 0] != np.float32(sc):
            fails.append(f"midpoints: scale {S.ravel()[0]} != {sc}")
        want = brute_nearest(m, "e4m3")
        bad = np.argwhere(q != want)
        if bad.size:
            r, c = bad[0]
            fails.append(f"midpoints x{sc}: element {r},{c} rounded to {q[r, c]:#x}, want {want[r, c]:#x}")
    # 4. padding beyond the columns is never read; zero blocks get scale 1
    x = np.full((40, 80), 1e30, np.float32)
    x[:, :70] = rng.standard_normal((40, 70)).astype(np.float32)
    x[:, 64:70] = 0.0
    x[33:, :] = 1e30
    q, S = orc.quantize_fp8(x[:33, :70], "f32", 32, "e4m3")
    q_ref, S_ref = orc.quantize_fp8(np.ascontiguousarray(x[:33, :70]), "f32", 32, "e4m3")
    if not (np.array_equal(q, q_ref) and np.array_equal(S, S_ref)) or not np.all(np.isfinite(S)):
        fails.append("quantize reads past the columns it was given")
    if S[0, 2] != 1.0 or np.any(q[:32, 64:70] != 0):
        fails.append("a block of zeros must get scale 1 and +0 codes")
    # 5. invariants: the amax element lands on +-F; reconstruction error bound
    for fmt, mb in (("e4m3", 3), ("e5m2", 2)):
        x = (rng.standard_normal((96, 96)) * 10).astype(np.float32)
        q, S = orc.quantize_fp8(x, "f32", 32, fmt)
        dq = orc.decode(q, fmt)
        for i in range(3):
            for j in range(3):
                b = dq[32 * i:32 * i + 32, 32 * j:32 * j + 32]
                if np.abs(b).max() != FP8_MAX[fmt]:
                    fails.append(f"{fmt}: block ({i},{j}) largest code is not +-{FP8_MAX[fmt]}")
        rec = dq * np.kron(S.astype(np.float64), np.ones((32, 32)))
        sub = 2.0 ** (-9 if fmt == "e4m3" else -16)
        bound = np.abs(x) * 2.0 ** -(mb + 1) * (1 + 1e-6) + np.kron(S, np.ones((32, 32))) * sub
        if np.any(np.abs(rec - x) > bound):
            fails.append(f"{fmt}: reconstruction error beyond half a step")
    # 6. bf16 input = fp32 input of the same values
    xb = gi.uniform_h16(50, 70, 13, "bf16")
    xf = np.ascontiguousarray(lib_decode(xb, "bf16").astype(np.float32) * np.float32(4.0))
    xb3 = gi.to_bf16_bits(xf)
    qa, Sa = orc.quantize_fp8(xb3, "bf16", 64, "e4m3")
    qb, Sb = orc.quantize_fp8(xf, "f32", 64, "e4m3")
    if not (np.array_equal(qa, qb) and np.array_equal(Sa, Sb)):
        fails.append("bf16 input differs from fp32 input of the same values")
    return fails


# ------------------------------------------------------------ fused epilogue

_NAN_BITS = {"f16": 0x7E00, "bf16": 0x7FC0}


def _prior(out: str, vals: np.ndarray, ldc: int) -> np.ndarray:
    """C's bits before the call: `vals` (exactly representable) in the first
    columns, NaN in the padding up to ldc (a reader that ignores ldc picks it up)."""
    M, N = vals.shape
    if out == "f32":
        buf = np.full((M, ldc), np.nan, dtype=np.float32)
        buf[:, :N] = vals
    else:
        buf = np.full((M, ldc), _NAN_BITS[out], dtype=np.uint16)
        buf[:, :N] = encode(vals, out)
    return buf


def pin_epilogue(orc) -> list:
    """act(alpha * A*B + beta * C_prior + bias[j]) on structured inputs whose
    results follow in closed form (worked out by hand, below), for every output
    type: all-ones products (every entry = K), per-column bias, a prior C that
    varies with row and column and sits in a padded buffer, relu thresholds on
    either side of zero, and a NaN-filled prior that must not be read when
    beta = 0."""
    fails = []
    M, N, K = 5, 7, 9
    i = np.arange(M, dtype=np.float64)[:, None]
    j = np.arange(N, dtype=np.float64)[None, :]
    for out in ("f16", "bf16", "f32"):
        op = "f32" if out == "f32" else out
        ones_a, ones_b = encode(np.ones((M, K)), op), encode(np.ones((K, N)), op)
        prod = orc.gemm(op, ones_a, ones_b, M, N, K)              # = K everywhere
        prior_vals = (i - 2.0 * j) + 0.375                        # exact in every type
        prior = _prior(out, prior_vals, N + 3)
        bias = (np.arange(N) / 4.0).astype(np.float32)
        cases = [
            # alpha * K + beta * (i - 2j + 3/8) + j/4 with alpha = 2, beta = -1/2:
            # 18 - i/2 + j - 3/16 + j/4
            ("scales, prior, bias", dict(alpha=2.0, beta=-0.5, c_prior=prior, bias=bias),
             18.0 - 0.5 * i + 1.25 * j - 0.1875),
            # no prior read: alpha = 1/2 -> K/2 + j/4
            ("bias only", dict(alpha=0.5, bias=bias), 4.5 + 0.25 * j + 0 * i),
            # relu after the bias: v = K + (j - 3 - K) = j - 3
            ("relu after bias", dict(bias=(np.arange(N) - 3.0 - K).astype(np.float32),
                                     act="relu"), np.maximum(j - 3.0, 0.0) + 0 * i),
            # relu of a negated product: v = -K + (K + 1 - j) = 1 - j
            ("relu, negative alpha", dict(alpha=-1.0, bias=(K + 1.0 - np.arange(N))
                                          .astype(np.float32), act="relu"),
             np.maximum(1.0 - j, 0.0) + 0 * i),
            # beta = 0: a NaN-filled C must not be read
            ("beta 0 ignores C", dict(alpha=1.0, beta=0.0,
                                      c_prior=_prior(out, np.full((M, N), np.nan), N)),
             np.full((M, N), float(K))),
            # only the prior: alpha = 0, beta = 4 -> 4i - 8j + 3/2
            ("prior only", dict(alpha=0.0, beta=4.0, c_prior=prior),
             4.0 * i - 8.0 * j + 1.5),
        ]
        for name, kw, want in cases:
            got = orc.epilogue(out, prod, **kw)
            if not np.array_equal(got, want):
                bad = np.argwhere(got != want)[0]
                fails.append(f"epilogue {out} {name}: at {tuple(bad)} got "
                             f"{got[tuple(bad)]} want {want[tuple(bad)]}")
        # identity settings leave any product unchanged
        rnd = orc.gemm(op, *[random_operand(r, c, op, s)[0] for r, c, s in
                             ((M, K, 11), (K, N, 12))], M, N, K)
        if not np.array_equal(orc.epilogue(out, rnd), rnd):
            fails.append(f"epilogue {out}: alpha=1, beta=0, no bias, no act changed the product")
    return fails


# ------------------------------------------------------------ convolution

CONV_CASES = [
    # n, h, w, c_in, c_out, kh, kw, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w
    dict(n=2, h=7, w=6, c_in=3, c_out=5, kh=3, kw=3, pad_h=1, pad_w=1),
    dict(n=1, h=9, w=11, c_in=4, c_out=2, kh=3, kw=2, stride_h=2, stride_w=3, pad_h=2, pad_w=0),
    dict(n=3, h=8, w=8, c_in=2, c_out=3, kh=2, kw=3, dil_h=2, dil_w=3, pad_h=1, pad_w=2),
    dict(n=1, h=5, w=4, c_in=6, c_out=4, kh=1, kw=1),
    dict(n=2, h=10, w=7, c_in=3, c_out=2, kh=7, kw=5, stride_h=2, stride_w=2, pad_h=3, pad_w=2),
]


def _torch_conv(xv, wv, g):
    """torch's float64 CPU conv2d on decoded NHWC / HWIO values (the library
    routine the oracle's convolution must agree with)."""
    n, h, w, ci, co, kh, kw, sh, sw, ph, pw, dh, dw = (int(v) for v in g)
    x = torch.from_numpy(xv.reshape(n, h, w, ci)).permute(0, 3, 1, 2)
    wt = torch.from_numpy(wv.reshape(kh, kw, ci, co)).permute(3, 2, 0, 1)
    y = torch.nn.functional.conv2d(x, wt, stride=(sh, sw), padding=(ph, pw), dilation=(dh, dw))
    return y.permute(0, 2, 3, 1).numpy()


def pin_conv(orc) -> list:
    """The direct convolution against torch's conv2d (float64, CPU) on random
    operands of every type over strides, paddings and dilations; closed forms:
    a centred delta kernel returns the input, a corner delta kernel shifts it
    by the padding, all-ones counts the taps inside the image, and a 1x1
    convolution is exactly the GEMM of the pixels by the weights."""
    fails = []
    for ci_, case in enumerate(CONV_CASES):
        g = orc.conv_geom(**case)
        n, h, w, ci, co, kh, kw = (int(v) for v in g[:7])
        for dtype in ("f16", "bf16", "f32"):
            X = random_operand(n * h * w, ci, dtype, 300 + ci_)[0]
            W = random_operand(kh * kw * ci, co, dtype, 400 + ci_)[0]
            got = orc.conv2d_nhwc(dtype, X, W, g)
            want = _torch_conv(lib_decode(X, dtype), lib_decode(W, dtype), g)
            if got.shape != want.shape or not np.allclose(got, want, rtol=1e-12, atol=1e-12):
                fails.append(f"conv {dtype} {case}: differs from torch conv2d")
    # closed forms (f32 operands; all values exact)
    n, h, w, c = 2, 5, 6, 3
    X = random_operand(n * h * w, c, "f32", 500)[0]
    xv = X.reshape(n, h, w, c).astype(np.float64)
    delta = np.zeros((3, 3, c, c), np.float32)
    delta[1, 1] = np.eye(c)
    y = orc.conv2d_nhwc("f32", X, delta, orc.conv_geom(n=n, h=h, w=w, c_in=c, c_out=c, kh=3,
                                                       kw=3, pad_h=1, pad_w=1))
    if not np.array_equal(y, xv):
        fails.append("conv: centred delta kernel does not return the input")
    corner = np.zeros((3, 3, c, c), np.float32)
    corner[0, 0] = np.eye(c)
    y = orc.conv2d_nhwc("f32", X, corner, orc.conv_geom(n=n, h=h, w=w, c_in=c, c_out=c, kh=3,
                                                        kw=3, pad_h=1, pad_w=1))
    shifted = np.zeros_like(xv)
    shifted[:, 1:, 1:, :] = xv[:, :-1, :-1, :]          # Y[oh][ow] = X[oh-1][ow-1]
    if not np.array_equal(y, shifted):
        fails.append("conv: corner delta kernel is not a shift by the padding")
    ones = orc.conv2d_nhwc("f32", np.ones((n * h * w, c), np.float32),
                           np.ones((3, 3, c, 2), np.float32),
                           orc.conv_geom(n=n, h=h, w=w, c_in=c, c_out=2, kh=3, kw=3, pad_h=1,
                                         pad_w=1))
    rows_in = np.array([2] + [3] * (h - 2) + [2])       # taps inside along each axis
    cols_in = np.array([2] + [3] * (w - 2) + [2])
    want = (rows_in[:, None] * cols_in[None, :] * c).astype(np.float64)
    if not all(np.array_equal(ones[b, :, :, o], want) for b in range(n) for o in range(2)):
        fails.append("conv: all-ones does not count the taps inside the image")
    W1 = random_operand(c, 4, "f32", 501)[0]
    y = orc.conv2d_nhwc("f32", X, W1, orc.conv_geom(n=n, h=h, w=w, c_in=c, c_out=4, kh=1, kw=1))
    if not np.array_equal(y.reshape(n * h * w, 4), orc.gemm("f32", X, W1, n * h * w, 4, c)):
        fails.append("conv: 1x1 convolution differs from the GEMM")
    return fails


def pin_im2col(orc) -> list:
    """The im2col matrix against torch's unfold (pure data movement, so exact),
    reordered from unfold's (channel, kh, kw) columns to (kh, kw, channel), and
    the 1x1 / stride 1 / no padding case, where it is the input itself."""
    fails = []
    for ci_, case in enumerate(CONV_CASES):
        g = orc.conv_geom(**case)
        n, h, w, ci, co, kh, kw, sh, sw, ph, pw, dh, dw = (int(v) for v in g)
        for dtype in ("bf16", "f32"):
            X = random_operand(n * h * w, ci, dtype, 600 + ci_)[0]
            got = orc.im2col_nhwc(X, g)
            x = torch.from_numpy(lib_decode(X, dtype).reshape(n, h, w, ci)).permute(0, 3, 1, 2)
            u = torch.nn.functional.unfold(x, (kh, kw), dilation=(dh, dw), padding=(ph, pw),
                                           stride=(sh, sw))            # (n, ci*kh*kw, L)
            L = u.shape[2]
            u = u.reshape(n, ci, kh, kw, L).permute(0, 4, 2, 3, 1).reshape(n * L, kh * kw * ci)
            if got.shape != tuple(u.shape) or not np.array_equal(lib_decode(got, dtype), u.numpy()):
                fails.append(f"im2col {dtype} {case}: differs from torch unfold")
    X = random_operand(30, 5, "bf16", 610)[0]
    if not np.array_equal(orc.im2col_nhwc(X, orc.conv_geom(n=2, h=3, w=5, c_in=5, c_out=1,
                                                           kh=1, kw=1)), X):
        fails.append("im2col: 1x1 case is not the input")
    return fails


ALL_PINS = (pin_decoders, pin_closed_forms, pin_bruteforce, pin_scale_blocks, pin_entries,
            pin_tolerance_checker, pin_fp8_encode, pin_quantize_fp8, pin_epilogue,
            pin_conv, pin_im2col)


def run_all(orc) -> list:
    fails = []
    for pin in ALL_PINS:
        try:
            fails += pin(orc)
        except Exception as e:  # a planted mistake may also make the oracle refuse
            fails.append(f"{pin.__name__} raised {type(e).__name__}: {e}")
    return fails
