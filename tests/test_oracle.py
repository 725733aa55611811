"""CPU oracle against its pins (decoders, closed forms, exact brute force), plus
mutation tests: a mistake planted in a copy of oracle.c must make a pin fail."""
import os
import subprocess
import sys
import tempfile

import numpy as np
import pytest

import oracle_pins as pins

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def test_decoders_exhaustive(orc):
    assert pins.pin_decoders(orc) == []


def test_closed_forms(orc):
    assert pins.pin_closed_forms(orc) == []


def test_bruteforce_exact_rationals(orc):
    assert pins.pin_bruteforce(orc) == []


def test_fp8_scale_blocks(orc):
    assert pins.pin_scale_blocks(orc) == []


def test_entries_path(orc):
    assert pins.pin_entries(orc) == []


def test_tolerance_checker(orc):
    assert pins.pin_tolerance_checker(orc) == []


def test_fp8_encoder(orc):
    assert pins.pin_fp8_encode(orc) == []


def test_fp8_quantiser(orc):
    assert pins.pin_quantize_fp8(orc) == []


def test_epilogue(orc):
    assert pins.pin_epilogue(orc) == []


def test_conv(orc):
    assert pins.pin_conv(orc) == []


def test_im2col(orc):
    assert pins.pin_im2col(orc) == []


def test_thread_count_does_not_change_result(orc):
    import gemm_inputs as gi
    A = gi.uniform_h16(67, 45, 1, "bf16")
    B = gi.uniform_h16(45, 53, 2, "bf16")
    r1 = orc.gemm("bf16", A, B, 67, 53, 45, nthreads=1)
    r7 = orc.gemm("bf16", A, B, 67, 53, 45, nthreads=7)
    assert np.array_equal(r1, r7)


def test_bad_arguments_rejected(orc):
    A = np.zeros((4, 4), np.uint16)
    with pytest.raises(RuntimeError):
        orc.gemm_entries("bf16", A, A, 4, 4, 4, np.array([4]), np.array([0]))
    with pytest.raises(ValueError):
        orc.gemm("fp8", A.astype(np.uint8), A.astype(np.uint8), 4, 4, 4,
                 np.ones((2, 2), np.float32), np.ones((1, 1), np.float32))


# (original text, planted mistake): each is a plausible slip in the oracle.
MUTANTS = {
    "sign": ("ci[j] = ci[j] + aik * bk[j]", "ci[j] = ci[j] - aik * bk[j]"),
    "dropped_last_term": ("kk < job->k; kk++", "kk + 1 < job->k; kk++"),
    "b_row_index": ("job->b + kk * job->n", "job->b + kk"),
    "a_index": ("job->a[i * job->k + kk]", "job->a[i * job->k]"),
    "no_zero_init": ("for (int64_t j = 0; j < job->n; j++) ci[j] = 0.0;", ""),
    "f16_exponent": ("e - 25);", "e - 24);"),
    "f16_subnormal": ("ldexp((double)f, -24)", "ldexp((double)f, -25)"),
    "bf16_exponent": ("e - 134);", "e - 133);"),
    "bf16_subnormal": ("ldexp((double)f, -133)", "ldexp((double)f, -126)"),
    "e4m3_nan_rule": ("if (e == 15 && m == 7)", "if (e == 15)"),
    "e4m3_subnormal": ("ldexp((double)m, -9)", "ldexp((double)m, -10)"),
    "f32_exponent": ("e - 150);", "e - 149);"),
    "scale_not_applied": ("* orc_f32_to_f64(sbits)", ""),
    "scale_grid_transposed": ("(r / ORC_SCALE_BLOCK) * scale_cols + (c / ORC_SCALE_BLOCK)",
                              "(c / ORC_SCALE_BLOCK) * scale_cols + (r / ORC_SCALE_BLOCK)"),
    "scale_block_32": ("#define ORC_SCALE_BLOCK 64", "#define ORC_SCALE_BLOCK 32"),
    "entries_wrong_scale_cols": ("int64_t sb_cols = (N + ORC_SCALE_BLOCK",
                                 "int64_t sb_cols = (K + ORC_SCALE_BLOCK"),
    # FP8 quantiser
    "e5m2_decoder_bias": ("ldexp((double)(4 | m), e - 17)", "ldexp((double)(4 | m), e - 16)"),
    "encode_ties_away": ("double n = rint(a / quantum);", "double n = floor(a / quantum + 0.5);"),
    "encode_truncates": ("double n = rint(a / quantum);", "double n = floor(a / quantum);"),
    "encode_no_binade_carry": ("if (n >= ldexp(1.0, mbits + 1)) {", "if (0) {"),
    "encode_sign_dropped": ("signbit(y) ? 0x80 : 0", "0"),
    "quant_scale_wrong_max": ("fmt == ORC_FP8_E4M3 ? 448.0f : 57344.0f;",
                              "fmt == ORC_FP8_E4M3 ? 240.0f : 57344.0f;"),
    "quant_multiplies": ("input_f32(dtype, X, ldx, r, c) / s;", "input_f32(dtype, X, ldx, r, c) * s;"),
    "quant_scale_grid_transposed": ("scales[bi * bc + bj] = s;", "scales[bj * br + bi] = s;"),
    "quant_amax_signed": ("const float a = fabsf(input_f32(dtype, X, ldx, r, c));",
                          "const float a = input_f32(dtype, X, ldx, r, c);"),
    "quant_zero_scale": ("amax > 0.0f ? amax / fmax : 1.0f", "amax > 0.0f ? amax / fmax : 0.5f"),
    # fused epilogue
    "epi_alpha_dropped": ("double v = alpha * prod[i * N + j];", "double v = prod[i * N + j];"),
    "epi_beta_sign": ("v = v + beta * operand_at", "v = v - beta * operand_at"),
    "epi_prior_read_when_beta_zero": ("if (beta != 0.0) v = v + beta", "v = v + beta"),
    "epi_prior_ignores_ldc": ("operand_at(out_dtype, c_bits, ldc, i, j",
                              "operand_at(out_dtype, c_bits, N, i, j"),
    "epi_prior_wrong_type": ("operand_at(out_dtype, c_bits", "operand_at(ORC_BF16, c_bits"),
    "epi_bias_by_row": ("memcpy(&bbits, &bias[j], 4);", "memcpy(&bbits, &bias[i], 4);"),
    "epi_relu_is_abs": ("if (act == 1 && !(v > 0.0)) v = 0.0;", "if (act == 1 && !(v > 0.0)) v = -v;"),
    "epi_relu_before_bias": ("""            if (bias) {
                uint32_t bbits;
                memcpy(&bbits, &bias[j], 4);
                v = v + orc_f32_to_f64(bbits);
            }
            if (act == 1 && !(v > 0.0)) v = 0.0;""", """            if (act == 1 && !(v > 0.0)) v = 0.0;
            if (bias) {
                uint32_t bbits;
                memcpy(&bbits, &bias[j], 4);
                v = v + orc_f32_to_f64(bbits);
            }"""),
    # convolution and im2col
    "conv_dilation_ignored": ("const int64_t ih = oh * SH - PH + kh * DH;",
                              "const int64_t ih = oh * SH - PH + kh;"),
    "conv_stride_ignored": ("const int64_t iw = ow * SW - PW + kw * DW;",
                            "const int64_t iw = ow - PW + kw * DW;"),
    "conv_padding_sign": ("const int64_t ih = oh * SH - PH + kh * DH;",
                          "const int64_t ih = oh * SH + PH + kh * DH;"),
    "conv_weight_taps_swapped": ("Wt, CO, (kh * KW + kw) * CI + ci", "Wt, CO, (kw * KH + kh) * CI + ci"),
    "conv_no_zero_padding": ("if (ih >= 0 && ih < H && iw >= 0 && iw < W)\n",
                             "if (ih >= 0 && iw >= 0 && (n * H + ih) * W + iw < N * H * W)\n"),
    "conv_output_size_floor": ("*ho = eh < 0 ? 0 : eh / g[7] + 1;", "*ho = eh < 0 ? 0 : (eh + g[7] - 1) / g[7] + 1;"),
    "im2col_channel_major": ("row * ldcol + (kh * KW + kw) * CI + ci;",
                             "row * ldcol + (ci * KH + kh) * KW + kw;"),
    "im2col_no_zero_fill": ("inside ? ((const uint16_t *)X)[src] : 0", "((const uint16_t *)X)[src < 0 ? 0 : src]"),
}

_RUNNER = r"""
import ctypes, sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import oracle, oracle_pins
oracle._lib = oracle.bind(ctypes.CDLL({lib!r}))
fails = oracle_pins.run_all(oracle)
print("PIN_FAILURES", len(fails))
for f in fails[:3]: print(f)
"""


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    src = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    old, new = MUTANTS[name]
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mutated = src.replace(old, new)
    with tempfile.TemporaryDirectory() as d:
        c_path, so_path = os.path.join(d, "m.c"), os.path.join(d, "libm.so")
        open(c_path, "w").write(mutated)
        subprocess.run(["gcc", "-O1", "-ffp-contract=off", "-fPIC", "-shared", "-pthread",
                        c_path, "-o", so_path, "-lm"], check=True)
        r = subprocess.run([sys.executable, "-c",
                            _RUNNER.format(root=ROOT, tests=HERE, lib=so_path)],
                           capture_output=True, text=True, timeout=300)
    out = r.stdout + r.stderr
    if r.returncode != 0:
        # the planted mistake crashed the oracle: detected, loudly
        return
    n = int(out.split("PIN_FAILURES")[1].split()[0])
    assert n > 0, f"planted mistake {name} passed every pin:\n{out}"
