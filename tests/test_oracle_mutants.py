"""The oracle's pins are strong enough to catch plausible mistakes.

Each case plants one mistake in a copy of oracle/hbl_oracle.c (a dropped
term, a wrong sign, index or constant, a transposed operand, another rounding
mode, a misplaced epsilon), builds that copy with the oracle's own compiler
flags, and runs tests/test_oracle_pins.py against it in a fresh process
(HBL_ORACLE_SO selects the library): at least one pin must fail.  The
unmodified source, built the same way, must pass every pin.  CPU only.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "hbl_oracle.c")

# (name, text in the source, replacement)
MUTANTS = [
    ("ternary_round_half_away", "float r = rintf(t);\n        if (r > 1.0f) r = 1.0f;",
     "float r = roundf(t);\n        if (r > 1.0f) r = 1.0f;"),
    ("codes_round_half_away", "float r = rintf(t);\n        if (r > hi) r = hi;",
     "float r = roundf(t);\n        if (r > hi) r = hi;"),
    ("alpha_without_abs", "for (int64_t i = 0; i < count; i++) s += fabs((double)W[i]);",
     "for (int64_t i = 0; i < count; i++) s += (double)W[i];"),
    ("weight_eps_dropped", "float den = alpha + eps;", "float den = alpha;"),
    ("act_eps_dropped", "float den = stat + eps;", "float den = stat;"),
    ("dequant_factor_wrong", "*d_out = stat / num;", "*d_out = stat / (num + 1.0f);"),
    ("hadamard_index_reversed", "(unsigned long long)(i & j)", "(unsigned long long)(i & (K - 1 - j))"),
    ("hadamard_sign_flipped", "acc += (odd ? -1.0 : 1.0) * r[j];", "acc += (odd ? 1.0 : -1.0) * r[j];"),
    ("hadamard_scale_missing", "z[i] = acc * inv;", "z[i] = acc;"),
    ("absmax_without_abs", "float a = fabsf(z[k]);", "float a = z[k];"),
    ("absmean_over_k_minus_1", "stat = (float)(s / (double)K);", "stat = (float)(s / (double)(K - 1));"),
    ("sqrt7_one_ulp_off", "v.u = 0x402953FDu;", "v.u = 0x402953FEu;"),
    ("int4_clip_symmetric", "lo = -8.0f; hi = 7.0f;", "lo = -7.0f; hi = 7.0f;"),
    ("int8_clip_narrow", "lo = -128.0f; hi = 127.0f;", "lo = -127.0f; hi = 126.0f;"),
    ("ternary_pack_field", "return (int)(2 * ((k % 16) / 4));", "return (int)(2 * (k % 4));"),
    ("ternary_pack_byte", "return 4 * (k / 16) + (k % 4);", "return 4 * (k / 16) + ((k / 4) % 4);"),
    ("int4_nibbles_swapped", "p[m * (K / 2) + k2] = (uint8_t)(lo | (hi << 4));",
     "p[m * (K / 2) + k2] = (uint8_t)(hi | (lo << 4));"),
    ("gemm_operand_transposed", "(int64_t)Wq[n * K + k]", "(int64_t)Wq[k * N + n]"),
    ("norm_eps_outside_sqrt", "double den = sqrt(ss / (double)K + (double)eps);",
     "double den = sqrt(ss / (double)K) + (double)eps;"),
    ("norm_gain_dropped", "r[k] = v * (gain ? (double)gain[k] : 1.0);", "r[k] = v;"),
    ("layernorm_mean_wrong", "mu /= (double)K;", "mu /= (double)(K - 1);"),
    ("rescale_without_d", "float t = (float)acc[m * N + n] * d[m];", "float t = (float)acc[m * N + n];"),
    ("rescale_without_alpha", "y[m * N + n] = t * alpha;", "y[m * N + n] = t;"),
    ("heads_eps_dropped", "const float s = gamma == 0.f ? 0.f : (float)qp / den;",
     "const float s = gamma == 0.f ? 0.f : (float)qp / gamma;"),
    ("heads_absmax_without_abs", "const float a = fabsf(x[j]);", "const float a = x[j];"),
    ("heads_round_half_away", "const int u = (int)rintf(t) + zp;", "const int u = (int)roundf(t) + zp;"),
    ("heads_zero_point_off", "const int zp = 1 << (bits - 1), qp = zp - 1;",
     "const int zp = (1 << (bits - 1)) - 1, qp = zp;"),
    ("heads_3bit_order_reversed", "if ((u >> b) & 1) out[(3 * j + b) / 8]", "if ((u >> (2 - b)) & 1) out[(3 * j + b) / 8]"),
    ("heads_nibbles_swapped", "out[j / 2] |= (uint8_t)(u << (4 * (j % 2)));",
     "out[j / 2] |= (uint8_t)(u << (4 * (1 - j % 2)));"),
    ("backward_alpha_dropped", "dz[k] = (double)alpha * acc;", "dz[k] = acc;"),
    ("backward_gemm_transposed", "acc += (double)dY[m * N + n] * (double)Wq[n * K + k];",
     "acc += (double)dY[m * N + n] * (double)Wq[k * N + n];"),
    ("backward_hadamard_skipped", "if (hadamard) hbo_hadamard_row(dz, K, dr);", "if (0) hbo_hadamard_row(dz, K, dr);"),
    ("backward_rms_c_cubed_wrong", "- c * c * c / (double)K * (double)x[k] * t;", "- c * c / (double)K * (double)x[k] * t;"),
    ("backward_ln_mean_term_dropped", "out[k] = c * (a - ma - ((double)x[k] - mu) * c * max_);",
     "out[k] = c * (a - ((double)x[k] - mu) * c * max_);"),
    ("backward_none_gain_dropped", "for (int64_t k = 0; k < K; k++) out[k] = (gain ? (double)gain[k] : 1.0) * dr[k];",
     "for (int64_t k = 0; k < K; k++) out[k] = dr[k];"),
    ("backward_dw_without_d", "acc += (double)dY[m * N + n] * (double)d[m] * (double)q[m * K + k];",
     "acc += (double)dY[m * N + n] * (double)q[m * K + k];"),
    ("heads_dequant_factor_wrong", "d_out[v] = gamma == 0.f ? 0.f : gamma / (float)qp;",
     "d_out[v] = gamma == 0.f ? 0.f : gamma / (float)(qp + 1);"),
    ("base3_digit_order_reversed", "v += (t + 1) * place;", "v += (t + 1) * (81 / place);"),
    ("base3_sign_convention_swapped", "v += (t + 1) * place;", "v += (1 - t) * place;"),
    ("base3_padding_weight_minus_one", "const int t = k < K ? Wq[n * K + k] : 0;",
     "const int t = k < K ? Wq[n * K + k] : -1;"),
    ("base3_row_bytes_wrong", "return 16 * ((K + 79) / 80);", "return 16 * (K / 80 + 1);"),
    ("base3_unpack_sign_swapped", "const int t = v % 3 - 1;", "const int t = 1 - v % 3;"),
    ("bf16_by_truncation", "out[i] = (uint16_t)((v.u + 0x7FFFu + lsb) >> 16);", "out[i] = (uint16_t)(v.u >> 16);"),
    ("bf16_round_half_away", "out[i] = (uint16_t)((v.u + 0x7FFFu + lsb) >> 16);",
     "out[i] = (uint16_t)((v.u + 0x8000u) >> 16);"),
    ("rescale_factors_premultiplied",
     "float t = (float)acc[m * N + n] * d[m];\n            y[m * N + n] = t * alpha;",
     "float t = (float)acc[m * N + n] * (d[m] * alpha);\n            y[m * N + n] = t;"),
    ("rescale_single_fp64_product",
     "float t = (float)acc[m * N + n] * d[m];\n            y[m * N + n] = t * alpha;",
     "double t = (double)acc[m * N + n] * (double)d[m];\n            y[m * N + n] = (float)(t * (double)alpha);"),
    ("fp4_nibbles_swapped", "b |= (uint8_t)(code << (4 * h));", "b |= (uint8_t)(code << (4 * (1 - h)));"),
    ("fp4_minus_one_code", "else if (t == -1) code = 0xA;", "else if (t == -1) code = 0x6;"),
    ("act_scale_overflow_kept", "if (isinf(s)) { *s_out = 0.0f; *d_out = 0.0f; return HBO_OK; }", ""),
]


def _build(src_text, out_dir, name):
    src = os.path.join(out_dir, name + ".c")
    so = os.path.join(out_dir, name + ".so")
    with open(src, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", src, "-o", so,
                    "-lm"], check=True)
    return so


def _run_pins(so):
    env = dict(os.environ, HBL_ORACLE_SO=so, OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle_pins.py"), "-x",
                        "-q", "-p", "no:cacheprovider", "-m", "not gpu"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout[-2000:]


@pytest.fixture(scope="module")
def source():
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    with open(SRC) as f:
        return f.read()


def test_unmodified_oracle_passes_pins(source, tmp_path):
    rc, out = _run_pins(_build(source, str(tmp_path), "unmodified"))
    assert rc == 0, out


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_fails_a_pin(source, tmp_path, name, old, new):
    assert source.count(old) == 1, "mutation site for %s not unique or not found" % name
    rc, out = _run_pins(_build(source.replace(old, new), str(tmp_path), name))
    assert rc != 0, "no pin caught the planted mistake %s" % name
