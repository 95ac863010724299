"""The oracle's pins catch plausible mistakes.

Each case plants one slip in a temporary copy of ``oracle/vqm_oracle.c`` (on
the CPU only), builds it, and runs the pin suite against it with
``VQM_ORACLE_LIB``: the suite must fail.  The unmodified source must pass.
"""

import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "vqm_oracle.c")

MUTANTS = {
    "no_half_window_shift": ("const int lo = -(scale / 2);", "const int lo = 0;",
                             "const int hi = scale - 1 - scale / 2;", "const int hi = scale - 1;"),
    "reflect_101_edges": ("i = -i - 1;", "i = -i;", "i = 2 * n - i - 1;", "i = 2 * n - i - 2;"),
    "fp32_window_sum": ("double acc = 0.0;", "float acc = 0.0f;", "acc += (double)p;", "acc += p;"),
    "sigma_1": ("#define SIGMA 1.5", "#define SIGMA 1.0"),
    "k2_wrong": ("#define SSIM_C2 ((0.03 * 255.0) * (0.03 * 255.0))",
                 "#define SSIM_C2 ((0.02 * 255.0) * (0.02 * 255.0))"),
    "covariance_sign": ("double sxy = m.exy - m.mx * m.my;", "double sxy = m.exy + m.mx * m.my;"),
    "c3_equals_c2": ("const double c3 = SSIM_C2 / 2.0;", "const double c3 = SSIM_C2;"),
    "exponents_reversed": ("{0.0448, 0.2856, 0.3001, 0.2363, 0.1333}",
                           "{0.1333, 0.2363, 0.3001, 0.2856, 0.0448}"),
    "exponents_b2_b4_swapped": ("{0.0448, 0.2856, 0.3001, 0.2363, 0.1333}",
                                "{0.0448, 0.2363, 0.3001, 0.2856, 0.1333}"),
    "exponent_b3_misread": ("{0.0448, 0.2856, 0.3001, 0.2363, 0.1333}",
                            "{0.0448, 0.2856, 0.3010, 0.2363, 0.1333}"),
    "luminance_every_level": ("msv *= pow(C[j], MS_EXPONENT[j]) * pow(S[j], MS_EXPONENT[j]);",
                              "msv *= pow(L[j], MS_EXPONENT[j]) * pow(C[j], MS_EXPONENT[j]) * pow(S[j], MS_EXPONENT[j]);"),
    "downsample_drops_sample": ("((a + b) + (c + d)) * 0.25f", "((a + b) + (c + c)) * 0.25f"),
    "integer_division_scale": ("double r = round((double)m / 256.0);", "double r = (double)(m / 256);"),
    "valid_region_off_by_one": ("const int mw = w - (WIN - 1), mh = h - (WIN - 1);\n    double total",
                                "const int mw = w - WIN, mh = h - WIN;\n    double total"),
    "db_natural_log": ("return -10.0 * log10(1.0 - ssim);", "return -10.0 * log(1.0 - ssim);"),
    "db_amplitude_form": ("return -10.0 * log10(1.0 - ssim);", "return -20.0 * log10(1.0 - ssim);"),
    "chroma_halves_down": ("*pw = sx ? (w + 1) / 2 : w;", "*pw = sx ? w / 2 : w;"),
    "ceil_dim_as_floor": ("return (n + scale - 1) / scale;", "return n / scale > 0 ? n / scale : 1;"),
}


# Slips in the ssimulacra2 statistics and the pair arithmetic (ss2_oracle.c).
SS2_SRC = os.path.join(ROOT, "oracle", "ss2_oracle.c")
SS2_MUTANTS = {
    "ss2_c2_wrong": ("#define SS2_C2 0.0009f", "#define SS2_C2 0.0001f"),
    "ss2_deficit_not_clamped": ("if (d < 0.0)\n            d = 0.0;", ""),
    "ss2_edge_ratio_inverted": ("(1.0 + (double)a2) / (1.0 + (double)a1)", "(1.0 + (double)a1) / (1.0 + (double)a2)"),
    "ss2_square_not_fourth_power": ("acc[1] += d2 * d2;", "acc[1] += d2;"),
    "ss2_covariance_sign": ("2.0f * (s12[i] - mu12)", "2.0f * (s12[i] + mu12)"),
    "ss2_detail_from_artifact": ("acc[4] += det;", "acc[4] += art;"),
    "two_prod_drops_error": ("out[1] = fmaf(a, b, -p);", "out[1] = 0.0f;"),
    "two_sum_drops_a_part": ("float e = (a - (s - bb)) + (b - bb);", "float e = b - bb;"),
    "ff_div_one_quotient": ("fast_two_sum(q1, q2, out);", "fast_two_sum(q1, 0.0f, out);"),
    "ff_mul_drops_cross_term": ("t = fmaf(a[1], b[0], t);", ""),
    "ff_add_sloppy_low_parts": ("vqm_oracle_two_sum(a[1], b[1], t);", "t[0] = a[1] + b[1];\n    t[1] = 0.0f;"),
}


# Slips in the per-scale chain (the recursion, the downsample, the filter
# design and the chain's stage wiring), caught by test_ss2_chain_pins.py.
CHAIN_MUTANTS = {
    "iir_causal_a1_a3_swapped": ("float t3 = a3 * p3;", "float t3 = a1 * p3;",
                                 "float t1 = a1 * p1;", "float t1 = a3 * p1;"),
    "iir_anticausal_drops_a2": ("float t2 = a2 * q2;", "float t2 = 0.0f * q2;"),
    "iir_anticausal_reads_input": ("float in = B * w[i];", "float in = B * x[(long)i * sx];"),
    "iir_state_shift_order": ("p3 = p2;\n        p2 = p1;", "p2 = p1;\n        p3 = p2;"),
    "iir_anticausal_start_one_early": ("for (int i = n - 1; i >= 0; i--) {", "for (int i = n - 2; i >= 0; i--) {"),
    "blur_columns_first": (
        "for (int r = 0; r < h; r++) /* every row first */\n"
        "        iir_line(in + (size_t)r * w, 1, rows + (size_t)r * w, 1, w, coef, line);\n"
        "    for (int c = 0; c < w; c++) /* then every column of the row pass's output */\n"
        "        iir_line(rows + c, w, out + c, w, h, coef, line);",
        "for (int c = 0; c < w; c++)\n"
        "        iir_line(in + c, w, rows + c, w, h, coef, line);\n"
        "    for (int r = 0; r < h; r++)\n"
        "        iir_line(rows + (size_t)r * w, 1, out + (size_t)r * w, 1, w, coef, line);"),
    "downsample_floor_dims": ("*ow = (w + 1) / 2;", "*ow = w / 2 > 0 ? w / 2 : 1;"),
    "downsample_drops_a_sample": ("out[(size_t)y * ow + x] = ((a + b) + (c + d)) * 0.25f;",
                                  "out[(size_t)y * ow + x] = ((a + b) + (c + c)) * 0.25f;"),
    "cascade_wrong_root": ("double p = ((s2 + 3.0) - sqrt(6.0 * s2 + 9.0)) / s2;",
                           "double p = ((s2 + 3.0) + sqrt(6.0 * s2 + 9.0)) / s2;"),
    "cascade_one_pass_variance": ("double p = ((s2 + 3.0) - sqrt(6.0 * s2 + 9.0)) / s2;",
                                  "double p = ((s2 + 1.0) - sqrt(2.0 * s2 + 1.0)) / s2;"),
    "cascade_a2_sign": ("coef[2] = (float)(-3.0 * p * p);", "coef[2] = (float)(3.0 * p * p);"),
    "chain_cross_product_as_square": ("ab[i] = a[i] * b[i];", "ab[i] = a[i] * a[i];"),
    "chain_means_swapped": ("const float *src[5] = {a, b, aa, bb, ab};", "const float *src[5] = {b, a, aa, bb, ab};"),
    "chain_never_downsamples": ("if (s > 0) { /* the next scale's images", "if (0) { /* the next scale's images"),
}


def _build_mutant(tmp_path, name, edits, path=SRC):
    src = open(path).read()
    for old, new in zip(edits[0::2], edits[1::2]):
        assert old in src, f"{name}: pattern not found: {old!r}"
        src = src.replace(old, new)
    cfile = tmp_path / os.path.basename(path)
    cfile.write_text(src)
    others = [f for f in oracle.SOURCES if os.path.basename(f) != os.path.basename(path)]
    so = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", *[f for f in oracle.CFLAGS if f != "-Werror"],
                    "-I", os.path.join(ROOT, "oracle"), "-o", str(so), str(cfile), *others, "-lm"],
                   check=True)
    return so


def _run_pins(lib_path, pin_file="test_oracle_pins.py"):
    env = dict(os.environ)
    if lib_path:
        env["VQM_ORACLE_LIB"] = str(lib_path)
    env["HYPOTHESIS_PROFILE"] = "ci"
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                           os.path.join(ROOT, "tests", pin_file)],
                          env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(tmp_path, name):
    so = _build_mutant(tmp_path, name, MUTANTS[name])
    r = _run_pins(so)
    assert r.returncode != 0, f"mutant {name} passed every pin:\n{r.stdout[-2000:]}"


@pytest.mark.parametrize("name", sorted(SS2_MUTANTS))
def test_ss2_pins_catch_mutant(tmp_path, name):
    so = _build_mutant(tmp_path, name, SS2_MUTANTS[name], SS2_SRC)
    r = _run_pins(so, "test_ss2_oracle_pins.py")
    assert r.returncode != 0, f"mutant {name} passed every pin:\n{r.stdout[-2000:]}"


@pytest.mark.parametrize("name", sorted(CHAIN_MUTANTS))
def test_chain_pins_catch_mutant(tmp_path, name):
    so = _build_mutant(tmp_path, name, CHAIN_MUTANTS[name], SS2_SRC)
    r = _run_pins(so, "test_ss2_chain_pins.py")
    assert r.returncode != 0, f"mutant {name} passed every pin:\n{r.stdout[-2000:]}"


def test_unmodified_sources_pass_the_pins(tmp_path):
    so = _build_mutant(tmp_path, "unmodified", ())
    for pins in ("test_oracle_pins.py", "test_ss2_oracle_pins.py", "test_ss2_chain_pins.py"):
        r = _run_pins(so, pins)
        assert r.returncode == 0, f"{pins}:\n{r.stdout[-2000:]}"
