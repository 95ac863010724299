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


def test_unmodified_sources_pass_the_pins(tmp_path):
    so = _build_mutant(tmp_path, "unmodified", ())
    for pins in ("test_oracle_pins.py", "test_ss2_oracle_pins.py"):
        r = _run_pins(so, pins)
        assert r.returncode == 0, f"{pins}:\n{r.stdout[-2000:]}"
