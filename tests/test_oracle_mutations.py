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


def _build_mutant(tmp_path, name, edits):
    src = open(SRC).read()
    for old, new in zip(edits[0::2], edits[1::2]):
        assert old in src, f"{name}: pattern not found: {old!r}"
        src = src.replace(old, new)
    cfile = tmp_path / f"{name}.c"
    cfile.write_text(src)
    so = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", *[f for f in oracle.CFLAGS if f != "-Werror"],
                    "-I", os.path.join(ROOT, "oracle"), "-o", str(so), str(cfile), "-lm"],
                   check=True)
    return so


def _run_pins(lib_path):
    env = dict(os.environ)
    if lib_path:
        env["VQM_ORACLE_LIB"] = str(lib_path)
    env["HYPOTHESIS_PROFILE"] = "ci"
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                           os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                          env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(tmp_path, name):
    so = _build_mutant(tmp_path, name, MUTANTS[name])
    r = _run_pins(so)
    assert r.returncode != 0, f"mutant {name} passed every pin:\n{r.stdout[-2000:]}"
