"""Plant plausible mistakes in copies of the oracle source (CPU only) and check that the pins in
``test_oracle.py`` catch every one of them: a dropped term, a wrong sign, a wrong index, a
transposed operand, the wrong rounding rule, the wrong scale denominator, a swapped nibble order."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "qvref.c")

MUTANTS = {
    "fwht_drops_normalisation": ("        for (int64_t j = 0; j < d; ++j) y[j] *= norm;\n    }\n    return 0;\n}\n\nint qvref_quantize_rows",
                                 "        for (int64_t j = 0; j < d; ++j) y[j] *= 1.0;\n    }\n    return 0;\n}\n\nint qvref_quantize_rows"),
    "fwht_wrong_sign": ("y[i + h] = u - v;", "y[i + h] = v - u;"),
    "closed_form_negated": ("? -1 : 1;", "? 1 : -1;"),
    "explicit_wrong_column": ("y[j] += xi * (double)h[j];", "y[j] += xi * (double)h[d - 1 - j];"),
    "scale_over_8": ("float s = amax / (float)qmax;", "float s = amax / (float)(qmax + 1);"),
    "round_half_away": ("float r = rintf(t);", "float r = roundf(t);"),
    "multiplier_ignored": ("xt[k] = xs * mk;", "xt[k] = xs; (void)mk;"),
    "no_zero_scale_guard": ("if (!(s >= FLT_MIN)) s = 0.0f;", ""),
    "nibbles_swapped": ("(uint8_t)((lo & 0xF) | ((hi & 0xF) << 4));", "(uint8_t)((hi & 0xF) | ((lo & 0xF) << 4));"),
    "unpack_no_sign_extension": ("if (lo >= 8) lo -= 16;", ""),
    "gemm_transposed_weight": ("(int64_t)qw[n * K + k];", "(int64_t)qw[k * N + n];"),
    "dequant_drops_bias": ("if (bias) y += (double)bias[n];", ""),
    "dequant_scale_index_swap": ("double y = (double)acc[m * N + n] * (double)sa[m] * (double)sw[n];",
                                 "double y = (double)acc[m * N + n] * (double)sa[n % M] * (double)sw[m % N];"),
    "gelu_wrong_sign": ("return 0.5 * y * erfc(-y / sqrt(2.0));", "return 0.5 * y * erfc(y / sqrt(2.0));"),
    "grouped_scale_ignores_group": ("y += (double)acc * (double)sa[m * groups + g] * (double)sw[n * groups + g];",
                                    "y += (double)acc * (double)sa[m * groups + g] * (double)sw[n * groups];"),
    "grouped_drops_last_channel": ("for (int64_t k = g * group; k < (g + 1) * group; ++k)",
                                   "for (int64_t k = g * group; k < (g + 1) * group - 1; ++k)"),
    "grouped_drops_bias": ("if (bias != NULL) y += (double)bias[n];", ""),
    "smoothing_alpha_swapped": ("sk = pow(ax, alpha) / pow(aw, 1.0 - alpha);", "sk = pow(ax, 1.0 - alpha) / pow(aw, alpha);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation site for {name} not unique"
    mdir = tmp_path / "oracle_mutant"
    mdir.mkdir()
    shutil.copy(os.path.join(ROOT, "oracle", "qvref.h"), mdir / "qvref.h")
    (mdir / "qvref.c").write_text(text.replace(old, new))
    so = mdir / "libqvref.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-shared", "-fPIC",
                    str(mdir / "qvref.c"), "-o", str(so), "-lm"], check=True)
    env = dict(os.environ, QVREF_LIB=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"mutant {name} survived the oracle pins:\n{r.stdout[-2000:]}"
