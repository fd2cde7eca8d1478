"""The oracle pins must catch plausible mistakes in the oracle.

Each case plants one mistake in a copy of the oracle's C source (on the
CPU, in a temporary folder), builds it, and runs the pin tests against the
mutated library in a subprocess: at least one pin has to fail.
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "gdn_oracle.c")

MUTATIONS = {
    "output_before_update": (
        "    if (o) {\n        for (int j = 0; j < dv; ++j) o[j] = 0.0;", "    if (0) {"),
    "delta_sign": ("beta * (v[j] - y[j])", "beta * (v[j] + y[j])"),
    "prediction_without_decay": ("const double w = a * k[i];", "const double w = k[i];"),
    "decay_after_write": ("row[j] = a * row[j] + k[i] * u[j]",
                          "row[j] = a * (row[j] + k[i] * u[j])"),
    "conv_taps_reversed": ("conv_w[c * CONV_W + r] * RAW(t - WIN + r)",
                           "conv_w[c * CONV_W + (CONV_W - 1 - r)] * RAW(t - WIN + r)"),
    "window_rows_reversed": ("win_out[(size_t)r * cc + c] = RAW(len - WIN + r);",
                             "win_out[(size_t)(WIN - 1 - r) * cc + c] = RAW(len - WIN + r);"),
    "replay_decay_sign": ("exp(lam_last - lam_e)", "exp(lam_e - lam_last)"),
    "norm_without_eps": ("1.0 / sqrt(ss + eps)", "1.0 / sqrt(ss)"),
    "readout_transposed": ("o[j] += row[j] * q[i];",
                           "o[j] += Sig[(size_t)j * dv + i] * q[i];"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    before, after = MUTATIONS[name]
    src = open(SRC).read()
    assert before in src, f"mutation site for {name} not found"
    mutated = tmp_path / "mutated.c"
    mutated.write_text(src.replace(before, after, 1))
    so = tmp_path / "liboracle_mutated.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", str(so),
                    str(mutated), "-lm"], check=True)
    env = dict(os.environ, ORACLE_LIB_OVERRIDE=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       env=env, capture_output=True, text=True, cwd=ROOT, timeout=300)
    assert r.returncode != 0, f"no pin failed for mutation {name}:\n{r.stdout[-2000:]}"
