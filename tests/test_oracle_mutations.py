"""The oracle pins must catch plausible mistakes in the oracle.

Each case plants one mistake in a copy of one of the oracle's C sources (on
the CPU, in a temporary folder), builds the library from it and the other
source unchanged, and runs the pin tests against the mutated library in a
subprocess: at least one pin has to fail.
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GDN_SRC = os.path.join(ROOT, "oracle", "gdn_oracle.c")
ATT_SRC = os.path.join(ROOT, "oracle", "fork_attention_oracle.c")
PINS = [os.path.join(ROOT, "tests", "test_oracle_pins.py"),
        os.path.join(ROOT, "tests", "test_attention_oracle_pins.py")]

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
ATT_MUTATIONS = {
    "attn_causal_off_by_one": ("for (int j = 0; j <= p; ++j) keys[n++] = t0 + j;",
                               "for (int j = 0; j <= p + 1 && j < len; ++j) keys[n++] = t0 + j;"),
    "attn_branch_without_trunk": ("for (int j = 0; j < plen; ++j) keys[n++] = p0 + j;",
                                  "for (int j = 1; j < plen; ++j) keys[n++] = p0 + j;"),
    "attn_scale_dropped": ("w[t] = scale * s;", "w[t] = s;"),
    "attn_group_mapping": ("const int hk = h / (H / Hkv);", "const int hk = h % Hkv;"),
    "attn_unnormalised": ("out[c] += (w[t] / den) * vj[c];", "out[c] += w[t] * vj[c];"),
}
CASES = {**{n: (GDN_SRC, m) for n, m in MUTATIONS.items()},
         **{n: (ATT_SRC, m) for n, m in ATT_MUTATIONS.items()}}


@pytest.mark.parametrize("name", sorted(CASES))
def test_pins_catch_planted_mistake(name, tmp_path):
    path, (before, after) = CASES[name]
    src = open(path).read()
    assert before in src, f"mutation site for {name} not found"
    mutated = tmp_path / os.path.basename(path)
    mutated.write_text(src.replace(before, after, 1))
    other = ATT_SRC if path == GDN_SRC else GDN_SRC
    so = tmp_path / "liboracle_mutated.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", str(so),
                    str(mutated), other, "-lm"], check=True)
    env = dict(os.environ, ORACLE_LIB_OVERRIDE=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        *PINS],
                       env=env, capture_output=True, text=True, cwd=ROOT, timeout=300)
    assert r.returncode != 0, f"no pin failed for mutation {name}:\n{r.stdout[-2000:]}"


def test_unmutated_library_passes_the_pins(tmp_path):
    """The same build and run without a planted mistake passes, so the
    failures above come from the mutations, not from the harness."""
    so = tmp_path / "liboracle_plain.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", str(so), GDN_SRC,
                    ATT_SRC, "-lm"], check=True)
    env = dict(os.environ, ORACLE_LIB_OVERRIDE=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        *PINS],
                       env=env, capture_output=True, text=True, cwd=ROOT, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:]
