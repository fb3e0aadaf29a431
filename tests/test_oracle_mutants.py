"""The oracle's pins must catch plausible mistakes.

Each case plants one slip into a copy of oracle.c (on the CPU, in a temporary
directory), rebuilds it and runs the pin suite against the copy; the suite must
fail.  This shows the pins constrain every step of the definition: the scale,
the causal mask in both directions, the key/value operands, the [B, N, H, d]
indexing, the logsumexp, the normalisation and each backward term.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCORE = ("const double* kj = k + at_bnhd(b, j, h, 0, N, H, d);\n"
         "    double dot = 0.0;\n"
         "    for (int64_t c = 0; c < d; ++c) dot += qi[c] * kj[c];\n"
         "    e[j]")

MUTANTS = {
    "drop_scale": ("e[j] = scale * dot;", "e[j] = dot;"),
    "mask_one_too_many": ("return causal ? i + 1 : N;",
                          "return causal ? (i + 2 < N ? i + 2 : N) : N;"),
    "mask_one_too_few": ("return causal ? i + 1 : N;",
                         "return causal ? (i > 0 ? i : 1) : N;"),
    "value_in_score": (SCORE, SCORE.replace("k + at_bnhd", "v + at_bnhd")),
    "layout_bhnd": ("return (size_t)(((b * N + n) * H + h) * d + c);",
                    "return (size_t)(((b * H + h) * N + n) * d + c);"),
    "lse_without_max": ("*lse_out = m + log(l);", "*lse_out = log(l);"),
    "no_normalisation": ("o_row[c] /= l;", "o_row[c] /= 1.0;"),
    "dk_uses_keys": ("dkj[c] += scale * dsij * qi[c];", "dkj[c] += scale * dsij * kj[c];"),
    "ds_without_D": ("const double dsij = pij * (dp[j] - Di);",
                     "const double dsij = pij * dp[j];"),
    "dq_without_scale": ("dqi[c] += scale * dsij * kj[c];", "dqi[c] += dsij * kj[c];"),
    "dv_uses_ds": ("dvj[c] += pij * doi[c];", "dvj[c] += dsij * doi[c];"),
    "ds_sign": ("const double dsij = pij * (dp[j] - Di);",
                "const double dsij = pij * (Di - dp[j]);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    src = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    before, after = MUTANTS[name]
    assert src.count(before) >= 1, f"mutation site for {name} not found"
    shutil.copytree(os.path.join(ROOT, "oracle"), tmp_path / "oracle",
                    ignore=shutil.ignore_patterns("*.so", "*.so.tmp", "__pycache__"))
    os.makedirs(tmp_path / "tests")
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), tmp_path / "tests" / "golden")
    for f in ("conftest.py", "test_oracle_pins.py"):
        shutil.copy(os.path.join(ROOT, "tests", f), tmp_path / "tests" / f)
    (tmp_path / "oracle" / "oracle.c").write_text(src.replace(before, after, 1))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "tests/test_oracle_pins.py"], cwd=tmp_path,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 1, f"pins did not catch {name}:\n{r.stdout[-2000:]}"
