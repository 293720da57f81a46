"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of oracle/mala_oracle.c, builds it,
and runs the pin suite (tests/test_oracle_pins.py: the worked example, the
hand-derived rules and margins, tau = 0 against brute force and autograd,
Proposition 1, nesting, the decode pins) against that build in a fresh
process.  The suite must fail on every mutant and pass on the unmodified
source.  The NumPy cross-check is deliberately not part of this run: it is a
second statement of the same rule, not a pin.  Rule: review page "Forward:
online sparse softmax", "Backward: offline sparse probabilities".
"""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle", "mala_oracle.c")

MUTANTS = {
    # the decision margin in log2 instead of ln (kept set unchanged: only the
    # hand-derived margins can see it)
    "margin_in_log2": [("            else x = M[r] - m[r] - log(l[r]) - th[r];",
                        "            else x = (M[r] - m[r] - log(l[r]) - th[r]) / log(2.0);"),
                       ("        const double x = mx - lz - th;",
                        "        const double x = (mx - lz - th) / log(2.0);")],
    # L_i = i instead of i + 1 in the forward threshold
    "visible_keys_off_by_one": [("log_threshold(c->tau, (double)(off + r0 + r + 1))",
                                 "log_threshold(c->tau, (double)(off + r0 + r + 2))")],
    # the candidate tile's own mass counted in the denominator
    "candidate_in_denominator": [
        ("            else x = M[r] - m[r] - log(l[r]) - th[r];",
         "            else { double zt = 0.0; for (int j = j0; j < j1; ++j) { const double s_ = "
         "S[(size_t)r * Bk + (j - j0)]; if (s_ > -INFINITY) zt += exp(s_ - m[r]); } "
         "x = M[r] - m[r] - log(l[r] + zt) - th[r]; }")],
    # dS = P (D - dP) in the dq pass
    "ds_sign_in_dq": [("                const double ds = p * (dp - D[i - r0]);\n"
                       "                for (int cc = 0; cc < d; ++cc) c->dq[row + cc] += c->scale * ds * kj[cc];",
                       "                const double ds = p * (D[i - r0] - dp);\n"
                       "                for (int cc = 0; cc < d; ++cc) c->dq[row + cc] += c->scale * ds * kj[cc];")],
    # GQA: q head h reading KV head h % Hkv instead of h / (Hq / Hkv)
    "gqa_mapping": [("    const int kh = h / (Hq / Hkv);\n    const int r0 = qb * c->Bq;\n    if (r0 >= Lq) return OR_OK;"
                     "       /* past this sequence's queries: not visited */",
                     "    const int kh = h % Hkv;\n    const int r0 = qb * c->Bq;\n    if (r0 >= Lq) return OR_OK;"
                     "       /* past this sequence's queries: not visited */")],
}


def _build(src_text, out):
    c = out.with_suffix(".c")
    c.write_text(src_text)
    subprocess.run(["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                    "-o", str(out), str(c), "-lm"], check=True, capture_output=True, text=True)
    return out


def _run_pins(lib):
    env = dict(os.environ, MALA_ORACLE_LIB=str(lib))
    return subprocess.run([sys.executable, "-m", "pytest", os.path.join(HERE, "test_oracle_pins.py"), "-x", "-q",
                           "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True,
                          timeout=600)


def test_pins_pass_on_the_unmodified_oracle(tmp_path):
    r = _run_pins(_build(open(SRC).read(), tmp_path / "control.so"))
    assert r.returncode == 0, r.stdout[-3000:]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_fail_on_mutant(name, tmp_path):
    text = open(SRC).read()
    for old, new in MUTANTS[name]:
        assert text.count(old) == 1, (name, old)
        text = text.replace(old, new)
    r = _run_pins(_build(text, tmp_path / f"{name}.so"))
    # exit status 1: tests ran and at least one failed (not a collection error)
    assert r.returncode == 1, (name, r.returncode, r.stdout[-3000:])
    assert "failed" in r.stdout
