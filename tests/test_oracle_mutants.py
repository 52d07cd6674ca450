"""Plant plausible mistakes in copies of the oracle's C source and require the
independent checks (tests/oracle_checks.py) to catch every one.  CPU only."""

import os
import subprocess

import pytest

from oracle import oracle
from tests import oracle_checks as oc

SRC = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")).read()

# (name, text in oracle.c, planted replacement)
MUTANTS = [
    ("forward traversal", "for (int kt = Tk - 1; kt >= 0; --kt) {\n                if (margin)",
     "for (int kt = 0; kt < Tk; ++kt) {\n                if (margin)"),
    ("skipped tiles visited", "continue; /* bypassed: no logits, m_run untouched */", "(void)0;"),
    ("any row passes", "if (d > mg)\n                        mg = d;",
     "if (mg == -INFINITY || d < mg)\n                        mg = d;"),
    ("sign flipped", "double d = mx - m_run[r];", "double d = m_run[r] - mx;"),
    ("non-strict test", "if (mg < tau)", "if (mg <= tau)"),
    ("missing keys as zero logits", "m_loc[r] = mx;", "m_loc[r] = (nc < BN && mx < 0.0) ? 0.0 : mx;"),
    ("missing rows vote", "if (margin)\n                    margin[i * Tk + kt] = mg;",
     "if (nr < BM && mg < 0.0)\n                    mg = 0.0;\n                if (margin)\n                    margin[i * Tk + kt] = mg;"),
    ("scale dropped", "s[r * nc + c] = scale * dot;", "s[r * nc + c] = dot;"),
    ("q used as k", "dot += elem(q, dtype, qo + e) * elem(k, dtype, ko + e);",
     "dot += elem(q, dtype, qo + e) * elem(q, dtype, ko + e);"),
    ("wrong head of k", "size_t ko = ((size_t)(b * (size_t)N + c0 + c) * H + h) * D;",
     "size_t ko = ((size_t)(b * (size_t)N + c0 + c) * H + 0) * D;"),
    ("no normalisation", "valid ? acc[r * D + e] / l[r] : 0.0", "valid ? acc[r * D + e] : 0.0"),
    ("mask_in not kept", "(in | nw) & keep_bits", "(nw) & keep_bits"),
    ("padding bits kept", "(in | nw) & keep_bits", "(in | nw)"),
    ("marked tile dropped at once", "for (int kt = Tk - 1; kt >= 0; --kt) {\n                if (is_skipped(mrow, kt))\n                    continue;\n                const int c0 = kt * BN, nc = (N - c0 < BN) ? N - c0 : BN;\n                tile_logits(q, k, dtype, N, H, D, b, h, r0, nr, c0, nc, scale, s);\n                for (int r = 0; r < nr; ++r) {\n                    for (int c = 0; c < nc; ++c) {",
     "for (int kt = Tk - 1; kt >= 0; --kt) {\n                if (is_skipped(mrow, kt) || ((newly[kt >> 5] >> (kt & 31)) & 1u))\n                    continue;\n                const int c0 = kt * BN, nc = (N - c0 < BN) ? N - c0 : BN;\n                tile_logits(q, k, dtype, N, H, D, b, h, r0, nr, c0, nc, scale, s);\n                for (int r = 0; r < nr; ++r) {\n                    for (int c = 0; c < nc; ++c) {"),
    ("running max frozen at first tile", "if (m_loc[r] > m_run[r])\n                        m_run[r] = m_loc[r];",
     "if (m_run[r] == -INFINITY)\n                        m_run[r] = m_loc[r];"),
    ("lse without max", "lse[i * BM + r] = valid ? m_run[r] + log(l[r]) : -INFINITY;",
     "lse[i * BM + r] = valid ? log(l[r]) : -INFINITY;"),
    ("v from wrong row", "size_t vo = ((size_t)(b * (size_t)N + c0 + c) * H + h) * D;",
     "size_t vo = ((size_t)(b * (size_t)N + c0 + (nc - 1 - c)) * H + h) * D;"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(name, old, new, tmp_path):
    assert SRC.count(old) >= 1, "mutation site not found: " + name
    src = tmp_path / "oracle_mutant.c"
    src.write_text(SRC.replace(old, new, 1))
    so = tmp_path / "liboracle_mutant.so"
    subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-o", str(so), str(src), "-lm"])
    lib = oracle.bind(str(so))
    fails = []
    for check in oc.ALL_CHECKS:
        fails += check(lib=lib)
        if fails:
            break
    assert fails, "planted mistake not caught: " + name
