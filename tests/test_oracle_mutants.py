"""Plant plausible mistakes in copies of the oracle's C source and Python helpers and require the
independent checks (tests/oracle_checks.py) to catch every one.  CPU only."""

import importlib.util
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
    ("non-strict test", "if (mg < tau && !must_do_t)", "if (mg <= tau && !must_do_t)"),
    ("missing keys as zero logits", "m_loc[r] = mx;", "m_loc[r] = (nc < BN && mx < 0.0) ? 0.0 : mx;"),
    ("missing rows vote", "if (margin)\n                    margin[i * Tk + kt] = mg;",
     "if (nr < BM && mg < 0.0)\n                    mg = 0.0;\n                if (margin)\n                    margin[i * Tk + kt] = mg;"),
    ("scale dropped", "s[r * nc + c] = scale * dot;", "s[r * nc + c] = dot;"),
    ("q used as k", "dot += elem(q, dtype, qo + e) * elem(k, dtype, ko + e);",
     "dot += elem(q, dtype, qo + e) * elem(q, dtype, ko + e);"),
    ("wrong head of k", "size_t ko = ((size_t)(b * (size_t)Nk + c0 + c) * H + h) * D;",
     "size_t ko = ((size_t)(b * (size_t)Nk + c0 + c) * H + 0) * D;"),
    ("k indexed with the query length", "size_t ko = ((size_t)(b * (size_t)Nk + c0 + c) * H + h) * D;",
     "size_t ko = ((size_t)(b * (size_t)Nq + c0 + c) * H + h) * D;"),
    ("no normalisation", "valid ? acc[r * D + e] / l[r] : 0.0", "valid ? acc[r * D + e] : 0.0"),
    ("mask_in not kept", "(in | nw) & keep_bits", "(nw) & keep_bits"),
    ("padding bits kept", "(in | nw) & keep_bits", "(in | nw)"),
    ("marked tile dropped at once", "                if (!tile_must_do(must_do, n_do, c0, nc) &&\n                    (is_skipped(mrow, kt) || tile_must_skip(must_skip, n_skip, c0, nc)))\n                    continue;\n                tile_logits(",
     "                if (!tile_must_do(must_do, n_do, c0, nc) &&\n                    (is_skipped(mrow, kt) || tile_must_skip(must_skip, n_skip, c0, nc) || ((newly[kt >> 5] >> (kt & 31)) & 1u)))\n                    continue;\n                tile_logits("),
    ("running max frozen at first tile", "if (m_loc[r] > m_run[r])\n                        m_run[r] = m_loc[r];",
     "if (m_run[r] == -INFINITY)\n                        m_run[r] = m_loc[r];"),
    ("lse without max", "lse[i * BM + r] = valid ? m_run[r] + log(l[r]) : -INFINITY;",
     "lse[i * BM + r] = valid ? log(l[r]) : -INFINITY;"),
    ("v from wrong row", "size_t vo = ((size_t)(b * (size_t)Nk + c0 + c) * H + h) * D;",
     "size_t vo = ((size_t)(b * (size_t)Nk + c0 + (nc - 1 - c)) * H + h) * D;"),
    ("range end inclusive", "if (rg[2 * i + 1] < t && t <= rg[2 * i])", "if (rg[2 * i + 1] <= t && t <= rg[2 * i])"),
    ("range start exclusive", "if (rg[2 * i + 1] < t && t <= rg[2 * i])", "if (rg[2 * i + 1] < t && t < rg[2 * i])"),
    ("must-skip on any key", "        if (!in_ranges(rg, n, t))\n            return 0;\n    return 1;",
     "        if (in_ranges(rg, n, t))\n            return 1;\n    return 0;"),
    ("must-do tiles may be marked", "if (mg < tau && !must_do_t)", "if (mg < tau)"),
    ("must-do does not override the mask", "if (!must_do_t && (is_skipped(mrow, kt) || tile_must_skip(must_skip, n_skip, c0, nc)))",
     "if (is_skipped(mrow, kt) || (!must_do_t && tile_must_skip(must_skip, n_skip, c0, nc)))"),
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


PY_SRC = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.py")).read()

# (name, text in oracle.py, planted replacement) -- mistakes in the Python helpers
PY_MUTANTS = [
    ("skip-list ascending", "for kt in range(tk - 1, -1, -1):\n            marked", "for kt in range(tk):\n            marked"),
    ("skip-list reads word 0 only", "marked = (int(m[r, kt // 32]) >> (kt % 32)) & 1",
     "marked = (int(m[r, 0]) >> (kt % 32)) & 1"),
    ("skip-list must-skip beats must-do", "if do or not (marked or sk):", "if (do and not sk) or not (marked or sk):"),
    ("skip-list must-do ignored", "if do or not (marked or sk):", "if not (marked or sk):"),
    ("tile flags end inclusive", "range(max(end + 1, 0), min(start, nk - 1) + 1)",
     "range(max(end, 0), min(start, nk - 1) + 1)"),
    ("tile flags start exclusive", "range(max(end + 1, 0), min(start, nk - 1) + 1)",
     "range(max(end + 1, 0), min(start, nk - 1))"),
    ("tile flags must-skip on any key", "cs[kt * tile_n:(kt + 1) * tile_n].all()", "cs[kt * tile_n:(kt + 1) * tile_n].any()"),
    ("tile flags last key of a tile dropped", "cd[kt * tile_n:(kt + 1) * tile_n].any()",
     "cd[kt * tile_n:(kt + 1) * tile_n - 1].any()"),
    ("merge without normalisation", "out = (w[..., None] * O).sum(axis=0) / np.where(empty, 1.0, s)[..., None]",
     "out = (w[..., None] * O).sum(axis=0)"),
    ("merge without the max shift", "m_safe = np.where(empty, 0.0, m)", "m_safe = np.where(empty, 0.0, 0.0 * m)"),
    ("merge lse is the max", "lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, s)))",
     "lse = np.where(empty, -np.inf, m_safe)"),
    ("merge weights by lse, not exp", "w = np.exp(L - m_safe)", "w = np.where(np.isneginf(L), 0.0, np.exp(L - m_safe) * 0 + 1)"),
    ("budgets reach 1.0 inside the early steps", "min(1.0, 0.5 + 0.5 * t / n)", "min(1.0, 0.5 + 0.5 * t / max(n - 1, 1))"),
    ("budgets rounded early count", "n = math.floor(num_steps * early_step_ratio)", "n = round(num_steps * early_step_ratio)"),
    ("budgets loosest first", "min(1.0, 0.5 + 0.5 * t / n)", "min(1.0, 1.0 - 0.5 * t / n)"),
    ("calibration takes the smallest feasible tau", "cands = sorted(set(float(t) for t in taus), reverse=True)",
     "cands = sorted(set(float(t) for t in taus))"),
    ("calibration forgets the carried mask", "        mask = m2\n    return out", "        mask = None\n    return out"),
    ("calibration error unnormalised", "err = float(np.sqrt(((o2 - od) ** 2).sum())) / norm if norm > 0 else 0.0",
     "err = float(np.sqrt(((o2 - od) ** 2).sum()))"),
    ("calibration budget unscaled", "budget = base_error * mult[t]", "budget = base_error"),
    ("calibration error before the marks take effect",
     "r2 = fwd(q, k, v, tile_m, tile_n, -math.inf, scale, mask_in=m2, want_mask_out=False, nthreads=nthreads)",
     "r2 = fwd(q, k, v, tile_m, tile_n, -math.inf, scale, mask_in=mask, want_mask_out=False, nthreads=nthreads)"),
    ("unpack swaps heads and q-tiles", "        qt = row % Tq\n        h = (row // Tq) % H",
     "        h = row % H\n        qt = (row // H) % Tq"),
]


@pytest.mark.filterwarnings("ignore::RuntimeWarning")
@pytest.mark.parametrize("name,old,new", PY_MUTANTS, ids=[m[0] for m in PY_MUTANTS])
def test_planted_python_mistake_is_caught(name, old, new, tmp_path, monkeypatch):
    assert PY_SRC.count(old) >= 1, "mutation site not found: " + name
    src = tmp_path / "oracle_mutant.py"
    src.write_text(PY_SRC.replace(old, new, 1))
    spec = importlib.util.spec_from_file_location("oracle_mutant", str(src))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod._lib = oracle._load()              # the unmodified fp64 C core
    monkeypatch.setattr(oc, "oracle", mod)
    fails = []
    for check in oc.PY_CHECKS + oc.ALL_CHECKS:
        fails += check()
        if fails:
            break
    assert fails, "planted mistake not caught: " + name
