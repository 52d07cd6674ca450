"""The oracle's C core under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).  oracle.c is compiled with both, and the independent checks run
against that build in a child process with the ASan runtime preloaded; any
out-of-bounds access, use of freed memory or undefined operation aborts the
child and fails the test."""

import os
import subprocess
import sys

import pytest

from oracle import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

CHILD = r"""
import sys
sys.path.insert(0, %(root)r)
from oracle import oracle
from tests import oracle_checks as oc
lib = oracle.bind(%(so)r)
fails = []
for check in (oc.run_golden, oc.check_edge_cases, oc.check_nonsquare, oc.check_ranges, oc.check_tile_invariance):
    fails += check(lib=lib)
fails += oc.check_masked_and_rule(lib=lib, seeds=range(2))
print("FAILS", fails)
sys.exit(1 if fails else 0)
"""


def _runtime(name):
    p = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.skipif(_runtime("libasan.so") is None, reason="gcc's ASan runtime is not installed")
def test_oracle_checks_pass_under_asan_and_ubsan(tmp_path):
    so = str(tmp_path / "liboracle_san.so")
    subprocess.check_call(["gcc", "-O1", "-g", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                           "-fno-omit-frame-pointer", "-o", so, SRC, "-lm"])
    env = dict(os.environ)
    env["LD_PRELOAD"] = _runtime("libasan.so")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["OMP_NUM_THREADS"] = "4"
    p = subprocess.run([sys.executable, "-c", CHILD % {"root": ROOT, "so": so}], env=env, capture_output=True,
                       text=True, timeout=600)
    assert p.returncode == 0, (p.stdout[-2000:], p.stderr[-4000:])
    assert "FAILS []" in p.stdout


@pytest.mark.skipif(_runtime("libasan.so") is None, reason="gcc's ASan runtime is not installed")
def test_sanitizer_catches_a_planted_overrun(tmp_path):
    """The same set-up with a key row read one row too far: the child must abort."""
    old = "size_t ko = ((size_t)(b * (size_t)Nk + c0 + c) * H + h) * D;"
    src = open(SRC).read()
    assert src.count(old) == 1
    bad = tmp_path / "oracle_overrun.c"
    bad.write_text(src.replace(old, "size_t ko = ((size_t)(b * (size_t)Nk + c0 + c + 1) * H + h) * D;"))
    so = str(tmp_path / "liboracle_overrun.so")
    subprocess.check_call(["gcc", "-O1", "-g", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                           "-fno-omit-frame-pointer", "-o", so, str(bad), "-lm"])
    env = dict(os.environ)
    env["LD_PRELOAD"] = _runtime("libasan.so")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["OMP_NUM_THREADS"] = "4"
    p = subprocess.run([sys.executable, "-c", CHILD % {"root": ROOT, "so": so}], env=env, capture_output=True,
                       text=True, timeout=600)
    assert p.returncode != 0 and "AddressSanitizer" in p.stderr
