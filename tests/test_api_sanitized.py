"""The library's host layer (lite_attn_api.cpp: descriptor, range, alignment
and alias validation) under AddressSanitizer, on the CPU.  It is built alone,
host code only, with stand-in launchers (tests/asan_launch_stubs.cpp), and the
CPU ABI tests run against it in a child process with the ASan runtime
preloaded and Python's allocator switched to malloc, so that the buffers the
tests pass through ctypes carry redzones."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"
API = os.path.join(ROOT, "temporal_block_sparse_amd", "csrc", "lite_attn_api.cpp")
STUBS = os.path.join(ROOT, "tests", "asan_launch_stubs.cpp")


def _asan_runtime():
    base = "/opt/rocm/llvm/lib/clang"
    if not os.path.isdir(base):
        return None
    for v in sorted(os.listdir(base), reverse=True):
        p = os.path.join(base, v, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(p):
            return p
    return None


RT = _asan_runtime()
pytestmark = pytest.mark.skipif(RT is None or not os.path.exists(HIPCC), reason="hipcc or clang's ASan runtime missing")


def _build(src, so):
    # host code only: the sanitizer flag applies to the host pass
    subprocess.check_call([HIPCC, "-O1", "-g", "-fPIC", "-shared", "-std=c++17", "-Xarch_host",
                           "-fsanitize=address", "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"),
                           "-I", os.path.dirname(API), "-o", so, src, STUBS],
                          stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)


def _env(so):
    env = dict(os.environ)
    env.update(LD_PRELOAD=RT, LITE_ATTN_LIBRARY=so, PYTHONMALLOC="malloc",
               ASAN_OPTIONS="detect_leaks=0:detect_odr_violation=0:abort_on_error=1")
    return env


def test_abi_checks_pass_under_asan(tmp_path):
    so = str(tmp_path / "liblite_attn_asan.so")
    _build(API, so)
    p = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       cwd=ROOT, env=_env(so), capture_output=True, text=True, timeout=600)
    assert p.returncode == 0, (p.stdout[-3000:], p.stderr[-3000:])


CHILD = r"""
import ctypes, sys
sys.path.insert(0, %(root)r)
from temporal_block_sparse_amd import lite_attn as la
d = la.make_desc(1, 1000, 2, 64, 128, 64, la.LITE_BF16)
do = (ctypes.c_int32 * 6)(80, 60, 45, 40, 12, 2)
sk = (ctypes.c_int32 * 1)(0)
r = la.Ranges(ctypes.cast(do, ctypes.POINTER(ctypes.c_int32)), 3, ctypes.cast(sk, ctypes.POINTER(ctypes.c_int32)), 0)
print("rc", la.LIB.lite_attn_build_skiplist(ctypes.byref(d), None, ctypes.c_void_p(1 << 40), ctypes.byref(r), None))
"""


def test_asan_catches_a_planted_overread(tmp_path):
    """Range validation reading one entry past the last pair: the child aborts."""
    src = open(API).read()
    old = "if (i + 1 < n && !(end > (int64_t)rg[2 * i + 2]))"
    assert src.count(old) == 1
    bad = tmp_path / "lite_attn_api_overread.cpp"
    bad.write_text(src.replace(old, "if (i < n && !(end > (int64_t)rg[2 * i + 2]))"))
    good_so, bad_so = str(tmp_path / "good.so"), str(tmp_path / "bad.so")
    _build(API, good_so)
    _build(str(bad), bad_so)
    ok = subprocess.run([sys.executable, "-c", CHILD % {"root": ROOT}], env=_env(good_so), capture_output=True,
                        text=True, timeout=300)
    assert ok.returncode == 0 and "rc" in ok.stdout, ok.stderr[-3000:]
    p = subprocess.run([sys.executable, "-c", CHILD % {"root": ROOT}], env=_env(bad_so), capture_output=True,
                       text=True, timeout=300)
    assert p.returncode != 0 and "AddressSanitizer" in p.stderr, (p.stdout, p.stderr[-3000:])
