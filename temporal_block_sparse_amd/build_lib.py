"""Build liblite_attn.so (the C-ABI library and its gfx950 kernels) in-tree with hipcc."""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "liblite_attn.so")
BUILD = os.path.join(ROOT, "_build")
SOURCES = ["lite_attn_api.cpp", "fwd_bf16.hip", "fwd_fp32.hip", "mask_ops.hip", "merge.hip", "calib_ops.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed-fp32 VALU forms are disabled for all device code.
FLAGS = ["-O3", "-fPIC", "-std=c++17", "--offload-arch=" + ARCH, "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    lines = [ln for ln in p.stdout.splitlines() if "packed-fp32-ops" not in ln]
    if p.returncode != 0:
        sys.stderr.write("\n".join(lines) + "\n")
        raise RuntimeError("command failed: " + " ".join(cmd))
    return "\n".join(lines)


def build(verbose=False, save_temps=False):
    """Compile every source for gfx950 and link the shared library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC] + FLAGS + ["-I", os.path.join(ROOT, "include")]
        if src.endswith(".hip"):
            cmd += ["-x", "hip"]
        if save_temps:
            cmd += ["-save-temps=obj"]
        cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
        msg = _run(cmd)
        if verbose and msg:
            print(msg)
        objs.append(obj)
    tmp = OUT + ".tmp%d" % os.getpid()
    _run([HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True, save_temps="--save-temps" in sys.argv))
