"""Python side of the CPU oracle (TEST INFRASTRUCTURE ONLY).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may use
this module; the product path never imports it.  It shares no code with the
HIP library: the fp64 arithmetic lives in oracle.c, and the Skip-List
reference below is a direct restatement of "list the live key tiles in the
order the kernel visits them".

Pages: [README] = the LiteAttention project README (moonmath-ai/LiteAttention);
[ABSTRACT] = arXiv 2511.11062 abstract.
"""

import ctypes
import os
import subprocess
import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

BF16, FP32, FP64 = 0, 1, 2


def build(force=False):
    """Compile oracle.c with gcc (plain -O2, IEEE semantics, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def bind(path):
    """Load a compiled oracle library (the default one, or a test's variant of it)."""
    lib = ctypes.CDLL(path)
    lib.oracle_fwd.restype = ctypes.c_int
    lib.oracle_fwd.argtypes = [ctypes.c_int] * 7 + [ctypes.c_void_p] * 4 + [
        ctypes.c_int, ctypes.c_double, ctypes.c_double, ctypes.c_void_p, ctypes.c_int64,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
    lib.oracle_max_threads.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        build()
        _lib = bind(_LIB)
    return _lib


def max_threads():
    return _load().oracle_max_threads()


def _as_host(x):
    """Contiguous CPU array + dtype code; bf16 is passed as its raw 16-bit patterns."""
    if isinstance(x, torch.Tensor):
        x = x.detach().cpu().contiguous()
        if x.dtype == torch.bfloat16:
            return x.view(torch.int16).numpy(), BF16
        if x.dtype == torch.float32:
            return x.numpy(), FP32
        if x.dtype == torch.float64:
            return x.numpy(), FP64
        raise TypeError("unsupported dtype %s" % x.dtype)
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return x, FP32
    if x.dtype == np.float64:
        return x, FP64
    raise TypeError("unsupported dtype %s" % x.dtype)


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def fwd(q, k, v, tile_m, tile_n, tau, scale, mask_in=None, want_mask_out=True, rows=None,
        nthreads=None, lib=None):
    """fp64 oracle forward on BSHD q, k, v (torch or numpy; bf16/fp32/fp64).

    mask_in: [B*H*Tq, W] words (int32 or uint32) or None (nothing skipped).
    rows:    row ids (b*H + h)*Tq + qt to compute, or None for all rows.
    Returns a dict of numpy arrays packed per computed row:
      out [nrows, BM, D], lse [nrows, BM], margin [nrows, Tk] (NaN = not visited),
      mask_out [nrows, W] (uint32), and 'rows'.
    """
    lib = lib or _load()
    qa, dt = _as_host(q)
    ka, dk = _as_host(k)
    va, dv = _as_host(v)
    if not (dt == dk == dv):
        raise TypeError("q, k, v must share a dtype")
    B, N, H, D = qa.shape
    if ka.shape != qa.shape or va.shape != qa.shape:
        raise ValueError("q, k, v shapes differ")
    Tq, Tk = -(-N // tile_m), -(-N // tile_n)
    W = -(-Tk // 32)
    if rows is None:
        rows_a = np.arange(B * H * Tq, dtype=np.int64)
    else:
        rows_a = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    nr = rows_a.shape[0]
    m_in = None
    if mask_in is not None:
        if isinstance(mask_in, torch.Tensor):
            mask_in = mask_in.detach().cpu().numpy()
        m_in = np.ascontiguousarray(np.asarray(mask_in).view(np.uint32).reshape(B * H * Tq, W))
    out = np.zeros((nr, tile_m, D), np.float64)
    lse = np.zeros((nr, tile_m), np.float64)
    margin = np.zeros((nr, Tk), np.float64)
    mask_out = np.zeros((nr, W), np.uint32)
    if nthreads is None:
        nthreads = lib.oracle_max_threads()
    rc = lib.oracle_fwd(B, N, H, D, tile_m, tile_n, dt, _ptr(qa), _ptr(ka), _ptr(va), _ptr(m_in),
                        int(bool(want_mask_out)), float(tau), float(scale), _ptr(rows_a), nr,
                        _ptr(out), _ptr(lse), _ptr(margin), _ptr(mask_out), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_fwd rejected its arguments")
    return {"out": out, "lse": lse, "margin": margin, "mask_out": mask_out, "rows": rows_a,
            "nthreads": int(nthreads)}


def unpack_rows(res, B, N, H, tile_m):
    """Scatter packed per-row outputs of a full-row oracle call back to BSHD / [B,H,N]."""
    D = res["out"].shape[2]
    Tq = -(-N // tile_m)
    out = np.zeros((B, Tq * tile_m, H, D))
    lse = np.full((B, H, Tq * tile_m), -np.inf)
    for i, row in enumerate(res["rows"]):
        qt = row % Tq
        h = (row // Tq) % H
        b = row // (Tq * H)
        out[b, qt * tile_m:(qt + 1) * tile_m, h, :] = res["out"][i]
        lse[b, h, qt * tile_m:(qt + 1) * tile_m] = res["lse"][i]
    return out[:, :N], lse[:, :, :N]


def skiplist(mask, tk):
    """Skip-List of each mask row: [count, live k-tiles in visiting (descending) order].

    mask: [rows, W] words; returns (counts [rows] int32, lists: list of int arrays).
    A tile is live when its bit is clear ([README] QK-Skip: marked tiles are bypassed).
    """
    m = np.asarray(mask).view(np.uint32)
    counts = np.zeros(m.shape[0], np.int32)
    lists = []
    for r in range(m.shape[0]):
        live = [kt for kt in range(tk - 1, -1, -1) if not (int(m[r, kt // 32]) >> (kt % 32)) & 1]
        counts[r] = len(live)
        lists.append(np.asarray(live, np.int32))
    return counts, lists
