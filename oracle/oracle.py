"""Python side of the CPU oracle (TEST INFRASTRUCTURE ONLY).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may use
this module; the product path never imports it.  It shares no code with the
HIP library: the fp64 arithmetic lives in oracle.c, and the Skip-List
reference below is a direct restatement of "list the live key tiles in the
order the kernel visits them".

Pages: [README] = the LiteAttention project README (moonmath-ai/LiteAttention);
[ABSTRACT] = arXiv 2511.11062 abstract; [SKILL] = the "Lite Attention
Temporal Sparse" skill page (its "Step 3: Error Calibration" gives the budget
multipliers used by error_budgets).
"""

import ctypes
import math
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
    lib.oracle_fwd.argtypes = [ctypes.c_int] * 8 + [ctypes.c_void_p] * 4 + [
        ctypes.c_int, ctypes.c_double, ctypes.c_double,
        ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_int64,
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


def _ranges(rg):
    """(start, end) pairs as a flat int32 array and the pair count."""
    if rg is None or len(rg) == 0:
        return None, 0
    a = np.ascontiguousarray(np.asarray(rg, dtype=np.int32).reshape(-1))
    if a.shape[0] % 2:
        raise ValueError("a range list holds (start, end) pairs")
    return a, a.shape[0] // 2


def fwd(q, k, v, tile_m, tile_n, tau, scale, mask_in=None, want_mask_out=True, rows=None,
        nthreads=None, lib=None, must_do=None, must_skip=None):
    """fp64 oracle forward on BSHD q [B,Nq,H,D] and k, v [B,Nk,H,D] (torch or numpy;
    bf16/fp32/fp64).

    mask_in: [B*H*Tq, W] words (int32 or uint32) or None (nothing skipped).
    rows:    row ids (b*H + h)*Tq + qt to compute, or None for all rows.
    must_do, must_skip: flat lists [start_0, end_0, start_1, end_1, ...] of key
             token ranges ([README] must_do_list / must_skip_list), or None.
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
    Nk = ka.shape[1]
    if ka.shape != (B, Nk, H, D) or va.shape != ka.shape:
        raise ValueError("q, k, v shapes differ")
    Tq, Tk = -(-N // tile_m), -(-Nk // tile_n)
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
    do_a, n_do = _ranges(must_do)
    sk_a, n_sk = _ranges(must_skip)
    rc = lib.oracle_fwd(B, N, Nk, H, D, tile_m, tile_n, dt, _ptr(qa), _ptr(ka), _ptr(va), _ptr(m_in),
                        int(bool(want_mask_out)), float(tau), float(scale),
                        _ptr(do_a), n_do, _ptr(sk_a), n_sk, _ptr(rows_a), nr,
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


def tile_flags(nk, tile_n, must_do=None, must_skip=None):
    """Per key tile: (must_do, must_skip) booleans from token ranges ([README]
    must_do_list / must_skip_list: pairs (start, end), start inclusive, end
    exclusive, descending, so pair i covers tokens end_i < t <= start_i).
    A tile is must-do when any of its keys is in a must-do range, must-skip
    when all of its keys are in must-skip ranges."""
    tk = -(-nk // tile_n)
    def covered(rg):
        c = np.zeros(nk, bool)
        if rg is not None:
            a = np.asarray(rg, np.int64).reshape(-1, 2)
            for start, end in a:
                for t in range(max(end + 1, 0), min(start, nk - 1) + 1):
                    c[t] = True
        return c
    cd, cs = covered(must_do), covered(must_skip)
    do = np.array([cd[kt * tile_n:(kt + 1) * tile_n].any() for kt in range(tk)], bool)
    sk = np.array([must_skip is not None and len(must_skip) > 0 and cs[kt * tile_n:(kt + 1) * tile_n].all()
                   for kt in range(tk)], bool)
    return do, sk


def skiplist(mask, tk, must_do_tiles=None, must_skip_tiles=None):
    """Skip-List of each mask row: [count, live k-tiles in visiting (descending) order].

    mask: [rows, W] words; returns (counts [rows] int32, lists: list of int arrays).
    A tile is live when its bit is clear ([README] QK-Skip: marked tiles are
    bypassed), or when it is must-do; must-skip tiles (not must-do) are never live.
    must_do_tiles / must_skip_tiles: boolean per tile (see tile_flags) or None.
    """
    m = np.asarray(mask).view(np.uint32)
    counts = np.zeros(m.shape[0], np.int32)
    lists = []
    for r in range(m.shape[0]):
        live = []
        for kt in range(tk - 1, -1, -1):
            marked = (int(m[r, kt // 32]) >> (kt % 32)) & 1
            do = must_do_tiles is not None and must_do_tiles[kt]
            sk = must_skip_tiles is not None and must_skip_tiles[kt]
            if do or not (marked or sk):
                live.append(kt)
        counts[r] = len(live)
        lists.append(np.asarray(live, np.int32))
    return counts, lists


def merge(outs, lses):
    """Combine partial attentions over disjoint key sets by their log-sum-exp
    ([README]: the softmax LSE is returned for combining partial attention
    results).  outs: list of [..., D] arrays, lses: list of matching [...]
    arrays (natural log, -inf for a part with no key).  For each query:
        lse = log(sum_i exp(lse_i)),   out = sum_i exp(lse_i - lse) * out_i
    with out = 0 and lse = -inf when every part is empty.  fp64."""
    L = np.stack([np.asarray(x, np.float64) for x in lses])            # [P, ...]
    O = np.stack([np.asarray(x, np.float64) for x in outs])            # [P, ..., D]
    m = L.max(axis=0)
    empty = np.isneginf(m)
    m_safe = np.where(empty, 0.0, m)
    w = np.exp(L - m_safe)                                              # exp(-inf) = 0
    s = w.sum(axis=0)
    lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, s)))
    out = (w[..., None] * O).sum(axis=0) / np.where(empty, 1.0, s)[..., None]
    out = np.where(empty[..., None], 0.0, out)
    return out, lse


def error_budgets(num_steps, early_step_ratio=0.3):
    """Per-timestep error-budget multipliers, in the form the "Lite Attention
    Temporal Sparse" skill page gives in "Implementation Steps", "Step 3: Error
    Calibration" (the LiteAttention README's "Error Calibration" says only that
    earlier timesteps get stricter bounds; it prints no schedule).

    With n = floor(T * r) early steps (T = num_steps, r = early_step_ratio):
        b_t = min(1, 0.5 + 0.5 * t / n)    for n >= 1,
    i.e. b_0 = 0.5, a rise of 0.5 / n per step, and 1 from t = n on; when
    T * r < 1 there is no early step and every b_t is 1."""
    n = math.floor(num_steps * early_step_ratio)
    if n < 1:
        return [1.0] * num_steps
    return [min(1.0, 0.5 + 0.5 * t / n) for t in range(num_steps)]


def calibrate(steps, tile_m, tile_n, scale, base_error, taus, early_step_ratio=0.3, nthreads=None):
    """Per-timestep thresholds from per-step output-error budgets, on given
    inputs.  [README] "Error Calibration": the timesteps get variable error
    budgets, stricter early; the multipliers are the skill page's (see
    error_budgets), and how a budget picks a threshold is this module's
    reading (the pages do not say).

    steps: list of (q, k, v) per denoising step.  taus: candidate thresholds.
    The budget of step t is base_error * error_budgets(T)[t].  At step t, with
    the mask M_t carried from the steps before (empty at step 0), a candidate
    tau gives the marks M' = mask_out(M_t, tau); its error is
        || attention(M') - attention(nothing skipped) ||_F / || attention(nothing skipped) ||_F
    over the whole step's output -- the deviation, accumulated over all
    earlier steps' marks, that the step would carry once the new marks take
    effect.  The step takes the largest candidate whose error is within its
    budget (-inf, which marks nothing new, when none is), and carries M'.
    Returns a list of dicts (tau, error, budget, sparsity, mask) per step.
    """
    T = len(steps)
    mult = error_budgets(T, early_step_ratio)
    cands = sorted(set(float(t) for t in taus), reverse=True)
    if -math.inf not in cands:
        cands.append(-math.inf)
    mask = None
    out = []
    for t, (q, k, v) in enumerate(steps):
        B, N, H, _ = np.asarray(q.shape)
        dense = fwd(q, k, v, tile_m, tile_n, -math.inf, scale, nthreads=nthreads)
        od, _ = unpack_rows(dense, B, N, H, tile_m)
        norm = float(np.sqrt((od * od).sum()))
        budget = base_error * mult[t]
        pick = None
        for tau in cands:
            r = fwd(q, k, v, tile_m, tile_n, tau, scale, mask_in=mask, nthreads=nthreads)
            m2 = r["mask_out"]
            r2 = fwd(q, k, v, tile_m, tile_n, -math.inf, scale, mask_in=m2, want_mask_out=False, nthreads=nthreads)
            o2, _ = unpack_rows(r2, B, N, H, tile_m)
            err = float(np.sqrt(((o2 - od) ** 2).sum())) / norm if norm > 0 else 0.0
            if err <= budget or tau == -math.inf:   # -inf (nothing new marked) when no candidate fits
                pick = (tau, err, m2)
                break
        tau, err, m2 = pick
        tk = -(-k.shape[1] // tile_n)
        bits = np.unpackbits(m2.view(np.uint8), bitorder="little").reshape(m2.shape[0], -1)[:, :tk]
        out.append({"tau": tau, "error": err, "budget": budget, "sparsity": float(bits.mean()), "mask": m2})
        mask = m2
    return out
