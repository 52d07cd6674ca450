"""Independent checks of the CPU oracle (shared by the pin tests and the mutant test).

Each check compares the oracle with something other than itself:
  * dense softmax attention written with numpy (the method with nothing
    skipped is plain attention; with a mask it is attention with the skipped
    tiles' logits at -inf -- the masked-softmax formulation of the skill page);
  * the hand-derived worked examples in tests/golden;
  * a closed form of the running max (max over the later live tiles);
  * consequences the pages fix (monotone masks, the e^tau bound on a marked
    tile's probabilities, the drop bound, invariance under tile size).
"""

import json
import math
import os

import numpy as np
import torch

from oracle import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def bits_of(mask_words, tk):
    m = np.asarray(mask_words).view(np.uint32)
    out = np.zeros((m.shape[0], tk), bool)
    for kt in range(tk):
        out[:, kt] = (m[:, kt // 32] >> np.uint32(kt % 32)) & np.uint32(1)
    return out


def words_of(bits):
    rows, tk = bits.shape
    W = -(-tk // 32)
    w = np.zeros((rows, W), np.uint64)
    for kt in range(tk):
        w[:, kt // 32] |= bits[:, kt].astype(np.uint64) << np.uint64(kt % 32)
    return w.astype(np.uint32)


def to64(x):
    if isinstance(x, torch.Tensor):
        return x.detach().to(torch.float64).cpu().numpy()
    return np.asarray(x, np.float64)


def dense_reference(q, k, v, scale, skip_bits=None, BM=None, BN=None):
    """Brute-force attention with numpy: logits of skipped tiles set to -inf.

    q [B,Nq,H,D], k and v [B,Nk,H,D].  Returns out [B,Nq,H,D], lse [B,H,Nq]
    and the probabilities [B,H,Nq,Nk]."""
    q, k, v = to64(q), to64(k), to64(v)
    B, N, H, D = q.shape
    Nk = k.shape[1]
    s = scale * np.einsum("bnhe,bmhe->bhnm", q, k)
    if skip_bits is not None:
        Tq, Tk = -(-N // BM), -(-Nk // BN)
        sb = np.asarray(skip_bits).reshape(B, H, Tq, Tk)
        full = np.repeat(np.repeat(sb, BM, axis=2), BN, axis=3)[:, :, :N, :Nk]
        s = np.where(full, -np.inf, s)
    m = s.max(axis=-1, keepdims=True)
    mf = np.where(np.isfinite(m), m, 0.0)
    p = np.exp(s - mf)
    l = p.sum(axis=-1, keepdims=True)
    with np.errstate(invalid="ignore", divide="ignore"):
        prob = np.where(l > 0, p / np.where(l > 0, l, 1.0), 0.0)
        lse = np.where(l[..., 0] > 0, mf[..., 0] + np.log(np.where(l[..., 0] > 0, l[..., 0], 1.0)), -np.inf)
    out = np.einsum("bhnm,bmhe->bnhe", prob, v)
    return out, lse, prob


def closed_form_margins(q, k, scale, BM, BN, skip_bits):
    """margin(qt, kt) = max_r [ max_{c in kt} s[r,c] - max_{c in live tiles after kt} s[r,c] ].

    The running max seen by a tile in a last-to-first sweep is the max over the
    live tiles with a larger index; written here as that max, not as a loop
    that updates a running value.  NaN for skipped tiles."""
    q, k = to64(q), to64(k)
    B, N, H, D = q.shape
    Tq, Tk = -(-N // BM), -(-N // BN)
    s = scale * np.einsum("bnhe,bmhe->bhnm", q, k)
    pad = np.full((B, H, Tq * BM, Tk * BN), -np.inf)
    pad[:, :, :N, :N] = s
    tiles = pad.reshape(B, H, Tq, BM, Tk, BN)
    loc = tiles.max(axis=5)                        # [B,H,Tq,BM,Tk] local row max
    sb = skip_bits.reshape(B, H, Tq, Tk)
    live_loc = np.where(sb[:, :, :, None, :], -np.inf, loc)
    out = np.full((B, H, Tq, Tk), np.nan)
    for kt in range(Tk):
        later = live_loc[..., kt + 1:].max(axis=-1) if kt + 1 < Tk else np.full(loc.shape[:-1], -np.inf)
        with np.errstate(invalid="ignore"):
            d = loc[..., kt] - later                    # [B,H,Tq,BM]
        valid_rows = (np.arange(Tq)[:, None] * BM + np.arange(BM)[None, :]) < N   # [Tq,BM]
        d = np.where(valid_rows[None, None], d, -np.inf)
        mg = d.max(axis=-1)
        out[..., kt] = np.where(sb[..., kt], np.nan, mg)
    return out.reshape(B * H * Tq, Tk)


def load_golden():
    with open(os.path.join(GOLDEN, "qkskip_worked_examples.json")) as f:
        return json.load(f)


def _tau(x):
    return -math.inf if x == "-inf" else float(x)


def run_golden(lib=None):
    """Run every worked example; return a list of failure strings."""
    doc = load_golden()
    fails = []
    rng = np.random.default_rng(0)
    for case in doc["cases"]:
        N, BM, BN = case["N"], case["BM"], case["BN"]
        qm = np.asarray(case["q"], np.float64)[None, :, None, :]        # [1,N,1,N]
        km = np.eye(N)[None, :, None, :]
        vm = rng.standard_normal((1, N, 1, N))
        Tq, Tk = -(-N // BM), -(-N // BN)
        variants = [("checks", case["mask_in"])]
        if "checks_without_mask_in" in case:
            variants.append(("checks_without_mask_in", []))
        for key, skipped in variants:
            bits = np.zeros((Tq, Tk), bool)
            for qt, kt in skipped:
                bits[qt, kt] = True
            for chk in case[key]:
                tau = _tau(chk["tau"])
                r = oracle.fwd(qm, km, vm, BM, BN, tau, 1.0, mask_in=words_of(bits), lib=lib)
                newly = bits_of(r["mask_out"], Tk) & ~bits
                want = np.zeros((Tq, Tk), bool)
                for qt, kt in chk["newly"]:
                    want[qt, kt] = True
                if not np.array_equal(newly, want):
                    fails.append("%s/%s tau=%s: newly %s want %s" % (case["name"], key, chk["tau"],
                                                                    np.argwhere(newly).tolist(), chk["newly"]))
                for tile, val in chk.get("margins", {}).items():
                    qt, kt = (int(x) for x in tile.split(","))
                    got = r["margin"][qt, kt]
                    exp_v = math.inf if val == "inf" else float(val)
                    if not (got == exp_v):
                        fails.append("%s/%s margin %s = %r want %r" % (case["name"], key, tile, got, exp_v))
                # the output of every worked example is plain masked attention
                o_ref, _, _ = dense_reference(qm, km, vm, 1.0, bits.reshape(-1, Tk), BM, BN)
                o, _ = oracle.unpack_rows(r, 1, N, 1, BM)
                if not np.allclose(o, o_ref, atol=1e-12, rtol=0):
                    fails.append("%s/%s: output differs from masked dense attention" % (case["name"], key))
    return fails


def random_case(seed, B, N, H, D, scale_in=1.0, dtype=torch.float64):
    g = torch.Generator().manual_seed(seed)
    q = (scale_in * torch.randn(B, N, H, D, generator=g, dtype=torch.float64)).to(dtype)
    k = (scale_in * torch.randn(B, N, H, D, generator=g, dtype=torch.float64)).to(dtype)
    v = torch.randn(B, N, H, D, generator=g, dtype=torch.float64).to(dtype)
    return q, k, v


def check_dense(lib=None, cases=None):
    """tau = -inf and an empty mask: the oracle is plain softmax attention."""
    fails = []
    cases = cases or [(0, 2, 37, 3, 8, 8, 4), (1, 1, 64, 2, 16, 16, 16), (2, 1, 5, 1, 4, 4, 2),
                      (3, 2, 100, 2, 8, 32, 16), (4, 1, 1, 1, 4, 4, 4), (5, 1, 70, 1, 32, 16, 64)]
    for seed, B, N, H, D, BM, BN in cases:
        q, k, v = random_case(seed, B, N, H, D, scale_in=1.5)
        scale = 1.0 / math.sqrt(D)
        r = oracle.fwd(q, k, v, BM, BN, -math.inf, scale, lib=lib)
        o, lse = oracle.unpack_rows(r, B, N, H, BM)
        o_ref, lse_ref, _ = dense_reference(q, k, v, scale)
        if not np.allclose(o, o_ref, atol=1e-12, rtol=1e-12):
            fails.append("dense out case %d: max err %.3g" % (seed, np.abs(o - o_ref).max()))
        if not np.allclose(lse, lse_ref, atol=1e-12, rtol=1e-12):
            fails.append("dense lse case %d" % seed)
        if np.any(bits_of(r["mask_out"], -(-N // BN))):
            fails.append("dense case %d marked a tile at tau=-inf" % seed)
    return fails


def check_masked_and_rule(lib=None, seeds=range(6)):
    """Random masks and thresholds: masked dense attention, closed-form margins,
    monotone masks, the e^tau bound and the first-visited-tile rule."""
    fails = []
    for seed in seeds:
        rng = np.random.default_rng(100 + seed)
        B, H = 1 + seed % 2, 1 + seed % 3
        N = int(rng.integers(9, 90))
        D = int(rng.choice([4, 8, 16]))
        BM, BN = int(rng.choice([4, 8, 16])), int(rng.choice([4, 8, 16]))
        q, k, v = random_case(seed, B, N, H, D, scale_in=2.0)
        scale = 1.0 / math.sqrt(D)
        Tq, Tk = -(-N // BM), -(-N // BN)
        bits = rng.random((B * H * Tq, Tk)) < 0.3
        tau = float(rng.choice([-4.0, -2.0, -1.0, -0.25]))
        r = oracle.fwd(q, k, v, BM, BN, tau, scale, mask_in=words_of(bits), lib=lib)
        o, lse = oracle.unpack_rows(r, B, N, H, BM)
        o_ref, lse_ref, prob = dense_reference(q, k, v, scale, bits, BM, BN)
        if not np.allclose(o, o_ref, atol=1e-12, rtol=1e-12):
            fails.append("masked out seed %d err %.3g" % (seed, np.nanmax(np.abs(o - o_ref))))
        if not np.array_equal(np.isneginf(lse), np.isneginf(lse_ref)) or not np.allclose(
                np.where(np.isfinite(lse), lse, 0), np.where(np.isfinite(lse_ref), lse_ref, 0), atol=1e-12):
            fails.append("masked lse seed %d" % seed)
        cf = closed_form_margins(q, k, scale, BM, BN, bits)
        got = r["margin"]
        same_nan = np.array_equal(np.isnan(got), np.isnan(cf))
        fin = np.isfinite(cf) & np.isfinite(got)
        if not same_nan or not np.array_equal(np.isposinf(got), np.isposinf(cf)) or \
                not np.allclose(got[fin], cf[fin], atol=1e-9, rtol=0):
            fails.append("margins differ from closed form, seed %d" % seed)
        out_bits = bits_of(r["mask_out"], Tk)
        if np.any(bits & ~out_bits):
            fails.append("mask_out dropped an input mark, seed %d" % seed)
        newly = out_bits & ~bits
        want = (~bits) & (np.nan_to_num(cf, nan=np.inf) < tau)
        clear = np.abs(np.nan_to_num(cf, nan=np.inf, posinf=1e300) - tau) > 1e-9
        if np.any((newly != want) & clear):
            fails.append("decisions differ from the closed form, seed %d" % seed)
        # a newly marked tile: each of its probabilities this step is below e^tau
        pb = prob.reshape(B * H, N, N)
        for row, kt in np.argwhere(newly):
            bh, qt = divmod(int(row), Tq)
            rr = slice(qt * BM, min(N, (qt + 1) * BM))
            cc = slice(kt * BN, min(N, (kt + 1) * BN))
            if not np.all(pb[bh, rr, cc] < math.exp(tau)):
                fails.append("marked tile above e^tau, seed %d" % seed)
                break
        # the first visited live tile of a row is never marked; a row with a live
        # tile keeps at least one
        for row in range(B * H * Tq):
            live = [kt for kt in range(Tk - 1, -1, -1) if not bits[row, kt]]
            if live and newly[row, live[0]]:
                fails.append("first visited tile marked, seed %d row %d" % (seed, row))
            if live and out_bits[row].all():
                fails.append("row emptied by the rule, seed %d row %d" % (seed, row))
    return fails


def check_tile_invariance(lib=None):
    """With nothing skipped the output does not depend on the tile grid."""
    q, k, v = random_case(7, 1, 77, 2, 8, scale_in=1.5)
    outs = []
    for BM, BN in ((4, 4), (8, 16), (32, 8), (128, 128)):
        r = oracle.fwd(q, k, v, BM, BN, -math.inf, 0.5, lib=lib)
        outs.append(oracle.unpack_rows(r, 1, 77, 2, BM)[0])
    return [] if all(np.allclose(outs[0], o, atol=1e-13) for o in outs[1:]) else ["tile-size dependence"]


def check_edge_cases(lib=None):
    """Padding bits past the last tile are cleared; a fully skipped row gives 0 / -inf;
    an input mark is never removed."""
    fails = []
    q, k, v = random_case(2, 1, 40, 1, 4)            # Tk = 5 with 8-wide tiles
    words = np.full((5, 1), 0xFFFFFFE0, np.uint32)   # only padding bits set
    r = oracle.fwd(q, k, v, 8, 8, -math.inf, 0.5, mask_in=words, lib=lib)
    if np.any(r["mask_out"] != 0):
        fails.append("padding bits survive")
    q, k, v = random_case(1, 1, 16, 1, 4)
    bits = np.ones((2, 2), bool)
    r = oracle.fwd(q, k, v, 8, 8, -3.0, 0.5, mask_in=words_of(bits), lib=lib)
    if not (np.all(r["out"] == 0) and np.all(np.isneginf(r["lse"]))):
        fails.append("fully skipped row")
    if not np.array_equal(bits_of(r["mask_out"], 2), bits):
        fails.append("input marks lost")
    return fails


def check_nonsquare(lib=None):
    """Queries and keys of different lengths (the text/video partial attentions
    and K/V splits of the pages): plain and masked attention, by brute force."""
    fails = []
    for seed, B, Nq, Nk, H, D, BM, BN in ((0, 1, 20, 53, 2, 8, 8, 16), (1, 2, 61, 9, 1, 4, 16, 4),
                                          (2, 1, 7, 100, 1, 8, 4, 32)):
        g = torch.Generator().manual_seed(300 + seed)
        q = 1.5 * torch.randn(B, Nq, H, D, generator=g, dtype=torch.float64)
        k = 1.5 * torch.randn(B, Nk, H, D, generator=g, dtype=torch.float64)
        v = torch.randn(B, Nk, H, D, generator=g, dtype=torch.float64)
        scale = 1.0 / math.sqrt(D)
        Tq, Tk = -(-Nq // BM), -(-Nk // BN)
        rng = np.random.default_rng(seed)
        for bits in (None, rng.random((B * H * Tq, Tk)) < 0.3):
            r = oracle.fwd(q, k, v, BM, BN, -2.0, scale, mask_in=None if bits is None else words_of(bits), lib=lib)
            o, lse = oracle.unpack_rows(r, B, Nq, H, BM)
            o_ref, lse_ref, _ = dense_reference(q, k, v, scale, bits, BM, BN)
            if not np.allclose(o, o_ref, atol=1e-12, rtol=1e-12):
                fails.append("non-square out case %d (masked=%s)" % (seed, bits is not None))
            fin = np.isfinite(lse_ref)
            if not (np.array_equal(fin, np.isfinite(lse)) and np.allclose(lse[fin], lse_ref[fin], atol=1e-12)):
                fails.append("non-square lse case %d" % seed)
    return fails


def load_range_golden():
    with open(os.path.join(GOLDEN, "token_ranges_examples.json")) as f:
        return json.load(f)


def check_ranges(lib=None):
    """must_do_list / must_skip_list: the hand-derived tile sets of the pages'
    examples, the output as brute-force attention over the visited tiles, and
    the rule that must-do tiles are never marked."""
    fails = []
    doc = load_range_golden()
    rng = np.random.default_rng(7)
    for case in doc["cases"]:
        N, BN = case["N"], case["BN"]
        Tk = -(-N // BN)
        BM = 8
        Tq = -(-N // BM)
        g = torch.Generator().manual_seed(len(case["name"]))
        q = 2.0 * torch.randn(1, N, 1, 8, generator=g, dtype=torch.float64)
        k = 2.0 * torch.randn(1, N, 1, 8, generator=g, dtype=torch.float64)
        v = torch.randn(1, N, 1, 8, generator=g, dtype=torch.float64)
        do_t = np.zeros(Tk, bool)
        do_t[case.get("must_do_tiles", [])] = True
        sk_t = np.zeros(Tk, bool)
        sk_t[case.get("must_skip_tiles", [])] = True
        for mask_kind in ("empty", "random", "full"):
            if mask_kind == "empty":
                bits = np.zeros((Tq, Tk), bool)
            elif mask_kind == "full":
                bits = np.ones((Tq, Tk), bool)
            else:
                bits = rng.random((Tq, Tk)) < 0.4
            for tau in (-math.inf, -1.0, 1e30):
                r = oracle.fwd(q, k, v, BM, BN, tau, 0.4, mask_in=words_of(bits), lib=lib,
                               must_do=case.get("must_do"), must_skip=case.get("must_skip"))
                eff = (bits | sk_t[None, :]) & ~do_t[None, :]
                o, _ = oracle.unpack_rows(r, 1, N, 1, BM)
                o_ref, _, _ = dense_reference(q, k, v, 0.4, eff, BM, BN)
                if not np.allclose(o, o_ref, atol=1e-12):
                    fails.append("%s (%s mask, tau %g): output is not attention over the visited tiles"
                                 % (case["name"], mask_kind, tau))
                out_bits = bits_of(r["mask_out"], Tk)
                newly = out_bits & ~bits
                if np.any(newly & do_t[None, :]):
                    fails.append("%s: a must-do tile was marked" % case["name"])
                if np.any(newly & eff):
                    fails.append("%s: a tile that was not visited was marked" % case["name"])
                if np.any(bits & ~out_bits):
                    fails.append("%s: an input mark was dropped" % case["name"])
                if tau == 1e30:
                    # every visited tile but the first of its row and the must-do ones is marked
                    for row in range(Tq):
                        vis = [kt for kt in range(Tk - 1, -1, -1) if not eff[row, kt]]
                        want = set(kt for kt in vis[1:] if not do_t[kt])
                        if set(np.flatnonzero(newly[row]).tolist()) != want:
                            fails.append("%s: marks at tau=+big, row %d" % (case["name"], row))
                            break
    return fails


ALL_CHECKS = (run_golden, check_dense, check_masked_and_rule, check_tile_invariance, check_edge_cases,
              check_nonsquare, check_ranges)


# ---- checks of the oracle's Python helpers (Skip-List reference, tile flags,
# LSE merge, error budgets, calibration).  They look the oracle up through this
# module's global, so a test can substitute a variant of it.

def check_tile_flags():
    """The tile sets derived by hand from the README's range examples."""
    fails = []
    for case in load_range_golden()["cases"]:
        do, sk = oracle.tile_flags(case["N"], case["BN"], case.get("must_do"), case.get("must_skip"))
        if np.flatnonzero(do).tolist() != case.get("must_do_tiles", []):
            fails.append("tile_flags must-do: " + case["name"])
        if np.flatnonzero(sk).tolist() != case.get("must_skip_tiles", []):
            fails.append("tile_flags must-skip: " + case["name"])
    return fails


def check_skiplist():
    """Skip-List reference: exactly the clear bits of each row, last tile
    first, across word boundaries; must-do beats a mark and must-skip,
    must-skip drops an unmarked tile."""
    fails = []
    rng = np.random.default_rng(0)
    for tk in (1, 5, 31, 32, 33, 70):
        bits = rng.random((6, tk)) < 0.4
        counts, lists = oracle.skiplist(words_of(bits), tk)
        for r in range(6):
            if counts[r] != (~bits[r]).sum() or list(lists[r]) != sorted(np.flatnonzero(~bits[r]).tolist(),
                                                                          reverse=True):
                fails.append("skiplist: Tk %d row %d" % (tk, r))
                break
    do = np.array([True, False, False, True, False])
    sk = np.array([False, True, False, True, False])
    bits = np.array([[1, 0, 0, 1, 0], [0, 0, 1, 0, 1]], bool)
    counts, lists = oracle.skiplist(words_of(bits), 5, do, sk)
    # row 0: 3 is must-do (beats its mark and its must-skip), 1 is must-skip
    # row 1: 4 and 2 are marked, 1 is must-skip
    if [list(x) for x in lists] != [[4, 3, 2, 0], [3, 0]] or list(counts) != [4, 2]:
        fails.append("skiplist with tile flags")
    return fails


def check_merge():
    """LSE merge: attention over a partition of the keys, merged, is attention
    over all keys (brute force), also through the oracle forward with an empty
    part; all parts empty give 0 and -inf; shifting every part's lse by the
    same constant (far outside exp's range) shifts the result and leaves the
    output unchanged."""
    fails = []
    g = torch.Generator().manual_seed(21)
    B, Nq, Nk, H, D = 2, 30, 70, 2, 8
    q = 1.5 * torch.randn(B, Nq, H, D, generator=g, dtype=torch.float64)
    k = 1.5 * torch.randn(B, Nk, H, D, generator=g, dtype=torch.float64)
    v = torch.randn(B, Nk, H, D, generator=g, dtype=torch.float64)
    scale = 0.4
    o_ref, lse_ref, _ = dense_reference(q, k, v, scale)
    lse_ref = np.transpose(lse_ref, (0, 2, 1))                    # [B, Nq, H] to match out[..., :]
    outs, lses = [], []
    for a, b in zip([0, 16, 17, 48], [16, 17, 48, 70]):
        o, lse, _ = dense_reference(q, k[:, a:b], v[:, a:b], scale)
        outs.append(o)
        lses.append(np.transpose(lse, (0, 2, 1)))
    out, lse = oracle.merge(outs, lses)
    if not (np.allclose(out, o_ref, atol=1e-12) and np.allclose(lse, lse_ref, atol=1e-12)):
        fails.append("merge of key splits is not full attention")
    with np.errstate(over="ignore", invalid="ignore"):
        for c in (1000.0, -1000.0):
            out2, lse2 = oracle.merge(outs, [x + c for x in lses])
            if not (np.allclose(out2, o_ref, atol=1e-12) and np.allclose(lse2, lse_ref + c, atol=1e-9)):
                fails.append("merge is not shift invariant (shift %g)" % c)
    outs, lses = [], []
    for a, b in ((0, 32), (32, 32), (32, 70)):
        r = oracle.fwd(q, k[:, a:b], v[:, a:b], 8, 16, -math.inf, scale)
        o, l = oracle.unpack_rows(r, B, Nq, H, 8)
        outs.append(o)
        lses.append(np.transpose(l, (0, 2, 1)))
    out, lse = oracle.merge(outs, lses)
    if not (np.allclose(out, o_ref, atol=1e-12) and np.allclose(lse, lse_ref, atol=1e-12)):
        fails.append("merge of forward partials with an empty part")
    out, lse = oracle.merge([np.ones((3, 4))] * 2, [np.full(3, -np.inf)] * 2)
    if not (np.all(out == 0) and np.all(np.isneginf(lse))):
        fails.append("merge of empty parts")
    return fails


def check_error_budgets():
    """Budget multipliers of the skill page "Lite Attention Temporal Sparse"
    (Implementation Steps, Step 3: Error Calibration), value by value: over
    the first floor(T*ratio) steps the multiplier goes 0.5 + 0.5*t/floor(T*ratio),
    later steps get 1.0, and with no early step every step gets 1.0."""
    fails = []
    b = oracle.error_budgets(50, 0.3)
    if not (len(b) == 50 and b[0] == 0.5 and b[1] == 0.5 + 0.5 / 15 and b[14] == 0.5 + 0.5 * 14 / 15
            and all(x == 1.0 for x in b[15:]) and b[:15] == sorted(b[:15])):
        fails.append("error budgets, 50 steps")
    if oracle.error_budgets(3, 0.3) != [1.0, 1.0, 1.0]:                 # int(0.9) = 0 early steps
        fails.append("error budgets, 3 steps")
    if oracle.error_budgets(10, 0.5)[:5] != [0.5, 0.6, 0.7, 0.8, 0.9]:
        fails.append("error budgets, 10 steps")
    return fails


def calib_inputs(steps=3, N=96, H=2, D=8, seed=0):
    """A tiny drifting trajectory with a locality bias, so thresholds matter."""
    g = torch.Generator().manual_seed(seed)
    pos = torch.arange(N, dtype=torch.float64)
    feat = torch.stack([torch.cos(pos / 6.0 * (j + 1)) for j in range(D)], -1)    # smooth in the position
    q0 = 3.0 * feat[None, :, None, :].expand(1, N, H, D) + torch.randn(1, N, H, D, generator=g, dtype=torch.float64)
    k0 = 3.0 * feat[None, :, None, :].expand(1, N, H, D) + torch.randn(1, N, H, D, generator=g, dtype=torch.float64)
    v0 = torch.randn(1, N, H, D, generator=g, dtype=torch.float64)
    out = []
    for t in range(steps):
        out.append((q0 + 0.05 * t * torch.randn(1, N, H, D, generator=g, dtype=torch.float64),
                    k0 + 0.05 * t * torch.randn(1, N, H, D, generator=g, dtype=torch.float64), v0))
    return out


def check_calibration():
    """Re-evaluated by brute force at every step: the chosen tau's error is
    within its budget and every larger candidate's is not (numpy attention over
    the visited tiles against numpy dense attention, with the mask carried from
    the earlier steps); an unbounded budget takes the largest candidate and a
    zero budget lets no new mark change the output."""
    fails = []
    steps = calib_inputs()
    BM = BN = 16
    taus = [0.0, -1.0, -2.0, -3.0, -5.0, -8.0]
    scale = 0.35
    # ratio 0.67 over 3 steps: int(2.01) = 2 early steps, multipliers 0.5, 0.75, 1.0
    res = oracle.calibrate(steps, BM, BN, scale, base_error=0.02, taus=taus, early_step_ratio=0.67)
    budgets = [0.5, 0.75, 1.0]
    mask = np.zeros((2 * 6, 1), np.uint32)
    saw_skip = False
    for t, ((q, k, v), r) in enumerate(zip(steps, res)):
        if r["budget"] != 0.02 * budgets[t]:
            fails.append("calibration budget, step %d" % t)
        o_dense, _, _ = dense_reference(q, k, v, scale)
        norm = np.sqrt((o_dense ** 2).sum())
        for tau in sorted(taus + [-math.inf], reverse=True):
            m2 = oracle.fwd(q, k, v, BM, BN, tau, scale, mask_in=mask)["mask_out"]
            o2, _, _ = dense_reference(q, k, v, scale, bits_of(m2, 6), BM, BN)
            err = np.sqrt(((o2 - o_dense) ** 2).sum()) / norm
            if tau > r["tau"]:
                if err <= r["budget"]:
                    fails.append("calibration skipped a feasible larger tau %g, step %d" % (tau, t))
            elif tau == r["tau"]:
                if abs(err - r["error"]) > 1e-12 or not (err <= r["budget"] or tau == -math.inf):
                    fails.append("calibration error of the chosen tau, step %d" % t)
                if not np.array_equal(np.asarray(r["mask"]).view(np.uint32), m2):
                    fails.append("calibration carries the wrong mask, step %d" % t)
                break
        saw_skip = saw_skip or r["sparsity"] > 0
        mask = np.asarray(r["mask"]).view(np.uint32)
    if not saw_skip:
        fails.append("calibration never marked a tile")
    steps = calib_inputs(steps=2)
    taus = [0.0, -2.0, -6.0]
    if [r["tau"] for r in oracle.calibrate(steps, 16, 16, 0.35, math.inf, taus)] != [0.0, 0.0]:
        fails.append("calibration with an unbounded budget")
    if any(r["error"] != 0.0 for r in oracle.calibrate(steps, 16, 16, 0.35, 0.0, taus)):
        fails.append("calibration with a zero budget")
    # marks accumulate across steps: a second step whose keys sit half a
    # sequence away from the first's keeps every mark the first step made
    (q, k, v), _ = steps
    moved = (q, torch.roll(k, 48, dims=1), torch.roll(v, 48, dims=1))
    res = oracle.calibrate([(q, k, v), moved], 16, 16, 0.35, math.inf, taus)
    b0, b1 = bits_of(res[0]["mask"], 6), bits_of(res[1]["mask"], 6)
    want = oracle.fwd(*moved, 16, 16, 0.0, 0.35, mask_in=res[0]["mask"])["mask_out"]
    if not b0.any() or np.any(b0 & ~b1) or not np.array_equal(np.asarray(res[1]["mask"]).view(np.uint32), want):
        fails.append("calibration does not carry the marks of earlier steps")
    return fails


PY_CHECKS = (check_tile_flags, check_skiplist, check_merge, check_error_budgets, check_calibration)
