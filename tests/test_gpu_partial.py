"""GPU parity of the partial-attention features against the CPU oracle:
queries and keys of different lengths, sequence slices passed by batch stride
(the text/video split), must-do / must-skip key ranges on both live-tile
paths, the LSE merge, and one GPU's share of the sequence-parallel K/V split.

Bars as in the other parity tests: outputs within 2e-2 (bf16) / 1e-5 (fp32)
max-abs, lse within 1e-3 / 1e-5, masks bit-exact except tiles whose oracle
margin is within 1e-3 of tau.  Inputs are the seeded locality-biased
video-token tensors; every mask_in comes from the generator or the oracle.
"""

import math
import sys

import numpy as np
import pytest
import torch

from oracle import oracle
from temporal_block_sparse_amd import configs, synth
from temporal_block_sparse_amd import lite_attn as la
from tests import parity as pa

pytestmark = pytest.mark.gpu


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def tokens(grid, heads, head_dim=128, batch=1):
    """Seeded locality-biased bf16 q, k, v [B, N, H, d] (CPU) of a small workload."""
    wl = configs.scaled(configs.C3 if head_dim == 128 else configs.C2, grid, heads=heads, batch=batch, steps=1)
    tr = synth.Trajectory(wl, "cpu")
    return tr.tensors()


def rand_mask(rows, tk, density, seed):
    return synth.random_mask(rows, tk, density, seed).numpy().view(np.uint32).reshape(rows, -1)


def mask_mismatches(got, ref, margin, tau, tk):
    """Tiles whose GPU and oracle marks differ, other than near-tau ties."""
    diff = np.asarray(got).view(np.uint32).reshape(ref.shape) ^ ref
    bad = 0
    for row, w in zip(*np.nonzero(diff)):
        for b in range(32):
            kt = int(w) * 32 + b
            if (int(diff[row, w]) >> b) & 1:
                mg = margin[row, kt] if kt < tk else np.nan
                if not (np.isfinite(mg) and abs(mg - tau) <= pa.NEAR_TAU):
                    bad += 1
    return bad


@pytest.mark.parametrize("D,BN,Nq,Nk", [(128, 128, 300, 1100), (128, 64, 1000, 129), (64, 128, 129, 1000),
                                        (64, 64, 700, 333)])
@pytest.mark.parametrize("skiplist", [False, True])
def test_queries_and_keys_of_different_lengths(D, BN, Nq, Nk, skiplist):
    q, k, v = tokens((8, 12, 12), 2, head_dim=D)                     # N = 1152
    q, k, v = q[:, :Nq].contiguous(), k[:, -Nk:].contiguous(), v[:, -Nk:].contiguous()
    Tq, Tk = -(-Nq // 128), -(-Nk // BN)
    mask = rand_mask(2 * Tq, Tk, 0.3, seed=Nq + Nk)
    log("  D %d BN %d Nq %d Nk %d skiplist %s" % (D, BN, Nq, Nk, skiplist))
    stats, _ = pa.check_full(q, k, v, 128, BN, -3.0, 1.0 / math.sqrt(D), mask_in=mask, use_skiplist=skiplist)
    log("   ", stats)


def test_fp32_queries_and_keys_of_different_lengths():
    g = torch.Generator().manual_seed(3)
    q = 1.5 * torch.randn(1, 300, 2, 64, generator=g)
    k = 1.5 * torch.randn(1, 700, 2, 64, generator=g)
    v = torch.randn(1, 700, 2, 64, generator=g)
    mask = rand_mask(2 * 5, 11, 0.3, seed=9)
    stats, _ = pa.check_full(q, k, v, 64, 64, -3.0, 0.125, mask_in=mask)
    log("  fp32 Nq 300 Nk 700", stats)


def test_no_keys_gives_zero_and_minus_inf():
    dev = torch.device("cuda")
    q = torch.randn(1, 200, 2, 128, device=dev).to(torch.bfloat16)
    k = torch.empty(1, 0, 2, 128, device=dev, dtype=torch.bfloat16)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((1, 2, 200), float("nan"), device=dev)
    la.lite_attn_fwd(q, k, k, out, tile_m=128, tile_n=128, tau=-3.0, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))


def _partial(q, k, v, BN, tau, mask, scale):
    """Oracle (out [B,Nq,H,D], lse [B,H,Nq], mask_out) of one partial attention."""
    B, Nq, H, _ = q.shape
    r = oracle.fwd(q, k, v, 128, BN, tau, scale, mask_in=mask)
    o, l = oracle.unpack_rows(r, B, Nq, H, 128)
    return o, l, r


def test_text_video_partial_attentions_and_merge():
    """The README's text/video example: t2t, t2v, v2t without skipping, v2v with
    a mask and tau, all on slices of the full tensors (batch strides, no copies),
    then the text and video queries' parts merged by LSE."""
    B, H, D, T = 2, 2, 128, 200
    q, k, v = tokens((6, 10, 16), H, head_dim=D, batch=B)             # N = 960 video + text at the front
    N = q.shape[1]
    scale = 1.0 / math.sqrt(D)
    dev = torch.device("cuda")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    out_full = torch.full_like(qd, float("nan"))
    Nv = N - T
    Tqv, Tkv = -(-Nv // 128), -(-Nv // 128)
    mask_vv = rand_mask(B * H * Tqv, Tkv, 0.3, seed=12)
    parts = {}
    for name, (qs, ks) in {"t2t": (slice(0, T), slice(0, T)), "t2v": (slice(0, T), slice(T, N)),
                           "v2t": (slice(T, N), slice(0, T)), "v2v": (slice(T, N), slice(T, N))}.items():
        mi = mask_vv if name == "v2v" else None
        tau = -3.0 if name == "v2v" else -math.inf
        nq = qs.stop - qs.start
        o = torch.full((B, nq, H, D), float("nan"), device=dev, dtype=qd.dtype)
        lse = torch.full((B, H, nq), float("nan"), device=dev)
        mo = None
        if mi is not None:
            mi_d = torch.as_tensor(mi.view(np.int32).reshape(-1)).to(dev)
            mo = torch.zeros_like(mi_d)
        la.lite_attn_fwd(qd[:, qs], kd[:, ks], vd[:, ks], o, tile_m=128, tile_n=128, tau=tau, softmax_scale=scale,
                         mask_in=mi_d if mi is not None else None, mask_out=mo, lse=lse)
        torch.cuda.synchronize()
        oo, lo, ro = _partial(q[:, qs].contiguous(), k[:, ks].contiguous(), v[:, ks].contiguous(), 128, tau, mi,
                              scale)
        got_o = o.cpu().double().numpy()
        assert np.abs(got_o - oo).max() <= 2e-2, name
        lg = lse.cpu().double().numpy()
        assert np.array_equal(np.isneginf(lg), np.isneginf(lo))
        fin = np.isfinite(lo)
        assert np.abs(lg[fin] - lo[fin]).max() <= 1e-3, name
        if mo is not None:
            assert mask_mismatches(mo.cpu().numpy(), ro["mask_out"], ro["margin"], tau, Tkv) == 0, name
        parts[name] = (o, lse, oo, lo)
    # merge into slices of the full output tensor (strided out)
    for qs, names in ((slice(0, T), ("t2t", "t2v")), (slice(T, N), ("v2t", "v2v"))):
        lse_m = torch.full((B, H, qs.stop - qs.start), float("nan"), device=dev)
        la.lite_attn_merge([parts[n][0] for n in names], [parts[n][1] for n in names], out_full[:, qs], lse_m)
        torch.cuda.synchronize()
        ref_o, ref_l = oracle.merge([parts[n][2] for n in names],
                                    [np.transpose(parts[n][3], (0, 2, 1)) for n in names])
        got = out_full[:, qs].cpu().double().numpy()
        assert np.abs(got - ref_o).max() <= 2e-2
        lm = np.transpose(lse_m.cpu().double().numpy(), (0, 2, 1))
        assert np.abs(lm - ref_l).max() <= 1e-3
    # with nothing skipped the merged result is full attention over all tokens
    r = oracle.fwd(q, k, v, 128, 128, -math.inf, scale, rows=None)
    full, _ = oracle.unpack_rows(r, B, N, H, 128)
    assert np.abs(out_full[:, :T].cpu().double().numpy() - full[:, :T]).max() <= 2e-2


@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.bfloat16, 64), (torch.float32, 64),
                                     (torch.float32, 128)])
@pytest.mark.parametrize("nparts", [1, 3, 8])
def test_merge_kernel(dtype, D, nparts):
    g = torch.Generator().manual_seed(nparts * 7 + D)
    B, N, H = 2, 333, 3
    outs = [torch.randn(B, N, H, D, generator=g).to(dtype) for _ in range(nparts)]
    lses = [3.0 * torch.randn(B, H, N, generator=g) for _ in range(nparts)]
    lses[0][0, 1, :50] = -math.inf                          # a part with no key for some queries
    for l in lses:
        l[1, 2, 7] = -math.inf                              # a query no part has a key for
    dev = torch.device("cuda")
    od = [o.to(dev) for o in outs]
    ld = [l.to(dev) for l in lses]
    out = torch.full_like(od[0], float("nan"))
    lse = torch.full_like(ld[0], float("nan"))
    la.lite_attn_merge(od, ld, out, lse)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.merge([o.double().numpy() for o in outs],
                                [np.transpose(l.double().numpy(), (0, 2, 1)) for l in lses])
    tol = 2e-2 if dtype == torch.bfloat16 else 1e-5
    assert np.abs(out.cpu().double().numpy() - ref_o).max() <= tol
    gl = np.transpose(lse.cpu().double().numpy(), (0, 2, 1))
    assert np.array_equal(np.isneginf(gl), np.isneginf(ref_l))
    fin = np.isfinite(ref_l)
    assert np.abs(gl[fin] - ref_l[fin]).max() <= 1e-5
    assert torch.all(out.cpu()[1, 7, 2] == 0)
    # in place: the merged result written over part 0 and its lse
    la.lite_attn_merge(od, ld, od[0], ld[0])
    torch.cuda.synchronize()
    assert torch.equal(od[0].cpu(), out.cpu())
    assert torch.equal(ld[0].cpu(), lse.cpu())


@pytest.mark.parametrize("skiplist", [False, True])
@pytest.mark.parametrize("BN", [64, 128])
def test_must_do_and_must_skip_ranges(skiplist, BN):
    """The README's range examples scaled to a 1152-token sequence, on a random
    mask and a trajectory step: outputs, lse and marks match the oracle."""
    q, k, v = tokens((8, 12, 12), 2)
    N = q.shape[1]
    scale = 1.0 / math.sqrt(128)
    must_do = [800, 600, 450, 400, 120, 20]
    must_skip = [1100, 900, 300, 129]
    Tq, Tk = -(-N // 128), -(-N // BN)
    mask = rand_mask(2 * Tq, Tk, 0.4, seed=BN)
    for tau in (-3.0, -0.5):
        stats, orc = pa.check_full(q, k, v, 128, BN, tau, scale, mask_in=mask, use_skiplist=skiplist,
                                   must_do=must_do, must_skip=must_skip)
        log("  ranges BN %d skiplist %s tau %g" % (BN, skiplist, tau), stats)
        do_t, sk_t = oracle.tile_flags(N, BN, must_do, must_skip)
        newly = (orc["mask_out"] & ~mask)
        for kt in np.flatnonzero(do_t):
            assert not np.any((newly[:, kt // 32] >> np.uint32(kt % 32)) & np.uint32(1))


def test_skiplist_with_ranges_matches_reference():
    N, BN, rows = 1000, 64, 6
    Tk = -(-N // BN)
    desc = la.make_desc(1, 128 * rows, 1, 128, 128, BN, la.LITE_BF16, seqlen_kv=N)
    mask = rand_mask(rows, Tk, 0.5, seed=4)
    must_do, must_skip = [800, 600, 45, 40], [999, 850, 300, 100]
    dev = torch.device("cuda")
    sl = torch.full((la.lite_attn_skiplist_len(desc),), -7, dtype=torch.int32, device=dev)
    la.lite_attn_build_skiplist(desc, torch.as_tensor(mask.view(np.int32).reshape(-1)).to(dev), sl, must_do,
                                must_skip)
    got = sl.cpu().numpy().reshape(rows, 1 + Tk)
    do_t, sk_t = oracle.tile_flags(N, BN, must_do, must_skip)
    counts, lists = oracle.skiplist(mask, Tk, do_t, sk_t)
    for r in range(rows):
        assert got[r, 0] == counts[r]
        assert list(got[r, 1:1 + counts[r]]) == list(lists[r])


def test_sequence_parallel_share_over_a_trajectory():
    """One GPU's share of the README's SeqParallelLiteAttention: the full
    queries against 3 K/V splits, each split with its own skip state
    (split_idx), over 3 steps of a drifting trajectory; the splits' (out, lse)
    merged by LSE.  Per split and merged, against the oracle run the same way."""
    wl = configs.scaled(configs.C3, (6, 10, 16), heads=2, batch=1, steps=3)
    tr = synth.Trajectory(wl, "cpu")
    N, H, D = wl.seqlen, wl.heads, wl.head_dim
    scale = 1.0 / math.sqrt(D)
    cuts = [0, 384, 640, N]                       # splits of 384, 256 and 320 keys
    sp = la.SeqParallelLiteAttention(num_nodes=3, threshold=-3.0, tile_m=128, tile_n=128)
    masks = [None] * 3
    dev = torch.device("cuda")
    for step in range(3):
        if step:
            tr.advance()
        q, k, v = tr.tensors()
        qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
        outs, lses, o_ref, l_ref = [], [], [], []
        for i in range(3):
            ks = slice(cuts[i], cuts[i + 1])
            if masks[i] is not None:          # every mask_in comes from the oracle's previous step
                sp._splits[i].mask.copy_(torch.from_numpy(masks[i].view(np.int32).reshape(-1)).to(dev))
            o, l = sp(qd, kd[:, ks], vd[:, ks], i, scale=scale, return_softmax_lse=True)
            outs.append(o)
            lses.append(l)
            r = oracle.fwd(q, k[:, ks].contiguous(), v[:, ks].contiguous(), 128, 128, -3.0, scale,
                           mask_in=masks[i])
            oo, lo = oracle.unpack_rows(r, 1, N, H, 128)
            o_ref.append(oo)
            l_ref.append(np.transpose(lo, (0, 2, 1)))
            torch.cuda.synchronize()
            assert np.abs(o.cpu().double().numpy() - oo).max() <= 2e-2, (step, i)
            # the split's own skip state matches the oracle's marks (near-tau ties aside)
            tk = -(-(cuts[i + 1] - cuts[i]) // 128)
            assert mask_mismatches(sp._splits[i].mask.cpu().numpy(), r["mask_out"], r["margin"], -3.0, tk) == 0, \
                (step, i)
            masks[i] = r["mask_out"]
        merged = torch.full_like(qd, float("nan"))
        la.lite_attn_merge(outs, lses, merged)
        torch.cuda.synchronize()
        ref, _ = oracle.merge(o_ref, l_ref)
        err = np.abs(merged.cpu().double().numpy() - ref).max()
        log("  SP share step %d merged err %.4g" % (step, err))
        assert err <= 2e-2


@pytest.mark.parametrize("D,BN", [(128, 128), (64, 64)])
@pytest.mark.parametrize("skiplist", [False, True])
def test_skipped_tiles_contribute_nothing(D, BN, skiplist):
    """Full-Stage Elimination: a k-tile set in mask_in is bypassed entirely, so
    its keys and values are never read.  Tiles skipped by every row get NaN K
    and V; outputs, lse and marks must equal the oracle's on the clean tensors
    (the q-tiles of a workgroup share K/V loads, so a tile that any row visits
    would be loaded; one that no row visits must not even be touched)."""
    q, k, v = tokens((6, 10, 16), 2, head_dim=D)                     # N = 960
    N = q.shape[1]
    Tq, Tk = -(-N // 128), -(-N // BN)
    rows = 2 * Tq
    mask = rand_mask(rows, Tk, 0.3, seed=17)
    dead = [1, Tk // 2, Tk - 2]
    for kt in dead:
        mask[:, kt >> 5] |= np.uint32(1 << (kt & 31))
    kp, vp = k.clone(), v.clone()
    for kt in dead:
        kp[:, kt * BN:(kt + 1) * BN] = float("nan")
        vp[:, kt * BN:(kt + 1) * BN] = float("nan")
    scale = 1.0 / math.sqrt(D)
    orc = oracle.fwd(q, k, v, 128, BN, -3.0, scale, mask_in=mask)
    gpu = pa.gpu_fwd(q, kp, vp, 128, BN, -3.0, scale, mask_in=mask, use_skiplist=skiplist)
    stats = pa.compare_rows(gpu, orc, orc["rows"], 1, N, 2, 128, BN, -3.0, q.dtype)
    log("  D %d BN %d skiplist %s dead tiles %s" % (D, BN, skiplist, dead), stats)
