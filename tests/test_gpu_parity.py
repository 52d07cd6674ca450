"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars: outputs within 2e-2 max-abs (bf16 storage, fp32 accumulation) and 1e-5
(fp32 storage); Skip-Mask decisions bit-exact except tiles whose oracle margin
is within 1e-3 of the threshold (counted).  Inputs are the seeded synthetic
video-token trajectories; every mask_in comes from the generator or from the
oracle's own previous step.
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


def small_wl(base, grid, heads, batch=1, steps=3):
    return configs.scaled(base, grid, heads=heads, batch=batch, steps=steps)


def run_trajectory(wl, steps, use_skiplist=False, nthreads=None):
    """Oracle trajectory from an empty mask; at each step the GPU gets the same
    inputs and the oracle's mask_in, and must match out, lse and mask_out."""
    tr = synth.Trajectory(wl, "cpu")
    mask = np.zeros((wl.rows, wl.mask_words), np.uint32)
    scale = 1.0 / math.sqrt(wl.head_dim)
    all_stats = []
    for step in range(steps):
        if step:
            tr.advance()
        q, k, v = tr.tensors()
        tau = wl.tau_at(step)
        log("  %s step %d tau %g" % (wl.name, step, tau))
        stats, orc = pa.check_full(q, k, v, wl.tile_m, wl.tile_n, tau, scale, mask_in=mask,
                                   use_skiplist=use_skiplist, nthreads=nthreads)
        stats["sparsity"] = float(np.unpackbits(orc["mask_out"].view(np.uint8)).sum()) / (wl.rows * wl.tk)
        all_stats.append(stats)
        mask = orc["mask_out"]
    return all_stats


def test_c1_fp32_trajectory():
    stats = run_trajectory(configs.C1, configs.C1.steps)
    log("C1", stats)
    assert stats[-1]["sparsity"] > 0.05


@pytest.mark.parametrize("D,BN", [(64, 64), (64, 128), (128, 64), (128, 128)])
def test_bf16_ragged_shapes_trajectory(D, BN):
    # 1000 tokens (5x10x20 grid): 8 q-tiles, the last holding 104 queries; the
    # last k-tile holds 104 (BN=128) or 40 (BN=64) keys.  At head_dim 128 the
    # positional bias is raised to 6 so that this short sequence marks tiles.
    base = configs.C3 if D == 128 else configs.C2
    wl = configs.Workload(**{**base.__dict__, "name": "ragged", "grid": (5, 10, 20), "heads": 3, "batch": 2,
                             "head_dim": D, "tile_m": 128, "tile_n": BN,
                             "bias_scale": (6.0, 6.0) if D == 128 else base.bias_scale})
    stats = run_trajectory(wl, 3)
    log("ragged", D, BN, stats)
    assert stats[-1]["sparsity"] > 0.0


def test_c2_trajectory_full_shape():
    """The 4,096-token, 12-head workload over all 10 of its steps, every row."""
    wl = configs.C2
    stats = run_trajectory(wl, wl.steps)
    log("C2", stats)
    assert stats[-1]["sparsity"] > 0.05


def test_c2_trajectory_skiplist_path():
    wl = configs.scaled(configs.C2, configs.C2.grid, heads=3, steps=6)
    stats = run_trajectory(wl, wl.steps, use_skiplist=True)
    log("C2 skiplist", stats)


def test_skiplist_path_bit_identical_to_bitmask():
    wl = small_wl(configs.C3, (6, 10, 20), heads=4, batch=2)
    q, k, v = synth.Trajectory(wl, "cpu").tensors()
    mask = synth.random_mask(wl.rows, wl.tk, 0.4, seed=3).numpy()
    a = pa.gpu_fwd(q, k, v, 128, 128, -3.0, 0.088, mask_in=mask)
    b = pa.gpu_fwd(q, k, v, 128, 128, -3.0, 0.088, mask_in=mask, use_skiplist=True)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]) and np.array_equal(a[2], b[2])


def test_mask_updated_in_place_equals_separate_buffers():
    wl = small_wl(configs.C2, (4, 16, 16), heads=2)
    q, k, v = synth.Trajectory(wl, "cpu").tensors()
    mask = synth.random_mask(wl.rows, wl.tk, 0.2, seed=4).numpy()
    a = pa.gpu_fwd(q, k, v, 128, 64, -3.0, 0.125, mask_in=mask)
    b = pa.gpu_fwd(q, k, v, 128, 64, -3.0, 0.125, mask_in=mask, inplace=True)
    assert torch.equal(a[0], b[0]) and np.array_equal(a[2], b[2])


def test_null_masks_and_minus_inf_threshold():
    wl = small_wl(configs.C2, (4, 16, 16), heads=2)
    q, k, v = synth.Trajectory(wl, "cpu").tensors()
    zeros = np.zeros((wl.rows, wl.mask_words), np.uint32)
    a = pa.gpu_fwd(q, k, v, 128, 64, -3.0, 0.125, mask_in=None)
    b = pa.gpu_fwd(q, k, v, 128, 64, -3.0, 0.125, mask_in=zeros)
    c = pa.gpu_fwd(q, k, v, 128, 64, -3.0, 0.125, mask_in=None, mark=False)
    d = pa.gpu_fwd(q, k, v, 128, 64, -math.inf, 0.125, mask_in=None)
    assert torch.equal(a[0], b[0]) and np.array_equal(a[2], b[2])
    assert torch.equal(a[0], c[0]) and c[2] is None
    assert torch.equal(a[0], d[0]) and not d[2].any()
    orc = oracle.fwd(q, k, v, 128, 64, -math.inf, 0.125)
    pa.compare_rows(d, orc, orc["rows"], 1, wl.seqlen, 2, 128, 64, -math.inf, torch.bfloat16)


def test_fully_skipped_rows_give_zero():
    wl = small_wl(configs.C2, (4, 16, 16), heads=2)
    q, k, v = synth.Trajectory(wl, "cpu").tensors()
    mask = synth.random_mask(wl.rows, wl.tk, 0.3, seed=5).numpy()
    mask[1, :] = -1                  # every tile of row 1 skipped (padding bits too: ignored)
    out, lse, mo = pa.gpu_fwd(q, k, v, 128, 64, -3.0, 0.125, mask_in=mask)
    b, h, qt = pa.row_coords(1, 2, wl.tq)
    assert torch.all(out[b, qt * 128:(qt + 1) * 128, h] == 0)
    assert torch.all(torch.isneginf(lse[b, h, qt * 128:(qt + 1) * 128]))
    orc = oracle.fwd(q, k, v, 128, 64, -3.0, 0.125, mask_in=mask)
    pa.compare_rows((out, lse, mo), orc, orc["rows"], 1, wl.seqlen, 2, 128, 64, -3.0, torch.bfloat16)


@pytest.mark.parametrize("tk", [1, 5, 31, 32, 33, 64, 65, 200, 591])
def test_build_skiplist_matches_reference(tk):
    rows = 37
    desc = la.make_desc(1, tk * 128, rows, 128, tk * 128, 128, la.LITE_BF16)   # one q-tile per head
    mask = synth.random_mask(rows, tk, 0.5, seed=tk)
    mask[3] = 0                                                          # all live
    mask[4] = -1                                                         # all skipped
    sl = torch.full((la.lite_attn_skiplist_len(desc),), -9, dtype=torch.int32, device="cuda")
    la.lite_attn_build_skiplist(desc, mask.cuda().reshape(-1), sl)
    got = sl.cpu().numpy().reshape(rows, 1 + tk)
    counts, lists = oracle.skiplist(mask.numpy(), tk)
    for r in range(rows):
        assert got[r, 0] == counts[r]
        assert list(got[r, 1:1 + counts[r]]) == list(lists[r])


@pytest.mark.parametrize("name", ["c4_bf16_76k", "c5_bf16_76k_pair"])
def test_build_skiplist_full_size(name):
    """The Skip-List build at the benchmark's shapes (23,640 and 47,280 rows of
    591 tiles): every row by properties that fix the list (the count is the
    number of live tiles; the entries are strictly descending and all live, so
    they are exactly the live tiles in visiting order), and 200 sampled rows
    against the oracle's reference."""
    wl = configs.ALL[name]
    desc = la.make_desc(wl.batch, wl.seqlen, wl.heads, wl.head_dim, wl.tile_m, wl.tile_n, la.LITE_BF16)
    mask = synth.random_mask(wl.rows, wl.tk, 0.6, seed=17)
    sl = torch.full((la.lite_attn_skiplist_len(desc),), -9, dtype=torch.int32, device="cuda")
    la.lite_attn_build_skiplist(desc, mask.cuda().reshape(-1), sl)
    got = sl.cpu().numpy().reshape(wl.rows, 1 + wl.tk)
    words = mask.numpy().view(np.uint32).reshape(wl.rows, wl.mask_words)
    bits = np.unpackbits(words.view(np.uint8), bitorder="little").reshape(wl.rows, -1)[:, :wl.tk].astype(bool)
    live = ~bits
    counts = got[:, 0]
    assert np.array_equal(counts, live.sum(axis=1))
    pos = np.arange(wl.tk)[None, :]
    valid = pos < counts[:, None]
    ent = np.where(valid, got[:, 1:], -1)
    assert np.all(ent[valid] >= 0) and np.all(ent[valid] < wl.tk)
    assert np.all(np.where(valid[:, 1:], ent[:, 1:] < ent[:, :-1], True))          # strictly descending
    rows_idx = np.broadcast_to(np.arange(wl.rows)[:, None], ent.shape)
    assert np.all(live[rows_idx[valid], ent[valid]])                                # every entry live
    sample = np.random.default_rng(3).choice(wl.rows, 200, replace=False)
    rc, rl = oracle.skiplist(words[sample], wl.tk)
    for i, r in enumerate(sample):
        assert got[r, 0] == rc[i] and list(got[r, 1:1 + rc[i]]) == list(rl[i])


def test_reset_mask_clears_every_word():
    desc = la.make_desc(2, 5000, 3, 128, 128, 128, la.LITE_BF16)
    m = torch.full((la.lite_attn_mask_words(desc) + 8,), -1, dtype=torch.int32, device="cuda")
    la.lite_attn_reset_mask(desc, m[:-8])
    torch.cuda.synchronize()
    assert int(m[:-8].abs().sum()) == 0 and bool((m[-8:] == -1).all())


@pytest.mark.parametrize("N", [1, 7, 64, 127, 128, 129, 300])
def test_edge_sequence_lengths(N):
    for D, BN in ((64, 64), (128, 128)):
        q, k, v = synth.random_qkv(1, N, 2, D, torch.bfloat16, seed=N, scale=2.0)
        pa.check_full(q, k, v, 128, BN, -1.0, 1.0 / math.sqrt(D))
    q, k, v = synth.random_qkv(1, N, 2, 64, torch.float32, seed=N, scale=2.0)
    pa.check_full(q, k, v, 64, 64, -1.0, 0.125)


def test_empty_sequence_is_noop():
    q = torch.empty(1, 0, 2, 128, dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(q)
    la.lite_attn_fwd(q, q.clone(), q.clone(), out, tile_m=128, tile_n=128, tau=-3.0)


@pytest.mark.parametrize("D,BN,skiplist", [(128, 128, False), (128, 128, True), (64, 64, True), (64, 128, False)])
def test_maximum_k_tiles(D, BN, skiplist):
    """Tk = 4096 (128 mask words per row: 524,288 tokens at 128-key tiles,
    262,144 at 64-key tiles) with 95% of tiles skipped, on both walks and
    both head dims; rows at the start, middle and end."""
    N, H = 4096 * BN, 1
    log("  bf16 N %d d %d tile 128x%d skiplist %s" % (N, D, BN, skiplist))
    q, k, v = synth.random_qkv(1, N, H, D, torch.bfloat16, seed=1, scale=1.0, device="cuda")
    Tq = N // 128
    mask = synth.random_mask(H * Tq, 4096, 0.95, seed=11).numpy()
    rows = np.array([0, Tq // 2, Tq - 1], np.int64)
    scale = 1.0 / math.sqrt(D)
    gpu = pa.gpu_fwd(q, k, v, 128, BN, -3.0, scale, mask_in=mask, use_skiplist=skiplist)
    orc = oracle.fwd(q.cpu(), k.cpu(), v.cpu(), 128, BN, -3.0, scale, mask_in=mask, rows=rows)
    log("  ", pa.compare_rows(gpu, orc, rows, 1, N, H, 128, BN, -3.0, torch.bfloat16))


@pytest.mark.parametrize("N,density,skiplist", [(4096 * 64 - 17, 0.95, False), (4096 * 64 - 17, 0.95, True),
                                                (20000, 0.5, False), (20000, 0.5, True)])
def test_fp32_long_sequences_sampled_rows(N, density, skiplist):
    """The fp32 kernel over many k-tiles: up to Tk = 4096 (128 mask words per
    row), ragged last tile, bitmask and Skip-List paths, on sampled rows."""
    H, D, T = 1, 64, 64
    Tq = Tk = -(-N // T)
    log("  fp32 N %d Tk %d density %.2f skiplist %s" % (N, Tk, density, skiplist))
    q, k, v = synth.random_qkv(1, N, H, D, torch.float32, seed=3, scale=1.5, device="cuda")
    mask = synth.random_mask(H * Tq, Tk, density, seed=12).numpy()
    rows = np.array([0, Tq // 3, Tq - 1], np.int64)
    gpu = pa.gpu_fwd(q, k, v, T, T, -3.0, 0.125, mask_in=mask, use_skiplist=skiplist)
    orc = oracle.fwd(q.cpu(), k.cpu(), v.cpu(), T, T, -3.0, 0.125, mask_in=mask, rows=rows)
    log("  ", pa.compare_rows(gpu, orc, rows, 1, N, H, T, T, -3.0, torch.float32))


@pytest.mark.parametrize("name", ["c3_bf16_33k", "c4_bf16_76k", "c5_bf16_76k_pair"])
def test_full_size_sampled_rows(name):
    """Full-size workloads in the benchmark's launch configuration: step 0 (empty
    mask) and a step from a synthetic 60%-sparse mask, on sampled rows against
    the oracle, and every row by properties."""
    wl = configs.ALL[name]
    tr = synth.Trajectory(wl, "cuda")
    q, k, v = tr.tensors()
    del tr
    torch.cuda.empty_cache()
    scale = 1.0 / math.sqrt(wl.head_dim)
    tau = wl.tau_at(0, -3.0)
    rows = pa.sample_rows(wl.batch, wl.heads, wl.tq, 10, seed=7)
    qc, kc, vc = q.cpu(), k.cpu(), v.cpu()
    for case, mask in (("empty", None), ("synthetic", synth.random_mask(wl.rows, wl.tk, 0.6, seed=8).numpy())):
        log("  %s %s tau %g rows %s" % (name, case, tau, rows.tolist()))
        gpu = pa.gpu_fwd(q, k, v, wl.tile_m, wl.tile_n, tau, scale, mask_in=mask,
                         use_skiplist=(wl.batch == 2))
        orc = oracle.fwd(qc, kc, vc, wl.tile_m, wl.tile_n, tau, scale, mask_in=mask, rows=rows)
        st = pa.compare_rows(gpu, orc, rows, wl.batch, wl.seqlen, wl.heads, wl.tile_m, wl.tile_n, tau,
                             torch.bfloat16)
        log("  ", st)
        pa.check_all_rows(gpu, vc, mask, wl.tk)
        log("   every row: outputs within V's range, lse finite, marks kept")


def test_binding_refuses_short_or_mistyped_buffers():
    """The kernels take plain pointers: the binding refuses any buffer smaller
    than the call uses (or of the wrong dtype) before launching anything."""
    q, k, v = synth.random_qkv(1, 300, 2, 64, torch.bfloat16, seed=0, scale=1.0, device="cuda")
    out = torch.empty_like(q)
    desc = la.desc_of(q, 128, 64, k)
    nw, nl = la.lite_attn_mask_words(desc), la.lite_attn_skiplist_len(desc)
    m = torch.zeros(nw, dtype=torch.int32, device="cuda")
    cases = ((dict(mask_in=m[:-1]), "mask_in holds"), (dict(mask_out=m[:-1]), "mask_out holds"),
             (dict(mask_in=m, skiplist=torch.zeros(nl - 1, dtype=torch.int32, device="cuda")), "skiplist holds"),
             (dict(lse=torch.zeros(1, 2, 299, device="cuda")), "lse holds"),
             (dict(lse=torch.zeros(1, 2, 300, dtype=torch.float64, device="cuda")), "lse must be"))
    for kw, msg in cases:
        with pytest.raises(ValueError, match=msg):
            la.lite_attn_fwd(q, k, v, out, tile_m=128, tile_n=64, tau=-3.0, **kw)
    lse = torch.zeros(1, 2, 300, device="cuda")
    with pytest.raises(ValueError, match=r"lses\[1\] holds"):
        la.lite_attn_merge([out, out], [lse, torch.zeros(1, 2, 299, device="cuda")], torch.empty_like(out))
    with pytest.raises(ValueError, match="sums must be"):
        la.lite_attn_error_sums(out, out, torch.zeros(2, dtype=torch.float32, device="cuda"))
    # the right buffers still work
    la.lite_attn_fwd(q, k, v, out, tile_m=128, tile_n=64, tau=-3.0, mask_in=m, mask_out=m, lse=lse)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
