"""GPU parity of carried-mask trajectories at full size: the 32,760-token,
75,600-token and cond/uncond-pair workloads, run the way the benchmark runs
them (Skip-List rebuilt from the carried mask before every step, the forward
writing the next step's mask), against the CPU oracle on sampled rows.

The Skip-Mask is state carried across denoising steps (LiteAttention README,
"QK-Skip Algorithm"), so a step's result depends on every earlier step.  The
oracle cannot run whole 75,600-token steps, but every row (batch, head,
q-tile) is independent: its mask after step t depends only on its own mask
and the inputs.  So the oracle runs its own trajectory on a fixed sample of
rows -- from an empty mask, carrying its own marks, never reading anything
the GPU produced -- while the GPU runs every row.  Before each step the
sampled rows of the GPU's mask are set to the oracle's carried rows (a GPU
input taken from the oracle; the other rows carry the GPU's own marks), so
that both sides start the step from the same mask even after a tile whose
margin lies within 1e-3 of the threshold, where either decision is accepted.
At each step the GPU's outputs, lse and new mask of the sampled rows must
match the oracle's at the bars of tests/parity.py; every other row is checked
by properties.  The key and value tensors sit at device addresses with bit
31 set (a sign-extension hazard of 64-bit addresses built from 32-bit
halves).
"""

import math
import os
import sys

import numpy as np
import pytest
import torch

from temporal_block_sparse_amd import configs, synth
from temporal_block_sparse_amd import lite_attn as la
from tests import parity as pa

pytestmark = pytest.mark.gpu


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def check_every_row(out, lse, v, m_in, m_out, tk):
    """Properties of every row, on the device: outputs finite and within the
    per-(batch, head, dim) range of V (a convex combination of V rows, up to
    bf16 rounding), lse finite (the rule never empties a row), mask_out keeps
    every bit of mask_in and sets no bit past the last tile."""
    of = out.float()
    assert bool(torch.isfinite(of).all()), "non-finite output"
    vmin = v.amin(dim=1, keepdim=True).float()
    vmax = v.amax(dim=1, keepdim=True).float()
    slack = 1e-2 * torch.maximum(vmin.abs(), vmax.abs()) + 1e-3
    assert bool(((of >= vmin - slack) & (of <= vmax + slack)).all()), "an output outside the range of V"
    del of
    assert bool(torch.isfinite(lse).all()), "non-finite lse"
    assert not bool((m_in & ~m_out).any()), "mask_out dropped a bit of mask_in"
    if tk % 32:
        w = -(-tk // 32)
        last = m_out.view(-1, w)[:, -1].to(torch.int64) & 0xFFFFFFFF
        assert not bool((last >> (tk % 32)).any()), "bits past the last tile"


def run_full_trajectory(wl, tau_of, steps, rows_small, rows_big=None, big_steps=(), use_skiplist=True):
    """Run `steps` steps of workload `wl` from an empty mask (tau_of(t) at step t)
    and check the sampled rows against the oracle's own trajectory at every
    step: rows_small always, rows_big (a superset) at the steps in big_steps,
    which must be the first steps (the oracle carries rows_big only that far)."""
    dev = torch.device("cuda")
    B, H, N, D, BM, BN = wl.batch, wl.heads, wl.seqlen, wl.head_dim, wl.tile_m, wl.tile_n
    Tq, Tk, W = wl.tq, wl.tk, wl.mask_words
    scale = 1.0 / math.sqrt(D)
    assert set(rows_small) <= set(rows_big if rows_big is not None else rows_small)
    assert list(big_steps) == list(range(len(big_steps)))
    tr = synth.Trajectory(wl, dev)
    desc = la.make_desc(B, N, H, D, BM, BN, la.LITE_BF16)
    nw = la.lite_attn_mask_words(desc)
    m_in = torch.zeros(nw, dtype=torch.int32, device=dev)
    m_out = torch.zeros(nw, dtype=torch.int32, device=dev)
    sl = la.alloc_skiplist(desc, dev) if use_skiplist else None
    out = torch.empty(B, N, H, D, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(B, H, N, dtype=torch.float32, device=dev)
    k31 = pa.bit31_empty((B, N, H, D), torch.bfloat16)
    v31 = pa.bit31_empty((B, N, H, D), torch.bfloat16)
    assert (k31.data_ptr() >> 31) & 1 and (v31.data_ptr() >> 31) & 1
    carried = {}                                    # row -> the oracle's own mask words for the next step
    stats = []
    for t in range(steps):
        if t:
            tr.advance()
        q, k, v = tr.tensors()
        k31.copy_(k)
        v31.copy_(v)
        del k, v
        tau = tau_of(t)
        rows = rows_big if t in big_steps else rows_small
        rm = np.stack([carried.get(int(r), np.zeros(W, np.uint32)) for r in rows])
        # the sampled rows start the step from the oracle's carried mask
        idx = torch.as_tensor(rows, device=dev)
        m_in.view(-1, W)[idx] = torch.as_tensor(rm.view(np.int32), device=dev)
        if sl is not None:
            la.lite_attn_build_skiplist(desc, m_in, sl)
        la.lite_attn_fwd(q, k31, v31, out, tile_m=BM, tile_n=BN, tau=tau, softmax_scale=scale, mask_in=m_in,
                         mask_out=m_out, skiplist=sl, lse=lse)
        torch.cuda.synchronize()
        check_every_row(out, lse, v31, m_in, m_out, Tk)
        orc = pa.oracle_sampled(q, k31, v31, BM, BN, tau, scale, rm, rows)
        g = pa.gpu_rows(out, lse, m_out, rows, H, BM)
        st = pa.packed_errors(g, orc, N, BM, Tk, tau)
        bits = np.unpackbits(m_out.cpu().numpy().view(np.uint8), bitorder="little").reshape(-1, W * 32)[:, :Tk]
        st.update(step=t, tau=tau, rows=len(rows), sparsity=round(float(bits.mean()), 4))
        log("  %s step %d tau %.3f rows %d: max_out %.4g max_lse %.3g mismatch %d near_tau %d sparsity %.4f"
            % (wl.name, t, tau, len(rows), st["max_out"], st["max_lse"], st["mask_mismatch"], st["near_tau"],
               st["sparsity"]))
        pa.assert_within_bars(st, torch.bfloat16)
        stats.append(st)
        carried = {int(r): orc["mask_out"][i].copy() for i, r in enumerate(rows)}
        m_in, m_out = m_out, m_in
        del q
    return stats


@pytest.mark.parametrize("use_skiplist", [True, False], ids=["skiplist", "bitmask"])
def test_c3_trajectory_full_size(use_skiplist):
    """32,760 tokens x 40 heads, 20 steps at tau = -3: 16 rows every step, 128
    rows at steps 0 and 1 (the Skip-List walk, and the bitmask walk)."""
    wl = configs.C3
    big = pa.sample_rows_in_heads(wl.batch, wl.heads, wl.tq, 128, 8, seed=31)
    small = big[np.random.default_rng(1).choice(len(big), 16, replace=False)]
    small = np.unique(np.concatenate([small, big[[0, -1]]]))
    steps = wl.steps if use_skiplist else 6
    stats = run_full_trajectory(wl, lambda t: -3.0, steps, small, big, big_steps=(0, 1),
                                use_skiplist=use_skiplist)
    assert stats[-1]["sparsity"] > 0.05


@pytest.mark.parametrize("tau", [-10.0, -3.0, 0.0])
def test_c4_trajectory_full_size(tau):
    """75,600 tokens x 40 heads on the Skip-List walk the benchmark times, 10
    steps at each finite threshold of the sweep: 16 rows every step, 128 rows
    at steps 0 and 1.  With LITE_ATTN_FULL_TRAJECTORIES=1 in the environment,
    all 50 steps of the sweep's trajectories (about 2.5 minutes each at
    tau = 0, too long for the default run)."""
    wl = configs.C4
    steps = wl.steps if os.environ.get("LITE_ATTN_FULL_TRAJECTORIES") == "1" else 10
    big = pa.sample_rows_in_heads(wl.batch, wl.heads, wl.tq, 128, 8, seed=41)
    small = big[np.random.default_rng(2).choice(len(big), 16, replace=False)]
    small = np.unique(np.concatenate([small, big[[0, -1]]]))
    stats = run_full_trajectory(wl, lambda t: tau, steps, small, big, big_steps=(0, 1))
    if tau >= -3.0:
        assert stats[-1]["sparsity"] > 0.1


def test_c5_pair_trajectory_full_size():
    """The cond/uncond pair (batch 2, 75,600 tokens, 40 heads) over its whole
    50-step schedule, tau_t = -10 + 10 t / 49, on the Skip-List walk: 8 rows
    of both batch entries carried by the oracle through every step, 64 at
    step 0."""
    wl = configs.C5
    big = pa.sample_rows_in_heads(wl.batch, wl.heads, wl.tq, 64, 4, seed=51)
    small = pa.sample_rows_in_heads(wl.batch, wl.heads, wl.tq, 8, 2, seed=52)
    big = np.unique(np.concatenate([big, small]))
    stats = run_full_trajectory(wl, wl.tau_at, wl.steps, small, big, big_steps=(0,))
    b_rows = [r for r in small if r >= wl.heads * wl.tq]
    assert b_rows, "no row of the second batch entry sampled"
    assert stats[-1]["sparsity"] > 0.3
