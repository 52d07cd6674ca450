"""Pins of the CPU oracle against what the pages and the mathematics fix (CPU only).

Pages: LiteAttention README (moonmath-ai/LiteAttention) -- 'QK-Skip Algorithm',
'Full-Stage Elimination', the threshold ablation table and the Python API
(reverse iteration, reset, debug flag for thresholds above 0); the
lite-attention-temporal-sparse skill page's masked-softmax formulation
(skipped positions get -inf logits, softmax renormalises over the rest).
"""

import math

import numpy as np
import pytest
import torch

from oracle import oracle
from temporal_block_sparse_amd import configs, synth
from tests import oracle_checks as oc


def test_golden_worked_examples():
    assert oc.run_golden() == []


def test_dense_is_plain_softmax_attention():
    assert oc.check_dense() == []


def test_masked_attention_and_decision_rule():
    assert oc.check_masked_and_rule() == []


def test_tile_grid_invariance_without_skipping():
    assert oc.check_tile_invariance() == []


def test_bf16_and_fp32_inputs_are_exact_upcasts():
    q, k, v = oc.random_case(11, 1, 40, 2, 8)
    for dt in (torch.bfloat16, torch.float32):
        qq, kk, vv = q.to(dt), k.to(dt), v.to(dt)
        r = oracle.fwd(qq, kk, vv, 16, 8, -3.0, 0.3)
        r64 = oracle.fwd(qq.double(), kk.double(), vv.double(), 16, 8, -3.0, 0.3)
        for key in ("out", "lse", "mask_out"):
            assert np.array_equal(r[key], r64[key])


def test_threshold_monotone_single_step():
    """newly(tau1) is a subset of newly(tau2) for tau1 <= tau2, from one mask_in
    (the running max does not depend on tau, since marked tiles still count in
    their own step)."""
    q, k, v = oc.random_case(3, 1, 96, 2, 8, scale_in=2.0)
    Tq, Tk = 96 // 16, 96 // 8
    rng = np.random.default_rng(5)
    bits = rng.random((2 * Tq, Tk)) < 0.2
    prev = None
    outs = []
    for tau in (-math.inf, -6.0, -3.0, -1.0, 0.0, 0.5):
        r = oracle.fwd(q, k, v, 16, 8, tau, 0.35, mask_in=oc.words_of(bits))
        newly = oc.bits_of(r["mask_out"], Tk) & ~bits
        if prev is not None:
            assert not np.any(prev & ~newly)
        prev = newly
        outs.append(r["out"])
    # the output depends on mask_in only, never on tau
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_drop_bound_when_marks_take_effect():
    """Re-running with mask_in := mask_out moves each output row by at most
    2*max|v|*delta/(1-delta), delta = probability mass of the dropped keys."""
    q, k, v = oc.random_case(9, 1, 64, 1, 8, scale_in=2.5)
    scale, BM, BN, tau = 0.35, 8, 8, -2.0
    r1 = oracle.fwd(q, k, v, BM, BN, tau, scale)
    _, _, prob = oc.dense_reference(q, k, v, scale)
    newly = oc.bits_of(r1["mask_out"], 8)
    assert newly.any()
    r2 = oracle.fwd(q, k, v, BM, BN, tau, scale, mask_in=r1["mask_out"])
    o1, _ = oracle.unpack_rows(r1, 1, 64, 1, BM)
    o2, _ = oracle.unpack_rows(r2, 1, 64, 1, BM)
    vmax = np.abs(oc.to64(v)).max()
    full = np.repeat(np.repeat(newly, BM, 0), BN, 1)[:64, :64]
    delta = (prob[0, 0] * full).sum(axis=1)                      # per query row
    bound = 2 * vmax * delta / (1 - delta)
    err = np.abs(o2[0, :, 0, :] - o1[0, :, 0, :]).max(axis=1)
    assert np.all(err <= bound + 1e-12)


def test_rows_subset_matches_full_call():
    q, k, v = oc.random_case(4, 2, 50, 3, 8)
    full = oracle.fwd(q, k, v, 16, 16, -2.0, 0.4)
    rows = np.array([7, 0, 3, 11], np.int64)
    part = oracle.fwd(q, k, v, 16, 16, -2.0, 0.4, rows=rows)
    for key in ("out", "lse", "margin", "mask_out"):
        np.testing.assert_array_equal(part[key], full[key][rows])


def test_fully_skipped_row_gives_zero_and_minus_inf():
    q, k, v = oc.random_case(1, 1, 16, 1, 4)
    bits = np.ones((2, 2), bool)
    r = oracle.fwd(q, k, v, 8, 8, -3.0, 0.5, mask_in=oc.words_of(bits))
    assert np.all(r["out"] == 0) and np.all(np.isneginf(r["lse"]))
    assert np.all(np.isnan(r["margin"]))
    assert np.array_equal(oc.bits_of(r["mask_out"], 2), bits)


def test_skipped_tiles_are_never_read():
    """Full-Stage Elimination (README): a skipped tile costs no K/V traffic, so
    NaN keys and values in tiles that every row skips change nothing."""
    q, k, v = oc.random_case(5, 1, 40, 2, 8)
    rng = np.random.default_rng(3)
    bits = rng.random((10, 5)) < 0.3
    bits[:, 2] = True
    words = oc.words_of(bits)
    kp, vp = k.clone(), v.clone()
    kp[:, 16:24] = float("nan")
    vp[:, 16:24] = float("nan")
    a = oracle.fwd(q, k, v, 8, 8, -2.0, 0.4, mask_in=words)
    b = oracle.fwd(q, kp, vp, 8, 8, -2.0, 0.4, mask_in=words)
    for key in ("out", "lse", "mask_out", "margin"):
        assert np.array_equal(np.asarray(a[key]), np.asarray(b[key]), equal_nan=True), key


def test_bits_past_last_tile_are_cleared():
    q, k, v = oc.random_case(2, 1, 40, 1, 4)     # Tk = 5 with 8-wide tiles
    words = np.full((5, 1), 0xFFFFFFE0, np.uint32)  # only padding bits set
    r = oracle.fwd(q, k, v, 8, 8, -math.inf, 0.5, mask_in=words)
    assert np.all(r["mask_out"] == 0)


def test_rejects_nan_threshold_and_bad_scale():
    q, k, v = oc.random_case(2, 1, 8, 1, 4)
    with pytest.raises(ValueError):
        oracle.fwd(q, k, v, 4, 4, float("nan"), 0.5)
    with pytest.raises(ValueError):
        oracle.fwd(q, k, v, 4, 4, -3.0, 0.0)


def test_skiplist_reference():
    """Skip-List reference: the clear bits of each row, last tile first, across
    word boundaries; must-do and must-skip tile flags applied."""
    assert oc.check_skiplist() == []


def test_c1_trajectory_masks_grow_and_stay_nondegenerate():
    """The fp32 1024-token workload over its 3 steps: marks only accumulate, and
    tau = -3 marks a non-trivial fraction of tiles on the locality-biased inputs."""
    wl = configs.C1
    tr = synth.Trajectory(wl, "cpu")
    mask = np.zeros((wl.rows, wl.mask_words), np.uint32)
    scale = 1.0 / math.sqrt(wl.head_dim)
    sparsity = []
    for step in range(wl.steps):
        if step:
            tr.advance()
        q, k, v = tr.tensors()
        r = oracle.fwd(q, k, v, wl.tile_m, wl.tile_n, wl.tau_at(step), scale, mask_in=mask)
        before = oc.bits_of(mask, wl.tk)
        after = oc.bits_of(r["mask_out"], wl.tk)
        assert not np.any(before & ~after)
        # given the mask, the output is plain masked attention
        o, _ = oracle.unpack_rows(r, 1, wl.seqlen, 1, wl.tile_m)
        o_ref, _, _ = oc.dense_reference(q, k, v, scale, before, wl.tile_m, wl.tile_n)
        assert np.allclose(o, o_ref, atol=1e-11)
        mask = r["mask_out"]
        sparsity.append(after.mean())
    assert 0.02 < sparsity[-1] < 0.9
    assert sparsity == sorted(sparsity)


def test_edge_case_checks():
    assert oc.check_edge_cases() == []


def test_queries_and_keys_of_different_lengths():
    assert oc.check_nonsquare() == []


def test_must_do_and_must_skip_ranges():
    assert oc.check_ranges() == []


def test_tile_flags_match_the_hand_derived_examples():
    """The Python tile-flag helper (used by the Skip-List reference) gives the
    tile sets derived by hand from the README's examples."""
    assert oc.check_tile_flags() == []


def test_lse_merge_of_key_splits_is_full_attention():
    """Attention over a partition of the keys, merged by LSE, is attention over
    all keys -- by brute force; also through the oracle's own forward on the
    K/V splits (the sequence-parallel use), with a part left empty."""
    assert oc.check_merge() == []


def test_error_budgets_follow_the_skill_page_schedule():
    assert oc.check_error_budgets() == []


def test_calibration_picks_the_largest_feasible_threshold():
    """Brute-force re-evaluation of every step's choice, plus the unbounded
    and zero budgets."""
    assert oc.check_calibration() == []
