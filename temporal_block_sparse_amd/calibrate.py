"""Per-timestep threshold calibration from output-error budgets.

LiteAttention README, "Error Calibration" ("Accumulated-Error Calibration" in
the architecture overview): denoising steps get variable error budgets, with
tighter budgets on the early steps, which weigh more on the final video.

The budget multiplier of step t follows the README's printed schedule: over
the first int(T * early_step_ratio) steps it rises linearly from 0.5 at step
0, every later step gets 1.0.  The calibration turns the budgets into
thresholds on given inputs (synthetic here; no model is needed): at step t,
with the Skip-Mask carried from the earlier steps, a candidate threshold is
run through the forward, the marks it would add are applied at once, and the
relative error of that output against plain attention,
    || out(marks) - out(nothing skipped) ||_F / || out(nothing skipped) ||_F,
is compared with base_error * multiplier(t).  The step takes the largest
candidate within its budget (-inf when none is) and carries its marks.  Every
forward and every error sum runs in the library's kernels.
"""

import math

import numpy as np
import torch

from . import lite_attn as la


def error_budgets(num_steps, early_step_ratio=0.3):
    """Budget multiplier per timestep (README "Error Calibration")."""
    n_early = int(num_steps * early_step_ratio)
    return [0.5 + 0.5 * t / n_early if t < n_early else 1.0 for t in range(num_steps)]


def _rel_error(a, b):
    s = la.lite_attn_error_sums(a, b).cpu().numpy()
    return math.sqrt(s[0] / s[1]) if s[1] > 0 else 0.0


def calibrate_thresholds(steps, tile_m, tile_n, base_error, taus, softmax_scale=None, early_step_ratio=0.3,
                         use_skiplist=False):
    """steps: sequence of (q, k, v) device tensors, one per denoising step.
    taus: candidate thresholds (natural-log units).  Returns one dict per step:
    tau, error, budget, sparsity (fraction of marked tiles) and the int32
    device mask carried to the next step."""
    steps = list(steps)
    mult = error_budgets(len(steps), early_step_ratio)
    cands = sorted({float(t) for t in taus}, reverse=True)
    if -math.inf not in cands:
        cands.append(-math.inf)
    mask = None
    res = []
    for t, (q, k, v) in enumerate(steps):
        desc = la.desc_of(q, tile_m, tile_n, k)
        nw = la.lite_attn_mask_words(desc)
        if mask is None:
            mask = torch.zeros(nw, dtype=torch.int32, device=q.device)
        dense = torch.empty_like(q)
        la.lite_attn_fwd(q, k, v, dense, tile_m=tile_m, tile_n=tile_n, tau=-math.inf, softmax_scale=softmax_scale)
        sl = la.alloc_skiplist(desc, q.device) if use_skiplist else None
        if sl is not None:
            la.lite_attn_build_skiplist(desc, mask, sl)
        budget = base_error * mult[t]
        trial = torch.empty_like(q)
        marks = torch.empty_like(mask)
        pick = None
        for tau in cands:
            la.lite_attn_fwd(q, k, v, trial, tile_m=tile_m, tile_n=tile_n, tau=tau, softmax_scale=softmax_scale,
                             mask_in=mask, mask_out=marks, skiplist=sl)
            la.lite_attn_fwd(q, k, v, trial, tile_m=tile_m, tile_n=tile_n, tau=-math.inf,
                             softmax_scale=softmax_scale, mask_in=marks)
            err = _rel_error(trial, dense)
            if err <= budget or tau == -math.inf:
                pick = (tau, err, marks.clone())
                break
        tau, err, mask = pick
        tk = -(-desc.seqlen_kv // tile_n)
        words = mask.cpu().numpy().view(np.uint32).reshape(-1, -(-tk // 32))
        bits = np.unpackbits(words.view(np.uint8), bitorder="little").reshape(words.shape[0], -1)[:, :tk]
        res.append({"tau": tau, "error": err, "budget": budget, "sparsity": float(bits.mean()), "mask": mask})
    return res
