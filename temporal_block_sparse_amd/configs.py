"""Workload definitions for the skip-masked attention forward.

Five synthetic video-token workloads, from a single-head fp32 toy up to the
75,600-token, 40-head shape of a 14B video DiT.  Tokens sit on an (F, H, W)
latent grid; token n maps to grid point (f, y, x) with n = (f*H + y)*W + x.

Pages cited by this package:
  [README]   "LiteAttention" project README (moonmath-ai/LiteAttention),
             sections on the QK-Skip algorithm, the threshold ablation table,
             the Python API (threshold, must-do list, LSE) and the debug flags.
  [ABSTRACT] "LiteAttention: A Temporal Sparse Attention for Diffusion
             Transformers" (arXiv 2511.11062), abstract.

Tile notation: "tile A x B" means A query rows (BM) by B key columns (BN).
"""

from dataclasses import dataclass, field
import math


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str            # "fp32" or "bf16": storage type of q, k, v and out
    batch: int
    heads: int
    grid: tuple           # (F, H, W) latent grid; seq = F*H*W
    head_dim: int
    tile_m: int           # BM, query rows per tile
    tile_n: int           # BN, key columns per tile
    steps: int
    taus: tuple           # thresholds swept (natural-log units); None -> schedule
    drift_qk: float       # per-step Gaussian drift on Q and K
    drift_v: float        # per-step Gaussian drift on V
    bias_scale: tuple     # (lo, hi) per-head scale of the positional feature
    v_locality: bool      # V's first 16 dims carry the positional feature
    shared_q_drift: bool  # batch entries share the Q drift increment (cond/uncond pair)
    seed: int = 0
    tau_schedule: tuple = field(default=None)  # (tau_first, tau_last): linear in step

    @property
    def seqlen(self):
        f, h, w = self.grid
        return f * h * w

    @property
    def tq(self):
        return -(-self.seqlen // self.tile_m)

    @property
    def tk(self):
        return -(-self.seqlen // self.tile_n)

    @property
    def mask_words(self):
        return -(-self.tk // 32)

    @property
    def rows(self):
        return self.batch * self.heads * self.tq

    def tau_at(self, step, tau=None):
        """Threshold used at denoising step `step` (natural-log units)."""
        if self.tau_schedule is not None:
            lo, hi = self.tau_schedule
            if self.steps <= 1:
                return float(lo)
            return float(lo + (hi - lo) * step / (self.steps - 1))
        return float(self.taus[0] if tau is None else tau)

    def dense_flops(self):
        n = self.seqlen
        return 4.0 * self.batch * self.heads * n * n * self.head_dim


NEG_INF = -math.inf

C1 = Workload("c1_fp32_1k", "fp32", 1, 1, (8, 8, 16), 64, 64, 64, 3, (-3.0,),
              0.05, 0.0, (4.0, 4.0), False, False)
C2 = Workload("c2_bf16_4k", "bf16", 1, 12, (16, 16, 16), 64, 128, 64, 10, (-3.0,),
              0.05, 0.0, (4.0, 4.0), False, False)
C3 = Workload("c3_bf16_33k", "bf16", 1, 40, (21, 30, 52), 128, 128, 128, 20, (-3.0,),
              0.05, 0.0, (2.0, 6.0), False, False)
C4 = Workload("c4_bf16_76k", "bf16", 1, 40, (21, 45, 80), 128, 128, 128, 50,
              (NEG_INF, -10.0, -3.0, 0.0), 0.03, 0.03, (2.0, 6.0), True, False)
C5 = Workload("c5_bf16_76k_pair", "bf16", 2, 40, (21, 45, 80), 128, 128, 128, 50,
              None, 0.03, 0.03, (2.0, 6.0), True, True, tau_schedule=(-10.0, 0.0))

ALL = {w.name: w for w in (C1, C2, C3, C4, C5)}


def scaled(w: Workload, grid, heads=None, batch=None, steps=None, name=None):
    """Same recipe on another grid (the parity tests use smaller ones, which the oracle finishes quickly)."""
    kw = dict(w.__dict__)
    kw["grid"] = tuple(grid)
    if heads is not None:
        kw["heads"] = heads
    if batch is not None:
        kw["batch"] = batch
    if steps is not None:
        kw["steps"] = steps
    kw["name"] = name or (w.name + "_small")
    return Workload(**kw)
