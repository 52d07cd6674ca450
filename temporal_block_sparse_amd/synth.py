"""Seeded synthetic video-token Q/K/V trajectories and synthetic Skip-Masks.

This module only draws inputs.  It holds none of the attention arithmetic, so
the HIP path and the CPU oracle can both consume its tensors without sharing
any of the method's code.

Recipe (the plainest construction of "locality-biased Gaussian Q/K/V that drift
slowly across denoising steps"; the pages give no activation statistics):

* Grid: token n <-> p = (f, y, x), n = (f*H + y)*W + x.
* Positional feature phi(p) in R^16, shared by Q and K and by all heads:
  random Fourier features of an RBF kernel with length scale 2 grid cells,
  phi_j(p) = sqrt(2) cos(w_j . p + b_j), w_j ~ N(0, I/4), b_j ~ U[0, 2 pi).
  Each component has unit variance and E[phi(p).phi(p')] decays with grid
  distance.
* Q, K: N(0,1) entries; dims 0..15 get + s_h * phi(p), s_h the per-head scale
  (a fixed value or U[lo, hi] per head).  K uses independent noise.
* V: N(0,1); for locality-biased V, dims 0..15 are (N(0,1) + phi)/sqrt(2).
* Drift: at each step X <- X + delta * N(0,1) with fresh noise.  For a
  cond/uncond pair the Q increment is shared by both batch entries.
* Values are drawn in fp32 and rounded to nearest-even into bf16 when the
  workload stores bf16.  Layout is BSHD: [batch, seq, heads, head_dim].
"""

import math
import torch

_TAG = {"phi": 1, "scale": 2, "q": 3, "k": 4, "v": 5, "dq": 6, "dk": 7, "dv": 8, "mask": 9}
_M63 = (1 << 63) - 1


def subseed(seed: int, tag: str, b: int = 0, step: int = 0) -> int:
    """Independent generator seed for (workload seed, tensor, batch entry, step)."""
    x = (seed * 0x9E3779B97F4A7C15 + _TAG[tag] * 0xBF58476D1CE4E5B9
         + (b + 1) * 0x94D049BB133111EB + (step + 1) * 0x2545F4914F6CDD1D)
    x &= _M63
    x ^= x >> 31
    return (x * 0xD6E8FEB86659FD93) & _M63


def _gen(device, s):
    g = torch.Generator(device=device)
    g.manual_seed(s)
    return g


def grid_positions(grid):
    f, h, w = grid
    ff, yy, xx = torch.meshgrid(torch.arange(f), torch.arange(h), torch.arange(w), indexing="ij")
    return torch.stack([ff, yy, xx], dim=-1).reshape(-1, 3).to(torch.float64)


def positional_feature(grid, seed, nfeat=16, length=2.0):
    """[N, nfeat] fp32 random Fourier features (CPU, identical on every device)."""
    g = _gen("cpu", subseed(seed, "phi"))
    w = torch.randn(nfeat, 3, generator=g, dtype=torch.float64) / length
    b = torch.rand(nfeat, generator=g, dtype=torch.float64) * (2.0 * math.pi)
    p = grid_positions(grid)
    return (math.sqrt(2.0) * torch.cos(p @ w.T + b)).to(torch.float32)


def head_scales(wl):
    lo, hi = wl.bias_scale
    if lo == hi:
        return torch.full((wl.heads,), float(lo), dtype=torch.float32)
    g = _gen("cpu", subseed(wl.seed, "scale"))
    return (lo + (hi - lo) * torch.rand(wl.heads, generator=g, dtype=torch.float64)).to(torch.float32)


class Trajectory:
    """fp32 Q/K/V state of one workload, advanced one denoising step at a time."""

    def __init__(self, wl, device="cpu"):
        self.wl = wl
        self.device = torch.device(device)
        self.step = 0
        n, H, d = wl.seqlen, wl.heads, wl.head_dim
        phi = positional_feature(wl.grid, wl.seed).to(self.device)           # [N,16]
        sc = head_scales(wl).to(self.device)                                 # [H]
        bias = sc[None, :, None] * phi[:, None, :]                           # [N,H,16]
        self.q = torch.empty(wl.batch, n, H, d, device=self.device)
        self.k = torch.empty_like(self.q)
        self.v = torch.empty_like(self.q)
        for b in range(wl.batch):
            for name, dst in (("q", self.q), ("k", self.k), ("v", self.v)):
                dst[b] = torch.randn(n, H, d, generator=_gen(self.device, subseed(wl.seed, name, b)),
                                     device=self.device)
            self.q[b, :, :, :16] += bias
            self.k[b, :, :, :16] += bias
            if wl.v_locality:
                self.v[b, :, :, :16] = (self.v[b, :, :, :16] + phi[:, None, :]) * (1.0 / math.sqrt(2.0))
        del bias

    def advance(self):
        """Apply one step of drift (step t -> t+1)."""
        wl = self.wl
        self.step += 1
        t = self.step
        shape = self.q.shape[1:]
        for b in range(wl.batch):
            if wl.drift_qk:
                bq = 0 if wl.shared_q_drift else b
                self.q[b].add_(torch.randn(shape, generator=_gen(self.device, subseed(wl.seed, "dq", bq, t)),
                                           device=self.device), alpha=wl.drift_qk)
                self.k[b].add_(torch.randn(shape, generator=_gen(self.device, subseed(wl.seed, "dk", b, t)),
                                           device=self.device), alpha=wl.drift_qk)
            if wl.drift_v:
                self.v[b].add_(torch.randn(shape, generator=_gen(self.device, subseed(wl.seed, "dv", b, t)),
                                           device=self.device), alpha=wl.drift_v)

    def tensors(self):
        """(q, k, v) in the workload's storage dtype, contiguous BSHD: new
        tensors, which later steps of drift do not change (the fp32 state is
        copied too, not returned by reference)."""
        dt = torch.bfloat16 if self.wl.dtype == "bf16" else torch.float32
        return tuple(x.to(dt, copy=True).contiguous() for x in (self.q, self.k, self.v))


def random_qkv(batch, seqlen, heads, head_dim, dtype=torch.float32, seed=0, scale=1.0, device="cpu"):
    """Plain BSHD tensors for shape sweeps and edge cases: q, k ~ N(0, scale^2),
    v ~ N(0, 1) (unit-variance values, as in the workload recipe)."""
    g = _gen(device, subseed(seed, "q", 0, 0))
    out = []
    for sc in (scale, scale, 1.0):
        out.append((sc * torch.randn(batch, seqlen, heads, head_dim, generator=g, device=device)).to(dtype))
    return tuple(out)


def random_mask(rows, tk, density, seed=0, device="cpu"):
    """Skip-Mask words [rows, ceil(tk/32)] uint32-as-int32 with each tile skipped
    independently with probability `density`; bits at positions >= tk are 0.
    Bit kt of a row lives in word kt // 32 at bit kt % 32."""
    words = -(-tk // 32)
    g = _gen("cpu", subseed(seed, "mask", 0, rows * 7 + tk))
    bits = (torch.rand(rows, words * 32, generator=g) < density)
    bits[:, tk:] = False
    w = torch.zeros(rows, words, dtype=torch.int64)
    for j in range(32):
        w |= bits[:, j::32].to(torch.int64) << j
    w = torch.where(w >= (1 << 31), w - (1 << 32), w).to(torch.int32)
    return w.to(device)
