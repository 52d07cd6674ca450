"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
compare it with the CPU oracle on the same inputs.

Comparison rules:
  * outputs: max |gpu - oracle| <= 2e-2 for bf16 storage, 1e-5 for fp32;
  * lse: <= 1e-3 (bf16 path, fp32 arithmetic) / 1e-5 (fp32 path), same -inf pattern;
  * masks: bit-exact, except a tile whose oracle margin lies within 1e-3 of
    tau (in natural-log units): either decision is accepted there, and such
    tiles are counted.
Inputs of the oracle never come from the HIP path: q/k/v come from the seeded
generator, mask_in from the generator or from the oracle's own previous step.
"""

import math
import time

import numpy as np
import torch

from oracle import oracle
from temporal_block_sparse_amd import lite_attn as la

TOL_OUT = {torch.bfloat16: 2e-2, torch.float32: 1e-5}
TOL_LSE = {torch.bfloat16: 1e-3, torch.float32: 1e-5}
NEAR_TAU = 1e-3


def words_to_u32(m):
    return np.asarray(m).view(np.uint32)


def gpu_fwd(q, k, v, BM, BN, tau, scale, mask_in=None, mark=True, use_skiplist=False, inplace=False,
            want_lse=True, must_do=None, must_skip=None):
    """Run the HIP forward on device copies of q [B,Nq,H,D] and k, v [B,Nk,H,D]
    (any device).  mask_in: host or device words or None.  must_do/must_skip:
    key ranges.  Returns (out, lse, mask_out) on the CPU (mask_out None when
    mark is False)."""
    dev = torch.device("cuda")
    qd, kd, vd = (t.to(dev).contiguous() for t in (q, k, v))
    desc = la.desc_of(qd, BM, BN, kd)
    nw = la.lite_attn_mask_words(desc)
    mi = None
    if mask_in is not None:
        mi = torch.as_tensor(np.asarray(mask_in).view(np.int32).reshape(-1)).to(dev) if not isinstance(
            mask_in, torch.Tensor) else mask_in.to(dev).view(torch.int32).reshape(-1).contiguous()
        assert mi.numel() == nw
    mo = None
    if mark:
        if inplace:
            if mi is None:
                mi = torch.zeros(nw, dtype=torch.int32, device=dev)
            mo = mi
        else:
            mo = torch.full((nw,), 0x5A5A5A5A, dtype=torch.int32, device=dev)
    sl = None
    if use_skiplist:
        sl = torch.full((la.lite_attn_skiplist_len(desc),), -7, dtype=torch.int32, device=dev)
        la.lite_attn_build_skiplist(desc, mi, sl, must_do, must_skip)
    out = torch.full_like(qd, float("nan"))
    lse = torch.full((qd.shape[0], qd.shape[2], qd.shape[1]), float("nan"), device=dev) if want_lse else None
    la.lite_attn_fwd(qd, kd, vd, out, tile_m=BM, tile_n=BN, tau=tau, softmax_scale=scale, mask_in=mi,
                     mask_out=mo, skiplist=sl, lse=lse, must_do=must_do, must_skip=must_skip)
    torch.cuda.synchronize()
    return (out.cpu(), lse.cpu() if lse is not None else None,
            mo.cpu().numpy().view(np.uint32).reshape(-1, desc_words(desc)) if mo is not None else None)


def desc_words(desc):
    tk = -(-desc.seqlen_kv // desc.tile_n)
    return -(-tk // 32)


def row_coords(row, H, Tq):
    return int(row // (Tq * H)), int((row // Tq) % H), int(row % Tq)


def compare_rows(gpu, orc, rows, B, N, H, BM, BN, tau, dtype, mask_checked=True, Nk=None):
    """Compare GPU results (full tensors) with packed oracle rows; N queries,
    Nk keys (default N).  Returns a dict of error statistics; raises
    AssertionError on a violation."""
    out_g, lse_g, mask_g = gpu
    Tq, Tk = -(-N // BM), -(-(N if Nk is None else Nk) // BN)
    W = -(-Tk // 32)
    og = out_g.to(torch.float64).numpy()
    lg = lse_g.numpy().astype(np.float64) if lse_g is not None else None
    max_out = 0.0
    max_lse = 0.0
    near, mism = 0, 0
    for i, row in enumerate(rows):
        b, h, qt = row_coords(row, H, Tq)
        r0, nr = qt * BM, min(BM, N - qt * BM)
        ref = orc["out"][i][:nr]
        got = og[b, r0:r0 + nr, h, :]
        assert np.all(np.isfinite(got)), "non-finite output in row %d" % row
        max_out = max(max_out, float(np.abs(got - ref).max()))
        if lg is not None:
            lr, lgot = orc["lse"][i][:nr], lg[b, h, r0:r0 + nr]
            assert np.array_equal(np.isneginf(lr), np.isneginf(lgot)), "lse -inf pattern, row %d" % row
            fin = np.isfinite(lr)
            if fin.any():
                max_lse = max(max_lse, float(np.abs(lgot[fin] - lr[fin]).max()))
        if mask_checked and mask_g is not None:
            mw = mask_g[row]
            mo = orc["mask_out"][i]
            diff = mw ^ mo
            for kt in range(Tk):
                if (int(diff[kt // 32]) >> (kt % 32)) & 1:
                    mg = orc["margin"][i][kt]
                    if np.isfinite(mg) and abs(mg - tau) <= NEAR_TAU:
                        near += 1
                    else:
                        mism += 1
            # padding bits must be zero
            if Tk % 32:
                assert (int(mw[W - 1]) >> (Tk % 32)) == 0, "padding bits set, row %d" % row
    stats = dict(max_out=max_out, max_lse=max_lse, near_tau=near, mask_mismatch=mism)
    assert max_out <= TOL_OUT[dtype], stats
    assert max_lse <= TOL_LSE[dtype], stats
    assert mism == 0, stats
    return stats


def oracle_sampled(q, k, v, BM, BN, tau, scale, row_masks, rows, nthreads=None):
    """The oracle on sampled rows of (device or host) BSHD q [B,N,H,D], k, v
    [B,Nk,H,D] in one call: the (batch, head) slices the rows need are gathered
    into a [G, N, 1, D] batch, so only those heads reach the host.
    row_masks: mask_in words of each sampled row [nrows, W] (host), or None for
    empty masks.  Returns a dict packed in the order of `rows`, like oracle.fwd's,
    plus "seconds", the time of the oracle call itself."""
    B, N, H, D = q.shape
    Tq = -(-N // BM)
    Tk = -(-k.shape[1] // BN)
    W = -(-Tk // 32)
    rows = np.asarray(rows, np.int64)
    groups = {}
    for r in rows:
        b, h, _ = row_coords(r, H, Tq)
        groups.setdefault((b, h), len(groups))
    gl = sorted(groups, key=groups.get)
    qg, kg, vg = (torch.stack([t[b, :, h, :] for b, h in gl]).unsqueeze(2).cpu() for t in (q, k, v))
    local = np.array([groups[row_coords(r, H, Tq)[:2]] * Tq + row_coords(r, H, Tq)[2] for r in rows], np.int64)
    mi = None
    if row_masks is not None:
        mi = np.zeros((len(gl) * Tq, W), np.uint32)
        mi[local] = np.asarray(row_masks).view(np.uint32).reshape(len(rows), W)
    t0 = time.perf_counter()
    res = oracle.fwd(qg, kg, vg, BM, BN, tau, scale, mask_in=mi, rows=local, nthreads=nthreads)
    res["seconds"] = time.perf_counter() - t0
    res["rows"] = rows
    return res


def gpu_rows(out, lse, mask_out, rows, H, BM):
    """The sampled rows of device results, packed like oracle_sampled's:
    out [nrows, BM, D] (fp64; rows past the sequence are NaN), lse [nrows, BM],
    mask_out [nrows, W] (uint32), gathered on the device."""
    B, N, _, D = out.shape
    Tq = -(-N // BM)
    o = np.full((len(rows), BM, D), np.nan)
    lo = np.full((len(rows), BM), np.nan)
    for i, r in enumerate(rows):
        b, h, qt = row_coords(r, H, Tq)
        r0, nr = qt * BM, min(BM, N - qt * BM)
        o[i, :nr] = out[b, r0:r0 + nr, h, :].to(torch.float64).cpu().numpy()
        if lse is not None:
            lo[i, :nr] = lse[b, h, r0:r0 + nr].to(torch.float64).cpu().numpy()
    m = None
    if mask_out is not None:
        idx = torch.as_tensor(np.asarray(rows, np.int64), device=mask_out.device)
        m = mask_out.view(B * H * Tq, -1)[idx].cpu().numpy().view(np.uint32)
    return {"out": o, "lse": lo if lse is not None else None, "mask_out": m}


def packed_errors(g, orc, N, BM, Tk, tau, H=None):
    """Error statistics of packed GPU rows (gpu_rows) against packed oracle rows
    (no assertion): max |out| and |lse| differences over the valid queries,
    mask bits that differ outside the 1e-3 band around tau (mismatches) and
    inside it (near_tau), non-finite outputs, lse -inf patterns that differ, and
    padding bits set."""
    W = -(-Tk // 32)
    Tq = -(-N // BM)
    st = dict(max_out=0.0, max_lse=0.0, near_tau=0, mask_mismatch=0, nonfinite=0, lse_pattern=0, padding=0)
    for i, row in enumerate(orc["rows"]):
        qt = int(row % Tq)
        nr = min(BM, N - qt * BM)
        got, ref = g["out"][i][:nr], orc["out"][i][:nr]
        if not np.all(np.isfinite(got)):
            st["nonfinite"] += 1
            continue
        st["max_out"] = max(st["max_out"], float(np.abs(got - ref).max()))
        if g["lse"] is not None:
            lr, lgot = orc["lse"][i][:nr], g["lse"][i][:nr]
            if not np.array_equal(np.isneginf(lr), np.isneginf(lgot)):
                st["lse_pattern"] += 1
            fin = np.isfinite(lr) & np.isfinite(lgot)
            if fin.any():
                st["max_lse"] = max(st["max_lse"], float(np.abs(lgot[fin] - lr[fin]).max()))
        if g["mask_out"] is not None:
            mw, mo = g["mask_out"][i], orc["mask_out"][i]
            diff = mw ^ mo
            for kt in range(Tk):
                if (int(diff[kt // 32]) >> (kt % 32)) & 1:
                    mg = orc["margin"][i][kt]
                    if np.isfinite(mg) and abs(mg - tau) <= NEAR_TAU:
                        st["near_tau"] += 1
                    else:
                        st["mask_mismatch"] += 1
            if Tk % 32 and (int(mw[W - 1]) >> (Tk % 32)):
                st["padding"] += 1
    return st


def assert_within_bars(st, dtype):
    assert st["nonfinite"] == 0 and st["lse_pattern"] == 0 and st["padding"] == 0, st
    assert st["max_out"] <= TOL_OUT[dtype], st
    assert st["max_lse"] <= TOL_LSE[dtype], st
    assert st["mask_mismatch"] == 0, st


def bit31_empty(shape, dtype, device="cuda"):
    """An uninitialised tensor whose first byte sits at a device address with
    bit 31 set (and 256-byte aligned): a view into a buffer 2 GiB larger than
    the tensor, which always holds such an address within its first 2 GiB."""
    nbytes = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
    buf = torch.empty(nbytes + (2 << 30) + 256, dtype=torch.uint8, device=device)
    base = buf.data_ptr()
    a = (base + 255) & ~255
    if not (a >> 31) & 1:
        a = ((a >> 31) + 1) << 31          # the next 2 GiB boundary: bit 31 set there
    off = a - base
    assert off + nbytes <= buf.numel() and (a >> 31) & 1
    return buf[off:off + nbytes].view(dtype).view(shape)


def check_full(q, k, v, BM, BN, tau, scale, mask_in=None, use_skiplist=False, nthreads=None, must_do=None,
               must_skip=None):
    """All rows: GPU vs oracle.  Returns (stats, oracle result)."""
    B, N, H, D = q.shape
    orc = oracle.fwd(q, k, v, BM, BN, tau, scale, mask_in=mask_in, nthreads=nthreads, must_do=must_do,
                     must_skip=must_skip)
    gpu = gpu_fwd(q, k, v, BM, BN, tau, scale, mask_in=mask_in, use_skiplist=use_skiplist, must_do=must_do,
                  must_skip=must_skip)
    stats = compare_rows(gpu, orc, orc["rows"], B, N, H, BM, BN, tau, q.dtype, Nk=k.shape[1])
    return stats, orc


def check_all_rows(gpu, v, mask_in, Tk):
    """Properties every row must have at any size, for the rows the oracle
    does not recompute: each output is a convex combination of V rows (so
    within V's per-(batch, head, dim) range, up to bf16 rounding), every lse is
    finite (no row of these masks is fully skipped), and mask_out keeps every
    bit of mask_in and no bit past the last tile."""
    out, lse, mo = gpu
    vf = v.float()
    vmin, vmax = vf.amin(dim=1, keepdim=True), vf.amax(dim=1, keepdim=True)      # [B, 1, H, D]
    slack = 1e-2 * torch.maximum(vmin.abs(), vmax.abs()) + 1e-3
    of = out.float()
    assert bool(torch.isfinite(of).all()), "non-finite output"
    assert bool(((of >= vmin - slack) & (of <= vmax + slack)).all()), "an output outside the range of V"
    assert bool(torch.isfinite(lse).all()), "non-finite lse"
    if mo is not None:
        mi = np.zeros_like(mo) if mask_in is None else np.asarray(mask_in).view(np.uint32).reshape(mo.shape)
        assert not np.any(mi & ~mo), "mask_out dropped a bit of mask_in"
        if Tk % 32:
            assert not np.any(mo[:, -1] >> np.uint32(Tk % 32)), "bits past the last tile"


def sample_rows(B, H, Tq, n, seed):
    rng = np.random.default_rng(seed)
    rows = set()
    rows.add((B * H - 1) * Tq + Tq - 1)          # last head's last (partial) q-tile
    rows.add(0)
    rows.add(Tq - 1)
    if B > 1:
        rows.add((H * Tq) + Tq // 2)             # second batch entry
    while len(rows) < n:
        rows.add(int(rng.integers(0, B * H * Tq)))
    return np.array(sorted(rows), np.int64)


def sample_rows_in_heads(B, H, Tq, n, n_heads, seed):
    """n distinct rows drawn from at most n_heads (batch, head) pairs, so that
    the oracle gathers few heads: always the last head's last (partial) q-tile
    and the first head's first q-tile, a row of the second batch entry when
    there is one, and both q-tiles of one workgroup pair."""
    rng = np.random.default_rng(seed)
    bh = {0, B * H - 1}
    if B > 1:
        bh.add(H + int(rng.integers(0, H)))
    while len(bh) < min(n_heads, B * H):
        bh.add(int(rng.integers(0, B * H)))
    bh = sorted(bh)
    rows = {(B * H - 1) * Tq + Tq - 1, 0}
    if B > 1:
        rows.add(bh[-2] * Tq + Tq // 2)
    p = int(rng.integers(0, Tq // 2)) if Tq >= 2 else 0
    rows.update({bh[0] * Tq + 2 * p, bh[0] * Tq + min(2 * p + 1, Tq - 1)})
    while len(rows) < min(n, len(bh) * Tq):
        rows.add(bh[int(rng.integers(0, len(bh)))] * Tq + int(rng.integers(0, Tq)))
    return np.array(sorted(rows), np.int64)
