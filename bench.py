"""Benchmark: skip-masked attention forward on the 75,600-token video-DiT shape.

One step = one denoising step of the hot path on one batch of synthetic input:
rebuild the Skip-List from the carried Skip-Mask, then run the skip-masked
forward, which also writes the next step's mask.  Inputs (seeded, drifting
video-token Q/K/V) are generated before the timed region and are resident in
HBM when it starts.

Printed (one JSON line on stdout):
  value            effective TFLOP/s on live tiles over the K timed steps
                   (4*d*sum over live tiles of valid rows x valid cols, / wall time)
  pct_mfma_peak    value / 2516.6 TFLOP/s (bf16 dense MFMA, 256 CUs x 4096 flop/clk x 2.4 GHz)
  speedup_vs_dense same kernel, empty mask and tau = -inf, same inputs
  roofline         dominant kernel (the forward): algorithmic flops per launch
                   / HIP-event launch duration, against the bf16 MFMA peak;
                   traffic from the committed rocprofv3 counter summary when
                   it was taken on the current kernel source, else null
  cpu_baseline     the CPU oracle timed on a bounded sample of the same step
  tau_sweep        per-threshold trajectories (-inf, -10, -3, 0): sparsity,
                   kernel time, speedup and a least-squares fit of t/t_dense
                   against the live fraction
  aux_kernels      HBM roofline of the Skip-List build, the mask reset, the
                   LSE merge and the error sums at the workload's shape
  dense_variants   with --dense-variants: every bf16 kernel instantiation
                   (head_dim, key-tile width) dense at 32,768 tokens x 32 heads

--workload c1_fp32_1k measures the fp32 path instead (fp64 arithmetic on the
fp64 matrix cores, against their 78.6 TFLOP/s peak).
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective TFLOP/s on live tiles + % MFMA peak + speedup vs dense, 75.6k-token DiT"
PEAK_BF16_TFLOPS = 2516.6
PEAK_FP64_TFLOPS = 78.6   # fp64 matrix (and vector) peak: the fp32 path computes in fp64
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_fwd_bf16_c4_76k.txt")
KERNEL_SOURCES = {dt: [os.path.join(ROOT, "temporal_block_sparse_amd", "csrc", f)
                      for f in (src, "lite_attn_internal.h")]
                  for dt, src in (("bf16", "fwd_bf16.hip"), ("fp32", "fwd_fp32.hip"))}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash(dtype="bf16"):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[dtype]:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def live_flops(mask_words, wl):
    """4*d*sum over live tiles of (valid query rows) x (valid key cols), exact for
    partial tiles; mask_words None = every tile live."""
    import torch
    N, BM, BN, d = wl.seqlen, wl.tile_m, wl.tile_n, wl.head_dim
    Tq, Tk = wl.tq, wl.tk
    device = mask_words.device if mask_words is not None else "cpu"
    vr = torch.full((Tq,), BM, dtype=torch.float64, device=device)
    vr[-1] = N - (Tq - 1) * BM
    vc = torch.full((Tk,), BN, dtype=torch.float64, device=device)
    vc[-1] = N - (Tk - 1) * BN
    if mask_words is None:
        return 4.0 * d * wl.batch * wl.heads * float(vr.sum() * vc.sum())
    w = mask_words.view(wl.rows, wl.mask_words).to(torch.int64) & 0xFFFFFFFF
    bits = (w[:, :, None] >> torch.arange(32, device=w.device)) & 1
    skip = bits.reshape(wl.rows, -1)[:, :Tk].to(torch.float64)
    live = (1.0 - skip) @ vc                                     # [rows] live cols per row
    rows_valid = vr.repeat(wl.batch * wl.heads)
    return 4.0 * d * float((live * rows_valid).sum())


def pair_occupancy(mask_words, wl):
    """Share of the walked steps that both q-tiles of a workgroup compute: one
    workgroup serves q-tiles 2j and 2j+1 of a (batch, head) and walks the union
    of their live tiles, so this is sum |live| / (2 sum |union|)."""
    import torch
    Tq, Tk = wl.tq, wl.tk
    w = mask_words.view(wl.batch * wl.heads, Tq, wl.mask_words).to(torch.int64) & 0xFFFFFFFF
    bits = (w[..., None] >> torch.arange(32, device=w.device)) & 1
    live = (1 - bits.reshape(wl.batch * wl.heads, Tq, -1)[..., :Tk]).to(torch.float64)
    if Tq % 2:
        live = torch.cat([live, torch.zeros_like(live[:, :1])], dim=1)
    a, b = live[:, 0::2], live[:, 1::2]
    union = torch.maximum(a, b).sum()
    return float((a.sum() + b.sum()) / (2.0 * union)) if union > 0 else 1.0


def hbm_entry(b, ms):
    return {"bound": "hbm", "us": round(ms * 1e3, 2), "bytes": b, "GB/s": round(b / (ms * 1e-3) / 1e9, 1),
            "frac": round(b / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}


def aux_kernels(mask_words, wl, sl_ms, reset_ms, merge_ms, err_ms):
    """HBM roofline of the other kernels, from algorithmic bytes and the
    HIP-event time of one call (mean of 10 back-to-back calls).

    Skip-List build: every mask word read once, and per row the count plus
    one entry per live tile written (4 bytes each).  Mask reset: every mask
    word written once.  LSE merge of 2 parts: per (query, head) both parts'
    d outputs and lse read, the merged ones written.  Error sums: both
    tensors read once."""
    import torch
    w = mask_words.view(wl.rows, wl.mask_words).to(torch.int64) & 0xFFFFFFFF
    bits = (w[:, :, None] >> torch.arange(32, device=w.device)) & 1
    marked = bits.reshape(wl.rows, -1)[:, :wl.tk].sum(dim=1)
    words = w.numel()
    out = {}
    if sl_ms is not None:
        out["skiplist_build"] = hbm_entry(4 * words + 4 * int((1 + wl.tk - marked).sum()), sl_ms)
    out["reset_mask"] = hbm_entry(4 * words, reset_ms)
    qh = wl.batch * wl.seqlen * wl.heads
    esz = 2 if wl.dtype == "bf16" else 4
    row_bytes = wl.head_dim * esz + 4                                    # output row + fp32 lse
    out["lse_merge_2_parts"] = hbm_entry(3 * qh * row_bytes, merge_ms)
    out["error_sums"] = hbm_entry(2 * qh * wl.head_dim * esz, err_ms)
    return out


def dense_variants(torch, la, N=32768, H=32):
    """Dense throughput of each bf16 kernel instantiation (head_dim, key-tile
    width) at one large shape: seeded N(0,1) q, k, v, no mask, tau = -inf;
    5 back-to-back launches after 2 warmups, timed with events."""
    res = []
    for D, BN in ((64, 64), (64, 128), (128, 64), (128, 128)):
        g = torch.Generator(device="cuda").manual_seed(0)
        q, k, v = (torch.randn(1, N, H, D, device="cuda", generator=g).to(torch.bfloat16) for _ in range(3))
        o = torch.empty_like(q)
        sc = 1.0 / math.sqrt(D)
        for _ in range(2):
            la.lite_attn_fwd(q, k, v, o, tile_m=128, tile_n=BN, tau=-math.inf, softmax_scale=sc)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            la.lite_attn_fwd(q, k, v, o, tile_m=128, tile_n=BN, tau=-math.inf, softmax_scale=sc)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 5
        res.append({"head_dim": D, "tile": "128x%d" % BN, "seq_len": N, "heads": H, "ms": round(ms, 3),
                    "tflops": round(4.0 * H * N * N * D / (ms * 1e-3) / 1e12, 1)})
        log("[bench] dense d=%d tile 128x%d: %.3f ms" % (D, BN, ms))
        del q, k, v, o
    return res


def read_traffic(src_hash):
    """(bytes per launch, note) from the committed counter summary, or (None, why)."""
    if not os.path.exists(TRAFFIC_FILE):
        return None, "no counter summary"
    kv = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != src_hash:
        return None, "kernel changed since the counters were taken"
    try:
        return float(kv["hbm_bytes_per_launch"]), kv.get("note", "")
    except (KeyError, ValueError):
        return None, "malformed counter summary"


def cpu_threads():
    n = os.environ.get("OMP_NUM_THREADS")
    try:
        n = int(n)
    except (TypeError, ValueError):
        n = len(os.sched_getaffinity(0))
    return max(1, min(n, 16))


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="c4_bf16_76k")
    ap.add_argument("--grid", default=None, help="F,H,W token grid overriding the workload's (same recipe)")
    ap.add_argument("--heads", type=int, default=None, help="head count overriding the workload's")
    ap.add_argument("--tau", type=float, default=None,
                    help="threshold of every step (default: the workload's per-step schedule if it has one, else -3)")
    ap.add_argument("--path", choices=("skiplist", "bitmask"), default="skiplist")
    ap.add_argument("--sweep-steps", type=int, default=50, help="steps of the tau sweep (0: skip)")
    ap.add_argument("--cpu-rows", type=int, default=0,
                    help="oracle rows for the CPU baseline (0: 6 per thread, ~10-15 s on 16 host threads)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--dense-variants", action="store_true",
                    help="also time every bf16 kernel instantiation (head_dim, key-tile width) dense at 32,768 "
                         "tokens x 32 heads")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (for scaling HBM counters)")
    args = ap.parse_args()

    if args.steps < 1 or args.warmup < 0 or args.sweep_steps < 0:
        ap.error("--steps must be at least 1; --warmup and --sweep-steps at least 0")
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this library has no multi-GPU path "
              "(the forward would shard by heads, each GPU running this kernel on its own heads).", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        src = torch.ones(256 * 1024 * 1024, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": src.numel() * 4, "copy_bytes_written": dst.numel() * 4}))
        return

    from temporal_block_sparse_amd import configs, synth
    from temporal_block_sparse_amd import lite_attn as la

    wl = configs.ALL[args.workload]
    if args.grid or args.heads:
        grid = tuple(int(x) for x in args.grid.split(",")) if args.grid else wl.grid
        wl = configs.scaled(wl, grid, heads=args.heads, name="%s_grid%s_h%d" % (
            wl.name, "x".join(str(x) for x in grid), args.heads or wl.heads))
    bf16 = wl.dtype == "bf16"   # else the fp32 path (fp64 arithmetic on the fp64 matrix cores)

    def tau_at(t):
        """Threshold of trajectory step t: --tau, else the workload's schedule, else -3."""
        if args.tau is not None:
            return args.tau
        return wl.tau_at(t) if wl.tau_schedule is not None else -3.0
    tau_desc = (args.tau if args.tau is not None else
                ("schedule %g..%g" % wl.tau_schedule if wl.tau_schedule is not None else -3.0))
    peak = PEAK_BF16_TFLOPS if bf16 else PEAK_FP64_TFLOPS
    dev = torch.device("cuda")
    scale = 1.0 / math.sqrt(wl.head_dim)
    K, W = args.steps, args.warmup
    log("[bench] workload %s: B=%d H=%d N=%d d=%d tile %dx%d, tau %s, path %s, warmup %d, steps %d"
        % (wl.name, wl.batch, wl.heads, wl.seqlen, wl.head_dim, wl.tile_m, wl.tile_n, tau_desc, args.path, W, K))

    tr = synth.Trajectory(wl, dev)
    desc = la.make_desc(wl.batch, wl.seqlen, wl.heads, wl.head_dim, wl.tile_m, wl.tile_n,
                        la.LITE_BF16 if bf16 else la.LITE_FP32)
    nw = la.lite_attn_mask_words(desc)
    masks = [torch.zeros(nw, dtype=torch.int32, device=dev) for _ in range(K + 1)]
    warm_mask = [torch.zeros(nw, dtype=torch.int32, device=dev), torch.zeros(nw, dtype=torch.int32, device=dev)]
    sl = la.alloc_skiplist(desc, dev) if args.path == "skiplist" else None
    out = torch.empty(wl.batch, wl.seqlen, wl.heads, wl.head_dim, dtype=torch.bfloat16 if bf16 else torch.float32,
                      device=dev)

    def step(q, k, v, m_in, m_out, tau, ev=None):
        if sl is not None:
            la.lite_attn_build_skiplist(desc, m_in, sl)
        if ev is not None:
            ev[0].record()
        la.lite_attn_fwd(q, k, v, out, tile_m=wl.tile_m, tile_n=wl.tile_n, tau=tau, softmax_scale=scale,
                         mask_in=m_in, mask_out=m_out, skiplist=sl if m_in is not None else None)
        if ev is not None:
            ev[1].record()

    # ---- warmup: the first W steps of the trajectory (untimed) ----
    step0 = None
    for t in range(W):
        q, k, v = tr.tensors()
        if t == 0:
            step0 = (q, k, v)
        step(q, k, v, warm_mask[t % 2], warm_mask[(t + 1) % 2], tau_at(t))
        tr.advance()
    if W == 0:
        step0 = tr.tensors()
    if W:
        masks[0].copy_(warm_mask[W % 2])
    # ---- inputs of the K timed steps, resident in HBM before timing ----
    inputs = []
    for t in range(K):
        inputs.append(tr.tensors())
        tr.advance()
    torch.cuda.synchronize()
    log("[bench] inputs ready: %.1f GB resident" % (torch.cuda.memory_allocated() / 1e9))

    # ---- timed region ----
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for t in range(K):
        q, k, v = inputs[t]
        step(q, k, v, masks[t], masks[t + 1], tau_at(W + t), evs[t])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = [a.elapsed_time(b) for a, b in evs]
    flops = [live_flops(masks[t], wl) for t in range(K)]
    dense_flops = live_flops(None, wl)
    log("[bench] timed %d steps: %.2f ms/step, kernel %.2f ms avg" % (K, wall * 1e3 / K, sum(kern_ms) / K))

    # ---- dense reference: same kernel, empty mask, tau = -inf, same inputs ----
    dev_ms = []
    for t in range(K):
        q, k, v = inputs[t]
        ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        ev[0].record()
        la.lite_attn_fwd(q, k, v, out, tile_m=wl.tile_m, tile_n=wl.tile_n, tau=-math.inf, softmax_scale=scale)
        ev[1].record()
        dev_ms.append(ev)
    # The two mask kernels, 10 calls each, enqueued behind the dense launches:
    # the host has submitted them all before the GPU gets there, so the events
    # time the kernels back to back, not the host's launch rate.  The Skip-List
    # is rebuilt from the last timed mask; the reset clears a spare mask.
    aux_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(2)]
    if sl is not None:
        aux_ev[0][0].record()
        for _ in range(10):
            la.lite_attn_build_skiplist(desc, masks[K], sl)
        aux_ev[0][1].record()
    aux_ev[1][0].record()
    for _ in range(10):
        la.lite_attn_reset_mask(desc, warm_mask[0])
    aux_ev[1][1].record()
    # LSE merge of two partial attentions and the calibration's error sums, at
    # this workload's shape (the forward's output as the data, lse 0)
    out_b, out_m = out.clone(), torch.empty_like(out)
    lses = [torch.zeros(wl.batch, wl.heads, wl.seqlen, dtype=torch.float32, device=dev) for _ in range(3)]
    sums = torch.empty(2, dtype=torch.float64, device=dev)
    aux_ev += [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(2)]
    aux_ev[2][0].record()
    for _ in range(10):
        la.lite_attn_merge([out, out_b], lses[:2], out_m, lses[2])
    aux_ev[2][1].record()
    aux_ev[3][0].record()
    for _ in range(10):
        la.lite_attn_error_sums(out_m, out, sums)
    aux_ev[3][1].record()
    torch.cuda.synchronize()
    dense_ms = [a.elapsed_time(b) for a, b in dev_ms]
    sl_ms = aux_ev[0][0].elapsed_time(aux_ev[0][1]) / 10 if sl is not None else None
    reset_ms = aux_ev[1][0].elapsed_time(aux_ev[1][1]) / 10
    aux = aux_kernels(masks[K], wl, sl_ms, reset_ms, aux_ev[2][0].elapsed_time(aux_ev[2][1]) / 10,
                      aux_ev[3][0].elapsed_time(aux_ev[3][1]) / 10)
    del out_b, out_m, lses
    del inputs

    value = sum(flops) / wall / 1e12
    achieved = sum(flops) / (sum(kern_ms) * 1e-3) / 1e12
    src_hash = kernel_source_hash(wl.dtype)
    if bf16 and wl.name == "c4_bf16_76k":
        traffic, traffic_note = read_traffic(src_hash)
    else:
        traffic, traffic_note = None, "the committed counter summary covers the 75,600-token bf16 workload only"
    sparsity = [1.0 - f / dense_flops for f in flops]
    occupancy = [pair_occupancy(masks[t], wl) for t in range(K)]

    # ---- tau sweep over a trajectory (kernel time per step, per threshold) ----
    sweep = None
    if args.sweep_steps > 0:
        # thresholds of the sweep: the workload's list, or dense and its schedule
        # (None stands for the schedule), or the one threshold given
        if wl.taus:
            taus = list(wl.taus)
        elif wl.tau_schedule is not None and args.tau is None:
            taus = [-math.inf, None]
        else:
            taus = [-math.inf, tau_at(0)]
        tr2 = synth.Trajectory(wl, dev)
        sm = {tau: [torch.zeros(nw, dtype=torch.int32, device=dev) for _ in range(2)] for tau in taus}
        rec = {tau: [] for tau in taus}
        for t in range(args.sweep_steps):
            q, k, v = tr2.tensors()
            pend = []
            for tau in taus:
                m_in, m_out = sm[tau][t % 2], sm[tau][(t + 1) % 2]
                ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                if tau is not None and math.isinf(tau):
                    ev[0].record()
                    la.lite_attn_fwd(q, k, v, out, tile_m=wl.tile_m, tile_n=wl.tile_n, tau=tau, softmax_scale=scale)
                    ev[1].record()
                    pend.append((tau, ev, None))
                else:
                    step(q, k, v, m_in, m_out, wl.tau_at(t) if tau is None else tau, ev)
                    pend.append((tau, ev, m_in))
            torch.cuda.synchronize()
            for tau, ev, m_in in pend:
                f = dense_flops if m_in is None else live_flops(m_in, wl)
                occ = 1.0 if m_in is None else pair_occupancy(m_in, wl)
                rec[tau].append((ev[0].elapsed_time(ev[1]), f, occ))
            if t % 10 == 0:
                log("[bench] sweep step %d/%d" % (t, args.sweep_steps))
            tr2.advance()
            del q, k, v
        del tr2
        dense_t = [x[0] for x in rec[taus[0]]] if math.isinf(taus[0]) else None
        sweep = []
        xs, ys = [], []
        for tau in taus:
            tms = [x[0] for x in rec[tau]]
            fl = [x[1] for x in rec[tau]]
            label = tau_desc if tau is None else (None if math.isinf(tau) else tau)   # None: -inf (dense)
            ent = {"tau": label, "steps": len(tms), "kernel_ms_total": round(sum(tms), 3),
                   "sparsity_first": round(1 - fl[0] / dense_flops, 4), "sparsity_last": round(1 - fl[-1] / dense_flops, 4),
                   "sparsity_mean": round(1 - sum(fl) / (dense_flops * len(fl)), 4),
                   "tflops_live": round(sum(fl) / (sum(tms) * 1e-3) / 1e12, 1),
                   "pair_occupancy_mean": round(sum(x[2] for x in rec[tau]) / len(tms), 4)}
            if dense_t:
                ent["speedup_vs_dense"] = round(sum(dense_t) / sum(tms), 3)
                for a, b, f in zip(tms, dense_t, fl):
                    xs.append(f / dense_flops)
                    ys.append(a / b)
            sweep.append(ent)
        fit = None
        if len(xs) > 2:
            n = len(xs)
            mx, my = sum(xs) / n, sum(ys) / n
            sxx = sum((x - mx) ** 2 for x in xs)
            sxy = sum((x - mx) * (y - my) for x, y in zip(xs, ys))
            slope = sxy / sxx if sxx > 0 else float("nan")
            icpt = my - slope * mx
            ss_res = sum((y - (icpt + slope * x)) ** 2 for x, y in zip(xs, ys))
            ss_tot = sum((y - my) ** 2 for y in ys)
            fit = {"t_over_tdense_vs_live_fraction": {"slope": round(slope, 4), "intercept": round(icpt, 4),
                                                      "r2": round(1 - ss_res / ss_tot, 4) if ss_tot > 0 else None,
                                                      "points": n}}
        sweep = {"per_tau": sweep, "fit": fit}

    # ---- CPU baseline: the oracle on a bounded sample of step 0 (empty mask) ----
    cpu = None
    if not args.no_cpu:
        import numpy as np
        from oracle import oracle
        nth = cpu_threads()
        nrows = args.cpu_rows or 6 * nth
        q0, k0, v0 = step0
        rng = np.random.default_rng(0)
        rows = np.sort(rng.choice(wl.rows, size=min(nrows, wl.rows), replace=False)).astype(np.int64)
        qc, kc, vc = q0.cpu(), k0.cpu(), v0.cpu()
        t0c = time.perf_counter()
        res = oracle.fwd(qc, kc, vc, wl.tile_m, wl.tile_n, tau_at(0), scale, rows=rows, nthreads=nth)
        tc = time.perf_counter() - t0c
        tq = wl.tq
        rf = 0.0
        for r in rows:
            qt = int(r % tq)
            vr = min(wl.tile_m, wl.seqlen - qt * wl.tile_m)
            rf += 4.0 * wl.head_dim * vr * wl.seqlen
        cpu = {"value": round(rf / tc / 1e12, 6), "unit": "TFLOP/s", "cores": res["nthreads"], "kind": "oracle",
               "sample": "%d of %d q-tile rows of step 0 (empty mask, every tile live), fp64, %.1f s on %d threads "
                         "of %s" % (len(rows), wl.rows, tc, res["nthreads"], cpu_model())}
        del qc, kc, vc

    variants = dense_variants(torch, la) if args.dense_variants else None

    res = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(wall * 1e3 / K, 3), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if bf16 else "fp64", "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "heads": wl.heads, "seq_len": wl.seqlen,
                   "grid": list(wl.grid), "head_dim": wl.head_dim, "tile": "%dx%d" % (wl.tile_m, wl.tile_n),
                   "tau": tau_desc, "path": args.path, "timed_steps": [W, W + K - 1]},
        "pct_mfma_peak": round(100.0 * value / peak, 2),
        "speedup_vs_dense": round(sum(dense_ms) / sum(kern_ms), 3),
        "dense_kernel_ms": round(sum(dense_ms) / K, 3), "kernel_ms": round(sum(kern_ms) / K, 3),
        "dense_tflops": round(dense_flops * K / (sum(dense_ms) * 1e-3) / 1e12, 1),
        "sparsity": [round(s, 4) for s in sparsity],
        "pair_occupancy": [round(o, 4) for o in occupancy],
        "skiplist_build_ms": round(sl_ms, 4) if sl_ms is not None else None,
        "aux_kernels": aux,
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4),
                     "traffic": traffic, "traffic_note": traffic_note,
                     "kernel": ("fwd_bf16_kernel<%d, %d, %s>" % (wl.head_dim, wl.tile_n,
                                                                  "true" if args.path == "skiplist" else "false"))
                     if bf16 else "fwd_fp32_kernel",
                     "kernel_source_sha256_16": src_hash},
        "cpu_baseline": cpu,
        "tau_sweep": sweep,
        "dense_variants": variants,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
