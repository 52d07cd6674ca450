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
                   it was taken on the current kernel code, else null; likewise
                   clock_ghz, the sustained clock of that counter run's timed
                   launches, and frac_at_clock, the fraction of the peak at
                   that clock (the chip runs power-limited below 2.4 GHz)
  cpu_baseline     the CPU oracle timed on a bounded sample of the same
                   trajectory: a fixed set of rows (one per host thread, at
                   most 16) that the oracle carries from an empty mask through
                   the warmup and timed steps by itself
  verification     the timed steps W, W + K/2 and W + K - 1 and a step of each
                   other threshold of the sweep against those oracle rows:
                   max-abs output and lse differences, mask mismatches and
                   near-threshold ties (the same bars as the parity tests)
  tau_sweep        per-threshold trajectories (-inf, -10, -3, 0): sparsity,
                   kernel time, speedup and a least-squares fit of t/t_dense
                   against the live fraction
  aux_kernels      HBM roofline of the Skip-List build, the mask reset, the
                   LSE merge and the error sums at the workload's shape
  dense_variants   with --dense-variants: every bf16 kernel instantiation
                   (head_dim, key-tile width) dense at 32,768 tokens x 32 heads
  pair_workload    default run only: the cond/uncond pair workload (batch 2,
                   threshold schedule -10 .. 0), 5 timed steps after 3 warmups,
                   with its own oracle check, run as a child process of this
                   script (--no-pair skips it)

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
PMC_FILE = os.path.join(ROOT, "profiles", "pmc_utilisation_fwd_bf16_c4_76k.txt")
PMC_NOTE = ("mean sustained clock of the timed masked launches in the committed counter run of this code "
            "(GRBM_GUI_ACTIVE / 8 / duration), not measured in this run; frac_at_clock = achieved / (peak x clock / 2.4 GHz)")
KERNEL_SOURCES = {dt: [os.path.join(ROOT, "temporal_block_sparse_amd", "csrc", f)
                      for f in (src, "lite_attn_internal.h")]
                  for dt, src in (("bf16", "fwd_bf16.hip"), ("fp32", "fwd_fp32.hip"))}


# keyword arguments of every forward call: empty for the library's default
# (the ticket schedule), {"sched": None} for one workgroup per q-tile pair
FWD_KW = {}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def strip_code(text):
    """C++ source with its comments removed, each line's blank space collapsed
    and empty lines dropped: what a comment or layout edit leaves unchanged."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":                 # a literal: copied whole, escapes included
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    lines = (" ".join(ln.split()) for ln in "".join(out).split("\n"))
    return "\n".join(ln for ln in lines if ln)


def kernel_code_hash(dtype="bf16"):
    """First 16 hex digits of the sha256 of the kernel's sources with comments
    and blank space removed: counters taken on one build stay valid across
    edits of its comments, and lapse with any change to the code."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[dtype]:
        with open(f, encoding="utf-8") as fh:
            h.update(strip_code(fh.read()).encode())
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


def rows_live_flops(row_masks, rows, wl):
    """4*d*sum over the sampled rows' live tiles of valid rows x valid cols;
    row_masks: the rows' mask_in words [nrows, W] (host) or None (all live)."""
    import numpy as np
    N, BM, BN, d, Tq, Tk = wl.seqlen, wl.tile_m, wl.tile_n, wl.head_dim, wl.tq, wl.tk
    vc = np.full(Tk, BN, np.float64)
    vc[-1] = N - (Tk - 1) * BN
    f = 0.0
    for i, r in enumerate(rows):
        qt = int(r % Tq)
        vr = min(BM, N - qt * BM)
        live = vc.sum()
        if row_masks is not None:
            bits = np.unpackbits(np.asarray(row_masks[i]).view(np.uint32).view(np.uint8),
                                 bitorder="little")[:Tk].astype(bool)
            live = vc[~bits].sum()
        f += 4.0 * d * vr * live
    return f


class OracleCheck:
    """The oracle's own trajectory on a fixed sample of rows, and the check of
    GPU steps against it (the CPU-baseline leg: the oracle's calls are also what
    cpu_baseline times).  Every row (batch, head, q-tile) is independent, so the
    oracle carries the sampled rows' masks by itself from an empty mask, from
    the seeded inputs alone; nothing the GPU computes reaches it.  A GPU step is
    compared on the rows whose carried mask equals the oracle's at that step
    (they differ only after a tile within 1e-3 of the threshold, where either
    decision is correct; such rows are counted as diverged)."""

    def __init__(self, wl, scale, rows, nthreads):
        from tests import parity as pa
        self.pa, self.wl, self.scale, self.rows, self.nth = pa, wl, scale, rows, nthreads
        self.carried = {}          # trajectory label -> mask_in words of the rows at the next step
        self.results = {}          # (label, step) -> (oracle result, its mask_in words)
        self.seconds = 0.0
        self.flops = 0.0
        self.threads = 0

    def step(self, label, t, q, k, v, tau, keep=False, timed=True):
        wl = self.wl
        rm = self.carried.get(label)
        res = self.pa.oracle_sampled(q, k, v, wl.tile_m, wl.tile_n, tau, self.scale, rm, self.rows,
                                     nthreads=self.nth)
        if timed:
            self.seconds += res["seconds"]
            self.flops += rows_live_flops(rm, self.rows, wl)
            self.threads = res["nthreads"]
        if keep:
            self.results[(label, t)] = (res, rm)
        self.carried[label] = res["mask_out"].copy()

    def compare(self, label, t, tau, out, lse, m_in, m_out):
        """Statistics of the GPU's rows at step t of trajectory `label` against
        the kept oracle result (m_in/m_out: the GPU's mask words, device)."""
        import numpy as np
        pa, wl = self.pa, self.wl
        res, rm = self.results[(label, t)]
        W = wl.mask_words
        g = pa.gpu_rows(out, lse, m_out, self.rows, wl.heads, wl.tile_m)
        if m_in is not None:
            import torch
            idx = torch.as_tensor(self.rows, device=m_in.device)
            gin = m_in.view(-1, W)[idx].cpu().numpy().view(np.uint32)
        else:
            gin = np.zeros((len(self.rows), W), np.uint32)
        oin = rm if rm is not None else np.zeros((len(self.rows), W), np.uint32)
        same = np.all(gin == oin, axis=1)
        sel = np.nonzero(same)[0]
        st = dict(max_out=0.0, max_lse=0.0, near_tau=0, mask_mismatch=0, nonfinite=0, lse_pattern=0, padding=0)
        if len(sel):
            gs = {key: (g[key][sel] if g[key] is not None else None) for key in ("out", "lse", "mask_out")}
            rs = {key: res[key][sel] for key in ("out", "lse", "margin", "mask_out")}
            rs["rows"] = self.rows[sel]
            st = pa.packed_errors(gs, rs, wl.seqlen, wl.tile_m, wl.tk, tau)
        ok = (st["max_out"] <= pa.TOL_OUT[out.dtype] and st["max_lse"] <= pa.TOL_LSE[out.dtype]
              and st["mask_mismatch"] == 0 and st["nonfinite"] == 0 and st["lse_pattern"] == 0
              and st["padding"] == 0)
        return {"trajectory": label, "step": t, "tau": None if math.isinf(tau) else tau,
                "rows": len(self.rows), "rows_compared": int(len(sel)), "diverged_rows": int(len(self.rows) - len(sel)),
                "max_abs_out": round(st["max_out"], 6), "max_lse": round(st["max_lse"], 7),
                "mask_mismatch": st["mask_mismatch"], "near_tau": st["near_tau"],
                "nonfinite": st["nonfinite"] + st["lse_pattern"] + st["padding"], "within_bars": bool(ok)}


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
            la.lite_attn_fwd(q, k, v, o, tile_m=128, tile_n=BN, tau=-math.inf, softmax_scale=sc, **FWD_KW)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            la.lite_attn_fwd(q, k, v, o, tile_m=128, tile_n=BN, tau=-math.inf, softmax_scale=sc, **FWD_KW)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 5
        res.append({"head_dim": D, "tile": "128x%d" % BN, "seq_len": N, "heads": H, "ms": round(ms, 3),
                    "tflops": round(4.0 * H * N * N * D / (ms * 1e-3) / 1e12, 1)})
        log("[bench] dense d=%d tile 128x%d: %.3f ms" % (D, BN, ms))
        del q, k, v, o
    return res


def pair_workload(args):
    """The cond/uncond pair workload (batch 2, its threshold schedule), run
    briefly as a child process of this script so that the default line also
    records it: 5 timed steps after 3 warmups, with the oracle check of those
    steps on 4 carried rows.  Returns a summary of the child's JSON line."""
    import subprocess
    cmd = [sys.executable, os.path.abspath(__file__), "--workload", "c5_bf16_76k_pair", "--steps", "5",
           "--warmup", "3", "--sweep-steps", "0", "--cpu-rows", "4", "--schedule", args.schedule]
    if args.no_cpu:
        cmd.append("--no-cpu")
    log("[bench] pair workload: %s" % " ".join(cmd[1:]))
    try:
        p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=sys.stderr, text=True, timeout=900)
    except subprocess.TimeoutExpired:
        return {"error": "child timed out after 900 s", "command": " ".join(cmd[1:])}
    lines = [l for l in p.stdout.splitlines() if l.startswith("{")]
    if p.returncode != 0 or not lines:
        return {"error": "child exited with %d" % p.returncode, "command": " ".join(cmd[1:])}
    j = json.loads(lines[-1])
    v = j.get("verification") or {}
    return {"command": "python bench.py " + " ".join(cmd[2:]), "value": j["value"], "unit": j["unit"],
            "pct_mfma_peak": j["pct_mfma_peak"], "ms_per_step": j["ms_per_step"],
            "speedup_vs_dense": j["speedup_vs_dense"], "dense_tflops": j["dense_tflops"],
            "config": j["config"], "sparsity": j["sparsity"], "pair_occupancy": j["pair_occupancy"],
            "roofline_frac": j["roofline"]["frac"],
            "verification": {k: v.get(k) for k in ("within_bars", "max_abs_out", "max_lse", "mask_mismatch",
                                                   "near_tau", "diverged_rows")} if v else None}


def read_traffic(code_hash):
    """(bytes per launch, note) from the committed counter summary, or (None, why)."""
    if not os.path.exists(TRAFFIC_FILE):
        return None, "no counter summary"
    kv = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_code_sha256_16") != code_hash:
        return None, "kernel changed since the counters were taken"
    try:
        return float(kv["hbm_bytes_per_launch"]), kv.get("note", "")
    except (KeyError, ValueError):
        return None, "malformed counter summary"


def read_clock(code_hash):
    """(GHz, note): the sustained clock of the timed masked launches in the
    committed utilisation-counter summary (GRBM_GUI_ACTIVE over each launch's
    duration), or (None, why).  The first skip-list dispatch there is the
    warmup step; the rest are timed steps.  Like the traffic figure it is
    taken from a counter run of the same code, not from this run."""
    if not os.path.exists(PMC_FILE):
        return None, "no counter summary"
    ghz, code = [], None
    for line in open(PMC_FILE):
        if line.startswith("kernel_code_sha256_16:"):
            code = line.split(":", 1)[1].strip()
        f = line.split()
        if len(f) >= 8 and f[0].isdigit() and "true>" in line and "skip-list" in line:
            try:
                ghz.append(float(f[f.index("skip-list") + 2]))
            except (ValueError, IndexError):
                return None, "malformed counter summary"
    if code != code_hash:
        return None, "kernel changed since the counters were taken"
    if len(ghz) < 2:
        return None, "malformed counter summary"
    return sum(ghz[1:]) / len(ghz[1:]), PMC_NOTE


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
                    help="rows the oracle carries through the trajectory for the CPU baseline and the check of "
                         "the timed steps (0: one per host thread, at most 16)")
    ap.add_argument("--check-sweep-steps", type=int, default=3,
                    help="steps of each other threshold's trajectory the oracle carries; the last is checked")
    ap.add_argument("--no-cpu", action="store_true", help="no CPU baseline and no oracle check")
    ap.add_argument("--dense-variants", action="store_true",
                    help="also time every bf16 kernel instantiation (head_dim, key-tile width) dense at 32,768 "
                         "tokens x 32 heads")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (for scaling HBM counters)")
    ap.add_argument("--schedule", choices=("tickets", "static"), default="tickets",
                    help="bf16 forward schedule: persistent workgroups drawing q-tile pairs from ticket counters "
                         "(the library's default), or one workgroup per pair")
    ap.add_argument("--no-pair", action="store_true",
                    help="skip the short run of the cond/uncond pair workload that the default run adds")
    ap.add_argument("--gemm-reference", action="store_true",
                    help="only time plain bf16 GEMMs (torch.matmul, the vendor library): what a dense "
                         "matrix-core kernel sustains on this GPU, for comparison with the forward")
    args = ap.parse_args()

    if args.steps < 1 or args.warmup < 0 or args.sweep_steps < 0:
        ap.error("--steps must be at least 1; --warmup and --sweep-steps at least 0")
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this library has no multi-GPU path "
              "(the forward would shard by heads, each GPU running this kernel on its own heads).", file=sys.stderr)
        sys.exit(2)

    if args.schedule == "static":
        FWD_KW["sched"] = None
    import torch
    if args.copy_calibration:
        src = torch.ones(256 * 1024 * 1024, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": src.numel() * 4, "copy_bytes_written": dst.numel() * 4}))
        return
    if args.gemm_reference:
        res = []
        for m, n, k in ((8192, 8192, 8192), (16384, 16384, 8192), (32768, 8192, 8192)):
            g = torch.Generator(device="cuda").manual_seed(0)
            a = torch.randn(m, k, device="cuda", generator=g).to(torch.bfloat16)
            b = torch.randn(k, n, device="cuda", generator=g).to(torch.bfloat16)
            for _ in range(3):
                c = a @ b
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(20):
                c = a @ b
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / 20
            tf = 2.0 * m * n * k / (ms * 1e-3) / 1e12
            res.append({"m": m, "n": n, "k": k, "ms": round(ms, 3), "tflops": round(tf, 1),
                        "pct_mfma_peak": round(100.0 * tf / PEAK_BF16_TFLOPS, 1)})
            log("[bench] gemm %dx%dx%d bf16: %.3f ms, %.0f TFLOP/s" % (m, n, k, ms, tf))
            del a, b, c
        print(json.dumps({"gemm_reference_bf16": res}))
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
                         mask_in=m_in, mask_out=m_out, skiplist=sl if m_in is not None else None, **FWD_KW)
        if ev is not None:
            ev[1].record()

    # ---- the oracle's own trajectory on sampled rows (CPU-baseline leg) ----
    # It runs on the host between the untimed GPU work, from the seeded inputs
    # alone, and keeps its results for the timed steps checked afterwards.
    chk = None
    check_steps = sorted({W, W + K // 2, W + K - 1})
    if not args.no_cpu:
        import numpy as np
        from tests import parity as pa
        nth = cpu_threads()
        nrows = args.cpu_rows or nth
        rows = pa.sample_rows_in_heads(wl.batch, wl.heads, wl.tq, nrows, max(2, nrows // 4), seed=0)
        chk = OracleCheck(wl, scale, rows, nth)
        log("[bench] oracle carries %d sampled rows through steps 0..%d (%d host threads)"
            % (len(rows), W + K - 1, nth))

    # ---- warmup: the first W steps of the trajectory (untimed) ----
    for t in range(W):
        q, k, v = tr.tensors()
        step(q, k, v, warm_mask[t % 2], warm_mask[(t + 1) % 2], tau_at(t))
        if chk is not None:
            chk.step("timed", t, q, k, v, tau_at(t), keep=t in check_steps)
        tr.advance()
    if W:
        masks[0].copy_(warm_mask[W % 2])
    # ---- inputs of the K timed steps, resident in HBM before timing ----
    inputs = []
    for t in range(K):
        inputs.append(tr.tensors())
        if chk is not None:
            chk.step("timed", W + t, *inputs[-1], tau_at(W + t), keep=W + t in check_steps)
            if t % 5 == 4:
                log("[bench] oracle at step %d" % (W + t))
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
        la.lite_attn_fwd(q, k, v, out, tile_m=wl.tile_m, tile_n=wl.tile_n, tau=-math.inf, softmax_scale=scale,
                         **FWD_KW)
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

    # ---- check of timed steps against the oracle's own trajectory ----
    # The step is run again (untimed) with lse into check buffers, from the
    # timed step's mask_in; its mask_out must equal the timed step's bit for bit.
    checks = []
    ck_out = ck_lse = ck_mask = None
    if chk is not None:
        ck_out = torch.empty_like(out)
        ck_lse = torch.empty(wl.batch, wl.heads, wl.seqlen, dtype=torch.float32, device=dev)
        ck_mask = torch.empty(nw, dtype=torch.int32, device=dev)

    def check_step(label, t, q, k, v, m_in, tau, m_timed=None):
        if sl is not None and m_in is not None:
            la.lite_attn_build_skiplist(desc, m_in, sl)
        la.lite_attn_fwd(q, k, v, ck_out, tile_m=wl.tile_m, tile_n=wl.tile_n, tau=tau, softmax_scale=scale,
                         mask_in=m_in, mask_out=ck_mask if m_in is not None else None,
                         skiplist=sl if m_in is not None else None, lse=ck_lse, **FWD_KW)
        torch.cuda.synchronize()
        c = chk.compare(label, t, tau, ck_out, ck_lse, m_in, ck_mask if m_in is not None else None)
        if m_timed is not None:
            c["mask_out_equals_measured_step"] = bool(torch.equal(ck_mask, m_timed))
            c["within_bars"] = c["within_bars"] and c["mask_out_equals_measured_step"]
        checks.append(c)
        log("[bench] check %s step %d: %s" % (label, t, c))

    if chk is not None:
        for t in check_steps:
            q, k, v = inputs[t - W]
            check_step("timed", t, q, k, v, masks[t - W], tau_at(t), masks[t - W + 1])
    sl_ms = aux_ev[0][0].elapsed_time(aux_ev[0][1]) / 10 if sl is not None else None
    reset_ms = aux_ev[1][0].elapsed_time(aux_ev[1][1]) / 10
    aux = aux_kernels(masks[K], wl, sl_ms, reset_ms, aux_ev[2][0].elapsed_time(aux_ev[2][1]) / 10,
                      aux_ev[3][0].elapsed_time(aux_ev[3][1]) / 10)
    del out_b, out_m, lses
    del inputs

    value = sum(flops) / wall / 1e12
    achieved = sum(flops) / (sum(kern_ms) * 1e-3) / 1e12
    code_hash = kernel_code_hash(wl.dtype)
    if bf16 and wl.name == "c4_bf16_76k" and args.path == "skiplist":
        traffic, traffic_note = read_traffic(code_hash)
        clock, clock_note = read_clock(code_hash)
    else:
        traffic, traffic_note = None, ("the committed counter summaries cover the 75,600-token bf16 workload "
                                       "on the Skip-List walk only")
        clock, clock_note = None, traffic_note
    sparsity = [1.0 - f / dense_flops for f in flops]
    occupancy = [pair_occupancy(masks[t], wl) for t in range(K)]

    # ---- tau sweep over a trajectory (kernel time per step, per threshold) ----
    sweep = None
    sweep_same_as_timed = None
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
        # the threshold whose trajectory is the timed one: its sweep masks must
        # equal the timed run's; the others are checked against the oracle
        head_tau = None if (wl.tau_schedule is not None and args.tau is None) else tau_at(0)
        S = min(args.check_sweep_steps, args.sweep_steps)
        for t in range(args.sweep_steps):
            q, k, v = tr2.tensors()
            pend = []
            for tau in taus:
                m_in, m_out = sm[tau][t % 2], sm[tau][(t + 1) % 2]
                ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                if tau is not None and math.isinf(tau):
                    ev[0].record()
                    la.lite_attn_fwd(q, k, v, out, tile_m=wl.tile_m, tile_n=wl.tile_n, tau=tau, softmax_scale=scale,
                                     **FWD_KW)
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
            if t == W + K - 1 and head_tau in sm:
                sweep_same_as_timed = bool(torch.equal(sm[head_tau][(t + 1) % 2], masks[K]))
            if chk is not None:
                for tau in taus:
                    dense = tau is not None and math.isinf(tau)
                    if tau == head_tau or t >= (1 if dense else S):
                        continue
                    tt = wl.tau_at(t) if tau is None else tau
                    label = "sweep tau %s" % ("-inf" if dense else tt if tau is not None else "schedule")
                    last = t == (0 if dense else S - 1)
                    chk.step(label, t, q, k, v, tt, keep=last, timed=False)
                    if last:
                        check_step(label, t, q, k, v, None if dense else sm[tau][t % 2], tt,
                                   None if dense else sm[tau][(t + 1) % 2])
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

    # ---- CPU baseline: the oracle's calls on the sampled rows of the timed trajectory ----
    cpu = None
    verification = None
    if chk is not None:
        cpu = {"value": round(chk.flops / chk.seconds / 1e12, 6), "unit": "TFLOP/s",
               "cores": min(chk.threads, len(chk.rows)), "kind": "oracle",
               "sample": "%d of %d q-tile rows (%d heads, incl. the last head's last partial q-tile), carried by "
                         "the oracle through steps 0..%d of the trajectory from an empty mask; live tiles only, "
                         "fp64, %.1f s on %d threads of %s"
                         % (len(chk.rows), wl.rows, len({int(r // wl.tq) for r in chk.rows}), W + K - 1,
                            chk.seconds, min(chk.threads, len(chk.rows)), cpu_model())}
        verification = {
            "rule": "outputs max-abs <= %g, lse <= %g, masks bit-exact off a 1e-3 band around tau (counted as "
                    "near_tau); rows compared where the carried masks agree" % (
                        pa.TOL_OUT[out.dtype], pa.TOL_LSE[out.dtype]),
            "max_abs_out": max((c["max_abs_out"] for c in checks), default=None),
            "max_lse": max((c["max_lse"] for c in checks), default=None),
            "mask_mismatch": sum(c["mask_mismatch"] for c in checks),
            "near_tau": sum(c["near_tau"] for c in checks),
            "diverged_rows": sum(c["diverged_rows"] for c in checks),
            "within_bars": all(c["within_bars"] for c in checks),
            "sweep_masks_equal_timed_run": sweep_same_as_timed if sweep else None,
            "steps": checks}

    variants = dense_variants(torch, la) if args.dense_variants else None
    pair = pair_workload(args) if (args.workload == "c4_bf16_76k" and not args.no_pair and not args.grid
                                   and not args.heads and args.tau is None) else None

    res = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(wall * 1e3 / K, 3), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if bf16 else "fp64", "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "heads": wl.heads, "seq_len": wl.seqlen,
                   "grid": list(wl.grid), "head_dim": wl.head_dim, "tile": "%dx%d" % (wl.tile_m, wl.tile_n),
                   "tau": tau_desc, "path": args.path, "timed_steps": [W, W + K - 1],
                   "schedule": args.schedule if bf16 else None},
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
                     "clock_ghz": round(clock, 3) if clock else None,
                     "frac_at_clock": round(achieved / (peak * clock / 2.4), 4) if clock else None,
                     "clock_note": clock_note,
                     "kernel": ("fwd_bf16_kernel<%d, %d, %s>" % (wl.head_dim, wl.tile_n,
                                                                  "true" if args.path == "skiplist" else "false"))
                     if bf16 else "fwd_fp32_kernel",
                     "kernel_code_sha256_16": code_hash},
        "cpu_baseline": cpu,
        "verification": verification,
        "tau_sweep": sweep,
        "dense_variants": variants,
        "pair_workload": pair,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
