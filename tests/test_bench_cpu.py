"""The benchmark's accounting, checked by brute force on the CPU: the live-tile
flop count behind every TFLOP/s figure, the pair occupancy, and the
algorithmic bytes of the HBM-bound kernels.  Also the one-GPU guard."""

import os
import subprocess
import sys

import numpy as np
import torch

import bench
from temporal_block_sparse_amd import configs, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _workloads():
    # ragged q- and k-tiles, several batch entries and heads, odd and even Tq
    yield configs.scaled(configs.C4, (3, 10, 30), heads=3, batch=2)     # N 900: Tq = Tk = 8, last tile 4
    yield configs.scaled(configs.C2, (4, 10, 25), heads=2, batch=1)     # N 1000: Tq 8, Tk 16 (128x64)
    yield configs.scaled(configs.C4, (5, 7, 9), heads=1, batch=1)       # N 315: Tq = Tk = 3 (odd)


def _bits(mask_words, wl):
    m = mask_words.numpy().view(np.uint32).reshape(wl.rows, wl.mask_words)
    return np.array([[(int(m[r, kt // 32]) >> (kt % 32)) & 1 for kt in range(wl.tk)] for r in range(wl.rows)], bool)


def test_live_flops_brute_force():
    for wl in _workloads():
        for density in (0.0, 0.4, 1.0):
            mw = synth.random_mask(wl.rows, wl.tk, density, seed=5).view(torch.int32).reshape(-1)
            bits = _bits(mw, wl)
            want = 0
            for r in range(wl.rows):
                qt = r % wl.tq
                rows_valid = min(wl.seqlen, (qt + 1) * wl.tile_m) - qt * wl.tile_m
                for kt in range(wl.tk):
                    if not bits[r, kt]:
                        cols_valid = min(wl.seqlen, (kt + 1) * wl.tile_n) - kt * wl.tile_n
                        want += 4 * wl.head_dim * rows_valid * cols_valid
            assert bench.live_flops(mw, wl) == want, (wl.name, density)
        assert bench.live_flops(None, wl) == 4.0 * wl.batch * wl.heads * wl.seqlen ** 2 * wl.head_dim


def test_pair_occupancy_brute_force():
    for wl in _workloads():
        mw = synth.random_mask(wl.rows, wl.tk, 0.5, seed=6).view(torch.int32).reshape(-1)
        bits = _bits(mw, wl)
        live = union = 0
        for bh in range(wl.batch * wl.heads):
            for j in range(0, wl.tq, 2):
                a = ~bits[bh * wl.tq + j]
                b = ~bits[bh * wl.tq + j + 1] if j + 1 < wl.tq else np.zeros(wl.tk, bool)
                live += a.sum() + b.sum()
                union += (a | b).sum()
        assert abs(bench.pair_occupancy(mw, wl) - live / (2.0 * union)) < 1e-12, wl.name
    # every tile live: 1 with an even number of q-tiles, (Tq) / (Tq + 1) with an odd one
    for wl in _workloads():
        occ = bench.pair_occupancy(torch.zeros(wl.rows * wl.mask_words, dtype=torch.int32), wl)
        assert abs(occ - (1.0 if wl.tq % 2 == 0 else wl.tq / (wl.tq + 1.0))) < 1e-12, wl.name


def test_aux_kernel_bytes_brute_force():
    for wl in _workloads():
        mw = synth.random_mask(wl.rows, wl.tk, 0.3, seed=7).view(torch.int32).reshape(-1)
        bits = _bits(mw, wl)
        aux = bench.aux_kernels(mw, wl, 1.0, 1.0, 1.0, 1.0)
        assert aux["skiplist_build"]["bytes"] == 4 * wl.rows * wl.mask_words + 4 * int((1 + (~bits).sum(axis=1)).sum())
        assert aux["reset_mask"]["bytes"] == 4 * wl.rows * wl.mask_words
        qh = wl.batch * wl.seqlen * wl.heads
        assert aux["lse_merge_2_parts"]["bytes"] == 3 * qh * (2 * wl.head_dim + 4)
        assert aux["error_sums"]["bytes"] == 2 * qh * 2 * wl.head_dim
        # 1 ms per call: bytes / 1e-3 s in GB/s
        e = aux["reset_mask"]
        assert abs(e["GB/s"] - round(e["bytes"] / 1e-3 / 1e9, 1)) < 1e-9
        assert abs(e["frac"] - round(e["bytes"] / 1e-3 / 1e9 / bench.PEAK_HBM_GBS, 4)) < 1e-12


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr


def test_step_count_must_be_positive():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "0"], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode == 2 and "--steps must be at least 1" in p.stderr


def test_every_workload_gets_to_its_first_gpu_call():
    """The host-side set-up of each workload (arguments, threshold schedule,
    descriptor, log line) runs cleanly; with no GPU visible the run then stops
    at its first device allocation."""
    for name in configs.ALL:
        env = dict(os.environ, HIP_VISIBLE_DEVICES="")
        p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", name, "--steps", "1",
                            "--warmup", "0", "--sweep-steps", "0", "--no-cpu"], env=env, capture_output=True,
                           text=True, timeout=300)
        assert "[bench] workload %s:" % name in p.stderr, (name, p.stderr[-1500:])
