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


def test_rows_live_flops_brute_force():
    wl = configs.scaled(configs.C4, (3, 10, 30), heads=3, batch=2)
    rows = np.array([0, wl.tq - 1, wl.rows - 1], np.int64)
    for density in (0.0, 0.5):
        mw = synth.random_mask(wl.rows, wl.tk, density, seed=9).numpy().view(np.uint32)
        bits = _bits(torch.from_numpy(mw.view(np.int32)).reshape(-1), wl)
        want = 0.0
        for r in rows:
            qt = r % wl.tq
            nr = min(wl.seqlen, (qt + 1) * wl.tile_m) - qt * wl.tile_m
            for kt in range(wl.tk):
                if not bits[r, kt]:
                    want += 4.0 * wl.head_dim * nr * (min(wl.seqlen, (kt + 1) * wl.tile_n) - kt * wl.tile_n)
        assert bench.rows_live_flops(mw[rows], rows, wl) == want


def test_oracle_check_compares_what_it_should():
    """The benchmark's check of timed steps: GPU results equal to the oracle's
    own (made here from the oracle's numbers, as a stand-in) are within the bars
    with every row compared; a row whose carried mask differs from the oracle's
    is counted as diverged and left out; a wrong output or mark is flagged."""
    import math
    wl = configs.scaled(configs.C4, (6, 10, 16), heads=2, batch=2)         # N 960: Tq = Tk = 8
    q, k, v = synth.Trajectory(wl, "cpu").tensors()
    rows = np.array([0, 3, wl.rows - 1, wl.rows - 2], np.int64)
    chk = bench.OracleCheck(wl, 1.0 / math.sqrt(wl.head_dim), rows, 2)
    chk.step("t", 0, q, k, v, 0.0, keep=True)
    chk.step("t", 1, q, k, v, 0.0, keep=True)
    res, rm = chk.results[("t", 1)]
    assert chk.flops > 0 and chk.seconds > 0
    B, N, H, D, BM, W = wl.batch, wl.seqlen, wl.heads, wl.head_dim, wl.tile_m, wl.mask_words
    out = torch.zeros(B, N, H, D, dtype=torch.bfloat16)
    lse = torch.zeros(B, H, N)
    m_in = torch.zeros(wl.rows * W, dtype=torch.int32)
    m_out = torch.zeros(wl.rows * W, dtype=torch.int32)
    for i, r in enumerate(rows):
        b, h, qt = int(r // (wl.tq * H)), int((r // wl.tq) % H), int(r % wl.tq)
        nr = min(BM, N - qt * BM)
        out[b, qt * BM:qt * BM + nr, h] = torch.from_numpy(res["out"][i][:nr]).to(torch.bfloat16)
        lse[b, h, qt * BM:qt * BM + nr] = torch.from_numpy(res["lse"][i][:nr]).float()
        m_in.view(-1, W)[r] = torch.from_numpy(rm[i].view(np.int32))
        m_out.view(-1, W)[r] = torch.from_numpy(res["mask_out"][i].view(np.int32))
    c = chk.compare("t", 1, 0.0, out, lse, m_in, m_out)
    assert c["within_bars"] and c["rows_compared"] == 4 and c["diverged_rows"] == 0, c
    assert rm.any(), "the carried mask is empty: the test would not see it compared"
    # a diverged carried mask: that row is left out
    m_in2 = m_in.clone()
    m_in2.view(-1, W)[rows[0], 0] ^= 1 << 2
    c = chk.compare("t", 1, 0.0, out, lse, m_in2, m_out)
    assert c["diverged_rows"] == 1 and c["rows_compared"] == 3 and c["within_bars"], c
    # a wrong output and a wrong mark are flagged
    out2 = out.clone()
    out2[0, 5, 0, 3] += 0.5
    assert not chk.compare("t", 1, 0.0, out2, lse, m_in, m_out)["within_bars"]
    m_out2 = m_out.clone()
    margins = res["margin"][1]
    kt = int(np.nanargmax(np.where(np.isfinite(margins), np.abs(margins), -1)))
    m_out2.view(-1, W)[rows[1], kt // 32] ^= 1 << (kt % 32)
    c = chk.compare("t", 1, 0.0, out, lse, m_in, m_out2)
    assert c["mask_mismatch"] == 1 and not c["within_bars"], c
    # a step without mask_in / mask_out (the dense check) compares outputs only
    chk.step("d", 0, q, k, v, -math.inf, keep=True)
    res, _ = chk.results[("d", 0)]
    for i, r in enumerate(rows):
        b, h, qt = int(r // (wl.tq * H)), int((r // wl.tq) % H), int(r % wl.tq)
        nr = min(BM, N - qt * BM)
        out[b, qt * BM:qt * BM + nr, h] = torch.from_numpy(res["out"][i][:nr]).to(torch.bfloat16)
        lse[b, h, qt * BM:qt * BM + nr] = torch.from_numpy(res["lse"][i][:nr]).float()
    c = chk.compare("d", 0, -math.inf, out, lse, None, None)
    assert c["within_bars"] and c["rows_compared"] == 4 and c["tau"] is None, c


def test_trajectory_tensors_are_snapshots():
    """A step's tensors must not change when the trajectory drifts on: the
    benchmark keeps the timed steps' inputs while it advances (the fp32
    workload's state was once returned by reference)."""
    for wl in (configs.C1, configs.scaled(configs.C2, (2, 4, 8), heads=1)):
        tr = synth.Trajectory(wl, "cpu")
        q, k, v = tr.tensors()
        q0 = q.clone()
        tr.advance()
        assert torch.equal(q, q0)
        assert not torch.equal(tr.tensors()[0], q0)


def test_code_hash_ignores_comments_and_layout_only():
    """The counter summaries are tied to the kernel's code: a comment or
    indentation edit keeps the hash, any change to code or to a literal
    changes it."""
    src = ('#include "a.h"  // header\n'
           '/* block\n   comment */ int f(int x) {\n'
           '    asm volatile("s_nop 0 // not a comment");\n'
           "    char c = '\"'; // a quote in a char literal\n"
           '    return x + 1;\n}\n')
    base = bench.strip_code(src)
    assert "block" not in base and "header" not in base
    assert '"s_nop 0 // not a comment"' in base and "'\"'" in base
    same = [src.replace("// header", "// the header, reworded"),
            src.replace("    return", "\t\treturn"),
            src.replace("/* block\n   comment */", "/* one line */"),
            src + "\n\n// trailing note\n"]
    for s in same:
        assert bench.strip_code(s) == base, s
    changed = [src.replace("x + 1", "x + 2"),
               src.replace("s_nop 0", "s_nop 1"),
               src.replace("int f", "long f")]
    for s in changed:
        assert bench.strip_code(s) != base, s
    assert len(bench.kernel_code_hash("bf16")) == 16
    assert bench.kernel_code_hash("bf16") != bench.kernel_code_hash("fp32")


def test_profiled_clock_reader(tmp_path, monkeypatch):
    """The clock reported next to the roofline comes from the committed counter
    summary of the same code: the timed masked launches (not the warmup, not the
    dense reference), and nothing when the code hash differs."""
    code = bench.kernel_code_hash("bf16")
    ghz, note = bench.read_clock(code)
    assert ghz is not None and 1.0 < ghz < 2.5, (ghz, note)
    assert bench.read_clock("0" * 16)[0] is None
    f = tmp_path / "pmc.txt"
    f.write_text("# header\nkernel_code_sha256_16: abc\n\n"
                 "dispatch  kernel  dur_ms GHz\n"
                 "24        <128, 128, true> skip-list       102.42   1.500     63.8%  32.0  57.8%  0.02%  6.18  67.5%\n"
                 "51        <128, 128, true> skip-list        86.19   1.800     58.4%  32.0  53.6%  0.02%  6.27  29.8%\n"
                 "53        <128, 128, true> skip-list        85.27   1.900     58.3%  32.0  53.6%  0.02%  6.27  29.7%\n"
                 "87        <128, 128, false> dense ref       99.71   1.648     68.0%  32.0  60.9%  0.01%  6.08  91.5%\n")
    monkeypatch.setattr(bench, "PMC_FILE", str(f))
    ghz, _ = bench.read_clock("abc")
    assert abs(ghz - 1.85) < 1e-12
    assert bench.read_clock("abd")[0] is None
