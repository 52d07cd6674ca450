"""GPU: the bf16 forward's two schedules give the same results bit for bit.

Without schedule counters the forward launches one workgroup per q-tile pair;
with them, one persistent workgroup per compute unit draws the pairs from an
atomic ticket.  Every pair is computed by the same code from the same inputs
either way, so out, lse and mask_out must be equal bit for bit, and the
counters must read zero after every call (the last workgroup resets them).
Parity of the ticket schedule with the oracle is the rest of the GPU suite:
the binding uses it by default."""

import sys

import pytest
import torch

from temporal_block_sparse_amd import lite_attn as la
from temporal_block_sparse_amd import synth

pytestmark = pytest.mark.gpu

# (batch, tokens, heads, head_dim, tile_n, tau, Skip-List walk, token ranges, mask density)
CASES = [
    (1, 1000, 2, 128, 128, -3.0, False, {}, 0.3),                       # 4 pairs: fewer than the CUs
    (1, 8200, 8, 128, 128, -3.0, True, {}, 0.5),                        # 65 q-tiles (odd): 264 pairs
    (2, 12000, 6, 64, 64, -2.0, True, {}, 0.6),                         # d = 64: 564 pairs
    (1, 16384, 16, 128, 64, -1.0, False,
     dict(must_do=[16383, 16200], must_skip=[9000, 7000]), 0.4),        # 1024 pairs, 4 per CU
]


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run(q, k, v, tile_n, tau, mask_in, use_skiplist, rg, sched):
    B, N, H, _ = q.shape
    desc = la.desc_of(q, 128, tile_n, k)
    out = torch.empty_like(q)
    lse = torch.empty(B, H, N, dtype=torch.float32, device=q.device)
    mask_out = torch.empty_like(mask_in)
    sl = None
    if use_skiplist:
        sl = la.alloc_skiplist(desc, q.device)
        la.lite_attn_build_skiplist(desc, mask_in, sl, **rg)
    la.lite_attn_fwd(q, k, v, out, tile_m=128, tile_n=tile_n, tau=tau, mask_in=mask_in, mask_out=mask_out,
                     skiplist=sl, lse=lse, sched=sched, **rg)
    return out, lse, mask_out


def test_ticket_schedule_equals_one_workgroup_per_pair():
    dev = torch.device("cuda")
    counters = torch.zeros(la.SCHED_WORDS, dtype=torch.int32, device=dev)  # one buffer for every call
    for i, (B, N, H, d, tile_n, tau, use_skiplist, rg, density) in enumerate(CASES):
        log("  case %d: B=%d N=%d H=%d d=%d tile 128x%d tau %g skiplist %s ranges %s"
            % (i, B, N, H, d, tile_n, tau, use_skiplist, bool(rg)))
        q, k, v = synth.random_qkv(B, N, H, d, dtype=torch.bfloat16, seed=40 + i, scale=2.0, device=dev)
        desc = la.desc_of(q, 128, tile_n, k)
        tq, tk = -(-N // 128), -(-N // tile_n)
        mask_in = synth.random_mask(B * H * tq, tk, density, seed=i).to(dev)  # pairs' costs differ
        assert mask_in.numel() == la.lite_attn_mask_words(desc)
        ref = run(q, k, v, tile_n, tau, mask_in, use_skiplist, rg, None)
        got = run(q, k, v, tile_n, tau, mask_in, use_skiplist, rg, counters)
        torch.cuda.synchronize()
        for name, a, b in zip(("out", "lse", "mask_out"), ref, got):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b), (i, name)
        assert counters.tolist() == [0, 0], (i, counters.tolist())
        log("    newly marked words: %d" % int((ref[2] != mask_in).sum()))


def test_counters_left_zero_by_back_to_back_calls():
    """Several calls in a row on one stream share one buffer; each starts from
    the zeros the previous one left, also when the grid shrinks (fewer pairs
    than compute units) and grows again."""
    dev = torch.device("cuda")
    counters = torch.zeros(la.SCHED_WORDS, dtype=torch.int32, device=dev)
    outs = []
    for N in (8200, 300, 8200):
        q, k, v = synth.random_qkv(1, N, 8, 128, dtype=torch.bfloat16, seed=7, scale=2.0, device=dev)
        o1, o2 = torch.empty_like(q), torch.empty_like(q)
        la.lite_attn_fwd(q, k, v, o1, tile_m=128, tile_n=128, tau=-3.0, sched=None)
        for _ in range(3):
            la.lite_attn_fwd(q, k, v, o2, tile_m=128, tile_n=128, tau=-3.0, sched=counters)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), N
        assert counters.tolist() == [0, 0], N
        outs.append(o2)
    assert torch.equal(outs[0].view(torch.int16), outs[2].view(torch.int16))


def test_binding_keeps_one_buffer_per_stream():
    dev = torch.device("cuda")
    q, k, v = synth.random_qkv(1, 1000, 2, 128, dtype=torch.bfloat16, seed=3, device=dev)
    ref = torch.empty_like(q)
    la.lite_attn_fwd(q, k, v, ref, tile_m=128, tile_n=128, tau=-3.0, sched=None)
    outs = [torch.empty_like(q), torch.empty_like(q)]
    torch.cuda.synchronize()                      # inputs ready before the side streams read them
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for s, o in zip((s1, s2), outs):
        with torch.cuda.stream(s):
            la.lite_attn_fwd(q, k, v, o, tile_m=128, tile_n=128, tau=-3.0)
    torch.cuda.synchronize()
    di = torch.cuda.current_device()
    b1, b2 = la._SCHED[(di, s1.cuda_stream)], la._SCHED[(di, s2.cuda_stream)]
    assert b1.data_ptr() != b2.data_ptr()
    assert b1.tolist() == [0, 0] and b2.tolist() == [0, 0]
    for o in outs:
        assert torch.equal(o.view(torch.int16), ref.view(torch.int16))


def _random_cases(n, seed):
    g = torch.Generator().manual_seed(seed)
    r = lambda lo, hi: int(torch.randint(lo, hi + 1, (1,), generator=g))  # noqa: E731
    cases = []
    for i in range(n):
        B, d, tile_n = r(1, 2), (64, 128)[r(0, 1)], (64, 128)[r(0, 1)]
        N, H = r(2000, 9000), r(4, 16)
        pph = (-(-N // 128) + 1) // 2                 # q-tile pairs per (batch entry, head)
        H = max(H, -(-300 // (B * pph)))              # at least 300 pairs: more than the CUs
        tk = -(-N // tile_n)
        rg = {}
        if r(0, 2) == 0:   # token ranges on a third of the cases
            a = r(N // 2, N - 1)
            rg = dict(must_do=[N - 1, N - 1 - r(1, 300)], must_skip=[a, a - r(1, 2000)])
            if rg["must_skip"][1] < -1 or rg["must_skip"][0] >= rg["must_do"][1]:
                rg = dict(must_do=rg["must_do"])
        cases.append((B, N, H, d, tile_n, -0.5 * r(0, 10), bool(r(0, 1)), rg, 0.1 * r(0, 9), tk))
    return cases


@pytest.mark.parametrize("i,case", list(enumerate(_random_cases(12, 2024))))
def test_random_shapes_with_several_pairs_per_workgroup(i, case):
    """Seeded shapes whose launches hold more q-tile pairs than the GPU has
    compute units, so persistent workgroups draw several tickets each; ragged
    last tiles, odd q-tile counts (a last pair with one q-tile), batch 2,
    token ranges.  The ticket schedule must equal one workgroup per pair bit
    for bit (that path is held to the oracle by the parity tests)."""
    B, N, H, d, tile_n, tau, use_skiplist, rg, density, tk = case
    dev = torch.device("cuda")
    tq = -(-N // 128)
    log("  case %d: B=%d N=%d H=%d d=%d tile 128x%d tau %g skiplist %s ranges %s density %.1f pairs %d"
        % (i, B, N, H, d, tile_n, tau, use_skiplist, rg, density, B * H * ((tq + 1) // 2)))
    q, k, v = synth.random_qkv(B, N, H, d, dtype=torch.bfloat16, seed=100 + i, scale=2.0, device=dev)
    mask_in = synth.random_mask(B * H * tq, tk, density, seed=200 + i).to(dev)
    counters = torch.zeros(la.SCHED_WORDS, dtype=torch.int32, device=dev)
    ref = run(q, k, v, tile_n, tau, mask_in, use_skiplist, rg, None)
    got = run(q, k, v, tile_n, tau, mask_in, use_skiplist, rg, counters)
    torch.cuda.synchronize()
    for name, a, b in zip(("out", "lse", "mask_out"), ref, got):
        if a.dtype == torch.bfloat16:
            a, b = a.view(torch.int16), b.view(torch.int16)
        assert torch.equal(a, b), (i, name)
    assert counters.tolist() == [0, 0]
