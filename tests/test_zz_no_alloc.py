"""GPU: lite_attn_fwd_noalloc, whose schedule counters are the library's own
static array, against lite_attn_fwd with caller-owned counters, through the
C ABI: out, lse and mask_out equal bit for bit, on two calls in a row, the
second with a smaller input (the array keeps the first call's contents until
the second clears it)."""

import sys

import pytest
import torch

from temporal_block_sparse_amd import lite_attn as la
from temporal_block_sparse_amd import synth

pytestmark = pytest.mark.gpu


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def call(fn, q, k, v, tile_n, tau, mask_in, use_skiplist, **kw):
    B, N, H, _ = q.shape
    desc = la.desc_of(q, 128, tile_n, k)
    out = torch.empty_like(q)
    lse = torch.empty(B, H, N, dtype=torch.float32, device=q.device)
    mask_out = torch.empty_like(mask_in)
    sl = None
    if use_skiplist:
        sl = la.alloc_skiplist(desc, q.device)
        la.lite_attn_build_skiplist(desc, mask_in, sl)
    fn(q, k, v, out, tile_m=128, tile_n=tile_n, tau=tau, mask_in=mask_in, mask_out=mask_out, skiplist=sl, lse=lse,
       **kw)
    return out, lse, mask_out


@pytest.mark.parametrize("use_skiplist", [False, True], ids=["bitmask", "skiplist"])
def test_noalloc_entry_point_matches_lite_attn_fwd(use_skiplist):
    dev = torch.device("cuda")
    counters = torch.zeros(la.SCHED_WORDS, dtype=torch.int32, device=dev)
    # (batch, tokens, heads, head_dim, tile_n): 1,056 q-tile pairs, then 6
    for i, (B, N, H, d, tile_n) in enumerate(((1, 16500, 16, 128, 128), (1, 1500, 2, 64, 64))):
        log("  call %d: B=%d N=%d H=%d d=%d tile 128x%d %s" % (i, B, N, H, d, tile_n,
                                                             "skiplist" if use_skiplist else "bitmask"))
        q, k, v = synth.random_qkv(B, N, H, d, dtype=torch.bfloat16, seed=60 + i, scale=2.0, device=dev)
        tq, tk = -(-N // 128), -(-N // tile_n)
        mask_in = synth.random_mask(B * H * tq, tk, 0.5, seed=70 + i).to(dev)
        ref = call(la.lite_attn_fwd, q, k, v, tile_n, -2.0, mask_in, use_skiplist, sched=counters)
        got = call(la.lite_attn_fwd_noalloc, q, k, v, tile_n, -2.0, mask_in, use_skiplist)
        torch.cuda.synchronize()
        for name, a, b in zip(("out", "lse", "mask_out"), ref, got):
            if a.dtype == torch.bfloat16:
                a, b = a.view(torch.int16), b.view(torch.int16)
            assert torch.equal(a, b), (i, name)
        assert counters.tolist() == [0, 0]


def test_noalloc_entry_point_fp32_path():
    """The fp32 forward has no schedule counters: through the allocation-free
    entry point it is the same call, bit for bit."""
    dev = torch.device("cuda")
    q, k, v = synth.random_qkv(1, 700, 2, 64, dtype=torch.float32, seed=80, scale=2.0, device=dev)
    mask_in = synth.random_mask(2 * 11, 11, 0.4, seed=81).to(dev)
    outs = []
    for fn in (la.lite_attn_fwd, la.lite_attn_fwd_noalloc):
        out = torch.empty_like(q)
        lse = torch.empty(1, 2, 700, dtype=torch.float32, device=dev)
        mask_out = torch.empty_like(mask_in)
        fn(q, k, v, out, tile_m=64, tile_n=64, tau=-2.0, mask_in=mask_in, mask_out=mask_out, lse=lse)
        outs.append((out, lse, mask_out))
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a, b)
