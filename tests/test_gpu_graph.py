"""HIP-graph capture of the per-layer step.

The library allocates nothing, clears memory with fill kernels (no
hipMemsetAsync) and makes no host-synchronising call, so one denoising step
of a layer -- Skip-List build from the mask, then the forward that reads the
mask and marks into it in place -- can be captured once and replayed every
step.  Each replay runs on the step's inputs copied into the captured
buffers, with eager work and a synchronisation between replays, and must give
exactly what the eager calls give at the same step (every kernel here is
deterministic: one workgroup per output row, no atomics on outputs).  A
second graph captures reset + forward: eager calls between its replays grow
the mask, and the captured reset has to clear it every time.  Two layers
stepping on two streams at once must match the same calls made one after the
other.  Last, the bf16 forward with its schedule counters is replayed from a
graph: the kernels reset the counters themselves, so no memset is captured.
"""

import sys

import pytest
import torch

from temporal_block_sparse_amd import configs, synth
from temporal_block_sparse_amd import lite_attn as la

pytestmark = pytest.mark.gpu

CASES = [
    ("bf16 d64 128x64 skiplist", configs.scaled(configs.C2, (4, 10, 25), heads=3, batch=1, steps=4), True),
    ("bf16 d128 128x128 mask", configs.scaled(configs.C3, (3, 10, 30), heads=2, batch=1, steps=4), False),
    ("fp32 d64 64x64 mask", configs.scaled(configs.C1, (4, 8, 20), heads=2, batch=1, steps=4), False),
]


def _steps(wl):
    tr = synth.Trajectory(wl, "cpu")
    out = []
    for s in range(wl.steps):
        if s:
            tr.advance()
        out.append(tuple(t.to("cuda") for t in tr.tensors()))
    return out


@pytest.mark.parametrize("name,wl,use_skiplist", CASES, ids=[c[0] for c in CASES])
def test_graph_replays_equal_eager_steps(name, wl, use_skiplist):
    print("  %s: N %d H %d d %d tile %dx%d steps %d" % (name, wl.seqlen, wl.heads, wl.head_dim, wl.tile_m,
                                                       wl.tile_n, wl.steps), flush=True)
    sys.stdout.flush()
    steps = _steps(wl)
    kw = dict(threshold=-3.0, tile_m=wl.tile_m, tile_n=wl.tile_n, use_skiplist=use_skiplist)

    # eager reference: one layer over the trajectory
    ref = la.LiteAttention(**kw)
    eager = []
    for q, k, v in steps:
        o, l = ref(q, k, v, return_softmax_lse=True)
        eager.append((o.clone(), l.clone(), ref.mask.clone()))
    torch.cuda.synchronize()
    assert (eager[-1][2] != 0).any(), "the trajectory marks nothing; the test would not see the mask carried"

    # the same layer, captured once
    qs, ks, vs = (t.clone() for t in steps[0])
    attn = la.LiteAttention(**kw)
    attn._state_for(qs, ks)                    # mask (and Skip-List) allocated and cleared before capture
    out = torch.empty_like(qs)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _, lse = attn(qs, ks, vs, out=out, return_softmax_lse=True)
    for s, (q, k, v) in enumerate(steps):
        qs.copy_(q)
        ks.copy_(k)
        vs.copy_(v)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager[s][0]), "%s: output differs at step %d" % (name, s)
        assert torch.equal(lse, eager[s][1]), "%s: lse differs at step %d" % (name, s)
        assert torch.equal(attn.mask, eager[s][2]), "%s: mask differs at step %d" % (name, s)

    # reset + forward captured together; eager calls in between grow the mask
    g2 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g2):
        attn.reset_skip_state()
        attn(qs, ks, vs, out=out)
    for r in range(3):
        qs.copy_(steps[0][0])
        ks.copy_(steps[0][1])
        vs.copy_(steps[0][2])
        g2.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager[0][0]), "%s: reset+forward replay %d output" % (name, r)
        assert torch.equal(attn.mask, eager[0][2]), "%s: reset+forward replay %d mask" % (name, r)
        for q, k, v in steps[1:]:
            attn(q, k, v)                      # eager steps on the same mask
        torch.cuda.synchronize()
        assert torch.equal(attn.mask, eager[-1][2])


def test_two_streams_equal_sequential_calls():
    """No state in the library, all work on the caller's stream: two layers
    stepping their own masks on two streams at once give exactly what they
    give one after the other (streams at the default priority)."""
    wls = [configs.scaled(configs.C2, (4, 10, 25), heads=3, batch=1, steps=3),
           configs.scaled(configs.C3, (3, 10, 30), heads=2, batch=1, steps=3)]
    kws = [dict(threshold=-3.0, tile_m=w.tile_m, tile_n=w.tile_n, use_skiplist=s) for w, s in zip(wls, (True, False))]
    steps = [_steps(w) for w in wls]
    # one after the other, on the current stream
    seq = []
    for kw, st in zip(kws, steps):
        a = la.LiteAttention(**kw)
        seq.append([(a(q, k, v).clone(), a.mask.clone()) for q, k, v in st])
    torch.cuda.synchronize()
    # both layers at once, each on its own stream
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    layers = [la.LiteAttention(**kw) for kw in kws]
    res = [[], []]
    torch.cuda.synchronize()
    for t in range(3):
        for i in range(2):
            with torch.cuda.stream(streams[i]):
                q, k, v = steps[i][t]
                res[i].append((layers[i](q, k, v).clone(), layers[i].mask.clone()))
    torch.cuda.synchronize()
    for i in range(2):
        for t in range(3):
            assert torch.equal(res[i][t][0], seq[i][t][0]), "layer %d step %d output" % (i, t)
            assert torch.equal(res[i][t][1], seq[i][t][1]), "layer %d step %d mask" % (i, t)


def test_ticket_counters_inside_a_graph():
    """The bf16 forward with caller-owned schedule counters, captured into a
    graph: the kernels reset the counters themselves (no memset node), so
    every replay -- with eager calls on the same counters in between --
    draws its tickets from zero and gives the eager result, and the counters
    read zero after each replay."""
    wl = configs.scaled(configs.C3, (10, 30, 60), heads=4, batch=1, steps=3)  # 18,000 tokens: 284 pairs
    steps = _steps(wl)
    print("  N %d H %d pairs %d" % (wl.seqlen, wl.heads, wl.heads * ((wl.tq + 1) // 2)), flush=True)
    counters = torch.zeros(la.SCHED_WORDS, dtype=torch.int32, device="cuda")
    desc = la.desc_of(steps[0][0], wl.tile_m, wl.tile_n)
    kw = dict(tile_m=wl.tile_m, tile_n=wl.tile_n, tau=-3.0)
    # eager reference over the trajectory, mask carried
    mask = torch.zeros(la.lite_attn_mask_words(desc), dtype=torch.int32, device="cuda")
    eager = []
    for q, k, v in steps:
        o = torch.empty_like(q)
        la.lite_attn_fwd(q, k, v, o, mask_in=mask, mask_out=mask, sched=counters, **kw)
        eager.append((o, mask.clone()))
    torch.cuda.synchronize()
    assert counters.tolist() == [0, 0]
    # capture one step with the same counters
    qs, ks, vs = (t.clone() for t in steps[0])
    out = torch.empty_like(qs)
    gmask = torch.zeros_like(mask)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        la.lite_attn_fwd(qs, ks, vs, out, mask_in=gmask, mask_out=gmask, sched=counters, **kw)
    for s, (q, k, v) in enumerate(steps):
        qs.copy_(q)
        ks.copy_(k)
        vs.copy_(v)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager[s][0].view(torch.int16)), "replay %d output" % s
        assert torch.equal(gmask, eager[s][1]), "replay %d mask" % s
        assert counters.tolist() == [0, 0], "replay %d left counters %s" % (s, counters.tolist())
        # an eager call on the same counters between replays
        scratch = torch.empty_like(q)
        la.lite_attn_fwd(q, k, v, scratch, sched=counters, **kw)
        torch.cuda.synchronize()
        assert counters.tolist() == [0, 0]


def test_binding_captures_without_counters_on_a_stream_that_has_them():
    """A stream whose eager calls already use the binding's counter buffer is
    then captured: while it captures, the binding passes no counters, so the
    graph holds the one-workgroup-per-pair launch and shares nothing with the
    eager calls.  Replays equal the eager result."""
    wl = configs.scaled(configs.C3, (10, 30, 60), heads=4, batch=1, steps=2)
    (q, k, v), _ = _steps(wl)
    s = torch.cuda.Stream()
    ref = torch.empty_like(q)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        la.lite_attn_fwd(q, k, v, ref, tile_m=wl.tile_m, tile_n=wl.tile_n, tau=-3.0)
    s.synchronize()
    di = torch.cuda.current_device()
    assert (di, s.cuda_stream) in la._SCHED          # the stream has its counters
    out = torch.empty_like(q)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        la.lite_attn_fwd(q, k, v, out, tile_m=wl.tile_m, tile_n=wl.tile_n, tau=-3.0)
    for _ in range(3):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
        with torch.cuda.stream(s):                     # eager calls on the same stream in between
            la.lite_attn_fwd(q, k, v, ref, tile_m=wl.tile_m, tile_n=wl.tile_n, tau=-3.0)
        s.synchronize()
    assert la._SCHED[(di, s.cuda_stream)].tolist() == [0, 0]
