"""The per-layer class mirroring the README's Python API, on the GPU, against
the oracle step by step: the carried Skip-Mask, set_threshold,
enable_skip_optimization(False) (plain attention, mask untouched) and
reset_skip_state; and the skip state's checkpoint round trip."""

import io
import math
import sys

import numpy as np
import pytest
import torch

from oracle import oracle
from temporal_block_sparse_amd import configs, synth
from temporal_block_sparse_amd import lite_attn as la
from tests import parity as pa

pytestmark = pytest.mark.gpu


def test_layer_class_against_the_oracle():
    wl = configs.scaled(configs.C3, (3, 10, 30), heads=2, batch=1, steps=4)
    tr = synth.Trajectory(wl, "cpu")
    scale = 1.0 / math.sqrt(wl.head_dim)
    attn = la.LiteAttention(threshold=-3.0, tile_m=wl.tile_m, tile_n=wl.tile_n)
    mask = np.zeros((wl.rows, wl.mask_words), np.uint32)
    steps = []
    for t in range(4):
        if t:
            tr.advance()
        steps.append(tr.tensors())

    def step(q, k, v, tau, mask_in):
        print("   oracle step, tau %g" % tau, flush=True)
        sys.stdout.flush()
        return oracle.fwd(q, k, v, wl.tile_m, wl.tile_n, tau, scale, mask_in=mask_in)

    def gpu_mask():
        return attn.mask.cpu().numpy().view(np.uint32).reshape(wl.rows, -1)

    def near_tau_ok(got, orc, tau):
        """Marks equal the oracle's, except tiles whose margin is within 1e-3 of tau."""
        want = orc["mask_out"]
        diff = got ^ want
        for r, kt in zip(*np.nonzero(np.unpackbits(diff.view(np.uint8), bitorder="little").reshape(wl.rows, -1))):
            assert abs(orc["margin"][r, kt] - tau) <= pa.NEAR_TAU, "mask differs at row %d tile %d" % (r, kt)

    # threshold -3 over two steps: the carried mask and the outputs
    for t in range(2):
        q, k, v = steps[t]
        out = attn(q.cuda(), k.cuda(), v.cuda())
        orc = step(q, k, v, -3.0, mask)
        o_ref, _ = oracle.unpack_rows(orc, wl.batch, wl.seqlen, wl.heads, wl.tile_m)
        assert float(np.abs(out.cpu().double().numpy() - o_ref).max()) <= pa.TOL_OUT[torch.bfloat16]
        near_tau_ok(gpu_mask(), orc, -3.0)
        # the oracle carries its own marks; the layer's state is set to them, so
        # both start the next step from one mask even after a near-tau tie
        mask = orc["mask_out"].copy()
        attn.mask.copy_(torch.from_numpy(mask.view(np.int32).reshape(-1)).cuda())
    assert mask.any(), "nothing marked: the test would not see the mask carried"

    # skipping off: plain attention, mask untouched
    attn.enable_skip_optimization(False)
    q, k, v = steps[2]
    out = attn(q.cuda(), k.cuda(), v.cuda())
    orc = step(q, k, v, -math.inf, None)
    o_ref, _ = oracle.unpack_rows(orc, wl.batch, wl.seqlen, wl.heads, wl.tile_m)
    assert float(np.abs(out.cpu().double().numpy() - o_ref).max()) <= pa.TOL_OUT[torch.bfloat16]
    assert np.array_equal(gpu_mask(), mask)
    attn.enable_skip_optimization(True)

    # a looser threshold marks more, on the carried mask
    attn.set_threshold(-1.0)
    out = attn(q.cuda(), k.cuda(), v.cuda())
    orc = step(q, k, v, -1.0, mask)
    o_ref, _ = oracle.unpack_rows(orc, wl.batch, wl.seqlen, wl.heads, wl.tile_m)
    assert float(np.abs(out.cpu().double().numpy() - o_ref).max()) <= pa.TOL_OUT[torch.bfloat16]
    near_tau_ok(gpu_mask(), orc, -1.0)
    assert not np.any(mask & ~gpu_mask())

    # reset: every tile live again, and the next call starts from an empty mask
    attn.reset_skip_state()
    torch.cuda.synchronize()
    assert not gpu_mask().any()
    q, k, v = steps[3]
    out = attn(q.cuda(), k.cuda(), v.cuda())
    orc = step(q, k, v, -1.0, None)
    o_ref, _ = oracle.unpack_rows(orc, wl.batch, wl.seqlen, wl.heads, wl.tile_m)
    assert float(np.abs(out.cpu().double().numpy() - o_ref).max()) <= pa.TOL_OUT[torch.bfloat16]
    near_tau_ok(gpu_mask(), orc, -1.0)


@pytest.mark.parametrize("use_skiplist", [False, True], ids=["bitmask", "skiplist"])
def test_checkpoint_round_trip_of_the_skip_state(use_skiplist):
    """The skip state is the layer's only state across denoising steps (README
    Python API: one instance per layer, reset_skip_state).  On the 4,096-token,
    12-head trajectory at tau = -3: 10 steps in one layer object equal 5 steps,
    the state saved to the host and through torch.save / torch.load
    (weights_only), restored into a new layer object, and 5 more steps -- bit
    for bit in outputs, lse and the mask after every step."""
    wl = configs.C2
    tr = synth.Trajectory(wl, "cuda")
    inputs = []
    for t in range(10):
        if t:
            tr.advance()
        inputs.append(tr.tensors())
    del tr
    kw = dict(threshold=-3.0, tile_m=wl.tile_m, tile_n=wl.tile_n, use_skiplist=use_skiplist)
    ref = la.LiteAttention(**kw)
    assert ref.skip_state() is None
    want = []
    for q, k, v in inputs:
        o, l = ref(q, k, v, return_softmax_lse=True)
        want.append((o, l, ref.mask.clone()))
    a = la.LiteAttention(**kw)
    got = []
    for q, k, v in inputs[:5]:
        o, l = a(q, k, v, return_softmax_lse=True)
        got.append((o, l, a.mask.clone()))
    state = a.skip_state()
    assert state["mask"].device.type == "cpu" and state["mask"].any()
    buf = io.BytesIO()
    torch.save(state, buf)
    buf.seek(0)
    state = torch.load(buf, weights_only=True)
    del a
    b = la.LiteAttention(**kw)
    b.load_skip_state(state)
    for q, k, v in inputs[5:]:
        o, l = b(q, k, v, return_softmax_lse=True)
        got.append((o, l, b.mask.clone()))
    torch.cuda.synchronize()
    for t, (w, g) in enumerate(zip(want, got)):
        assert torch.equal(w[0], g[0]) and torch.equal(w[1], g[1]), "step %d output/lse" % t
        assert torch.equal(w[2], g[2]), "step %d mask" % t
    sp = [float((w[2] != 0).float().mean()) for w in want]
    assert sp[9] >= sp[4] > 0, sp
    # clearing the state starts again from an empty mask
    b.load_skip_state(None)
    o, l = b(*inputs[0], return_softmax_lse=True)
    assert torch.equal(o, want[0][0]) and torch.equal(b.mask, want[0][2])
