"""The C-ABI library loads, exports every declared symbol and validates its
arguments on the host.  No kernel is launched: every call here is rejected
(or is an empty no-op) before the library touches the device."""

import ctypes
import math
import os
import re

import pytest
import torch

from temporal_block_sparse_amd import lite_attn as la

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lite_attn.h")

BF16 = dict(batch=1, seqlen=1000, heads=2, head_dim=128, tile_m=128, tile_n=128, dtype=la.LITE_BF16)
FAKE = 1 << 40  # an address that is never dereferenced: every call below fails validation first


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(lite_attn_\w+)\s*\(", src)))


def desc(**kw):
    d = dict(BF16)
    d.update(kw)
    return la.Desc(d["batch"], d["seqlen"], d["heads"], d["head_dim"], d["tile_m"], d["tile_n"], d["dtype"],
                   d.get("seqlen_kv", d["seqlen"]), d.get("q_batch_stride", 0), d.get("kv_batch_stride", 0),
                   d.get("out_batch_stride", 0))


def fwd(d, q=FAKE, k=FAKE + (1 << 30), v=FAKE + (2 << 30), mask_in=None, mask_out=None, skiplist=None,
        tau=-3.0, scale=0.125, out=FAKE + (3 << 30), lse=None, ranges=None, sched=None):
    P = lambda x: None if x is None else ctypes.c_void_p(x)  # noqa: E731
    return la.LIB.lite_attn_fwd(ctypes.byref(d) if d is not None else None, P(q), P(k), P(v), P(mask_in),
                                P(mask_out), P(skiplist), tau, scale, P(out), P(lse),
                                ctypes.byref(ranges) if ranges is not None else None, P(sched), None)


def merge(d, outs, lses, out, lse=None):
    n = len(outs)
    po = (ctypes.c_void_p * max(n, 1))(*[ctypes.c_void_p(x) if x else None for x in outs])
    pl = (ctypes.c_void_p * max(n, 1))(*[ctypes.c_void_p(x) if x else None for x in lses])
    return la.LIB.lite_attn_merge(ctypes.byref(d), n, po, pl, ctypes.c_void_p(out) if out else None,
                                  ctypes.c_void_p(lse) if lse else None, None)


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert set(la.EXPORTS) <= set(names) and len(names) == len(la.EXPORTS)
    lib = ctypes.CDLL(la.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert la.LIB.lite_attn_abi_version() == 3


def test_sizes():
    d = desc()
    tq, tk = 8, 8
    assert la.lite_attn_mask_words(d) == 1 * 2 * tq * 1
    assert la.lite_attn_skiplist_len(d) == 1 * 2 * tq * (1 + tk)
    d = desc(seqlen=75600, heads=40)
    assert la.lite_attn_mask_words(d) == 40 * 591 * 19
    assert la.lite_attn_skiplist_len(d) == 40 * 591 * 592
    assert la.lite_attn_mask_words(desc(seqlen=-1)) == 0


def test_strerror_covers_every_code():
    for code in range(0, 10):
        assert la.lite_attn_strerror(code)
    assert "unknown" in la.lite_attn_strerror(1234)


@pytest.mark.parametrize("kw,code", [
    (dict(seqlen=-1), 2), (dict(batch=-2), 2), (dict(head_dim=0), 2), (dict(tile_n=0), 2),
    (dict(head_dim=96), 3), (dict(tile_m=64), 3), (dict(tile_n=32), 3), (dict(dtype=7), 3),
    (dict(dtype=la.LITE_FP32), 3), (dict(dtype=la.LITE_FP32, head_dim=64, tile_m=64, tile_n=32), 3),
    (dict(seqlen=4097 * 128), 3),
])
def test_descriptor_errors(kw, code):
    assert fwd(desc(**kw)) == code


def test_null_arguments():
    assert fwd(None) == 1
    assert fwd(desc(), q=None) == 1
    assert fwd(desc(), out=None) == 1
    assert la.LIB.lite_attn_build_skiplist(ctypes.byref(desc()), None, None, None, None) == 1
    assert la.LIB.lite_attn_reset_mask(ctypes.byref(desc()), None, None) == 1


def test_threshold_rules(monkeypatch):
    assert fwd(desc(), tau=float("nan")) == 4
    monkeypatch.delenv("LITE_ATTENTION_DEBUG", raising=False)
    assert fwd(desc(), tau=0.5) == 4
    monkeypatch.setenv("LITE_ATTENTION_DEBUG", "FALSE")
    assert fwd(desc(), tau=0.5) == 4
    monkeypatch.setenv("LITE_ATTENTION_DEBUG", "1")
    assert fwd(desc(), tau=0.5, q=None) == 1           # threshold accepted, then the NULL q is reported
    assert fwd(desc(), tau=0.0, q=None) == 1
    assert fwd(desc(), tau=-math.inf, q=None) == 1


def test_scale_rules():
    for s in (0.0, -1.0, float("inf"), float("nan")):
        assert fwd(desc(), scale=s) == 5


def test_alignment():
    assert fwd(desc(), q=FAKE + 8) == 6
    assert fwd(desc(), out=FAKE + (3 << 30) + 2) == 6
    assert fwd(desc(), mask_in=FAKE + (5 << 30) + 1) == 6
    assert fwd(desc(), lse=FAKE + (6 << 30) + 2) == 6


def test_aliasing():
    assert fwd(desc(), out=FAKE) == 7                                   # out is q
    assert fwd(desc(), out=FAKE + 4096) == 7                            # out overlaps q
    assert fwd(desc(), lse=FAKE + (2 << 30) + 64) == 7                  # lse inside v
    m = FAKE + (5 << 30)
    assert fwd(desc(), mask_in=m, mask_out=m + 4, q=None) == 1          # partial overlap is checked after NULL
    assert fwd(desc(), mask_in=m, mask_out=m + 4) == 7
    assert fwd(desc(), mask_in=m, mask_out=m, skiplist=m + 32) == 7      # mask_out overlaps the skip-list


def test_schedule_counters_validation():
    """The forward's schedule counters (LITE_ATTN_SCHED_WORDS words) are
    written by the kernel: 4-byte aligned, and sharing no byte with any other
    buffer of the call."""
    c = FAKE + (7 << 30)
    assert fwd(desc(), sched=c + 2) == 6
    m = FAKE + (5 << 30)
    assert fwd(desc(), sched=FAKE + 64) == 7                                  # inside q
    assert fwd(desc(), sched=FAKE + (2 << 30)) == 7                           # at v
    assert fwd(desc(), sched=FAKE + (3 << 30) + 4096) == 7                    # inside out
    assert fwd(desc(), mask_in=m, mask_out=m, sched=m + 8) == 7              # inside the masks
    assert fwd(desc(), lse=FAKE + (6 << 30), sched=FAKE + (6 << 30) - 4) == 7  # its last word is lse's first
    # checked only when there is work: an empty call ignores it
    assert fwd(desc(seqlen=0), q=None, k=None, v=None, out=None, sched=c + 2) == 0


def test_binding_schedule_argument():
    with pytest.raises(ValueError, match="sched must be"):
        t = torch.zeros(1, 8, 1, 64, dtype=torch.bfloat16)
        la.lite_attn_fwd(t, t.clone(), t.clone(), t.clone(), tile_m=128, tile_n=64, tau=-3.0, sched="tickets")
    with pytest.raises(ValueError, match="sched holds"):
        la._buf(torch.zeros(1, dtype=torch.int32), 4 * la.SCHED_WORDS, "sched", torch.int32)
    with pytest.raises(ValueError, match="sched must be torch.int32"):
        la._buf(torch.zeros(2, dtype=torch.int64), 4 * la.SCHED_WORDS, "sched", torch.int32)


def fwd_noalloc(d, q=FAKE, k=FAKE + (1 << 30), v=FAKE + (2 << 30), mask_in=None, mask_out=None, skiplist=None,
                tau=-3.0, scale=0.125, out=FAKE + (3 << 30), lse=None):
    P = lambda x: None if x is None else ctypes.c_void_p(x)  # noqa: E731
    return la.LIB.lite_attn_fwd_noalloc(ctypes.byref(d) if d is not None else None, P(q), P(k), P(v),
                                        P(mask_in), P(mask_out), P(skiplist), tau, scale, P(out), P(lse), None,
                                        None)


def test_noalloc_entry_point_validates_like_lite_attn_fwd():
    """lite_attn_fwd_noalloc rejects what lite_attn_fwd rejects, with the same
    codes, before it looks up its counters or touches the device."""
    cases = [dict(d=None), dict(d=desc(tile_m=0)), dict(d=desc(head_dim=96)), dict(d=desc(), tau=float("nan")),
             dict(d=desc(), scale=0.0), dict(d=desc(), q=None), dict(d=desc(), q=FAKE + 8),
             dict(d=desc(), out=FAKE + 4096), dict(d=desc(seqlen=4097 * 128))]
    for kw in cases:
        want = fwd(**kw)
        assert want != 0 and fwd_noalloc(**kw) == want, kw
    assert fwd_noalloc(desc(seqlen=0), q=None, k=None, v=None, out=None) == 0


def test_empty_descriptor_is_a_noop():
    for kw in (dict(seqlen=0), dict(batch=0), dict(heads=0)):
        assert fwd(desc(**kw), q=None, k=None, v=None, out=None) == 0
        assert la.LIB.lite_attn_reset_mask(ctypes.byref(desc(**kw)), None, None) == 0
        assert la.LIB.lite_attn_build_skiplist(ctypes.byref(desc(**kw)), None, None, None, None) == 0
    # an empty call still rejects a bad threshold or scale
    assert fwd(desc(seqlen=0), tau=float("nan")) == 4


def test_skiplist_and_reset_validation():
    d = desc()
    m = FAKE
    assert la.LIB.lite_attn_build_skiplist(ctypes.byref(d), ctypes.c_void_p(m), ctypes.c_void_p(m + 2), None, None) == 6
    assert la.LIB.lite_attn_build_skiplist(ctypes.byref(d), ctypes.c_void_p(m), ctypes.c_void_p(m + 8), None, None) == 7
    assert la.LIB.lite_attn_reset_mask(ctypes.byref(d), ctypes.c_void_p(m + 1), None) == 6
    assert la.LIB.lite_attn_reset_mask(ctypes.byref(desc(tile_m=-3)), ctypes.c_void_p(m), None) == 2
    # more than 4096 k-tiles: unsupported for the Skip-List build too (checked before any pointer)
    assert la.LIB.lite_attn_build_skiplist(ctypes.byref(desc(seqlen=4097 * 128)), ctypes.c_void_p(m),
                                           ctypes.c_void_p(FAKE + (1 << 30)), None, None) == 3


def test_binding_raises_with_code():
    with pytest.raises(la.LiteAttnError) as ei:
        la._check(3)
    assert ei.value.code == 3


def test_sizes_with_separate_key_length():
    d = desc(seqlen=300, seqlen_kv=1000)          # Tq = 3, Tk = 8
    assert la.lite_attn_mask_words(d) == 2 * 3 * 1
    assert la.lite_attn_skiplist_len(d) == 2 * 3 * 9
    d = desc(seqlen=300, seqlen_kv=0)             # no keys: Tk = 0
    assert la.lite_attn_mask_words(d) == 0 and la.lite_attn_skiplist_len(d) == 2 * 3
    assert la.lite_attn_mask_words(desc(seqlen_kv=-1)) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(q_batch_stride=-1), 2), (dict(kv_batch_stride=-8), 2),
    (dict(batch=2, q_batch_stride=1000 * 2 * 128 - 8), 2),     # batch entries would overlap
    (dict(batch=2, kv_batch_stride=100), 2),
    (dict(batch=2, out_batch_stride=1000 * 2 * 128 - 1), 2), (dict(out_batch_stride=-1), 2),
    (dict(batch=2, out_batch_stride=1000 * 2 * 128 + 2), 6),
    (dict(batch=2, q_batch_stride=1000 * 2 * 128 + 4), 6),     # 8-byte stride: entries misaligned
    (dict(batch=2, kv_batch_stride=1000 * 2 * 128 + 8), 0),    # 16-byte multiple: accepted, then ...
])
def test_batch_strides(kw, code):
    if code == 0:
        assert fwd(desc(**kw), q=None) == 1                   # ... the NULL q is reported
    else:
        assert fwd(desc(**kw)) == code


def test_strided_extents_are_checked_for_aliasing():
    d = desc(batch=2, q_batch_stride=4 * 1000 * 2 * 128)
    # q spans (1 * 4 + 1) * 256000 elements * 2 bytes = 2.56 MB from its start, so buffers starting 1 MB
    # and 2.5 MB in overlap it (the second lies in the gap-free extent of the second batch entry)
    assert fwd(d, out=FAKE + (1 << 20)) == 7
    assert fwd(d, lse=FAKE + 2500000) == 7


def _ranges(do=(), skip=()):
    a = (ctypes.c_int32 * max(len(do), 1))(*do)
    b = (ctypes.c_int32 * max(len(skip), 1))(*skip)
    r = la.Ranges(ctypes.cast(a, ctypes.POINTER(ctypes.c_int32)), len(do) // 2,
                  ctypes.cast(b, ctypes.POINTER(ctypes.c_int32)), len(skip) // 2)
    r._keep = (a, b)
    return r


@pytest.mark.parametrize("do,skip,code", [
    ((80, 60, 45, 40, 12, 2), (), 0),       # the README's must_do example
    ((), (80, 40), 0),                      # the README's must_skip example
    ((10, -1), (), 0),                      # end -1: the range reaches token 0
    ((60, 80), (), 9),                      # start must exceed end
    ((80, 60, 70, 65), (), 9),              # pairs must descend
    ((80, 60, 60, 50), (), 9),              # ... strictly: end_0 > start_1
    ((10, -2), (), 9),                      # end below -1
    ((5, 5), (), 9),
])
def test_range_validation(do, skip, code):
    r = _ranges(do, skip)
    if code == 0:
        assert fwd(desc(), ranges=r, q=None) == 1
    else:
        assert fwd(desc(), ranges=r) == code
        assert la.LIB.lite_attn_build_skiplist(ctypes.byref(desc()), None, ctypes.c_void_p(FAKE), ctypes.byref(r),
                                               None) == code


def test_range_list_with_null_pointer():
    r = la.Ranges(None, 1, None, 0)
    assert fwd(desc(), ranges=r) == 9
    r = la.Ranges(None, 0, None, 0)                     # no ranges at all is fine
    assert fwd(desc(), ranges=r, q=None) == 1


def test_merge_validation():
    d = desc()
    o = [FAKE, FAKE + (1 << 30)]
    l = [FAKE + (2 << 30), FAKE + (2 << 30) + (1 << 20)]
    out, lse = FAKE + (3 << 30), FAKE + (4 << 30)
    assert merge(d, o, l, None) == 1
    assert merge(d, [FAKE, 0], l, out) == 1
    assert merge(d, [], [], out) == 3
    assert merge(d, o * 5, l * 5, out) == 3                          # more than 8 parts
    assert merge(desc(head_dim=24), o, l, out) == 3                  # head_dim / 8 not a power of two
    assert merge(desc(head_dim=1024), o, l, out) == 3
    assert merge(d, [FAKE + 8, o[1]], l, out) == 6
    assert merge(d, o, [l[0] + 2, l[1]], out) == 6
    assert merge(d, o, l, out + 2) == 6
    assert merge(d, o, l, FAKE + 4096) == 7                          # out partly overlaps a part
    assert merge(d, o, l, out, lse=l[0] + 4) == 7                    # lse partly overlaps a part's lse
    assert merge(d, o, l, out, lse=out + 64) == 7                    # lse inside out
    assert merge(desc(batch=0), o, l, out) == 0                      # empty: no-op


def test_error_sums_validation():
    P = ctypes.c_void_p
    d = desc()
    a, b, s = P(FAKE), P(FAKE + (1 << 30)), P(FAKE + (2 << 30))
    f = la.LIB.lite_attn_error_sums
    assert f(None, a, b, s, None) == 1
    assert f(ctypes.byref(d), a, b, None, None) == 1
    assert f(ctypes.byref(d), None, b, s, None) == 1
    assert f(ctypes.byref(d), a, b, P(FAKE + (2 << 30) + 4), None) == 6
    assert f(ctypes.byref(d), P(FAKE + 8), b, s, None) == 6
    assert f(ctypes.byref(desc(head_dim=12)), a, b, s, None) == 3
    assert f(ctypes.byref(desc(dtype=5)), a, b, s, None) == 3
    assert f(ctypes.byref(d), a, b, P(FAKE + 4096), None) == 7         # sums inside a


def test_binding_refuses_short_mask_and_skiplist_buffers():
    """The kernels take plain pointers; the binding checks every buffer holds
    what the call will touch before anything is launched."""
    d = la.make_desc(1, 1000, 2, 64, 128, 64, la.LITE_BF16)
    nw, nl = la.lite_attn_mask_words(d), la.lite_attn_skiplist_len(d)
    with pytest.raises(ValueError, match="mask holds"):
        la.lite_attn_build_skiplist(d, torch.zeros(nw - 1, dtype=torch.int32), torch.zeros(nl, dtype=torch.int32))
    with pytest.raises(ValueError, match="skiplist holds"):
        la.lite_attn_build_skiplist(d, None, torch.zeros(nl - 1, dtype=torch.int32))   # no mask: nothing skipped
    with pytest.raises(ValueError, match="mask holds"):
        la.lite_attn_reset_mask(d, torch.zeros(nw - 1, dtype=torch.int32))
    # right sizes, host memory: refused for the device
    with pytest.raises(ValueError, match="device tensor expected"):
        la.lite_attn_reset_mask(d, torch.zeros(nw, dtype=torch.int32))


def test_verbose_flag_prints_one_line_per_call():
    """[README] debug flags: LITE_ATTENTION_VERBOSE (not "FALSE") prints the
    launch of each validated forward on stderr.  Run in a child process, so
    the C library's stderr can be read; without a GPU the launch itself then
    fails, after the line."""
    import subprocess
    import sys
    child = ("import ctypes, sys; sys.path.insert(0, %r)\n"
             "from tests import test_abi_cpu as t\n"
             "print('rc', t.fwd(t.desc()))\n") % os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    for flag, want in (("1", True), ("FALSE", False)):
        env = dict(os.environ, LITE_ATTENTION_VERBOSE=flag, HIP_VISIBLE_DEVICES="")
        p = subprocess.run([sys.executable, "-c", child], env=env, capture_output=True, text=True, timeout=120)
        assert ("[lite_attn] fwd bf16" in p.stderr) == want, (flag, p.stderr[-500:])


@pytest.mark.parametrize("make", [
    lambda: torch.zeros(1, 300, 2, 64, dtype=torch.bfloat16).expand(2, 300, 2, 64),        # batch stride 0
    lambda: torch.zeros(1, 600, 2, 64, dtype=torch.bfloat16).as_strided((2, 300, 2, 64), (100 * 128, 128, 64, 1)),
])
def test_binding_refuses_overlapping_batch_entries(make):
    """The C ABI reads a batch stride of 0 as "dense": a batch-expanded tensor
    would be read (or written) a whole batch entry past its allocation.  The
    binding refuses any tensor whose batch entries overlap, before it looks at
    the device or calls the library."""
    t = make()
    with pytest.raises(ValueError, match="batch entries overlap"):
        la._bshd(t)
    with pytest.raises(ValueError, match="batch entries overlap"):
        la.desc_of(t, 128, 64)
    with pytest.raises(ValueError, match="batch entries overlap"):
        la.lite_attn_fwd(t, t, t, t, tile_m=128, tile_n=64, tau=-3.0)
    # a sequence slice of a larger tensor keeps a batch stride >= its own entry: not refused by this check
    sl = torch.zeros(2, 600, 2, 64, dtype=torch.bfloat16)[:, :300]
    with pytest.raises(ValueError, match="device tensor expected"):
        la._bshd(sl)


def test_layer_classes_refuse_batches_over_max_batch_size():
    """README Python API: the constructor takes max_batch_size (default 4);
    a larger batch is refused before anything is allocated or launched."""
    q = torch.zeros(5, 8, 1, 64, dtype=torch.bfloat16)
    attn = la.LiteAttention(threshold=-3.0)
    assert attn.max_batch_size == 4
    with pytest.raises(ValueError, match="max_batch_size"):
        attn(q, q, q)
    assert attn.mask is None
    attn = la.LiteAttention(True, -3.0, 2)
    with pytest.raises(ValueError, match="max_batch_size"):
        attn(q[:3], q[:3], q[:3])
    sp = la.SeqParallelLiteAttention(num_nodes=2, max_batch_size=2)
    with pytest.raises(ValueError, match="max_batch_size"):
        sp(q[:3], q[:3], q[:3], split_idx=0)
    assert all(s.max_batch_size == 2 for s in sp._splits)
