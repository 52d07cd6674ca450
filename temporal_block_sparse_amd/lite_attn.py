"""Thin Python binding of liblite_attn.so (argument marshalling only).

Every function here forwards to the C entry point of the same name; all
arithmetic runs in the library's HIP kernels.  Tensors are torch tensors used
as plain device memory: the binding reads their shapes, strides, dtypes and
data pointers and passes the current HIP stream.  If the library is missing
the import of this module fails loudly -- there is no fallback path.

Pages: LiteAttention README (moonmath-ai/LiteAttention), "QK-Skip Algorithm"
and the Python API (threshold, reset of the skip state, turning skipping off,
must_do_list / must_skip_list, SeqParallelLiteAttention with split_idx, LSE
return and the text/video partial attentions, one instance per layer).
"""

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("LITE_ATTN_LIBRARY") or os.path.join(_HERE, "liblite_attn.so")

LITE_BF16, LITE_FP32 = 0, 1
LITE_OK = 0
SCHED_WORDS = 2  # LITE_ATTN_SCHED_WORDS
MAX_MERGE_PARTS = 8
ERRORS = {1: "LITE_ERR_NULL_ARG", 2: "LITE_ERR_BAD_SHAPE", 3: "LITE_ERR_UNSUPPORTED", 4: "LITE_ERR_BAD_THRESHOLD",
          5: "LITE_ERR_BAD_SCALE", 6: "LITE_ERR_MISALIGNED", 7: "LITE_ERR_ALIAS", 8: "LITE_ERR_HIP",
          9: "LITE_ERR_BAD_RANGES"}
EXPORTS = ("lite_attn_fwd", "lite_attn_fwd_noalloc", "lite_attn_build_skiplist", "lite_attn_reset_mask", "lite_attn_merge",
           "lite_attn_error_sums", "lite_attn_mask_words", "lite_attn_skiplist_len", "lite_attn_strerror",
           "lite_attn_abi_version")


class Desc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seqlen", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("tile_m", ctypes.c_int32), ("tile_n", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("seqlen_kv", ctypes.c_int32), ("q_batch_stride", ctypes.c_int64),
                ("kv_batch_stride", ctypes.c_int64), ("out_batch_stride", ctypes.c_int64)]


class Ranges(ctypes.Structure):
    _fields_ = [("must_do", ctypes.POINTER(ctypes.c_int32)), ("n_must_do", ctypes.c_int32),
                ("must_skip", ctypes.POINTER(ctypes.c_int32)), ("n_must_skip", ctypes.c_int32)]


class LiteAttnError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__("%s (%d): %s" % (ERRORS.get(code, "?"), code, msg))
        self.code = code


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("liblite_attn.so is not built (run __graft_entry__.build() or "
                          "python temporal_block_sparse_amd/build_lib.py); there is no fallback")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    D = ctypes.POINTER(Desc)
    R = ctypes.POINTER(Ranges)
    lib.lite_attn_fwd.restype = ctypes.c_int
    lib.lite_attn_fwd.argtypes = [D, P, P, P, P, P, P, ctypes.c_float, ctypes.c_float, P, P, R, P, P]
    lib.lite_attn_fwd_noalloc.restype = ctypes.c_int
    lib.lite_attn_fwd_noalloc.argtypes = [D, P, P, P, P, P, P, ctypes.c_float, ctypes.c_float, P, P, R, P]
    lib.lite_attn_build_skiplist.restype = ctypes.c_int
    lib.lite_attn_build_skiplist.argtypes = [D, P, P, R, P]
    lib.lite_attn_reset_mask.restype = ctypes.c_int
    lib.lite_attn_reset_mask.argtypes = [D, P, P]
    lib.lite_attn_merge.restype = ctypes.c_int
    lib.lite_attn_merge.argtypes = [D, ctypes.c_int32, ctypes.POINTER(P), ctypes.POINTER(P), P, P, P]
    lib.lite_attn_error_sums.restype = ctypes.c_int
    lib.lite_attn_error_sums.argtypes = [D, P, P, P, P]
    lib.lite_attn_mask_words.restype = ctypes.c_size_t
    lib.lite_attn_mask_words.argtypes = [D]
    lib.lite_attn_skiplist_len.restype = ctypes.c_size_t
    lib.lite_attn_skiplist_len.argtypes = [D]
    lib.lite_attn_strerror.restype = ctypes.c_char_p
    lib.lite_attn_strerror.argtypes = [ctypes.c_int]
    lib.lite_attn_abi_version.restype = ctypes.c_int
    lib.lite_attn_abi_version.argtypes = []
    return lib


LIB = _load()


def lite_attn_strerror(code):
    return LIB.lite_attn_strerror(int(code)).decode()


def _check(code):
    if code != LITE_OK:
        raise LiteAttnError(code, lite_attn_strerror(code))


def _dtype_code(dtype):
    if isinstance(dtype, torch.dtype):
        return LITE_BF16 if dtype == torch.bfloat16 else (LITE_FP32 if dtype == torch.float32 else 99)
    return dtype


def make_desc(batch, seqlen, heads, head_dim, tile_m, tile_n, dtype, seqlen_kv=None, q_batch_stride=0,
              kv_batch_stride=0, out_batch_stride=0):
    """Descriptor of contiguous (or, with batch strides, sliced) BSHD tensors;
    seqlen_kv defaults to seqlen."""
    return Desc(batch, seqlen, heads, head_dim, tile_m, tile_n, _dtype_code(dtype),
                seqlen if seqlen_kv is None else seqlen_kv, q_batch_stride, kv_batch_stride, out_batch_stride)


def lite_attn_mask_words(desc):
    return int(LIB.lite_attn_mask_words(ctypes.byref(desc)))


def lite_attn_skiplist_len(desc):
    return int(LIB.lite_attn_skiplist_len(ctypes.byref(desc)))


def _on_device(t):
    if t.numel() and not t.is_cuda:
        raise ValueError("device tensor expected")
    if t.is_cuda and t.device.index != torch.cuda.current_device():
        raise ValueError("tensor on cuda:%d, but the current device is cuda:%d"
                         % (t.device.index, torch.cuda.current_device()))


def _ptr(t):
    """Device pointer of a contiguous tensor (masks, skip-lists, lse)."""
    if t is None:
        return None
    _on_device(t)
    if not t.is_contiguous():
        raise ValueError("contiguous tensor expected")
    return ctypes.c_void_p(t.data_ptr())


def _buf(t, nbytes, what, dtype=None):
    """_ptr of a buffer the library reads or writes nbytes of: the kernels take
    plain pointers, so a short tensor would be overrun -- refuse it here."""
    if t is None:
        return None
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must be %s, not %s" % (what, dtype, t.dtype))
    if t.numel() * t.element_size() < nbytes:
        raise ValueError("%s holds %d bytes; this call uses %d" % (what, t.numel() * t.element_size(), nbytes))
    return _ptr(t)


def _bshd(t):
    """(B, N, H, D, batch stride in elements, pointer) of a BSHD tensor that is
    contiguous within each batch entry -- a whole tensor, or a slice of one
    along the sequence such as q[:, :text_len]."""
    if t.dim() != 4:
        raise ValueError("BSHD tensor expected")
    B, N, H, D = t.shape
    if N > 1 and t.stride(1) != H * D or H > 1 and t.stride(2) != D or D > 1 and t.stride(3) != 1:
        raise ValueError("each batch entry must be a contiguous [N][H][D] block")
    # The C ABI reads a batch stride of 0 as "dense", so a batch-expanded
    # tensor (stride 0, e.g. k.expand(2, ...)) would make the kernels read or
    # write a whole batch entry past the allocation: refuse any stride that
    # lets batch entries overlap.
    if B > 1 and N * H * D > 0 and t.stride(0) < N * H * D:
        raise ValueError("batch entries overlap (batch stride %d < %d elements); pass a tensor whose batch "
                         "entries are separate, e.g. .contiguous()" % (t.stride(0), N * H * D))
    _on_device(t)
    return B, N, H, D, (t.stride(0) if B > 1 else 0), ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _ranges(must_do, must_skip):
    """ctypes Ranges for the README's flat [start_0, end_0, start_1, end_1, ...] lists, or None."""
    if not must_do and not must_skip:
        return None
    def arr(x):
        x = list(x or [])
        if len(x) % 2:
            raise ValueError("a range list holds (start, end) pairs")
        return (ctypes.c_int32 * max(len(x), 1))(*x), len(x) // 2
    do_a, n_do = arr(must_do)
    sk_a, n_sk = arr(must_skip)
    r = Ranges(ctypes.cast(do_a, ctypes.POINTER(ctypes.c_int32)), n_do,
               ctypes.cast(sk_a, ctypes.POINTER(ctypes.c_int32)), n_sk)
    r._keep = (do_a, sk_a)
    return r


# Schedule counters of the forward, one buffer per (device, stream): calls on
# one stream never overlap, so they may share it; the kernels leave it zero.
_SCHED = {}


def _torch_stream(stream):
    if stream is None:
        return torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream.cuda_stream if hasattr(stream, "cuda_stream") else stream))


def _sched_auto(stream, device):
    """The counters for calls on this stream, or None (one workgroup per pair)
    while the stream is being captured into a graph: a graph replayed on
    another stream could then run at the same time as eager calls sharing
    the buffer.  A new buffer is zeroed by a fill kernel on the stream itself,
    ahead of the forward that uses it, so no synchronisation is needed."""
    ts = _torch_stream(stream)
    with torch.cuda.stream(ts):
        if torch.cuda.is_current_stream_capturing():
            return None
        key = (device.index, ts.cuda_stream)
        buf = _SCHED.get(key)
        if buf is None:
            buf = torch.zeros(SCHED_WORDS, dtype=torch.int32, device=device)
            _SCHED[key] = buf
    return buf


def desc_of(q, tile_m, tile_n, k=None, out=None):
    """Descriptor of the q (and k, v, out) tensors as passed to lite_attn_fwd."""
    B, N, H, D, qs, _ = _bshd(q)
    os_ = _bshd(out)[4] if out is not None else qs
    if k is None:
        return make_desc(B, N, H, D, tile_m, tile_n, q.dtype, N, qs, qs, os_)
    Bk, Nk, Hk, Dk, ks, _ = _bshd(k)
    if (Bk, Hk, Dk) != (B, H, D):
        raise ValueError("q and k must share batch, heads and head_dim")
    return make_desc(B, N, H, D, tile_m, tile_n, q.dtype, Nk, qs, ks, os_)


def _fwd_args(q, k, v, out, tile_m, tile_n, tau, softmax_scale, mask_in, mask_out, skiplist, lse, rg):
    """The C forward's arguments up to its token ranges, checked."""
    desc = desc_of(q, tile_m, tile_n, k, out)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(q.shape[-1])
    if v.shape != k.shape or v.dtype != k.dtype or k.dtype != q.dtype:
        raise ValueError("k and v must match, and share q's dtype")
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    if _bshd(v)[4] != desc.kv_batch_stride:
        raise ValueError("v must be laid out like k")
    mb = 4 * lite_attn_mask_words(desc)
    return (ctypes.byref(desc), _bshd(q)[5], _bshd(k)[5], _bshd(v)[5], _buf(mask_in, mb, "mask_in"),
            _buf(mask_out, mb, "mask_out"), _buf(skiplist, 4 * lite_attn_skiplist_len(desc), "skiplist"),
            float(tau), float(softmax_scale), _bshd(out)[5],
            _buf(lse, 4 * desc.batch * desc.heads * desc.seqlen, "lse", torch.float32),
            ctypes.byref(rg) if rg is not None else None)


def lite_attn_fwd(q, k, v, out, *, tile_m, tile_n, tau, softmax_scale=None, mask_in=None, mask_out=None,
                  skiplist=None, lse=None, must_do=None, must_skip=None, sched="auto", stream=None):
    """C lite_attn_fwd on BSHD tensors: q and out [B, Nq, H, d], k and v
    [B, Nk, H, d], each a whole tensor or a sequence slice of one.
    mask_in/mask_out: int32 tensors of lite_attn_mask_words() words; skiplist:
    int32 of lite_attn_skiplist_len(); lse: fp32 [B, H, Nq]; must_do/must_skip:
    the README's [start_0, end_0, ...] key ranges.  sched: the schedule
    counters (int32 tensor of SCHED_WORDS zeros), "auto" for the stream's own
    (none while a graph is being captured), or None for one workgroup per
    q-tile pair.  Raises LiteAttnError on a non-zero return code."""
    if isinstance(sched, str) and sched != "auto":
        raise ValueError('sched must be a tensor, "auto" or None')
    rg = _ranges(must_do, must_skip)
    args = _fwd_args(q, k, v, out, tile_m, tile_n, tau, softmax_scale, mask_in, mask_out, skiplist, lse, rg)
    st = _stream(stream)
    if isinstance(sched, str):
        sched = _sched_auto(stream, q.device) if q.dtype == torch.bfloat16 and q.is_cuda else None
    _check(LIB.lite_attn_fwd(*args, _buf(sched, 4 * SCHED_WORDS, "sched", torch.int32), st))
    return out


def lite_attn_fwd_noalloc(q, k, v, out, *, tile_m, tile_n, tau, softmax_scale=None, mask_in=None,
                          mask_out=None, skiplist=None, lse=None, must_do=None, must_skip=None, stream=None):
    """C lite_attn_fwd_noalloc: lite_attn_fwd with the library's own schedule
    counters (one static array per GPU; calls that overlap in time on one GPU
    must not be made).  Neither the library nor this function allocates."""
    rg = _ranges(must_do, must_skip)
    args = _fwd_args(q, k, v, out, tile_m, tile_n, tau, softmax_scale, mask_in, mask_out, skiplist, lse, rg)
    _check(LIB.lite_attn_fwd_noalloc(*args, _stream(stream)))
    return out


def lite_attn_build_skiplist(desc, mask, skiplist, must_do=None, must_skip=None, stream=None):
    rg = _ranges(must_do, must_skip)
    _check(LIB.lite_attn_build_skiplist(ctypes.byref(desc), _buf(mask, 4 * lite_attn_mask_words(desc), "mask"),
                                        _buf(skiplist, 4 * lite_attn_skiplist_len(desc), "skiplist"),
                                        ctypes.byref(rg) if rg is not None else None, _stream(stream)))
    return skiplist


def lite_attn_reset_mask(desc, mask, stream=None):
    _check(LIB.lite_attn_reset_mask(ctypes.byref(desc), _buf(mask, 4 * lite_attn_mask_words(desc), "mask"),
                                    _stream(stream)))
    return mask


def lite_attn_merge(outs, lses, out, lse=None, stream=None):
    """C lite_attn_merge: combine partial attentions (outs[i] [B, Nq, H, d],
    all with one batch stride; lses[i] fp32 [B, H, Nq]) by their log-sum-exp
    into out (and lse)."""
    B, N, H, D, os_, optr = _bshd(out)
    n = len(outs)
    if n != len(lses) or not 1 <= n <= MAX_MERGE_PARTS:
        raise ValueError("1..%d parts, one lse per part" % MAX_MERGE_PARTS)
    ps = _bshd(outs[0])[4]
    for o in outs:
        if o.shape != out.shape or o.dtype != out.dtype or _bshd(o)[4] != ps:
            raise ValueError("every part must match out's shape and share one layout")
    desc = make_desc(B, N, H, D, 1, 1, out.dtype, N, ps, ps, os_)
    po = (ctypes.c_void_p * n)(*[_bshd(o)[5] for o in outs])
    lb = 4 * B * H * N
    pl = (ctypes.c_void_p * n)(*[_buf(x, lb, "lses[%d]" % i, torch.float32) for i, x in enumerate(lses)])
    _check(LIB.lite_attn_merge(ctypes.byref(desc), n, po, pl, optr, _buf(lse, lb, "lse", torch.float32),
                               _stream(stream)))
    return out


def lite_attn_error_sums(a, b, sums=None, stream=None):
    """C lite_attn_error_sums: (sum (a-b)^2, sum b^2) in fp64 for two BSHD
    tensors of one shape.  Returns the device tensor of the two sums."""
    B, N, H, D, as_, ap = _bshd(a)
    bs = _bshd(b)
    if b.shape != a.shape or b.dtype != a.dtype:
        raise ValueError("a and b must share shape and dtype")
    if sums is None:
        sums = torch.empty(2, dtype=torch.float64, device=a.device)
    desc = make_desc(B, N, H, D, 1, 1, a.dtype, N, as_, 0, bs[4])
    _check(LIB.lite_attn_error_sums(ctypes.byref(desc), ap, bs[5], _buf(sums, 16, "sums", torch.float64),
                                    _stream(stream)))
    return sums


def alloc_mask(desc, device="cuda"):
    return torch.empty(lite_attn_mask_words(desc), dtype=torch.int32, device=device)


def alloc_skiplist(desc, device="cuda"):
    return torch.empty(lite_attn_skiplist_len(desc), dtype=torch.int32, device=device)


class LiteAttention:
    """Per-layer skip state plus the forward call (README Python API).

    Holds the persistent Skip-Mask of one attention layer -- one instance per
    layer, never shared -- updated in place by each call.  `threshold` is in
    natural-log units (README ablation: -10, -3, 0); thresholds above 0 need
    LITE_ATTENTION_DEBUG.  With skipping disabled the call is plain attention
    and the mask is neither read nor written.  `max_batch_size` (README
    constructor argument) bounds the batch a call may pass: the skip state
    holds one mask row per (batch entry, head, q-tile).  `use_skiplist` walks the
    compacted Skip-List (rebuilt from the mask before each call) instead of
    the bitmask.  must_do_list / must_skip_list are the README's key ranges."""

    def __init__(self, enable_skipping=True, threshold=-10.0, max_batch_size=4, tile_m=128, tile_n=128,
                 use_skiplist=False):
        self.enable_skipping = enable_skipping
        self.max_batch_size = int(max_batch_size)
        self.threshold = float(threshold)
        self.tile_m, self.tile_n = tile_m, tile_n
        self.use_skiplist = use_skiplist
        self._key = None
        self._desc = None
        self.mask = None
        self.skiplist = None

    def set_threshold(self, threshold):
        self.threshold = float(threshold)

    def enable_skip_optimization(self, enable=True):
        self.enable_skipping = bool(enable)

    def reset_skip_state(self):
        if self.mask is not None:
            lite_attn_reset_mask(self._desc, self.mask)

    def skip_state(self):
        """The layer's skip state for a checkpoint: a host copy of the Skip-Mask
        and the shape key it belongs to (batch, seqlen, heads, head_dim, tile_m,
        tile_n, dtype, seqlen_kv), or None before the first skipping call.
        Plain tensors and ints: torch.save / torch.load(weights_only=True)
        round-trip it."""
        if self.mask is None:
            return None
        return {"key": tuple(int(x) for x in self._key), "mask": self.mask.cpu()}

    def load_skip_state(self, state, device=None):
        """Restore a state from skip_state() (None clears it).  A later call
        with other shapes starts again from an empty mask, as it would after
        any change of shape."""
        if state is None:
            self._key = self._desc = self.mask = self.skiplist = None
            return
        key = tuple(int(x) for x in state["key"])
        d = make_desc(*key[:7], seqlen_kv=key[7])
        mask = state["mask"]
        if mask.dtype != torch.int32 or mask.numel() != lite_attn_mask_words(d):
            raise ValueError("skip state does not match its shape key")
        device = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
        self._key, self._desc = key, d
        self.mask = mask.to(device).contiguous()
        self.skiplist = alloc_skiplist(d, device) if self.use_skiplist else None

    def _state_for(self, q, k):
        d = desc_of(q, self.tile_m, self.tile_n, k)
        key = (d.batch, d.seqlen, d.heads, d.head_dim, d.tile_m, d.tile_n, d.dtype, d.seqlen_kv)
        if key != self._key:
            self._key = key
            self._desc = d
            self.mask = alloc_mask(d, q.device)
            lite_attn_reset_mask(d, self.mask)
            self.skiplist = alloc_skiplist(d, q.device) if self.use_skiplist else None
        return d

    def __call__(self, q, k, v, scale=None, return_softmax_lse=False, out=None, must_do_list=None,
                 must_skip_list=None):
        if q.shape[0] > self.max_batch_size:
            raise ValueError("batch %d larger than max_batch_size %d" % (q.shape[0], self.max_batch_size))
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device) if out is None else out
        lse = None
        if return_softmax_lse:
            lse = torch.empty(q.shape[0], q.shape[2], q.shape[1], dtype=torch.float32, device=q.device)
        if not self.enable_skipping:
            lite_attn_fwd(q, k, v, out, tile_m=self.tile_m, tile_n=self.tile_n, tau=-math.inf,
                          softmax_scale=scale, lse=lse, must_do=must_do_list, must_skip=must_skip_list)
        else:
            d = self._state_for(q, k)
            sl = None
            if self.use_skiplist:
                lite_attn_build_skiplist(d, self.mask, self.skiplist, must_do_list, must_skip_list)
                sl = self.skiplist
            lite_attn_fwd(q, k, v, out, tile_m=self.tile_m, tile_n=self.tile_n, tau=self.threshold,
                          softmax_scale=scale, mask_in=self.mask, mask_out=self.mask, skiplist=sl, lse=lse,
                          must_do=must_do_list, must_skip=must_skip_list)
        return (out, lse) if return_softmax_lse else out


class SeqParallelLiteAttention:
    """One GPU's share of the README's SeqParallelLiteAttention: the caller
    passes the full queries with the K/V split it owns and that split's index;
    the skip state is kept per split (`split_idx`), since each split has its
    own running max and so its own decisions.  Combining the splits' (out,
    lse) pairs -- across GPUs in the README's setting -- is lite_attn_merge."""

    def __init__(self, num_nodes, enable_skipping=True, threshold=-10.0, max_batch_size=4, **kw):
        self.num_nodes = int(num_nodes)
        self.max_batch_size = int(max_batch_size)
        self._splits = [LiteAttention(enable_skipping, threshold, max_batch_size, **kw)
                        for _ in range(self.num_nodes)]

    def set_threshold(self, threshold):
        for s in self._splits:
            s.set_threshold(threshold)

    def enable_skip_optimization(self, enable=True):
        for s in self._splits:
            s.enable_skip_optimization(enable)

    def reset_skip_state(self):
        for s in self._splits:
            s.reset_skip_state()

    def __call__(self, q, k, v, split_idx, scale=None, return_softmax_lse=False, **kw):
        if not 0 <= split_idx < self.num_nodes:
            raise ValueError("split_idx out of range")
        if q.shape[0] > self.max_batch_size:
            raise ValueError("batch larger than max_batch_size")
        return self._splits[split_idx](q, k, v, scale, return_softmax_lse, **kw)
