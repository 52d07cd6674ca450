"""Thin Python binding of liblite_attn.so (argument marshalling only).

Every function here forwards to the C entry point of the same name; all
arithmetic runs in the library's HIP kernels.  Tensors are torch tensors used
as plain device memory: the binding reads their shapes, dtypes and data
pointers and passes the current HIP stream.  If the library is missing the
import of this module fails loudly -- there is no fallback path.

Pages: LiteAttention README (moonmath-ai/LiteAttention), "QK-Skip Algorithm"
and the Python API (threshold, reset of the skip state, turning skipping off,
LSE return, one instance per layer).
"""

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("LITE_ATTN_LIBRARY") or os.path.join(_HERE, "liblite_attn.so")

LITE_BF16, LITE_FP32 = 0, 1
LITE_OK = 0
ERRORS = {1: "LITE_ERR_NULL_ARG", 2: "LITE_ERR_BAD_SHAPE", 3: "LITE_ERR_UNSUPPORTED", 4: "LITE_ERR_BAD_THRESHOLD",
          5: "LITE_ERR_BAD_SCALE", 6: "LITE_ERR_MISALIGNED", 7: "LITE_ERR_ALIAS", 8: "LITE_ERR_HIP"}
EXPORTS = ("lite_attn_fwd", "lite_attn_build_skiplist", "lite_attn_reset_mask", "lite_attn_mask_words",
           "lite_attn_skiplist_len", "lite_attn_strerror", "lite_attn_abi_version")


class Desc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seqlen", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("tile_m", ctypes.c_int32), ("tile_n", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


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
    lib.lite_attn_fwd.restype = ctypes.c_int
    lib.lite_attn_fwd.argtypes = [ctypes.POINTER(Desc), P, P, P, P, P, P, ctypes.c_float, ctypes.c_float, P, P, P]
    lib.lite_attn_build_skiplist.restype = ctypes.c_int
    lib.lite_attn_build_skiplist.argtypes = [ctypes.POINTER(Desc), P, P, P]
    lib.lite_attn_reset_mask.restype = ctypes.c_int
    lib.lite_attn_reset_mask.argtypes = [ctypes.POINTER(Desc), P, P]
    lib.lite_attn_mask_words.restype = ctypes.c_size_t
    lib.lite_attn_mask_words.argtypes = [ctypes.POINTER(Desc)]
    lib.lite_attn_skiplist_len.restype = ctypes.c_size_t
    lib.lite_attn_skiplist_len.argtypes = [ctypes.POINTER(Desc)]
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


def make_desc(batch, seqlen, heads, head_dim, tile_m, tile_n, dtype):
    if isinstance(dtype, torch.dtype):
        dtype = LITE_BF16 if dtype == torch.bfloat16 else (LITE_FP32 if dtype == torch.float32 else 99)
    return Desc(batch, seqlen, heads, head_dim, tile_m, tile_n, dtype)


def lite_attn_mask_words(desc):
    return int(LIB.lite_attn_mask_words(ctypes.byref(desc)))


def lite_attn_skiplist_len(desc):
    return int(LIB.lite_attn_skiplist_len(ctypes.byref(desc)))


def _ptr(t):
    if t is None:
        return None
    if t.numel() and not t.is_cuda:
        raise ValueError("device tensor expected")
    if not t.is_contiguous():
        raise ValueError("contiguous tensor expected")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def desc_of(q, tile_m, tile_n):
    B, N, H, D = q.shape
    return make_desc(B, N, H, D, tile_m, tile_n, q.dtype)


def lite_attn_fwd(q, k, v, out, *, tile_m, tile_n, tau, softmax_scale=None, mask_in=None, mask_out=None,
                  skiplist=None, lse=None, stream=None):
    """C lite_attn_fwd on BSHD tensors.  mask_in/mask_out: int32 tensors of
    lite_attn_mask_words() words; skiplist: int32 of lite_attn_skiplist_len();
    lse: fp32 [B, H, N].  Raises LiteAttnError on a non-zero return code."""
    desc = desc_of(q, tile_m, tile_n)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(q.shape[-1])
    for t in (k, v, out):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError("q, k, v, out must share shape and dtype")
    _check(LIB.lite_attn_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(mask_in), _ptr(mask_out),
                             _ptr(skiplist), float(tau), float(softmax_scale), _ptr(out), _ptr(lse), _stream(stream)))
    return out


def lite_attn_build_skiplist(desc, mask, skiplist, stream=None):
    _check(LIB.lite_attn_build_skiplist(ctypes.byref(desc), _ptr(mask), _ptr(skiplist), _stream(stream)))
    return skiplist


def lite_attn_reset_mask(desc, mask, stream=None):
    _check(LIB.lite_attn_reset_mask(ctypes.byref(desc), _ptr(mask), _stream(stream)))
    return mask


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
    and the mask is neither read nor written.  `use_skiplist` walks the
    compacted Skip-List (rebuilt from the mask before each call) instead of
    the bitmask."""

    def __init__(self, enable_skipping=True, threshold=-10.0, tile_m=128, tile_n=128, use_skiplist=False):
        self.enable_skipping = enable_skipping
        self.threshold = float(threshold)
        self.tile_m, self.tile_n = tile_m, tile_n
        self.use_skiplist = use_skiplist
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

    def _state_for(self, q):
        d = desc_of(q, self.tile_m, self.tile_n)
        key = (d.batch, d.seqlen, d.heads, d.head_dim, d.tile_m, d.tile_n, d.dtype)
        if self._desc is None or key != tuple(getattr(self._desc, f) for f, _ in Desc._fields_):
            self._desc = d
            self.mask = alloc_mask(d, q.device)
            lite_attn_reset_mask(d, self.mask)
            self.skiplist = alloc_skiplist(d, q.device) if self.use_skiplist else None
        return self._desc

    def __call__(self, q, k, v, scale=None, return_softmax_lse=False, out=None):
        out = torch.empty_like(q) if out is None else out
        lse = None
        if return_softmax_lse:
            lse = torch.empty(q.shape[0], q.shape[2], q.shape[1], dtype=torch.float32, device=q.device)
        if not self.enable_skipping:
            lite_attn_fwd(q, k, v, out, tile_m=self.tile_m, tile_n=self.tile_n, tau=-math.inf,
                          softmax_scale=scale, lse=lse)
        else:
            d = self._state_for(q)
            sl = None
            if self.use_skiplist:
                lite_attn_build_skiplist(d, self.mask, self.skiplist)
                sl = self.skiplist
            lite_attn_fwd(q, k, v, out, tile_m=self.tile_m, tile_n=self.tile_n, tau=self.threshold,
                          softmax_scale=scale, mask_in=self.mask, mask_out=self.mask, skiplist=sl, lse=lse)
        return (out, lse) if return_softmax_lse else out
