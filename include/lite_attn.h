/*
 * lite_attn.h -- C ABI of the skip-masked tiled attention forward for MI355X
 * (gfx950): LiteAttention's temporal-sparse attention hot path.
 *
 * Pages cited:
 *   [README]   LiteAttention project README (moonmath-ai/LiteAttention):
 *              "QK-Skip Algorithm", "Full-Stage Elimination", the threshold
 *              ablation table, the Python API (threshold, reset of the skip
 *              state, turning skipping off, must_do_list / must_skip_list and
 *              the note that the kernel iterates in reverse order,
 *              SeqParallelLiteAttention with split_idx, LSE return and the
 *              text/video partial-attention example) and the debug flags.
 *   [ABSTRACT] "LiteAttention: A Temporal Sparse Attention for Diffusion
 *              Transformers", arXiv 2511.11062, abstract.
 *   [SKILL]    "Lite Attention Temporal Sparse" skill page: Skip-Mask as a
 *              bitmask, or a Skip-List for high sparsity ("Architecture
 *              Overview").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensors are BSHD: element (n, h, e) of batch entry b of q sits at
 *   b*q_batch_stride + (n*heads + h)*head_dim + e, of out at
 *   b*out_batch_stride + ..., and of k and v at b*kv_batch_stride + ....
 *   With zero strides the tensors are contiguous [B][seqlen][H][d] and
 *   [B][seqlen_kv][H][d]; a non-zero stride passes a slice along the sequence
 *   of a larger tensor without a copy (the [README] text/video split,
 *   q[:, :text_len], and the K/V splits of SeqParallelLiteAttention).  [README] Wan integration: the
 *   attention takes (batch, seq_len, heads, head_dim).
 * - Tiles: a q-tile is tile_m consecutive query tokens, a k-tile tile_n
 *   consecutive key tokens.  Tq = ceil(seqlen/tile_m), Tk = ceil(seqlen_kv/tile_n).
 *   A "row" is one (b, h, q-tile); row id = (b*heads + h)*Tq + qt.
 * - Skip-Mask (the persistent per-layer state, [README] QK-Skip Algorithm):
 *   W = ceil(Tk/32) uint32 words per row, row-major; k-tile kt of a row is
 *   bit (kt % 32) of word (kt / 32); 1 = skip.  Bits at positions >= Tk are
 *   ignored on input and written 0 on output.
 * - Skip-List ([SKILL]): int32 per row, stride 1 + Tk: element 0 is the
 *   number of live k-tiles L, elements 1..L are the live k-tiles in the order
 *   the forward visits them (descending).  Elements after L are not written.
 * - Token ranges ([README] must_do_list / must_skip_list): pairs (start, end)
 *   of key token indices, start inclusive and end exclusive, listed in
 *   descending order because the kernel iterates in reverse: pair i covers
 *   the keys t with end_i < t <= start_i.  A k-tile holding any must-do key
 *   is visited whatever the mask says and is never marked; a k-tile whose
 *   keys all lie in must-skip ranges (and that is not must-do) is never
 *   visited.  Ranges are the same for every row.
 * - Device pointers are plain HIP device addresses owned by the caller; the
 *   library allocates nothing, keeps no pointer and no state between calls,
 *   and is reentrant.  `stream` is a hipStream_t (NULL = the null stream).
 *   All work is enqueued asynchronously on `stream`; argument errors are
 *   returned synchronously before anything is enqueued.
 * - Every function returns LITE_OK (0) or a LITE_ERR_* code;
 *   lite_attn_strerror gives its text (for LITE_ERR_HIP, with the HIP error
 *   of the failing call of this thread).
 * - A descriptor with batch, seqlen or heads equal to 0 describes empty
 *   tensors: the call validates the rest and does nothing.  seqlen_kv = 0
 *   with queries present gives every query no key: out 0, lse -inf.
 */
#ifndef LITE_ATTN_H
#define LITE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LITE_ATTN_ABI_VERSION 3

/* uint32 words of the forward's schedule counters (lite_attn_fwd, sched). */
#define LITE_ATTN_SCHED_WORDS 2

typedef enum {
    LITE_BF16 = 0, /* bf16 q, k, v, out; fp32 accumulation */
    LITE_FP32 = 1  /* fp32 q, k, v, out; fp64 logits */
} lite_attn_dtype;

typedef struct {
    int32_t batch;           /* B >= 0 */
    int32_t seqlen;          /* Nq >= 0 queries per batch entry (the last tiles may be partial) */
    int32_t heads;           /* H >= 0 */
    int32_t head_dim;        /* d */
    int32_t tile_m;          /* BM: query rows per tile */
    int32_t tile_n;          /* BN: key columns per tile */
    int32_t dtype;           /* lite_attn_dtype */
    int32_t seqlen_kv;       /* Nk >= 0 keys (and values) per batch entry */
    int64_t q_batch_stride;  /* elements between batch entries of q and out; 0 = seqlen*heads*head_dim */
    int64_t kv_batch_stride; /* elements between batch entries of k and v; 0 = seqlen_kv*heads*head_dim */
    int64_t out_batch_stride; /* elements between batch entries of out; 0 = seqlen*heads*head_dim */
} lite_attn_desc;

/* must-do / must-skip key token ranges (host memory, read during the call). */
typedef struct {
    const int32_t *must_do;   /* 2*n_must_do values: start_0, end_0, start_1, end_1, ...; NULL if n is 0 */
    int32_t n_must_do;        /* number of (start, end) pairs, >= 0 */
    const int32_t *must_skip; /* same convention */
    int32_t n_must_skip;
} lite_attn_ranges;

/* Supported (dtype, head_dim, tile_m x tile_n):
 *   LITE_BF16: head_dim 64 or 128; tile 128x64 or 128x128.
 *   LITE_FP32: head_dim 64; tile 64x64.
 * Anything else is LITE_ERR_UNSUPPORTED (never a silent fallback).
 * Tk may be at most 4096.  lite_attn_merge takes head_dim 8, 16, 32, 64,
 * 128, 256 or 512, in either dtype. */

enum {
    LITE_OK = 0,
    LITE_ERR_NULL_ARG = 1,      /* a required pointer is NULL */
    LITE_ERR_BAD_SHAPE = 2,     /* negative size or stride, batch entries overlapping, or sizes overflow */
    LITE_ERR_UNSUPPORTED = 3,   /* (dtype, head_dim, tile) not built, Tk too large, too many merge parts */
    LITE_ERR_BAD_THRESHOLD = 4, /* tau is NaN, or > 0 without LITE_ATTENTION_DEBUG */
    LITE_ERR_BAD_SCALE = 5,     /* softmax_scale not finite and > 0 */
    LITE_ERR_MISALIGNED = 6,    /* q/k/v/out or a batch stride not 16-byte, mask/skiplist/lse not 4-byte */
    LITE_ERR_ALIAS = 7,         /* out or lse overlaps an input; mask_out partly overlaps mask_in */
    LITE_ERR_HIP = 8,           /* a HIP call failed (launch or device query) */
    LITE_ERR_BAD_RANGES = 9     /* a token range list is malformed (see the conventions above) */
};

/* Words of one Skip-Mask for all rows: B*H*Tq*ceil(Tk/32).  0 for a bad descriptor. */
size_t lite_attn_mask_words(const lite_attn_desc *desc);

/* int32 elements of one Skip-List for all rows: B*H*Tq*(1+Tk).  0 for a bad descriptor. */
size_t lite_attn_skiplist_len(const lite_attn_desc *desc);

/*
 * lite_attn_fwd -- one denoising step of skip-masked attention.
 *
 * For every row (b, h, qt), the k-tiles not set in mask_in ("live") are
 * visited from the last to the first ([README] must-do list: the kernel
 * iterates in reverse order).  Skipped tiles cost nothing: no K/V load, no
 * QK^T, no softmax, no PV ([README] "Full-Stage Elimination").  Each visited
 * tile runs flash-style online softmax (QK^T, running max and sum, PV;
 * [ABSTRACT]: built on FlashAttention) and the QK-Skip test ([README]
 * "QK-Skip Algorithm"): with m_loc the tile's local max logit of a query and
 * m_run that query's running max over the tiles visited before it, the tile
 * is newly marked when every valid query of the q-tile has
 *     m_loc - m_run < tau          (logits scale*q.k, natural-log units),
 * i.e. max over the q-tile's queries of (m_loc - m_run) < tau.  A newly
 * marked tile still counts in this call's output and is skipped from the
 * next call on (the mask carried to the next denoising step).
 *
 *   q, k, v   device, of dtype, laid out as in the conventions, 16-byte
 *             aligned; read only.  k and v may be NULL when seqlen_kv is 0.
 *   mask_in   device, lite_attn_mask_words() uint32; NULL = nothing skipped
 *             (the "skipping off" path of the [README] API: plain attention).
 *   mask_out  device, same size; NULL = no marking.  Receives
 *             mask_in | newly-marked (marks only accumulate).  May be the
 *             same pointer as mask_in (updated in place); any other overlap
 *             with an input is LITE_ERR_ALIAS.
 *   skiplist  device, lite_attn_skiplist_len() int32, or NULL.  When given,
 *             the live tiles are read from it instead of from mask_in; it
 *             must have been built by lite_attn_build_skiplist from this
 *             mask_in with the same ranges (mask_in is still read for
 *             mask_out).
 *   tau       threshold in natural-log units.  -inf never marks.  NaN is
 *             LITE_ERR_BAD_THRESHOLD; tau > 0 is too unless the environment
 *             variable LITE_ATTENTION_DEBUG is set to anything other than
 *             "FALSE" ([README] debug flags).
 *   softmax_scale  multiplier of q.k; finite and > 0 (1/sqrt(d) is usual).
 *   out       device, [B][seqlen][H][d] with out_batch_stride, 16-byte
 *             aligned; written for every query.  A query whose row has no
 *             live tile gets 0.
 *   lse       device, fp32 [B][H][seqlen] contiguous, or NULL: natural-log
 *             log-sum-exp of the query's live logits ([README]: softmax LSE
 *             for merging partial attentions); -inf when the row has no live
 *             tile.
 *   ranges    host, or NULL for none: must-do / must-skip key ranges.
 *   sched     device, LITE_ATTN_SCHED_WORDS uint32, 4-byte aligned, or NULL:
 *             schedule counters of the bf16 forward (ignored for LITE_FP32).
 *             With counters, one persistent workgroup per compute unit takes
 *             the q-tile pairs in order from an atomic ticket, which keeps
 *             every compute unit busy when the pairs' costs differ (sparse
 *             masks); NULL launches one workgroup per pair.  Results are the
 *             same bit for bit either way.  The words must be zero before the
 *             first call that uses them; every call leaves them zero again
 *             (the last workgroup resets them, no memset), so a buffer zeroed
 *             once serves any number of calls, also inside HIP graph capture.
 *             Calls that may run at the same time (on different streams, or
 *             replays of graphs that captured it) must not share one buffer;
 *             calls on one stream never overlap.  Owned by the caller; may not
 *             overlap any other buffer of the call (LITE_ERR_ALIAS).
 *   stream    hipStream_t.
 * With the environment variable LITE_ATTENTION_VERBOSE set to anything other
 * than "FALSE" ([README] debug flags), each call that passes validation prints
 * one line describing its launch to stderr.
 */
int lite_attn_fwd(const lite_attn_desc *desc, const void *q, const void *k, const void *v,
                  const uint32_t *mask_in, uint32_t *mask_out, const int32_t *skiplist,
                  float tau, float softmax_scale, void *out, float *lse, const lite_attn_ranges *ranges,
                  uint32_t *sched, void *stream);

/*
 * lite_attn_fwd_noalloc -- for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): lite_attn_fwd with its schedule counters taken from the
 * library instead of from a sched argument.  Same arguments otherwise, same
 * validation, same results bit for bit.
 * The counters are a static array of LITE_ATTN_SCHED_WORDS words per GPU,
 * held until the process ends; its address on a device is looked up once, at
 * the first call on that device.  Each call clears the counters with a fill
 * kernel (no memset) and then runs the ticket schedule; nothing is allocated.
 * The array's size does not grow with the call: every size lite_attn_fwd
 * accepts fits, so no size is refused for lack of room.
 * Every call on one GPU shares the array and finds the last call's contents:
 * calls that overlap in time on one GPU (different streams, or graphs
 * replayed concurrently) race on it and must not be made.
 */
int lite_attn_fwd_noalloc(const lite_attn_desc *desc, const void *q, const void *k, const void *v,
                          const uint32_t *mask_in, uint32_t *mask_out, const int32_t *skiplist, float tau,
                          float softmax_scale, void *out, float *lse, const lite_attn_ranges *ranges,
                          void *stream);

/*
 * lite_attn_build_skiplist -- compact each row of a Skip-Mask into its
 * Skip-List ([SKILL] "Skip-List for high sparsity"): the tiles the forward
 * would visit under this mask and these ranges, in visiting order.
 *   mask      device, lite_attn_mask_words() uint32 (NULL = nothing skipped).
 *   skiplist  device, lite_attn_skiplist_len() int32; must not overlap mask.
 *   ranges    host, or NULL: the ranges the forward will be called with.
 * Tk > 4096 is LITE_ERR_UNSUPPORTED, as for the forward.
 */
int lite_attn_build_skiplist(const lite_attn_desc *desc, const uint32_t *mask, int32_t *skiplist,
                             const lite_attn_ranges *ranges, void *stream);

/*
 * lite_attn_reset_mask -- clear a Skip-Mask: every tile live again ([README]
 * Python API: resetting the skip state).  Uses a fill kernel, so it is safe
 * inside HIP graph capture.
 *   mask      device, lite_attn_mask_words() uint32.
 */
int lite_attn_reset_mask(const lite_attn_desc *desc, uint32_t *mask, void *stream);

/* Most partial attentions one lite_attn_merge call combines. */
#define LITE_ATTN_MAX_MERGE_PARTS 8

/*
 * lite_attn_merge -- combine partial attentions of the same queries over
 * disjoint key sets into the attention over their union ([README]: the
 * softmax LSE is returned "for combining results from multiple partial
 * attention computations" -- the text/video split and the K/V splits of
 * SeqParallelLiteAttention).  For every query (b, n, h):
 *     lse = ln(sum_i exp(lse_i)),   out = sum_i exp(lse_i - lse) * out_i,
 * computed in fp32; a part with lse_i = -inf (no key) contributes nothing;
 * when every part has -inf the query gets out 0 and lse -inf.
 *   desc      batch, seqlen (queries), heads, head_dim and dtype; every
 *             out_i has batch stride q_batch_stride, out has
 *             out_batch_stride; tiles and seqlen_kv are not used.
 *   nparts    1..LITE_ATTN_MAX_MERGE_PARTS.
 *   outs      host array of nparts device pointers, 16-byte aligned.
 *   lses      host array of nparts device pointers, fp32 [B][H][seqlen].
 *   out       device.  May be exactly one of outs when the two strides are
 *             equal (in place); any other overlap is LITE_ERR_ALIAS.
 *   lse       device, fp32 [B][H][seqlen], or NULL.  May be exactly one of lses.
 */
int lite_attn_merge(const lite_attn_desc *desc, int32_t nparts, const void *const *outs,
                    const float *const *lses, void *out, float *lse, void *stream);

/*
 * lite_attn_error_sums -- the two sums behind the relative output error used
 * by the per-timestep threshold calibration ([README] "Error Calibration":
 * error budgets assigned per timestep, stricter early):
 *     sums[0] = sum over all elements of (a - b)^2,   sums[1] = sum of b^2,
 * accumulated in fp64 (order unspecified), so ||a - b|| / ||b|| =
 * sqrt(sums[0] / sums[1]).
 *   desc      batch, seqlen, heads, head_dim (a multiple of 8) and dtype; a is
 *             laid out with q_batch_stride, b with out_batch_stride.
 *   a, b      device, 16-byte aligned; read only.
 *   sums      device, 2 doubles, 8-byte aligned; overwritten (not added to).
 */
int lite_attn_error_sums(const lite_attn_desc *desc, const void *a, const void *b, double *sums, void *stream);

/* Text of a return code.  For LITE_ERR_HIP it includes the HIP error text of
 * this thread's last failing call.  Never NULL. */
const char *lite_attn_strerror(int code);

/* LITE_ATTN_ABI_VERSION of the loaded library. */
int lite_attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LITE_ATTN_H */
