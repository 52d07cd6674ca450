/*
 * lite_attn.h -- C ABI of the skip-masked tiled attention forward for MI355X
 * (gfx950): LiteAttention's temporal-sparse attention hot path.
 *
 * Pages cited:
 *   [README]   LiteAttention project README (moonmath-ai/LiteAttention):
 *              "QK-Skip Algorithm", "Full-Stage Elimination", the threshold
 *              ablation table, the Python API (threshold, reset of the skip
 *              state, turning skipping off, must-do list note that the kernel
 *              iterates in reverse order, LSE return) and the debug flags.
 *   [ABSTRACT] "LiteAttention: A Temporal Sparse Attention for Diffusion
 *              Transformers", arXiv 2511.11062, abstract.
 *   [SKILL]    "Lite Attention Temporal Sparse" skill page: Skip-Mask as a
 *              bitmask, or a Skip-List for high sparsity ("Architecture
 *              Overview").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensors are BSHD and contiguous: element (b, n, h, e) of q, k, v and out
 *   sits at ((b*seqlen + n)*heads + h)*head_dim + e.  [README] Wan
 *   integration: the attention takes (batch, seq_len, heads, head_dim) and
 *   returns (batch, seq_len, heads*head_dim) -- the same bytes.
 * - Tiles: a q-tile is tile_m consecutive query tokens, a k-tile tile_n
 *   consecutive key tokens.  Tq = ceil(seqlen/tile_m), Tk = ceil(seqlen/tile_n).
 *   A "row" is one (b, h, q-tile); row id = (b*heads + h)*Tq + qt.
 * - Skip-Mask (the persistent per-layer state, [README] QK-Skip Algorithm):
 *   W = ceil(Tk/32) uint32 words per row, row-major; k-tile kt of a row is
 *   bit (kt % 32) of word (kt / 32); 1 = skip.  Bits at positions >= Tk are
 *   ignored on input and written 0 on output.
 * - Skip-List ([SKILL]): int32 per row, stride 1 + Tk: element 0 is the
 *   number of live k-tiles L, elements 1..L are the live k-tiles in the order
 *   the forward visits them (descending).  Elements after L are not written.
 * - Device pointers are plain HIP device addresses owned by the caller; the
 *   library allocates nothing, keeps no pointer and no state between calls,
 *   and is reentrant.  `stream` is a hipStream_t (NULL = the null stream).
 *   All work is enqueued asynchronously on `stream`; argument errors are
 *   returned synchronously before anything is enqueued.
 * - Every function returns LITE_OK (0) or a LITE_ERR_* code;
 *   lite_attn_strerror gives its text (for LITE_ERR_HIP, with the HIP error
 *   of the failing call of this thread).
 * - A descriptor with batch, seqlen or heads equal to 0 describes empty
 *   tensors: the call validates the rest and does nothing.
 */
#ifndef LITE_ATTN_H
#define LITE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LITE_ATTN_ABI_VERSION 1

typedef enum {
    LITE_BF16 = 0, /* bf16 q, k, v, out; fp32 accumulation */
    LITE_FP32 = 1  /* fp32 q, k, v, out; fp64 logits */
} lite_attn_dtype;

typedef struct {
    int32_t batch;    /* B >= 0 */
    int32_t seqlen;   /* N >= 0, any value (the last tiles may be partial) */
    int32_t heads;    /* H >= 0 */
    int32_t head_dim; /* d */
    int32_t tile_m;   /* BM: query rows per tile */
    int32_t tile_n;   /* BN: key columns per tile */
    int32_t dtype;    /* lite_attn_dtype */
} lite_attn_desc;

/* Supported (dtype, head_dim, tile_m x tile_n):
 *   LITE_BF16: head_dim 64 or 128; tile 128x64 or 128x128.
 *   LITE_FP32: head_dim 64; tile 64x64.
 * Anything else is LITE_ERR_UNSUPPORTED (never a silent fallback).
 * Tk may be at most 4096. */

enum {
    LITE_OK = 0,
    LITE_ERR_NULL_ARG = 1,      /* a required pointer is NULL */
    LITE_ERR_BAD_SHAPE = 2,     /* negative size, or sizes overflow */
    LITE_ERR_UNSUPPORTED = 3,   /* (dtype, head_dim, tile) not built, or Tk too large */
    LITE_ERR_BAD_THRESHOLD = 4, /* tau is NaN, or > 0 without LITE_ATTENTION_DEBUG */
    LITE_ERR_BAD_SCALE = 5,     /* softmax_scale not finite and > 0 */
    LITE_ERR_MISALIGNED = 6,    /* q/k/v/out not 16-byte, mask/skiplist/lse not 4-byte aligned */
    LITE_ERR_ALIAS = 7,         /* out or lse overlaps an input; mask_out partly overlaps mask_in */
    LITE_ERR_HIP = 8            /* a HIP call failed (launch or device query) */
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
 *   q, k, v   device, [B][N][H][d] of dtype, 16-byte aligned; read only.
 *   mask_in   device, lite_attn_mask_words() uint32; NULL = nothing skipped
 *             (the "skipping off" path of the [README] API: plain attention).
 *   mask_out  device, same size; NULL = no marking.  Receives
 *             mask_in | newly-marked (marks only accumulate).  May be the
 *             same pointer as mask_in (updated in place); any other overlap
 *             with an input is LITE_ERR_ALIAS.
 *   skiplist  device, lite_attn_skiplist_len() int32, or NULL.  When given,
 *             the live tiles are read from it instead of from mask_in; it
 *             must have been built by lite_attn_build_skiplist from this
 *             mask_in (mask_in is still read for mask_out).
 *   tau       threshold in natural-log units.  -inf never marks.  NaN is
 *             LITE_ERR_BAD_THRESHOLD; tau > 0 is too unless the environment
 *             variable LITE_ATTENTION_DEBUG is set to anything other than
 *             "FALSE" ([README] debug flags).
 *   softmax_scale  multiplier of q.k; finite and > 0 (1/sqrt(d) is usual).
 *   out       device, [B][N][H][d] of dtype, 16-byte aligned; written for
 *             every query.  A query whose row has no live tile gets 0.
 *   lse       device, fp32 [B][H][N], or NULL: natural-log log-sum-exp of the
 *             query's live logits ([README]: softmax LSE for merging partial
 *             attentions); -inf when the row has no live tile.
 *   stream    hipStream_t.
 */
int lite_attn_fwd(const lite_attn_desc *desc, const void *q, const void *k, const void *v,
                  const uint32_t *mask_in, uint32_t *mask_out, const int32_t *skiplist,
                  float tau, float softmax_scale, void *out, float *lse, void *stream);

/*
 * lite_attn_build_skiplist -- compact each row of a Skip-Mask into its
 * Skip-List ([SKILL] "Skip-List for high sparsity").
 *   mask      device, lite_attn_mask_words() uint32 (NULL = nothing skipped).
 *   skiplist  device, lite_attn_skiplist_len() int32; must not overlap mask.
 */
int lite_attn_build_skiplist(const lite_attn_desc *desc, const uint32_t *mask, int32_t *skiplist,
                             void *stream);

/*
 * lite_attn_reset_mask -- clear a Skip-Mask: every tile live again ([README]
 * Python API: resetting the skip state).  Uses a fill kernel, so it is safe
 * inside HIP graph capture.
 *   mask      device, lite_attn_mask_words() uint32.
 */
int lite_attn_reset_mask(const lite_attn_desc *desc, uint32_t *mask, void *stream);

/* Text of a return code.  For LITE_ERR_HIP it includes the HIP error text of
 * this thread's last failing call.  Never NULL. */
const char *lite_attn_strerror(int code);

/* LITE_ATTN_ABI_VERSION of the loaded library. */
int lite_attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LITE_ATTN_H */
