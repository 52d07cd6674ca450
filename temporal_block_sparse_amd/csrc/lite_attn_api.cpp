// C-ABI host layer: argument validation, error reporting and dispatch to the
// HIP kernels.  Every check runs before anything is enqueued, so a rejected
// call has no effect on the stream.
#include "../../include/lite_attn.h"
#include "lite_attn_internal.h"

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>

static_assert(lite_attn::NOALLOC_SCHED_WORDS == LITE_ATTN_SCHED_WORDS, "one counter layout");

namespace {

thread_local char g_hip_msg[256] = "";

bool env_flag(const char *name)
{
    const char *v = std::getenv(name);
    return v != nullptr && std::strcmp(v, "FALSE") != 0;
}

struct Dims {
    int64_t Tq = 0, Tk = 0, W = 0, rows = 0;
    int64_t q_sb = 0, kv_sb = 0, o_sb = 0;              // effective batch strides (elements)
    int64_t q_extent = 0, kv_extent = 0, o_extent = 0;  // elements spanned by q, k/v, out
};

constexpr int64_t kMaxElems = (int64_t)1 << 56;

// Shape checks shared by every entry point: sizes and strides non-negative,
// tiles positive, batch entries not overlapping, products representable.
int check_desc(const lite_attn_desc *d, Dims *out)
{
    if (!d)
        return LITE_ERR_NULL_ARG;
    if (d->batch < 0 || d->seqlen < 0 || d->seqlen_kv < 0 || d->heads < 0 || d->head_dim <= 0 || d->tile_m <= 0 ||
        d->tile_n <= 0 || d->q_batch_stride < 0 || d->kv_batch_stride < 0 || d->out_batch_stride < 0)
        return LITE_ERR_BAD_SHAPE;
    if (d->q_batch_stride > kMaxElems || d->kv_batch_stride > kMaxElems || d->out_batch_stride > kMaxElems)
        return LITE_ERR_BAD_SHAPE;
    Dims r;
    r.Tq = (d->seqlen + (int64_t)d->tile_m - 1) / d->tile_m;
    r.Tk = (d->seqlen_kv + (int64_t)d->tile_n - 1) / d->tile_n;
    r.W = (r.Tk + 31) / 32;
    r.rows = (int64_t)d->batch * d->heads * r.Tq;
    const int64_t tok = (int64_t)d->heads * d->head_dim;  // < 2^62
    const int64_t q_dense = d->seqlen * tok, kv_dense = d->seqlen_kv * tok;
    r.q_sb = d->q_batch_stride ? d->q_batch_stride : q_dense;
    r.kv_sb = d->kv_batch_stride ? d->kv_batch_stride : kv_dense;
    r.o_sb = d->out_batch_stride ? d->out_batch_stride : q_dense;
    if (d->batch > 1 && (r.q_sb < q_dense || r.kv_sb < kv_dense || r.o_sb < q_dense))
        return LITE_ERR_BAD_SHAPE;  // batch entries would overlap
    if (q_dense > kMaxElems || kv_dense > kMaxElems)
        return LITE_ERR_BAD_SHAPE;
    r.q_extent = d->batch ? (d->batch - 1) * r.q_sb + q_dense : 0;
    r.kv_extent = d->batch ? (d->batch - 1) * r.kv_sb + kv_dense : 0;
    r.o_extent = d->batch ? (d->batch - 1) * r.o_sb + q_dense : 0;
    if (r.q_extent > kMaxElems || r.kv_extent > kMaxElems || r.o_extent > kMaxElems)
        return LITE_ERR_BAD_SHAPE;
    if (r.rows > (int64_t)std::numeric_limits<int32_t>::max() / 2)
        return LITE_ERR_BAD_SHAPE;  // grid size
    if (r.rows * (1 + r.Tk) > std::numeric_limits<int64_t>::max() / 8)
        return LITE_ERR_BAD_SHAPE;
    *out = r;
    return LITE_OK;
}

bool empty(const lite_attn_desc *d) { return d->batch == 0 || d->seqlen == 0 || d->heads == 0; }

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Half-open byte ranges [a, a+na) and [b, b+nb) overlap.
bool overlap(const void *a, size_t na, const void *b, size_t nb)
{
    if (!a || !b || na == 0 || nb == 0)
        return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

int hip_fail(hipError_t e)
{
    std::snprintf(g_hip_msg, sizeof g_hip_msg, "%s", hipGetErrorString(e));
    return LITE_ERR_HIP;
}

bool supported(const lite_attn_desc *d)
{
    if (d->dtype == LITE_BF16)
        return (d->head_dim == 64 || d->head_dim == 128) && d->tile_m == 128 &&
               (d->tile_n == 64 || d->tile_n == 128);
    if (d->dtype == LITE_FP32)
        return d->head_dim == 64 && d->tile_m == 64 && d->tile_n == 64;
    return false;
}

size_t elem_size(int dtype) { return dtype == LITE_BF16 ? 2 : 4; }

// Batch strides must keep every batch entry 16-byte aligned.
bool strides_aligned(const lite_attn_desc *d, const Dims &r)
{
    const size_t es = elem_size(d->dtype);
    return ((size_t)r.q_sb * es) % 16 == 0 && ((size_t)r.kv_sb * es) % 16 == 0 && ((size_t)r.o_sb * es) % 16 == 0;
}

// One range list: pairs (start, end) with start > end >= -1, strictly
// descending (end_i > start_{i+1}).
bool ranges_ok(const int32_t *rg, int32_t n)
{
    if (n < 0 || (n > 0 && !rg))
        return false;
    for (int32_t i = 0; i < n; ++i) {
        const int64_t start = rg[2 * i], end = rg[2 * i + 1];
        if (!(start > end) || end < -1)
            return false;
        if (i + 1 < n && !(end > (int64_t)rg[2 * i + 2]))
            return false;
    }
    return true;
}

// Keys of [c0, c1] covered by the ranges (disjoint, so the counts add up).
int64_t covered(const int32_t *rg, int32_t n, int64_t c0, int64_t c1)
{
    int64_t k = 0;
    for (int32_t i = 0; i < n; ++i) {
        const int64_t lo = std::max<int64_t>(c0, (int64_t)rg[2 * i + 1] + 1), hi = std::min<int64_t>(c1, rg[2 * i]);
        if (hi >= lo)
            k += hi - lo + 1;
    }
    return k;
}

// Validate the ranges and reduce them to per-tile bits.
int tile_ranges(const lite_attn_ranges *ranges, int32_t Nk, int32_t BN, int64_t Tk, lite_attn::TileRanges *rg)
{
    std::memset(rg, 0, sizeof *rg);
    if (!ranges)
        return LITE_OK;
    if (!ranges_ok(ranges->must_do, ranges->n_must_do) || !ranges_ok(ranges->must_skip, ranges->n_must_skip))
        return LITE_ERR_BAD_RANGES;
    if (ranges->n_must_do == 0 && ranges->n_must_skip == 0)
        return LITE_OK;
    if (Tk > 32 * lite_attn::MAX_TILE_WORDS)
        return LITE_ERR_UNSUPPORTED;
    rg->any = 1;
    for (int64_t kt = 0; kt < Tk; ++kt) {
        const int64_t c0 = kt * BN, c1 = std::min<int64_t>(c0 + BN, Nk) - 1;
        const bool d = covered(ranges->must_do, ranges->n_must_do, c0, c1) > 0;
        const bool s = ranges->n_must_skip > 0 && covered(ranges->must_skip, ranges->n_must_skip, c0, c1) == c1 - c0 + 1;
        if (d)
            rg->do_bits[kt >> 5] |= 1u << (kt & 31);
        else if (s)
            rg->skip_bits[kt >> 5] |= 1u << (kt & 31);
    }
    return LITE_OK;
}

}  // namespace

extern "C" {

int lite_attn_abi_version(void) { return LITE_ATTN_ABI_VERSION; }

size_t lite_attn_mask_words(const lite_attn_desc *desc)
{
    Dims r;
    if (check_desc(desc, &r) != LITE_OK)
        return 0;
    return (size_t)(r.rows * r.W);
}

size_t lite_attn_skiplist_len(const lite_attn_desc *desc)
{
    Dims r;
    if (check_desc(desc, &r) != LITE_OK)
        return 0;
    return (size_t)(r.rows * (1 + r.Tk));
}

const char *lite_attn_strerror(int code)
{
    static thread_local char buf[320];
    switch (code) {
    case LITE_OK: return "success";
    case LITE_ERR_NULL_ARG: return "a required pointer argument is NULL";
    case LITE_ERR_BAD_SHAPE:
        return "invalid shape: negative size or stride, non-positive head_dim or tile, batch entries overlapping, "
               "or sizes too large";
    case LITE_ERR_UNSUPPORTED:
        return "unsupported configuration: bf16 needs head_dim 64/128 and tile 128x64 or 128x128; "
               "fp32 needs head_dim 64 and tile 64x64; at most 4096 k-tiles; merge needs head_dim 8, 16, 32, ..., "
               "512 and 1..8 parts";
    case LITE_ERR_BAD_THRESHOLD:
        return "invalid threshold: NaN, or > 0 without LITE_ATTENTION_DEBUG set to a value other than FALSE";
    case LITE_ERR_BAD_SCALE: return "invalid softmax_scale: must be finite and > 0";
    case LITE_ERR_MISALIGNED:
        return "misaligned pointer: q, k, v, out and their batch strides need 16-byte alignment; masks, skip-list "
               "and lse 4-byte";
    case LITE_ERR_ALIAS:
        return "overlapping buffers: out/lse overlap an input, or mask_out partly overlaps another buffer";
    case LITE_ERR_HIP:
        std::snprintf(buf, sizeof buf, "HIP error: %s", g_hip_msg);
        return buf;
    case LITE_ERR_BAD_RANGES:
        return "malformed token ranges: pairs (start, end) need start > end >= -1, in strictly descending order";
    default: return "unknown error code";
    }
}

namespace {

// The forward behind both entry points: with own_sched the schedule counters
// are the library's static per-device array (cleared first) instead of sched.
int fwd_impl(const lite_attn_desc *desc, const void *q, const void *k, const void *v, const uint32_t *mask_in,
             uint32_t *mask_out, const int32_t *skiplist, float tau, float softmax_scale, void *out, float *lse,
             const lite_attn_ranges *ranges, uint32_t *sched, bool own_sched, void *stream)
{
    Dims r;
    int rc = check_desc(desc, &r);
    if (rc != LITE_OK)
        return rc;
    if (desc->dtype != LITE_BF16 && desc->dtype != LITE_FP32)
        return LITE_ERR_UNSUPPORTED;
    if (!supported(desc) || r.Tk > 4096)
        return LITE_ERR_UNSUPPORTED;
    if (std::isnan(tau) || (tau > 0.f && !env_flag("LITE_ATTENTION_DEBUG")))
        return LITE_ERR_BAD_THRESHOLD;
    if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f))
        return LITE_ERR_BAD_SCALE;
    lite_attn::FwdParams p;
    rc = tile_ranges(ranges, desc->seqlen_kv, desc->tile_n, r.Tk, &p.rg);
    if (rc != LITE_OK)
        return rc;
    if (empty(desc))
        return LITE_OK;
    if (!q || !out || (desc->seqlen_kv > 0 && (!k || !v)))
        return LITE_ERR_NULL_ARG;  // k and v may be NULL when there are no keys
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(mask_in, 4) ||
        !aligned(mask_out, 4) || !aligned(skiplist, 4) || !aligned(lse, 4) || !aligned(sched, 4) ||
        !strides_aligned(desc, r))
        return LITE_ERR_MISALIGNED;

    const size_t esz = elem_size(desc->dtype);
    const size_t qbytes = (size_t)r.q_extent * esz, kvbytes = (size_t)r.kv_extent * esz;
    const size_t obytes = (size_t)r.o_extent * esz;
    const size_t mbytes = (size_t)(r.rows * r.W) * 4;
    const size_t sbytes = (size_t)(r.rows * (1 + r.Tk)) * 4;
    const size_t lbytes = (size_t)desc->batch * desc->heads * desc->seqlen * 4;
    const void *ins[] = {q, k, v};
    const size_t inb[] = {qbytes, kvbytes, kvbytes};
    for (int i = 0; i < 3; ++i) {
        if (overlap(out, obytes, ins[i], inb[i]) || overlap(lse, lbytes, ins[i], inb[i]) ||
            overlap(mask_out, mbytes, ins[i], inb[i]))
            return LITE_ERR_ALIAS;
    }
    if (overlap(lse, lbytes, out, obytes) || overlap(mask_out, mbytes, out, obytes) ||
        overlap(mask_out, mbytes, lse, lbytes) || overlap(mask_out, mbytes, skiplist, sbytes) ||
        overlap(out, obytes, mask_in, mbytes) || overlap(out, obytes, skiplist, sbytes) ||
        overlap(lse, lbytes, mask_in, mbytes) || overlap(lse, lbytes, skiplist, sbytes))
        return LITE_ERR_ALIAS;
    if (mask_out != mask_in && overlap(mask_out, mbytes, mask_in, mbytes))
        return LITE_ERR_ALIAS;
    // the schedule counters are written by the kernel: they share no byte with any other buffer
    const size_t cbytes = LITE_ATTN_SCHED_WORDS * sizeof(uint32_t);
    const void *bufs[] = {q, k, v, out, lse, mask_in, mask_out, skiplist};
    const size_t bufb[] = {qbytes, kvbytes, kvbytes, obytes, lbytes, mbytes, mbytes, sbytes};
    for (int i = 0; i < 8; ++i)
        if (overlap(sched, cbytes, bufs[i], bufb[i]))
            return LITE_ERR_ALIAS;

    p.q = q;
    p.k = k;
    p.v = v;
    p.mask_in = mask_in;
    p.mask_out = mask_out;
    p.skiplist = skiplist;
    p.out = out;
    p.lse = lse;
    p.B = desc->batch;
    p.Nq = desc->seqlen;
    p.Nk = desc->seqlen_kv;
    p.H = desc->heads;
    p.D = desc->head_dim;
    p.BM = desc->tile_m;
    p.BN = desc->tile_n;
    p.Tq = (int32_t)r.Tq;
    p.Tk = (int32_t)r.Tk;
    p.W = (int32_t)r.W;
    p.q_sb = r.q_sb;
    p.kv_sb = r.kv_sb;
    p.o_sb = r.o_sb;
    p.rows = r.rows;
    p.tau = (double)tau;
    p.scale = (double)softmax_scale;
    p.sched = desc->dtype == LITE_BF16 ? sched : nullptr;

    if (env_flag("LITE_ATTENTION_VERBOSE"))
        std::fprintf(stderr,
                     "[lite_attn] fwd %s d=%d tile=%dx%d B=%d Nq=%d Nk=%d H=%d rows=%lld Tk=%d mask_in=%d "
                     "mask_out=%d skiplist=%d ranges=%d sched=%d tau=%g\n",
                     desc->dtype == LITE_BF16 ? "bf16" : "fp32", p.D, p.BM, p.BN, p.B, p.Nq, p.Nk, p.H,
                     (long long)p.rows, p.Tk, mask_in != nullptr, mask_out != nullptr, skiplist != nullptr,
                     p.rg.any, p.sched != nullptr, (double)tau);

    hipStream_t s = static_cast<hipStream_t>(stream);
    if (own_sched && desc->dtype == LITE_BF16) {
        // the array keeps the last call's contents: clear the counters with
        // a fill kernel (no memset, no allocation) before this call uses them
        hipError_t e = lite_attn::noalloc_sched(&p.sched);
        if (e == hipSuccess)
            e = lite_attn::launch_reset_mask(p.sched, lite_attn::NOALLOC_SCHED_WORDS, s);
        if (e != hipSuccess)
            return hip_fail(e);
    }
    const hipError_t e =
        desc->dtype == LITE_BF16 ? lite_attn::launch_fwd_bf16(p, s) : lite_attn::launch_fwd_fp32(p, s);
    return e == hipSuccess ? LITE_OK : hip_fail(e);
}

}  // namespace

int lite_attn_fwd(const lite_attn_desc *desc, const void *q, const void *k, const void *v,
                  const uint32_t *mask_in, uint32_t *mask_out, const int32_t *skiplist, float tau,
                  float softmax_scale, void *out, float *lse, const lite_attn_ranges *ranges, uint32_t *sched,
                  void *stream)
{
    return fwd_impl(desc, q, k, v, mask_in, mask_out, skiplist, tau, softmax_scale, out, lse, ranges, sched, false,
                    stream);
}

int lite_attn_fwd_noalloc(const lite_attn_desc *desc, const void *q, const void *k, const void *v,
                          const uint32_t *mask_in, uint32_t *mask_out, const int32_t *skiplist, float tau,
                          float softmax_scale, void *out, float *lse, const lite_attn_ranges *ranges, void *stream)
{
    return fwd_impl(desc, q, k, v, mask_in, mask_out, skiplist, tau, softmax_scale, out, lse, ranges, nullptr, true,
                    stream);
}

int lite_attn_build_skiplist(const lite_attn_desc *desc, const uint32_t *mask, int32_t *skiplist,
                             const lite_attn_ranges *ranges, void *stream)
{
    Dims r;
    int rc = check_desc(desc, &r);
    if (rc != LITE_OK)
        return rc;
    if (r.Tk > 32 * lite_attn::MAX_TILE_WORDS)
        return LITE_ERR_UNSUPPORTED;  // the documented bound on k-tiles, as for the forward
    lite_attn::TileRanges rg;
    rc = tile_ranges(ranges, desc->seqlen_kv, desc->tile_n, r.Tk, &rg);
    if (rc != LITE_OK)
        return rc;
    if (empty(desc))
        return LITE_OK;
    if (!skiplist)
        return LITE_ERR_NULL_ARG;
    if (!aligned(mask, 4) || !aligned(skiplist, 4))
        return LITE_ERR_MISALIGNED;
    if (overlap(mask, (size_t)(r.rows * r.W) * 4, skiplist, (size_t)(r.rows * (1 + r.Tk)) * 4))
        return LITE_ERR_ALIAS;
    const hipError_t e = lite_attn::launch_build_skiplist(mask, skiplist, r.rows, (int32_t)r.Tk, rg,
                                                          static_cast<hipStream_t>(stream));
    return e == hipSuccess ? LITE_OK : hip_fail(e);
}

int lite_attn_reset_mask(const lite_attn_desc *desc, uint32_t *mask, void *stream)
{
    Dims r;
    int rc = check_desc(desc, &r);
    if (rc != LITE_OK)
        return rc;
    if (empty(desc))
        return LITE_OK;
    if (!mask)
        return LITE_ERR_NULL_ARG;
    if (!aligned(mask, 4))
        return LITE_ERR_MISALIGNED;
    const hipError_t e = lite_attn::launch_reset_mask(mask, r.rows * r.W, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? LITE_OK : hip_fail(e);
}

int lite_attn_merge(const lite_attn_desc *desc, int32_t nparts, const void *const *outs, const float *const *lses,
                    void *out, float *lse, void *stream)
{
    Dims r;
    int rc = check_desc(desc, &r);
    if (rc != LITE_OK)
        return rc;
    const int32_t cpq = desc->head_dim / 8;  // threads per query: a power of two up to a wave
    if ((desc->dtype != LITE_BF16 && desc->dtype != LITE_FP32) || desc->head_dim % 8 != 0 || cpq > 64 ||
        (cpq & (cpq - 1)) != 0 || nparts < 1 || nparts > LITE_ATTN_MAX_MERGE_PARTS)
        return LITE_ERR_UNSUPPORTED;
    if (empty(desc))
        return LITE_OK;
    if (!outs || !lses || !out)
        return LITE_ERR_NULL_ARG;
    for (int32_t i = 0; i < nparts; ++i)
        if (!outs[i] || !lses[i])
            return LITE_ERR_NULL_ARG;
    if (!aligned(out, 16) || !aligned(lse, 4) || !strides_aligned(desc, r))
        return LITE_ERR_MISALIGNED;
    for (int32_t i = 0; i < nparts; ++i)
        if (!aligned(outs[i], 16) || !aligned(lses[i], 4))
            return LITE_ERR_MISALIGNED;
    const size_t pbytes = (size_t)r.q_extent * elem_size(desc->dtype);  // one part
    const size_t obytes = (size_t)r.o_extent * elem_size(desc->dtype);
    const size_t lbytes = (size_t)desc->batch * desc->heads * desc->seqlen * 4;
    // out may be exactly one of the parts when both use the same stride (each
    // query's values are read before they are written); any other overlap is
    // refused.
    for (int32_t i = 0; i < nparts; ++i) {
        if (!(out == outs[i] && r.o_sb == r.q_sb) && overlap(out, obytes, outs[i], pbytes))
            return LITE_ERR_ALIAS;
        if (lse != lses[i] && overlap(lse, lbytes, lses[i], lbytes))
            return LITE_ERR_ALIAS;
        if (overlap(out, obytes, lses[i], lbytes) || overlap(lse, lbytes, outs[i], pbytes))
            return LITE_ERR_ALIAS;
    }
    if (overlap(out, obytes, lse, lbytes))
        return LITE_ERR_ALIAS;
    lite_attn::MergeParams p;
    std::memset(&p, 0, sizeof p);
    for (int32_t i = 0; i < nparts; ++i) {
        p.outs[i] = outs[i];
        p.lses[i] = lses[i];
    }
    p.out = out;
    p.lse = lse;
    p.nparts = nparts;
    p.B = desc->batch;
    p.N = desc->seqlen;
    p.H = desc->heads;
    p.D = desc->head_dim;
    p.dtype = desc->dtype;
    p.q_sb = r.q_sb;
    p.o_sb = r.o_sb;
    const hipError_t e = lite_attn::launch_merge(p, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? LITE_OK : hip_fail(e);
}

int lite_attn_error_sums(const lite_attn_desc *desc, const void *a, const void *b, double *sums, void *stream)
{
    Dims r;
    int rc = check_desc(desc, &r);
    if (rc != LITE_OK)
        return rc;
    if ((desc->dtype != LITE_BF16 && desc->dtype != LITE_FP32) || desc->head_dim % 8 != 0)
        return LITE_ERR_UNSUPPORTED;
    if (!sums)
        return LITE_ERR_NULL_ARG;
    if (!aligned(sums, 8))
        return LITE_ERR_MISALIGNED;
    if (!empty(desc)) {
        if (!a || !b)
            return LITE_ERR_NULL_ARG;
        if (!aligned(a, 16) || !aligned(b, 16) || !strides_aligned(desc, r))
            return LITE_ERR_MISALIGNED;
        const size_t es = elem_size(desc->dtype);
        if (overlap(sums, 16, a, (size_t)r.q_extent * es) || overlap(sums, 16, b, (size_t)r.o_extent * es))
            return LITE_ERR_ALIAS;
    }
    lite_attn::ErrParams p;
    p.a = a;
    p.b = b;
    p.sums = sums;
    p.B = desc->batch;
    p.N = desc->seqlen;
    p.H = desc->heads;
    p.D = desc->head_dim;
    p.dtype = desc->dtype;
    p.a_sb = r.q_sb;
    p.b_sb = r.o_sb;
    const hipError_t e = lite_attn::launch_error_sums(p, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? LITE_OK : hip_fail(e);
}

}  // extern "C"
