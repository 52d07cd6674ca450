// C-ABI host layer: argument validation, error reporting and dispatch to the
// HIP kernels.  Every check runs before anything is enqueued, so a rejected
// call has no effect on the stream.
#include "../../include/lite_attn.h"
#include "lite_attn_internal.h"

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>

namespace {

thread_local char g_hip_msg[256] = "";

bool env_flag(const char *name)
{
    const char *v = std::getenv(name);
    return v != nullptr && std::strcmp(v, "FALSE") != 0;
}

struct Dims {
    int64_t Tq = 0, Tk = 0, W = 0, rows = 0, elems = 0;
};

// Shape checks shared by every entry point: sizes non-negative, tiles
// positive, products representable.
int check_desc(const lite_attn_desc *d, Dims *out)
{
    if (!d)
        return LITE_ERR_NULL_ARG;
    if (d->batch < 0 || d->seqlen < 0 || d->heads < 0 || d->head_dim <= 0 || d->tile_m <= 0 || d->tile_n <= 0)
        return LITE_ERR_BAD_SHAPE;
    Dims r;
    r.Tq = (d->seqlen + (int64_t)d->tile_m - 1) / d->tile_m;
    r.Tk = (d->seqlen + (int64_t)d->tile_n - 1) / d->tile_n;
    r.W = (r.Tk + 31) / 32;
    r.rows = (int64_t)d->batch * d->heads * r.Tq;
    r.elems = (int64_t)d->batch * d->seqlen * d->heads * d->head_dim;  // < 2^62: no overflow
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
    case LITE_ERR_BAD_SHAPE: return "invalid shape: negative size, non-positive head_dim or tile, or sizes too large";
    case LITE_ERR_UNSUPPORTED:
        return "unsupported configuration: bf16 needs head_dim 64/128 and tile 128x64 or 128x128; "
               "fp32 needs head_dim 64 and tile 64x64; at most 4096 k-tiles";
    case LITE_ERR_BAD_THRESHOLD:
        return "invalid threshold: NaN, or > 0 without LITE_ATTENTION_DEBUG set to a value other than FALSE";
    case LITE_ERR_BAD_SCALE: return "invalid softmax_scale: must be finite and > 0";
    case LITE_ERR_MISALIGNED:
        return "misaligned pointer: q, k, v, out need 16-byte alignment; masks, skip-list and lse 4-byte";
    case LITE_ERR_ALIAS:
        return "overlapping buffers: out/lse overlap an input, or mask_out partly overlaps another buffer";
    case LITE_ERR_HIP:
        std::snprintf(buf, sizeof buf, "HIP error: %s", g_hip_msg);
        return buf;
    default: return "unknown error code";
    }
}

int lite_attn_fwd(const lite_attn_desc *desc, const void *q, const void *k, const void *v,
                  const uint32_t *mask_in, uint32_t *mask_out, const int32_t *skiplist, float tau,
                  float softmax_scale, void *out, float *lse, void *stream)
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
    if (empty(desc))
        return LITE_OK;
    if (!q || !k || !v || !out)
        return LITE_ERR_NULL_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(mask_in, 4) ||
        !aligned(mask_out, 4) || !aligned(skiplist, 4) || !aligned(lse, 4))
        return LITE_ERR_MISALIGNED;

    const size_t esz = desc->dtype == LITE_BF16 ? 2 : 4;
    const size_t tbytes = (size_t)r.elems * esz;
    const size_t mbytes = (size_t)(r.rows * r.W) * 4;
    const size_t sbytes = (size_t)(r.rows * (1 + r.Tk)) * 4;
    const size_t lbytes = (size_t)desc->batch * desc->heads * desc->seqlen * 4;
    const void *ins[] = {q, k, v};
    for (const void *in : ins) {
        if (overlap(out, tbytes, in, tbytes) || overlap(lse, lbytes, in, tbytes) ||
            overlap(mask_out, mbytes, in, tbytes))
            return LITE_ERR_ALIAS;
    }
    if (overlap(lse, lbytes, out, tbytes) || overlap(mask_out, mbytes, out, tbytes) ||
        overlap(mask_out, mbytes, lse, lbytes) || overlap(mask_out, mbytes, skiplist, sbytes) ||
        overlap(out, tbytes, mask_in, mbytes) || overlap(out, tbytes, skiplist, sbytes) ||
        overlap(lse, lbytes, mask_in, mbytes) || overlap(lse, lbytes, skiplist, sbytes))
        return LITE_ERR_ALIAS;
    if (mask_out != mask_in && overlap(mask_out, mbytes, mask_in, mbytes))
        return LITE_ERR_ALIAS;

    lite_attn::FwdParams p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.mask_in = mask_in;
    p.mask_out = mask_out;
    p.skiplist = skiplist;
    p.out = out;
    p.lse = lse;
    p.B = desc->batch;
    p.N = desc->seqlen;
    p.H = desc->heads;
    p.D = desc->head_dim;
    p.BM = desc->tile_m;
    p.BN = desc->tile_n;
    p.Tq = (int32_t)r.Tq;
    p.Tk = (int32_t)r.Tk;
    p.W = (int32_t)r.W;
    p.rows = r.rows;
    p.tau = (double)tau;
    p.scale = (double)softmax_scale;

    if (env_flag("LITE_ATTENTION_VERBOSE"))
        std::fprintf(stderr,
                     "[lite_attn] fwd %s d=%d tile=%dx%d B=%d N=%d H=%d rows=%lld Tk=%d mask_in=%d mask_out=%d "
                     "skiplist=%d tau=%g\n",
                     desc->dtype == LITE_BF16 ? "bf16" : "fp32", p.D, p.BM, p.BN, p.B, p.N, p.H,
                     (long long)p.rows, p.Tk, mask_in != nullptr, mask_out != nullptr, skiplist != nullptr,
                     (double)tau);

    hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t e =
        desc->dtype == LITE_BF16 ? lite_attn::launch_fwd_bf16(p, s) : lite_attn::launch_fwd_fp32(p, s);
    return e == hipSuccess ? LITE_OK : hip_fail(e);
}

int lite_attn_build_skiplist(const lite_attn_desc *desc, const uint32_t *mask, int32_t *skiplist, void *stream)
{
    Dims r;
    int rc = check_desc(desc, &r);
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
    const hipError_t e =
        lite_attn::launch_build_skiplist(mask, skiplist, r.rows, (int32_t)r.Tk, static_cast<hipStream_t>(stream));
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

}  // extern "C"
