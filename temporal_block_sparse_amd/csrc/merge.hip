// LSE merge of partial attentions (README Python API: the softmax LSE is
// returned for combining the results of several partial attention calls --
// the text/video split and the K/V splits of SeqParallelLiteAttention).
//
// For every query (b, n, h), over the parts i with lse_i > -inf:
//   lse = m + ln(sum_i exp(lse_i - m)),  m = max_i lse_i,
//   out = sum_i exp(lse_i - lse) * out_i.
// HBM-bound: P*(d*esz + 4) bytes read and d*esz + 4 written per query.
//
// Layout: one thread per 8 consecutive head-dim elements of one (b, n, h);
// the d/8 threads of a query sit in one wave (d/8 is a power of two <= 64),
// so every thread of the query reads the part LSEs before any of them writes
// the merged one -- which makes the in-place call (out == outs[i], lse ==
// lses[i]) safe.
#include "lite_attn_internal.h"

#include <math.h>

namespace lite_attn {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void load8(const void *base, int64_t off, int dtype, float (&x)[8])
{
    if (dtype == 0) {
        const u32x4 w = *(const u32x4 *)((const __bf16 *)base + off);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[2 * j] = __builtin_bit_cast(float, w[j] << 16);
            x[2 * j + 1] = __builtin_bit_cast(float, w[j] & 0xffff0000u);
        }
    } else {
        const f32x4 a = *(const f32x4 *)((const float *)base + off);
        const f32x4 b = *(const f32x4 *)((const float *)base + off + 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[j] = a[j];
            x[4 + j] = b[j];
        }
    }
}

__device__ __forceinline__ void store8(void *base, int64_t off, int dtype, const float (&x)[8])
{
    if (dtype == 0) {
        u32x4 w;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t lo = __builtin_bit_cast(uint16_t, (__bf16)x[2 * j]);
            const uint32_t hi = __builtin_bit_cast(uint16_t, (__bf16)x[2 * j + 1]);
            w[j] = lo | (hi << 16);
        }
        *(u32x4 *)((__bf16 *)base + off) = w;
    } else {
        f32x4 a, b;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            a[j] = x[j];
            b[j] = x[4 + j];
        }
        *(f32x4 *)((float *)base + off) = a;
        *(f32x4 *)((float *)base + off + 4) = b;
    }
}

__global__ void __launch_bounds__(256) merge_kernel(MergeParams p)
{
    const int cpq = p.D / 8;  // threads per query
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t nq = (int64_t)p.B * p.N * p.H;
    const int64_t qid = t / cpq;  // (b, n, h) in BSHD order
    const int c = (int)(t % cpq);
    const bool on = qid < nq;
    int64_t off = 0, ooff = 0, lo = 0;
    float lse[MAX_MERGE_PARTS];
    float m = -INFINITY;
    if (on) {
        const int h = (int)(qid % p.H);
        const int64_t bn = qid / p.H;
        const int n = (int)(bn % p.N), b = (int)(bn / p.N);
        off = (int64_t)b * p.q_sb + ((int64_t)n * p.H + h) * p.D + 8 * c;
        ooff = (int64_t)b * p.o_sb + ((int64_t)n * p.H + h) * p.D + 8 * c;
        lo = ((int64_t)b * p.H + h) * p.N + n;
#pragma unroll
        for (int i = 0; i < MAX_MERGE_PARTS; ++i) {
            lse[i] = i < p.nparts ? p.lses[i][lo] : -INFINITY;
            m = fmaxf(m, lse[i]);
        }
    }
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float s = 0.f;
    if (on && m != -INFINITY) {
#pragma unroll
        for (int i = 0; i < MAX_MERGE_PARTS; ++i) {
            if (i < p.nparts && lse[i] != -INFINITY) {
                const float w = expf(lse[i] - m);
                s += w;
                float x[8];
                load8(p.outs[i], off, p.dtype, x);
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    acc[j] = fmaf(w, x[j], acc[j]);
            }
        }
        const float inv = 1.0f / s;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            acc[j] *= inv;
    }
    // every thread of this wave has read its part values before any writes
    __builtin_amdgcn_wave_barrier();
    if (on) {
        store8(p.out, ooff, p.dtype, acc);
        if (p.lse && c == 0)
            p.lse[lo] = m == -INFINITY ? -INFINITY : m + logf(s);
    }
}

}  // namespace

hipError_t launch_merge(const MergeParams &p, hipStream_t stream)
{
    if (p.D % 8 != 0 || p.D > 512 || p.nparts < 1 || p.nparts > MAX_MERGE_PARTS)
        return hipErrorInvalidValue;
    const int64_t threads = (int64_t)p.B * p.N * p.H * (p.D / 8);
    if (threads <= 0)
        return hipSuccess;
    const int64_t blocks = (threads + 255) / 256;
    if (blocks > 0x7fffffff)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(merge_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace lite_attn
