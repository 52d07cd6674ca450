// Skip-masked tiled attention forward for fp32 storage (head_dim 64, 64x64
// tiles).  Same method as the bf16 kernel (LiteAttention README: "QK-Skip
// Algorithm", "Full-Stage Elimination", reverse iteration over k-tiles), for
// callers that keep activations in fp32.
//
// One wave64 per (batch, head, q-tile); lane = query, so every row reduction
// is in-register.  Logits are accumulated in fp64: at this shape's logit
// magnitudes (|s| of a few tens) a plain fp32 dot product of 64 terms is off
// by a few 1e-5, more than an fp32 output can afford.  The exponent argument
// is formed in fp64 and rounded once to fp32 for exp; sums and the output
// accumulator stay in fp64.  This instantiation is latency-bound (a few
// hundred tiles per call), so it uses plain VALU arithmetic, not MFMA.
#include "lite_attn_internal.h"

#include <math.h>

namespace lite_attn {
namespace {

constexpr int TILE = 64;  // BM = BN = 64
constexpr int DIM = 64;
constexpr int MAXW = 128;

__global__ void __attribute__((amdgpu_flat_work_group_size(64, 64), amdgpu_waves_per_eu(1, 1)))
fwd_fp32_kernel(FwdParams p)
{
    __shared__ float Ks[TILE][DIM];
    __shared__ float Vs[TILE][DIM];
    __shared__ uint32_t keep[MAXW];

    const int lane = threadIdx.x;
    const int N = p.N, H = p.H, Tq = p.Tq, Tk = p.Tk, W = p.W;
    const int64_t row = blockIdx.x;
    const int qt = (int)(row % Tq);
    const int64_t bh = row / Tq;
    const int h = (int)(bh % H), b = (int)(bh / H);
    const int64_t rs = (int64_t)H * DIM;
    const int64_t base = (int64_t)b * N * rs + (int64_t)h * DIM;
    const float *Qb = (const float *)p.q + base;
    const float *Kb = (const float *)p.k + base;
    const float *Vb = (const float *)p.v + base;
    const uint32_t *mrow = p.mask_in ? p.mask_in + row * W : nullptr;
    const int32_t *list = p.skiplist ? p.skiplist + row * (1 + Tk) : nullptr;
    const bool vote = p.mask_out != nullptr;
    const double scale = p.scale, tau = p.tau;

    for (int w = lane; w < W; w += 64)
        keep[w] = 0u;

    const int qi = qt * TILE + lane;
    const bool qvalid = qi < N;
    float qv[DIM];
#pragma unroll
    for (int e = 0; e < DIM; ++e)
        qv[e] = qvalid ? Qb[(int64_t)qi * rs + e] : 0.f;

    double o[DIM];
#pragma unroll
    for (int e = 0; e < DIM; ++e)
        o[e] = 0.0;
    double m_run = -INFINITY, l_run = 0.0;

    // live k-tiles in visiting order (descending): Skip-List or mask words
    int cnt = 0, idx = 0, wi = W - 1;
    uint32_t cur = 0;
    if (list) {
        cnt = list[0];
        cnt = cnt < 0 ? 0 : (cnt > Tk ? Tk : cnt);
    } else {
        cur = mrow ? ~mrow[wi] : 0xffffffffu;
        if (Tk & 31)
            cur &= (1u << (Tk & 31)) - 1u;
    }

    for (;;) {
        int kt = -1;
        if (list) {
            if (idx < cnt) {
                kt = list[1 + idx++];
                if (kt < 0 || kt >= Tk)
                    kt = -1;
            }
        } else {
            while (cur == 0 && wi > 0) {
                --wi;
                cur = mrow ? ~mrow[wi] : 0xffffffffu;
            }
            if (cur != 0) {
                const int bit = 31 - __builtin_clz(cur);
                cur &= ~(1u << bit);
                kt = wi * 32 + bit;
            }
        }
        if (kt < 0)
            break;

        const int key0 = kt * TILE;
        __syncthreads();  // previous tile fully consumed
        for (int c = 0; c < TILE; ++c) {
            const int key = key0 + c;
            Ks[c][lane] = key < N ? Kb[(int64_t)key * rs + lane] : 0.f;
            Vs[c][lane] = key < N ? Vb[(int64_t)key * rs + lane] : 0.f;
        }
        __syncthreads();

        double s[TILE];
        double mloc = -INFINITY;
#pragma unroll
        for (int c = 0; c < TILE; ++c) {
            double dot = 0.0;
#pragma unroll
            for (int e = 0; e < DIM; ++e)
                dot = fma((double)qv[e], (double)Ks[c][e], dot);
            s[c] = (key0 + c < N) ? dot * scale : -INFINITY;
            mloc = fmax(mloc, s[c]);
        }
        if (vote) {
            const bool keep_lane = qvalid && !(mloc - m_run < tau);
            if (__ballot(keep_lane) != 0ull && lane == 0)
                atomicOr(&keep[kt >> 5], 1u << (kt & 31));
        }
        const double m_new = fmax(m_run, mloc);
        const double alpha = exp(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int e = 0; e < DIM; ++e)
            o[e] *= alpha;
#pragma unroll
        for (int c = 0; c < TILE; ++c) {
            const double pc = (double)expf((float)(s[c] - m_new));
            l_run += pc;
#pragma unroll
            for (int e = 0; e < DIM; ++e)
                o[e] = fma(pc, (double)Vs[c][e], o[e]);
        }
        m_run = m_new;
    }

    if (qvalid) {
        float *Ob = (float *)p.out + base + (int64_t)qi * rs;
        const double inv = l_run > 0.0 ? 1.0 / l_run : 0.0;
#pragma unroll
        for (int e = 0; e < DIM; ++e)
            Ob[e] = (float)(o[e] * inv);
        if (p.lse)
            p.lse[bh * N + qi] = l_run > 0.0 ? (float)(m_run + log(l_run)) : -INFINITY;
    }
    if (vote) {
        __syncthreads();
        for (int w = lane; w < W; w += 64) {
            uint32_t valid = 0xffffffffu;
            if (w == W - 1 && (Tk & 31))
                valid = (1u << (Tk & 31)) - 1u;
            const uint32_t in = mrow ? mrow[w] : 0u;
            p.mask_out[row * W + w] = (in | ~keep[w]) & valid;
        }
    }
}

}  // namespace

hipError_t launch_fwd_fp32(const FwdParams &p, hipStream_t stream)
{
    if (p.D != DIM || p.BM != TILE || p.BN != TILE || p.W > MAXW)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(fwd_fp32_kernel, dim3((unsigned)p.rows), dim3(64), 0, stream, p);
    return hipGetLastError();
}

}  // namespace lite_attn
