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
    const int Nq = p.Nq, Nk = p.Nk, H = p.H, Tq = p.Tq, Tk = p.Tk, W = p.W;
    const int64_t row = blockIdx.x;
    const int qt = (int)(row % Tq);
    const int64_t bh = row / Tq;
    const int h = (int)(bh % H), b = (int)(bh / H);
    const int64_t rs = (int64_t)H * DIM;
    const int64_t qbase = (int64_t)b * p.q_sb + (int64_t)h * DIM;
    const int64_t kvbase = (int64_t)b * p.kv_sb + (int64_t)h * DIM;
    const float *Qb = (const float *)p.q + qbase;
    const float *Kb = (const float *)p.k + kvbase;
    const float *Vb = (const float *)p.v + kvbase;
    const uint32_t *mrow = p.mask_in ? p.mask_in + row * W : nullptr;
    const int32_t *list = p.skiplist ? p.skiplist + row * (1 + Tk) : nullptr;
    const bool vote = p.mask_out != nullptr;
    const bool ranges = p.rg.any != 0;
    const double scale = p.scale, tau = p.tau;

    // keep-vector: a clear bit marks the tile in mask_out.  Must-skip tiles are
    // never visited and never marked, so their bits start set.
    for (int w = lane; w < W; w += 64)
        keep[w] = ranges ? p.rg.skip_bits[w] : 0u;

    const int qi = qt * TILE + lane;
    const bool qvalid = qi < Nq;
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
    // (must-do tiles live whatever the mask says, must-skip tiles never)
    auto live_word = [&](int w) -> uint32_t {
        uint32_t bits = mrow ? ~mrow[w] : 0xffffffffu;
        if (ranges)
            bits = (bits & ~p.rg.skip_bits[w]) | p.rg.do_bits[w];
        if (w == W - 1 && (Tk & 31))
            bits &= (1u << (Tk & 31)) - 1u;
        return bits;
    };
    int cnt = 0, idx = 0, wi = W - 1;
    uint32_t cur = 0;
    if (list) {
        cnt = list[0];
        cnt = cnt < 0 ? 0 : (cnt > Tk ? Tk : cnt);
    } else if (W > 0) {
        cur = live_word(wi);
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
                cur = live_word(wi);
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
            Ks[c][lane] = key < Nk ? Kb[(int64_t)key * rs + lane] : 0.f;
            Vs[c][lane] = key < Nk ? Vb[(int64_t)key * rs + lane] : 0.f;
        }
        __syncthreads();

        // The tile in two 32-key halves, each folded into the online softmax
        // (exact in any grouping; half the logits live at a time keeps the
        // fp64 state in registers).  The QK-Skip test uses the maximum over
        // the whole tile against the running max taken before it.
        const double m_before = m_run;
        double m_tile = -INFINITY;
#pragma unroll
        for (int hc = 0; hc < TILE; hc += TILE / 2) {
            double s[TILE / 2];
            double mloc = -INFINITY;
#pragma unroll
            for (int c = 0; c < TILE / 2; ++c) {
                double dot = 0.0;
#pragma unroll
                for (int e = 0; e < DIM; ++e)
                    dot = fma((double)qv[e], (double)Ks[hc + c][e], dot);
                s[c] = (key0 + hc + c < Nk) ? dot * scale : -INFINITY;
                mloc = fmax(mloc, s[c]);
            }
            m_tile = fmax(m_tile, mloc);
            const double m_new = fmax(m_run, mloc);
            if (m_new > -INFINITY) {
                const double alpha = exp(m_run - m_new);
                l_run *= alpha;
#pragma unroll
                for (int e = 0; e < DIM; ++e)
                    o[e] *= alpha;
#pragma unroll
                for (int c = 0; c < TILE / 2; ++c) {
                    const double pc = (double)expf((float)(s[c] - m_new));
                    l_run += pc;
#pragma unroll
                    for (int e = 0; e < DIM; ++e)
                        o[e] = fma(pc, (double)Vs[hc + c][e], o[e]);
                }
                m_run = m_new;
            }
        }
        if (vote) {
            // a must-do tile is never marked
            const bool must_do = ranges && ((p.rg.do_bits[kt >> 5] >> (kt & 31)) & 1u);
            const bool keep_lane = must_do || (qvalid && !(m_tile - m_before < tau));
            if (__ballot(keep_lane) != 0ull && lane == 0)
                atomicOr(&keep[kt >> 5], 1u << (kt & 31));
        }
    }

    if (qvalid) {
        float *Ob = (float *)p.out + (int64_t)b * p.o_sb + (int64_t)h * DIM + (int64_t)qi * rs;
        const double inv = l_run > 0.0 ? 1.0 / l_run : 0.0;
#pragma unroll
        for (int e = 0; e < DIM; ++e)
            Ob[e] = (float)(o[e] * inv);
        if (p.lse)
            p.lse[bh * Nq + qi] = l_run > 0.0 ? (float)(m_run + log(l_run)) : -INFINITY;
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
