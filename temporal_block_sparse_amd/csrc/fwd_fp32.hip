// Skip-masked tiled attention forward for fp32 storage (head_dim 64, 64x64
// tiles).  Same method as the bf16 kernel (LiteAttention README: "QK-Skip
// Algorithm", "Full-Stage Elimination", reverse iteration over k-tiles), for
// callers that keep activations in fp32.
//
// One workgroup of 8 waves per (batch, head, q-tile); lane = query in every
// wave.  Per visited k-tile, the waves split the work three ways:
//   logits  -- wave w computes keys 8w .. 8w+7 of the tile for all 64 queries;
//   softmax -- the tile's row max comes from the waves' partial maxima, and
//              wave w turns its own 8 logits into weights;
//   PV      -- wave w accumulates head-dim entries 8w .. 8w+7 of the output
//              over all 64 keys.
// K and V are staged in LDS as fp64 (converted once, on load).  Logits are
// accumulated in fp64: at this shape's logit magnitudes (|s| of a few tens) a
// plain fp32 dot product of 64 terms is off by a few 1e-5, more than an fp32
// output can afford.  The exponent argument is formed in fp64 and rounded
// once to fp32 for exp; sums and the output accumulator stay in fp64.  The
// online softmax is folded once per tile; the QK-Skip test compares the
// tile's maximum with the running max taken before it.  Plain VALU
// arithmetic, not MFMA: the fp32 workloads are small and latency-bound.
#include "lite_attn_internal.h"

#include <math.h>

namespace lite_attn {
namespace {

constexpr int TILE = 64;  // BM = BN = 64
constexpr int DIM = 64;
constexpr int MAXW = 128;
constexpr int NWAVE = 8;
constexpr int KPW = TILE / NWAVE;  // keys (logits) and head-dim entries (PV) per wave

__global__ void __attribute__((amdgpu_flat_work_group_size(512, 512))) fwd_fp32_kernel(FwdParams p)
{
    __shared__ double Kd[TILE][DIM];
    __shared__ double Vd[TILE][DIM];
    __shared__ double S[TILE][TILE];   // [key][query]: logits, then weights
    __shared__ double mx[NWAVE][TILE]; // per-wave maximum over its keys, per query
    __shared__ double ps[NWAVE][TILE]; // per-wave sum of its weights, per query
    __shared__ uint32_t keep[MAXW];

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
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
    for (int w = tid; w < W; w += 512)
        keep[w] = ranges ? p.rg.skip_bits[w] : 0u;

    // this lane's query, in fp64
    const int qi = qt * TILE + lane;
    const bool qvalid = qi < Nq;
    double qd[DIM];
#pragma unroll
    for (int e = 0; e < DIM; e += 4) {
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (qvalid)
            x = *(const float4 *)(Qb + (int64_t)qi * rs + e);
        qd[e] = x.x;
        qd[e + 1] = x.y;
        qd[e + 2] = x.z;
        qd[e + 3] = x.w;
    }

    double o[KPW];  // head-dim entries wv*KPW .. +KPW of this lane's output
#pragma unroll
    for (int e = 0; e < KPW; ++e)
        o[e] = 0.0;
    double m_run = -INFINITY, l_run = 0.0;  // identical in every wave

    // live k-tiles in visiting order (descending): Skip-List or mask words
    // (must-do tiles live whatever the mask says, must-skip tiles never).
    // Every wave walks the same sequence.
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

    // K/V tile staging: thread tid converts 8 consecutive elements of key
    // row tid / 8 (columns (tid % 8) * 8 ..) of each
    const int lc = tid >> 3, le = (tid & 7) * 8;

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

        __syncthreads();  // the previous tile is fully consumed
        {
            const int key = key0 + lc;
            float4 k0 = make_float4(0.f, 0.f, 0.f, 0.f), k1 = k0, v0 = k0, v1 = k0;
            if (key < Nk) {
                const float *kr = Kb + (int64_t)key * rs + le;
                const float *vr = Vb + (int64_t)key * rs + le;
                k0 = *(const float4 *)kr;
                k1 = *(const float4 *)(kr + 4);
                v0 = *(const float4 *)vr;
                v1 = *(const float4 *)(vr + 4);
            }
            double *kd = &Kd[lc][le];
            double *vd = &Vd[lc][le];
            *(double2 *)(kd + 0) = make_double2(k0.x, k0.y);
            *(double2 *)(kd + 2) = make_double2(k0.z, k0.w);
            *(double2 *)(kd + 4) = make_double2(k1.x, k1.y);
            *(double2 *)(kd + 6) = make_double2(k1.z, k1.w);
            *(double2 *)(vd + 0) = make_double2(v0.x, v0.y);
            *(double2 *)(vd + 2) = make_double2(v0.z, v0.w);
            *(double2 *)(vd + 4) = make_double2(v1.x, v1.y);
            *(double2 *)(vd + 6) = make_double2(v1.z, v1.w);
        }
        __syncthreads();

        // logits of this wave's keys (fp64 dot products in head-dim order)
        {
            double s[KPW];
#pragma unroll
            for (int j = 0; j < KPW; ++j)
                s[j] = 0.0;
#pragma unroll
            for (int e = 0; e < DIM; e += 2) {
#pragma unroll
                for (int j = 0; j < KPW; ++j) {
                    const double2 kk = *(const double2 *)&Kd[wv * KPW + j][e];
                    s[j] = fma(qd[e], kk.x, s[j]);
                    s[j] = fma(qd[e + 1], kk.y, s[j]);
                }
            }
            double m = -INFINITY;
#pragma unroll
            for (int j = 0; j < KPW; ++j) {
                const double sj = (key0 + wv * KPW + j < Nk) ? s[j] * scale : -INFINITY;
                S[wv * KPW + j][lane] = sj;
                m = fmax(m, sj);
            }
            mx[wv][lane] = m;
        }
        __syncthreads();

        // the tile's row max, the online-softmax update, this wave's weights
        double m_tile = mx[0][lane];
#pragma unroll
        for (int w = 1; w < NWAVE; ++w)
            m_tile = fmax(m_tile, mx[w][lane]);
        const double m_before = m_run;
        const double m_new = fmax(m_run, m_tile);
        const bool upd = m_new > -INFINITY;
        const double alpha = upd ? exp(m_run - m_new) : 1.0;
        {
            double sum = 0.0;
#pragma unroll
            for (int j = 0; j < KPW; ++j) {
                const double pj = upd ? (double)expf((float)(S[wv * KPW + j][lane] - m_new)) : 0.0;
                S[wv * KPW + j][lane] = pj;
                sum += pj;
            }
            ps[wv][lane] = sum;
        }
        m_run = m_new;
        if (vote && wv == 0) {
            // a must-do tile is never marked
            const bool must_do = ranges && ((p.rg.do_bits[kt >> 5] >> (kt & 31)) & 1u);
            const bool keep_lane = must_do || (qvalid && !(m_tile - m_before < tau));
            if (__ballot(keep_lane) != 0ull && lane == 0)
                keep[kt >> 5] |= 1u << (kt & 31);
        }
        __syncthreads();

        // row sum and this wave's slice of the output
        {
            double tsum = 0.0;
#pragma unroll
            for (int w = 0; w < NWAVE; ++w)
                tsum += ps[w][lane];
            l_run = l_run * alpha + tsum;
#pragma unroll
            for (int e = 0; e < KPW; ++e)
                o[e] *= alpha;
#pragma unroll 8
            for (int c = 0; c < TILE; ++c) {
                const double pc = S[c][lane];
                const double *vr = &Vd[c][wv * KPW];
#pragma unroll
                for (int e = 0; e < KPW; e += 2) {
                    const double2 vv = *(const double2 *)(vr + e);
                    o[e] = fma(pc, vv.x, o[e]);
                    o[e + 1] = fma(pc, vv.y, o[e + 1]);
                }
            }
        }
    }

    if (qvalid) {
        float *Ob = (float *)p.out + (int64_t)b * p.o_sb + (int64_t)h * DIM + (int64_t)qi * rs + wv * KPW;
        const double inv = l_run > 0.0 ? 1.0 / l_run : 0.0;
        float4 r0, r1;
        r0.x = (float)(o[0] * inv);
        r0.y = (float)(o[1] * inv);
        r0.z = (float)(o[2] * inv);
        r0.w = (float)(o[3] * inv);
        r1.x = (float)(o[4] * inv);
        r1.y = (float)(o[5] * inv);
        r1.z = (float)(o[6] * inv);
        r1.w = (float)(o[7] * inv);
        *(float4 *)Ob = r0;
        *(float4 *)(Ob + 4) = r1;
        if (p.lse && wv == 0)
            p.lse[bh * Nq + qi] = l_run > 0.0 ? (float)(m_run + log(l_run)) : -INFINITY;
    }
    if (vote) {
        __syncthreads();
        for (int w = tid; w < W; w += 512) {
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
    hipLaunchKernelGGL(fwd_fp32_kernel, dim3((unsigned)p.rows), dim3(512), 0, stream, p);
    return hipGetLastError();
}

}  // namespace lite_attn
