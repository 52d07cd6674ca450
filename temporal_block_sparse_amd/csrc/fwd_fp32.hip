// Skip-masked tiled attention forward for fp32 storage (head_dim 64, 64x64
// tiles).  Same method as the bf16 kernel (LiteAttention README: "QK-Skip
// Algorithm", "Full-Stage Elimination", reverse iteration over k-tiles), for
// callers that keep activations in fp32.
//
// One workgroup of 8 waves per (batch, head, q-tile).  Both contractions
// run on the fp64 matrix cores (v_mfma_f64_16x16x4f64: 16x16 blocks, 4 terms
// per step):
//   logits  S^T = K Q^T -- wave w owns key block w/2 (16 keys) and query
//           blocks 2(w%2), 2(w%2)+1, with Q^T in registers and K from LDS;
//   softmax on the accumulators: the tile's row max from per-wave maxima
//           (LDS), the weights into an LDS buffer P[key][query];
//   PV      O^T = V^T P^T -- wave w owns head-dim block w/2 for the same two
//           query blocks, so a lane's online-softmax state (two queries) is
//           the same in both phases.
// Matrix-core operands: lane l holds A[l%16][l/16] and B[l/16][l%16] of each
// 16x4 / 4x16 step, and D[l/16 + 4r][l%16], r = 0..3, of the 16x16 result.
// K (transposed), V and P sit in LDS as fp64 with a row stride of 80
// doubles, so each 32-lane half of an operand read touches distinct banks.
// The next tile's K and V are loaded into registers a whole tile ahead.
// Arithmetic: fp64 logits (at this shape's logit magnitudes, |s| of a few
// tens, a plain fp32 dot product of 64 terms is off by a few 1e-5, more than
// an fp32 output can afford); the exponent argument formed in fp64 and
// rounded once to fp32 for exp; sums and the output accumulator in fp64.
// The online softmax is folded once per tile; the QK-Skip test compares the
// tile's maximum with the running max taken before it.
#include "lite_attn_internal.h"

#include <math.h>

namespace lite_attn {
namespace {

constexpr int TILE = 64;  // BM = BN = 64
constexpr int DIM = 64;
constexpr int MAXW = 128;
constexpr int NWAVE = 8;
constexpr int LD = 80;  // LDS row stride (doubles) of Kt, Vd and P

typedef double f64x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ double xor_max(double x, int m) { return fmax(x, __shfl_xor(x, m)); }
__device__ __forceinline__ double xor_sum(double x, int m) { return x + __shfl_xor(x, m); }

__global__ void __attribute__((amdgpu_flat_work_group_size(512, 512))) fwd_fp32_kernel(FwdParams p)
{
    __shared__ double Kt[DIM][LD];   // K transposed: [head-dim][key]
    __shared__ double Vd[TILE][LD];  // [key][head-dim]
    __shared__ double P[TILE][LD];   // [key][query]: the tile's weights
    __shared__ double mx[4][TILE];   // per key block: maximum logit, per query
    __shared__ double ps[4][TILE];   // per key block: sum of weights, per query
    __shared__ uint32_t keep[MAXW];

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int l16 = lane & 15, g = lane >> 4;
    const int xb = wv >> 1;             // key block (logits) / head-dim block (PV)
    const int qb0 = 2 * (wv & 1);       // first of this wave's two query blocks
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

    // this lane's two queries (one per query block) and their Q^T operands:
    // step s of block j takes Q[query_j][4s + g]
    int qi[2];
    bool qv[2];
    double qf[2][DIM / 4];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        qi[j] = qt * TILE + (qb0 + j) * 16 + l16;
        qv[j] = qi[j] < Nq;
        const float *qr = Qb + (int64_t)qi[j] * rs + g;
#pragma unroll
        for (int st = 0; st < DIM / 4; ++st)
            qf[j][st] = qv[j] ? (double)qr[4 * st] : 0.0;
    }

    f64x4 O[2];  // O^T block (head-dim block xb, query block qb0 + j)
#pragma unroll
    for (int j = 0; j < 2; ++j)
        O[j] = (f64x4){0.0, 0.0, 0.0, 0.0};
    double m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.0, 0.0};

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
    auto next_tile = [&]() -> int {
        if (list) {
            if (idx < cnt) {
                const int kt = list[1 + idx++];
                return (kt < 0 || kt >= Tk) ? -1 : kt;
            }
            return -1;
        }
        while (cur == 0 && wi > 0) {
            --wi;
            cur = live_word(wi);
        }
        if (cur == 0)
            return -1;
        const int bit = 31 - __builtin_clz(cur);
        cur &= ~(1u << bit);
        return wi * 32 + bit;
    };

    // K/V staging: thread tid holds 8 consecutive elements (head-dim (tid % 8) * 8 ..)
    // of key row tid / 8 of the next tile, loaded a tile ahead
    const int lc = tid >> 3, le = (tid & 7) * 8;
    float4 pk0, pk1, pv0, pv1;
    auto fetch = [&](int kt) {
        const int key = kt * TILE + lc;
        pk0 = pk1 = pv0 = pv1 = make_float4(0.f, 0.f, 0.f, 0.f);
        if (kt >= 0 && key < Nk) {
            const float *kr = Kb + (int64_t)key * rs + le;
            const float *vr = Vb + (int64_t)key * rs + le;
            pk0 = *(const float4 *)kr;
            pk1 = *(const float4 *)(kr + 4);
            pv0 = *(const float4 *)vr;
            pv1 = *(const float4 *)(vr + 4);
        }
    };

    int kt = next_tile();
    fetch(kt);
    while (kt >= 0) {
        const int key0 = kt * TILE;
        __syncthreads();  // the previous tile is fully consumed
        {
            const float kx[8] = {pk0.x, pk0.y, pk0.z, pk0.w, pk1.x, pk1.y, pk1.z, pk1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e)
                Kt[le + e][lc] = kx[e];
            double *vd = &Vd[lc][le];
            *(double2 *)(vd + 0) = make_double2(pv0.x, pv0.y);
            *(double2 *)(vd + 2) = make_double2(pv0.z, pv0.w);
            *(double2 *)(vd + 4) = make_double2(pv1.x, pv1.y);
            *(double2 *)(vd + 6) = make_double2(pv1.z, pv1.w);
        }
        const int kt_next = next_tile();
        fetch(kt_next);
        __syncthreads();

        // logits S^T of key block xb for this wave's two query blocks
        f64x4 Sacc[2] = {(f64x4){0.0, 0.0, 0.0, 0.0}, (f64x4){0.0, 0.0, 0.0, 0.0}};
#pragma unroll
        for (int st = 0; st < DIM / 4; ++st) {
            const double a = Kt[4 * st + g][xb * 16 + l16];
#pragma unroll
            for (int j = 0; j < 2; ++j)
                Sacc[j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, qf[j][st], Sacc[j], 0, 0, 0);
        }
        // lane holds keys xb*16 + g + 4r of query qi[j]
        double sv[2][4];
        double wmax[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            double m = -INFINITY;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = key0 + xb * 16 + g + 4 * r;
                sv[j][r] = key < Nk ? Sacc[j][r] * scale : -INFINITY;
                m = fmax(m, sv[j][r]);
            }
            m = xor_max(m, 16);
            m = xor_max(m, 32);
            wmax[j] = m;
        }
        if (g == 0) {
#pragma unroll
            for (int j = 0; j < 2; ++j)
                mx[xb][(qb0 + j) * 16 + l16] = wmax[j];
        }
        __syncthreads();

        // the tile's row max, the online-softmax update, this wave's weights
        double alpha[2];
        bool keep_lane = false;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int qc = (qb0 + j) * 16 + l16;
            const double m_tile = fmax(fmax(mx[0][qc], mx[1][qc]), fmax(mx[2][qc], mx[3][qc]));
            const double m_before = m_run[j];
            const double m_new = fmax(m_run[j], m_tile);
            const bool upd = m_new > -INFINITY;
            alpha[j] = upd ? exp(m_run[j] - m_new) : 1.0;
            double sum = 0.0;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const double pj = upd ? (double)expf((float)(sv[j][r] - m_new)) : 0.0;
                P[xb * 16 + g + 4 * r][qc] = pj;
                sum += pj;
            }
            sum = xor_sum(sum, 16);
            sum = xor_sum(sum, 32);
            if (g == 0)
                ps[xb][qc] = sum;
            m_run[j] = m_new;
            keep_lane = keep_lane || (qv[j] && !(m_tile - m_before < tau));
        }
        if (vote && xb == 0) {
            // a must-do tile is never marked
            const bool must_do = ranges && ((p.rg.do_bits[kt >> 5] >> (kt & 31)) & 1u);
            if (__ballot(keep_lane || must_do) != 0ull && lane == 0)
                atomicOr(&keep[kt >> 5], 1u << (kt & 31));
        }
        __syncthreads();

        // row sums, and this wave's block of the output: O^T += V^T P^T
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int qc = (qb0 + j) * 16 + l16;
            l_run[j] = l_run[j] * alpha[j] + (((ps[0][qc] + ps[1][qc]) + ps[2][qc]) + ps[3][qc]);
            O[j] *= alpha[j];
        }
#pragma unroll
        for (int st = 0; st < TILE / 4; ++st) {
            const double a = Vd[4 * st + g][xb * 16 + l16];
#pragma unroll
            for (int j = 0; j < 2; ++j)
                O[j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, P[4 * st + g][(qb0 + j) * 16 + l16], O[j], 0, 0, 0);
        }
        kt = kt_next;
    }

    // lane holds head-dim entries xb*16 + g + 4r of queries qi[0], qi[1]
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        if (!qv[j])
            continue;
        float *Ob = (float *)p.out + (int64_t)b * p.o_sb + (int64_t)h * DIM + (int64_t)qi[j] * rs + xb * 16 + g;
        const double inv = l_run[j] > 0.0 ? 1.0 / l_run[j] : 0.0;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            Ob[4 * r] = (float)(O[j][r] * inv);
        if (p.lse && xb == 0 && g == 0)
            p.lse[bh * Nq + qi[j]] = l_run[j] > 0.0 ? (float)(m_run[j] + log(l_run[j])) : -INFINITY;
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
