// Skip-masked tiled attention forward, bf16 in / bf16 out, fp32 accumulation,
// hand-written for gfx950 (CDNA4): one workgroup of 4 wave64s per
// (batch, head, q-tile of 128 queries); each wave owns 32 queries; two
// workgroups share a CU.
//
// Method (LiteAttention README, "QK-Skip Algorithm" and "Full-Stage
// Elimination"; arXiv 2511.11062 abstract): k-tiles set in the Skip-Mask are
// bypassed entirely -- no K/V traffic, no QK^T, no softmax, no PV.  Live
// k-tiles are visited last-to-first (README Python API: the kernel iterates in
// reverse order) with flash-style online softmax; every visited tile also
// runs the QK-Skip test (tile-local max logit minus the running max before
// the tile, below the threshold for every query of the q-tile) and, when it
// passes, is marked in the mask carried to the next denoising step.
//
// gfx950 layout choices
// * Both contractions are transposed, S^T = K Q^T and O^T = V^T P^T, on
//   v_mfma_f32_32x32x16_bf16.  The accumulator layout then gives every lane a
//   single query (lane % 32): its row max needs only in-register max plus one
//   v_permlane32_swap with the other half-wave, P^T feeds the second MFMA
//   straight from registers, and the O rescale uses the lane's own factor.
// * A k-tile is consumed in steps of 64 keys.  The online softmax is updated
//   per step (exact in any grouping); the QK-Skip test uses the maximum over
//   all steps of the tile against the running max taken before its first step.
// * Two 64-key steps are double-buffered in LDS (64 KB at head_dim 128), so
//   two workgroups fit on a CU and each SIMD interleaves two waves: one wave's
//   softmax (VALU, v_exp) runs under the other's MFMAs.  The next step's
//   global loads are issued before the current step's MFMAs and land in the
//   other buffer afterwards; one barrier per step.
// * K rows are stored in LDS with rows 4..7 and 8..11 of every 16 swapped, so
//   that the 8 scores a lane holds per 16-key MFMA step are 8 consecutive
//   keys; V is stored transposed (V^T, e-major) via an in-register 4x8
//   transpose (v_perm_b32), so the PV A-operand is one 16-byte LDS read, with
//   its rows permuted so a lane's O^T values are 16 consecutive head-dim
//   entries (two 16-byte global stores).
// * 16-byte chunks are XOR-swizzled per row against LDS bank conflicts.
// * Loads use a wave-uniform tile base plus a per-lane 32-bit offset fixed for
//   the whole kernel; only the ragged last tile takes the predicated path.
// * The QK-Skip vote is one ballot per wave and tile; a wave that wants to
//   keep the tile sets its bit in an LDS keep-vector with one atomic OR.  The
//   mask row is written once, in the epilogue.
// * Workgroups are remapped so each XCD runs contiguous q-tiles of a head
//   (shared K/V in that XCD's L2).
#include "lite_attn_internal.h"

#include <math.h>

namespace lite_attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BM = 128;       // queries per workgroup (one q-tile)
constexpr int NWAVES = 4;
constexpr int NT = 64 * NWAVES;
constexpr int HK = 64;        // keys per step
constexpr int MAXW = 128;     // mask words per row (Tk <= 4096)

// LDS row r of a K step holds key kperm(r): rows 4..7 and 8..11 of each 16 swapped.
__device__ __forceinline__ int kperm(int r)
{
    const int m = r & 15;
    return (m >= 4 && m < 8) ? r + 4 : ((m >= 8 && m < 12) ? r - 4 : r);
}

// LDS row of head-dim entry e in a V^T step: within each 32-block,
// e = 16*g + 4*a + b is stored at row 8*a + 4*g + b.
__device__ __forceinline__ int vt_row(int e)
{
    const int x = e & 31;
    return (e & ~31) | (((x >> 2) & 3) << 3) | ((x >> 4) << 2) | (x & 3);
}

// 16-byte chunk swizzle: a bijection on the low 3 chunk bits for any 8
// consecutive rows, and across rows that differ in bits 2, 4, 5 (the V^T
// store pattern).
__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 4) & 3); }

__device__ __forceinline__ float other_half(float x)
{
    // v_permlane32_swap(x, x): first = x of lane l % 32, second = x of lane l % 32 + 32
    auto s = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                              __builtin_bit_cast(uint32_t, x), false, false);
    const float a = __builtin_bit_cast(float, (uint32_t)s[0]);
    const float b = __builtin_bit_cast(float, (uint32_t)s[1]);
    return (threadIdx.x & 32) ? a : b;
}

// Live k-tiles of one row in visiting order (descending), from the Skip-List
// when one is given, else from the mask words.  All values are wave-uniform.
struct LiveTiles {
    const uint32_t *mask;
    const int32_t *list;
    int Tk, W, w, idx, cnt;
    uint32_t cur;

    __device__ uint32_t live_word(int wi) const
    {
        uint32_t bits = mask ? ~mask[wi] : 0xffffffffu;
        if (wi == W - 1 && (Tk & 31))
            bits &= (1u << (Tk & 31)) - 1u;
        return bits;
    }
    __device__ void init(const uint32_t *m, const int32_t *l, int tk)
    {
        mask = m;
        list = l;
        Tk = tk;
        W = (tk + 31) >> 5;
        idx = 0;
        if (list) {
            const int c = list[0];
            cnt = c < 0 ? 0 : (c > tk ? tk : c);
            w = 0;
            cur = 0;
        } else {
            cnt = 0;
            w = W - 1;
            cur = live_word(w);
        }
    }
    __device__ int next()
    {
        if (list) {
            if (idx >= cnt)
                return -1;
            const int kt = list[1 + idx++];
            return (kt >= 0 && kt < Tk) ? kt : -1;
        }
        while (cur == 0) {
            if (w <= 0)
                return -1;
            cur = live_word(--w);
        }
        const int bit = 31 - __builtin_clz(cur);
        cur &= ~(1u << bit);
        return w * 32 + bit;
    }
};

template <int D>
struct Geo {
    static constexpr int KCH = HK * D / 8;   // 16-byte chunks of a K step (= of a V^T step)
    static constexpr int STAGE = 2 * KCH;    // K then V^T, in 16-byte chunks
    static constexpr int KPT = KCH / NT;     // K chunks per thread
    static constexpr int VK = HK * D / 8 / NT;  // keys per thread's V block (VK x 8 head-dim entries)
    static_assert(KCH % NT == 0 && (VK == 2 || VK == 4), "unsupported step geometry");
};

template <int D, int BN>
__global__ void __attribute__((amdgpu_flat_work_group_size(NT, NT), amdgpu_waves_per_eu(2, 2)))
fwd_bf16_kernel(FwdParams p, float c2, float tau2)
{
    using G = Geo<D>;
    constexpr int SPT = BN / HK;  // steps per k-tile
    __shared__ u32x4 smem[2 * G::STAGE];
    __shared__ uint32_t keep[MAXW];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, lq = lane & 31;
    const int N = p.N, H = p.H, Tq = p.Tq, Tk = p.Tk, W = p.W;
    const int64_t row = xcd_remap(blockIdx.x, p.rows);
    const int qt = (int)(row % Tq);
    const int64_t bh = row / Tq;
    const int h = (int)(bh % H), b = (int)(bh / H);
    const int rs = H * D;  // token stride (elements)
    const int64_t base = (int64_t)b * N * rs + (int64_t)h * D;
    const __bf16 *Qb = (const __bf16 *)p.q + base;
    const char *Kb = (const char *)((const __bf16 *)p.k + base);
    const char *Vb = (const char *)((const __bf16 *)p.v + base);
    const uint32_t *mrow = p.mask_in ? p.mask_in + row * W : nullptr;
    const bool vote = p.mask_out != nullptr;

    if (tid < W)
        keep[tid] = 0u;

    // this lane's query and its Q^T B-operand fragments
    const int qi = qt * BM + wave * 32 + lq;
    const bool qvalid = qi < N;
    bf16x8 qf[D / 16];
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) {
        u32x4 x = {0u, 0u, 0u, 0u};
        if (qvalid)
            x = *(const u32x4 *)(Qb + (int64_t)qi * rs + ds * 16 + 8 * g);
        qf[ds] = __builtin_bit_cast(bf16x8, x);
    }

    // per-thread load slots (fixed for the kernel): K chunk i is key row kr[i],
    // 16-byte column kc[i]; V block j covers keys 4*vk[j]..+3, head-dim 8*vc..+7
    int koff[G::KPT], kr[G::KPT], klds[G::KPT];
#pragma unroll
    for (int i = 0; i < G::KPT; ++i) {
        const int C = tid + i * NT, r = C / (D / 8), c = C % (D / 8);
        kr[i] = r;
        koff[i] = r * rs * 2 + c * 16;
        const int lr = kperm(r);
        klds[i] = lr * (D / 8) + (c ^ swz(lr));
    }
    const int vc = tid % (D / 8);              // V block: head-dim entries 8*vc..+7
    const int vk = tid / (D / 8);              //          keys VK*vk..+VK-1 of the step
    const int voff = vk * G::VK * rs * 2 + vc * 16;

    u32x4 kreg[G::KPT];
    u32x4 vreg[G::VK];
    auto load_step = [&](int key0) {
        const char *kb = Kb + (int64_t)key0 * rs * 2;
        const char *vb = Vb + (int64_t)key0 * rs * 2;
        if (key0 + HK <= N) {
#pragma unroll
            for (int i = 0; i < G::KPT; ++i)
                kreg[i] = *(const u32x4 *)(kb + koff[i]);
#pragma unroll
            for (int r = 0; r < G::VK; ++r)
                vreg[r] = *(const u32x4 *)(vb + voff + r * rs * 2);
        } else {
            const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int i = 0; i < G::KPT; ++i)
                kreg[i] = (key0 + kr[i] < N) ? *(const u32x4 *)(kb + koff[i]) : z;
#pragma unroll
            for (int r = 0; r < G::VK; ++r)
                vreg[r] = (key0 + G::VK * vk + r < N) ? *(const u32x4 *)(vb + voff + r * rs * 2) : z;
        }
    };
    auto store_step = [&](int stage) {
        u32x4 *Ks = smem + stage * G::STAGE;
        char *Vs = (char *)(Ks + G::KCH);
#pragma unroll
        for (int i = 0; i < G::KPT; ++i)
            Ks[klds[i]] = kreg[i];
        // VK keys x 8 head-dim entries -> 8 rows of V^T holding VK keys (2*VK bytes) each
        constexpr int PER_CHUNK = 8 / G::VK;    // key groups per 16-byte chunk
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
            const int lr = vt_row(vc * 8 + e);
            char *dst = Vs + (lr * (HK / 8) + ((vk / PER_CHUNK) ^ swz(lr))) * 16 + (vk % PER_CHUNK) * 2 * G::VK;
            if constexpr (G::VK == 4) {
                u32x2 o;
                o[0] = __builtin_amdgcn_perm(vreg[1][e >> 1], vreg[0][e >> 1], sel);
                o[1] = __builtin_amdgcn_perm(vreg[3][e >> 1], vreg[2][e >> 1], sel);
                *(u32x2 *)dst = o;
            } else {
                *(uint32_t *)dst = __builtin_amdgcn_perm(vreg[1][e >> 1], vreg[0][e >> 1], sel);
            }
        }
    };

    f32x16 O[D / 32];
#pragma unroll
    for (int eb = 0; eb < D / 32; ++eb)
#pragma unroll
        for (int v = 0; v < 16; ++v)
            O[eb][v] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;
    float m_before = -INFINITY, m_tile = -INFINITY;

    LiveTiles it;
    it.init(mrow, p.skiplist ? p.skiplist + row * (1 + Tk) : nullptr, Tk);
    int kt = it.next();
    int sub = 0;
    if (kt >= 0) {
        load_step(kt * BN);
        store_step(0);
    }
    __syncthreads();
    int kt_after = kt >= 0 ? it.next() : -1;  // next live tile after kt
    int stage = 0;

    while (kt >= 0) {
        // the step after this one
        int kt_n = kt, sub_n = sub + 1;
        if (sub_n == SPT) {
            kt_n = kt_after;
            sub_n = 0;
        }
        const int key0 = kt * BN + sub * HK;
        if (kt_n >= 0 && kt_n * BN + sub_n * HK < N)
            load_step(kt_n * BN + sub_n * HK);

        const u32x4 *Ks = smem + stage * G::STAGE;
        const u32x4 *Vs = Ks + G::KCH;
        if (sub == 0) {
            m_before = m_run;
            m_tile = -INFINITY;
        }

        if (key0 < N) {
            // ---- S^T = K Q^T (raw logits, fp32) ----
            f32x16 S[HK / 32];
#pragma unroll
            for (int kb = 0; kb < HK / 32; ++kb) {
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    S[kb][v] = 0.f;
                const int lr = kb * 32 + lq;
#pragma unroll
                for (int ds = 0; ds < D / 16; ++ds) {
                    const u32x4 a = Ks[lr * (D / 8) + ((2 * ds + g) ^ swz(lr))];
                    S[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), qf[ds], S[kb],
                                                                    0, 0, 0);
                }
            }

            // keys past the end of the sequence do not exist
            if (key0 + HK > N) {
#pragma unroll
                for (int kb = 0; kb < HK / 32; ++kb)
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        if (key0 + kb * 32 + 16 * (v >> 3) + 8 * g + (v & 7) >= N)
                            S[kb][v] = -INFINITY;
            }

            // ---- step-local max (log2 units) ----
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < HK / 32; ++kb)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    mx = fmaxf(mx, S[kb][v]);
            mx = fmaxf(mx, other_half(mx));
            const float m_loc = mx * c2;
            m_tile = fmaxf(m_tile, m_loc);

            // ---- online softmax ----
            const float m_new = fmaxf(m_run, m_loc);
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            const float neg = -m_new;
            float rsum = 0.f;
            bf16x8 P[HK / 16];
#pragma unroll
            for (int kb = 0; kb < HK / 32; ++kb)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kb][v], c2, neg));
                    rsum += pv;
                    P[kb * 2 + (v >> 3)][v & 7] = (__bf16)pv;
                }
            l_run = l_run * alpha + rsum;
            m_run = m_new;
            if (__ballot(alpha != 1.0f) != 0ull) {
#pragma unroll
                for (int eb = 0; eb < D / 32; ++eb)
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        O[eb][v] *= alpha;
            }

            // ---- O^T += V^T P^T ----
#pragma unroll
            for (int eb = 0; eb < D / 32; ++eb) {
                const int lr = eb * 32 + lq;
#pragma unroll
                for (int ks = 0; ks < HK / 16; ++ks) {
                    const u32x4 a = Vs[lr * (HK / 8) + ((2 * ks + g) ^ swz(lr))];
                    O[eb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), P[ks], O[eb],
                                                                    0, 0, 0);
                }
            }
        }

        // ---- QK-Skip vote once the whole tile has been seen ----
        if (vote && sub == SPT - 1) {
            const bool keep_lane = qvalid && !(m_tile - m_before < tau2);
            if (__ballot(keep_lane) != 0ull && lane == 0)
                atomicOr(&keep[kt >> 5], 1u << (kt & 31));
        }

        if (kt_n >= 0 && kt_n * BN + sub_n * HK < N)
            store_step(stage ^ 1);
        __syncthreads();
        if (sub_n == 0) {
            kt = kt_after;
            kt_after = kt >= 0 ? it.next() : -1;
        }
        sub = sub_n;
        stage ^= 1;
    }

    // ---- epilogue ----
    const float l_tot = l_run + other_half(l_run);
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    if (qvalid) {
        __bf16 *Ob = (__bf16 *)p.out + base + (int64_t)qi * rs;
#pragma unroll
        for (int eb = 0; eb < D / 32; ++eb) {
            bf16x8 lo, hi;
#pragma unroll
            for (int v = 0; v < 8; ++v) {
                lo[v] = (__bf16)(O[eb][v] * inv);
                hi[v] = (__bf16)(O[eb][v + 8] * inv);
            }
            u32x4 *dst = (u32x4 *)(Ob + eb * 32 + 16 * g);
            dst[0] = __builtin_bit_cast(u32x4, lo);
            dst[1] = __builtin_bit_cast(u32x4, hi);
        }
        if (p.lse && g == 0)
            p.lse[bh * N + qi] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
    }
    if (vote) {
        __syncthreads();
        if (tid < W) {
            uint32_t valid = 0xffffffffu;
            if (tid == W - 1 && (Tk & 31))
                valid = (1u << (Tk & 31)) - 1u;
            const uint32_t in = mrow ? mrow[tid] : 0u;
            p.mask_out[row * W + tid] = (in | ~keep[tid]) & valid;
        }
    }
}

template <int D, int BN>
hipError_t launch(const FwdParams &p, hipStream_t stream)
{
    const double LOG2E = 1.4426950408889634;
    const float c2 = (float)(p.scale * LOG2E);
    const float tau2 = isinf(p.tau) ? (float)p.tau : (float)(p.tau * LOG2E);
    hipLaunchKernelGGL((fwd_bf16_kernel<D, BN>), dim3((unsigned)p.rows), dim3(NT), 0, stream, p, c2, tau2);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdParams &p, hipStream_t stream)
{
    if (p.BM != BM || p.W > MAXW)
        return hipErrorInvalidValue;
    if (p.D == 128 && p.BN == 128)
        return launch<128, 128>(p, stream);
    if (p.D == 128 && p.BN == 64)
        return launch<128, 64>(p, stream);
    if (p.D == 64 && p.BN == 128)
        return launch<64, 128>(p, stream);
    if (p.D == 64 && p.BN == 64)
        return launch<64, 64>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace lite_attn
