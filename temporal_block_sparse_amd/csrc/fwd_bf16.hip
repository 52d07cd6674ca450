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
// * K and V steps go global -> LDS by direct-to-LDS loads
//   (global_load_lds_dwordx4): no staging registers, no LDS store
//   instructions.  Two steps are double-buffered (64 KB at head_dim 128), so
//   two workgroups fit on a CU and each SIMD interleaves two waves: one
//   wave's softmax (VALU, v_exp) runs under the other's MFMAs.  The next
//   step's loads are issued before the current step's MFMAs; one barrier per
//   step.
// * K rows sit in LDS with rows 4..7 and 8..11 of every 16 swapped, so the 8
//   scores a lane holds per 16-key MFMA step are 8 consecutive keys.  V stays
//   in natural (key x head-dim) layout and the PV A-operand (V^T) is read with
//   ds_read_b64_tr_b16, the LDS transpose read.
// * 16-byte chunks (K) and 64-byte segments (V) are XOR-swizzled per row,
//   measured free of bank conflicts for these read patterns.
// * Workgroups run in plain row order: at any time all XCDs work on the q-tiles
//   of one or two heads, whose K/V (39 MB per head at 75,600 tokens) then stay
//   in the 256 MB Infinity Cache, so L2 misses are served there, not by HBM.
// * The QK-Skip vote is one ballot per wave and tile; a wave that wants to
//   keep the tile sets its bit in an LDS keep-vector with one atomic OR.  The
//   mask row is written once, in the epilogue.
#include "lite_attn_internal.h"

#include <math.h>

namespace lite_attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
#define LDS_S16X4(p) ((__attribute__((address_space(3))) s16x4 *)(p))
#define LDS_VOID(p) ((__attribute__((address_space(3))) void *)(p))

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

// LDS layout of one 64-key step.  K and V arrive by direct-to-LDS loads
// (global_load_lds_dwordx4): each wave instruction writes 64 consecutive
// 16-byte chunks, lane i to chunk i, so the layout is any permutation of the
// step's chunks -- chosen per lane by the global address it loads.
// K: key x head-dim with the kperm row order; chunk c of LDS row r holds
//    head-dim chunk c ^ fk(r).  The MFMA A-operand reads (16-byte, 16 lanes
//    per LDS cycle over 32 consecutive rows) then hit 16 distinct 16-byte bank
//    groups: fk(r) = r mod 16 for 16-chunk rows, (r/2) mod 8 for 8-chunk rows.
// V: key x head-dim, natural row order; its 64-byte segments are XOR-swizzled
//    by the row so that the 4 rows touched by one ds_read_b64_tr_b16 (see the
//    PV step) land in 4 different bank groups.
template <int D>
struct Geo {
    static constexpr int CPR = D / 8;            // 16-byte chunks per row
    static constexpr int CH = HK * CPR;          // chunks of a K (or V) step
    static constexpr int STAGE = 2 * CH;         // K then V, in chunks
    static constexpr int IPW = CH / 64 / NWAVES; // DMA instructions per wave, per tensor
    static_assert(CH % (64 * NWAVES) == 0, "unsupported step geometry");
};

// One 16-byte direct-to-LDS load: each lane's `src`, into `dst` + 16 * lane
// (dst is wave-uniform).
__device__ __forceinline__ void dma16(const char *src, char *dst)
{
    __builtin_amdgcn_global_load_lds((const void *)src, LDS_VOID(dst), 16, 0, 0);
}

template <int D>
__device__ __forceinline__ int k_swz(int r)
{
    return D == 128 ? (r & 15) : ((r >> 1) & 7);
}

// chunk offset (within a row) that the 64-byte-segment swizzle of row r applies
template <int D>
__device__ __forceinline__ int v_swz(int r)
{
    return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
}

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
    const int64_t row = blockIdx.x;
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

    // Direct-to-LDS slots (fixed for the kernel): DMA instruction i of this wave
    // fills LDS chunks [(i*NWAVES + wave)*64, +64) of the K (and V) step; this
    // lane's chunk comes from key row kr[i], head-dim chunk kc[i] (K) / vc[i] (V).
    int kr[G::IPW], kgo[G::IPW], vr[G::IPW], vgo[G::IPW];
#pragma unroll
    for (int i = 0; i < G::IPW; ++i) {
        const int P = (i * NWAVES + wave) * 64 + lane;
        const int lr = P / G::CPR, pos = P % G::CPR;
        kr[i] = kperm(lr);
        kgo[i] = kr[i] * rs * 2 + (pos ^ k_swz<D>(lr)) * 16;
        vr[i] = lr;
        vgo[i] = lr * rs * 2 + (pos ^ v_swz<D>(lr)) * 16;
    }
    // Issue the DMA of one 64-key step into LDS stage `stage`.  Keys past the
    // end of the sequence are clamped to the last key: their logits are set
    // to -inf before use, so their K and V rows never contribute.
    auto load_step = [&](int key0, int stage) {
        char *kdst = (char *)(smem + stage * G::STAGE) + wave * 64 * 16;
        char *vdst = kdst + G::CH * 16;
        const char *kb = Kb + (int64_t)key0 * rs * 2;
        const char *vb = Vb + (int64_t)key0 * rs * 2;
        if (key0 + HK <= N) {
#pragma unroll
            for (int i = 0; i < G::IPW; ++i) {
                dma16(kb + kgo[i], kdst + i * NWAVES * 64 * 16);
                dma16(vb + vgo[i], vdst + i * NWAVES * 64 * 16);
            }
        } else {
            const int64_t back = (int64_t)rs * 2;
#pragma unroll
            for (int i = 0; i < G::IPW; ++i) {
                const int ko = key0 + kr[i] < N ? kgo[i] : kgo[i] - (int)((key0 + kr[i] - (N - 1)) * back);
                const int vo = key0 + vr[i] < N ? vgo[i] : vgo[i] - (int)((key0 + vr[i] - (N - 1)) * back);
                dma16(kb + ko, kdst + i * NWAVES * 64 * 16);
                dma16(vb + vo, vdst + i * NWAVES * 64 * 16);
            }
        }
    };

    // This lane's slot as a source of the transposed V read: key row 8g + a of
    // the 16-key group, 4 head-dim entries starting at sigma(16*(lane/16 % 2) + 4b),
    // where lane % 16 = 4a + b.  The lane that receives column i of a 32-entry
    // block then holds head-dim entry sigma(i) = 16*((i>>2)&1) + 4*(i>>3) + (i&3),
    // which makes the O^T accumulator layout give every lane 16 consecutive
    // head-dim entries (16*g + v, v = 0..15).
    // Rows 8g + a + 16ks + 4h keep (row & 3) = a and ((row >> 1) & 1) = a >> 1,
    // so the segment swizzle of the row depends only on this lane's a.
    const int ts = lane & 15, tb = ts & 3;
    const int vtr_row = 8 * g + (ts >> 2);
    const int vtr_col = (16 * (tb & 1) + 8 * ((lane >> 4) & 1) + 4 * (tb >> 1)) * 2;  // bytes in a 64-B segment
    const int vtr_seg = v_swz<D>(vtr_row) / 4;                                       // segment XOR

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
    if (kt >= 0)
        load_step(kt * BN, 0);
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
            load_step(kt_n * BN + sub_n * HK, stage ^ 1);

        const u32x4 *Ks = smem + stage * G::STAGE;
        const char *Vs = (const char *)(Ks + G::CH);
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
                const int kr0 = kb * 32 + lq;
                const u32x4 *ka = Ks + kr0 * G::CPR;
                const int ksw = k_swz<D>(kr0);
#pragma unroll
                for (int ds = 0; ds < D / 16; ++ds) {
                    const u32x4 a = ka[(2 * ds + g) ^ ksw];
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
            // Exponents are taken against the exact running max, so the largest
            // weight of a row is exactly 1 (exact in bf16); O and l are rescaled
            // only when some query's max moved (wave-uniform test).
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
#pragma unroll
                for (int ks = 0; ks < HK / 16; ++ks) {
                    const char *va = Vs + (vtr_row + 16 * ks) * G::CPR * 16 + ((eb ^ vtr_seg) * 64) + vtr_col;
                    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_S16X4(va));
                    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_S16X4(va + 4 * G::CPR * 16));
                    const s16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
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
