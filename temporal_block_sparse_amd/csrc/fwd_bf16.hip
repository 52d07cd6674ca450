// Skip-masked tiled attention forward, bf16 in / bf16 out, fp32 accumulation,
// hand-written for gfx950 (CDNA4): one workgroup of 4 wave64s per
// (batch, head, q-tile of 128 queries); each wave owns 32 queries.
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
// * K tile rows are stored in LDS with rows 4..7 and 8..11 of every 16 swapped,
//   so that the 8 scores a lane holds per 16-key step are 8 consecutive keys;
//   V is stored transposed (V^T, e-major) so the PV A-operand is one 16-byte
//   LDS read.  Its rows are permuted so a lane's O^T values are 16
//   consecutive head-dim entries (two 16-byte global stores).
// * 16-byte chunks are XOR-swizzled per row against LDS bank conflicts.
// * K/V tiles are double-buffered in LDS; the next live tile's global loads
//   are issued before the current tile's MFMAs and land in the other buffer
//   afterwards; one barrier per tile.
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

constexpr int BM = 128;       // queries per workgroup (one q-tile)
constexpr int NWAVES = 4;
constexpr int NT = 64 * NWAVES;
constexpr int MAXW = 128;     // mask words per row (Tk <= 4096)

// LDS row r of a K tile holds key kperm(r): rows 4..7 and 8..11 of each 16 swapped.
__device__ __forceinline__ int kperm(int r)
{
    const int m = r & 15;
    return (m >= 4 && m < 8) ? r + 4 : ((m >= 8 && m < 12) ? r - 4 : r);
}

// LDS row of head-dim entry e in a V^T tile: within each 32-block,
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

template <int D, int BN>
struct Tile {
    static constexpr int KCHUNKS = BN * D / 8;          // 16-byte chunks of a K tile
    static constexpr int VCHUNKS = BN * D / 8;          // of a V^T tile
    static constexpr int STAGE = KCHUNKS + VCHUNKS;
    static constexpr int KPT = KCHUNKS / NT;            // K chunks per thread
    static constexpr int VBLK = BN * D / 64;            // 8x8 V blocks
    static constexpr int WAVES_PER_EU = (BN * D <= 64 * 64) ? 2 : 1;
    static_assert(KCHUNKS % NT == 0, "tile too small");
    static_assert(VBLK <= NT, "tile too large");
};

template <int D, int BN>
__global__ void __attribute__((amdgpu_flat_work_group_size(NT, NT),
                               amdgpu_waves_per_eu(Tile<D, BN>::WAVES_PER_EU, Tile<D, BN>::WAVES_PER_EU)))
fwd_bf16_kernel(FwdParams p, float c2, float tau2)
{
    using T = Tile<D, BN>;
    __shared__ u32x4 smem[2 * T::STAGE];
    __shared__ uint32_t keep[MAXW];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, lq = lane & 31;
    const int N = p.N, H = p.H, Tq = p.Tq, Tk = p.Tk, W = p.W;
    const int64_t row = xcd_remap(blockIdx.x, p.rows);
    const int qt = (int)(row % Tq);
    const int64_t bh = row / Tq;
    const int h = (int)(bh % H), b = (int)(bh / H);
    const int64_t rs = (int64_t)H * D;  // token stride (elements)
    const int64_t base = (int64_t)b * N * rs + (int64_t)h * D;
    const __bf16 *Qb = (const __bf16 *)p.q + base;
    const __bf16 *Kb = (const __bf16 *)p.k + base;
    const __bf16 *Vb = (const __bf16 *)p.v + base;
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

    u32x4 kreg[T::KPT];
    u32x4 vreg[8];
    auto load_tile = [&](int kt) {
        const int key0 = kt * BN;
#pragma unroll
        for (int i = 0; i < T::KPT; ++i) {
            const int C = tid + i * NT, r = C / (D / 8), c = C % (D / 8);
            const int key = key0 + r;
            u32x4 x = {0u, 0u, 0u, 0u};
            if (key < N)
                x = *(const u32x4 *)(Kb + (int64_t)key * rs + c * 8);
            kreg[i] = x;
        }
        if (tid < T::VBLK) {
            const int c = tid % (D / 8), kg = tid / (D / 8);
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const int key = key0 + kg * 8 + r;
                u32x4 x = {0u, 0u, 0u, 0u};
                if (key < N)
                    x = *(const u32x4 *)(Vb + (int64_t)key * rs + c * 8);
                vreg[r] = x;
            }
        }
    };
    auto store_tile = [&](int stage) {
        u32x4 *Ks = smem + stage * T::STAGE;
        u32x4 *Vs = Ks + T::KCHUNKS;
#pragma unroll
        for (int i = 0; i < T::KPT; ++i) {
            const int C = tid + i * NT, r = C / (D / 8), c = C % (D / 8);
            const int lr = kperm(r);
            Ks[lr * (D / 8) + (c ^ swz(lr))] = kreg[i];
        }
        if (tid < T::VBLK) {
            const int c = tid % (D / 8), kg = tid / (D / 8);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                // column j of the 8x8 block (8 keys of head-dim entry c*8 + j)
                u32x4 o;
#pragma unroll
                for (int pr = 0; pr < 4; ++pr) {
                    const uint32_t lo = vreg[2 * pr][j >> 1], hi = vreg[2 * pr + 1][j >> 1];
                    o[pr] = (j & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
                }
                const int lr = vt_row(c * 8 + j);
                Vs[lr * (BN / 8) + (kg ^ swz(lr))] = o;
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

    LiveTiles it;
    it.init(mrow, p.skiplist ? p.skiplist + row * (1 + Tk) : nullptr, Tk);
    int kt = it.next();
    if (kt >= 0) {
        load_tile(kt);
        store_tile(0);
    }
    __syncthreads();
    int kt_next = kt >= 0 ? it.next() : -1;
    int stage = 0;

    while (kt >= 0) {
        if (kt_next >= 0)
            load_tile(kt_next);

        const u32x4 *Ks = smem + stage * T::STAGE;
        const u32x4 *Vs = Ks + T::KCHUNKS;

        // ---- S^T = K Q^T (raw logits, fp32) ----
        f32x16 S[BN / 32];
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb) {
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
        const int key0 = kt * BN;
        if (key0 + BN > N) {
#pragma unroll
            for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    if (key0 + kb * 32 + 16 * (v >> 3) + 8 * g + (v & 7) >= N)
                        S[kb][v] = -INFINITY;
        }

        // ---- tile-local max (log2 units), QK-Skip vote ----
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                mx = fmaxf(mx, S[kb][v]);
        mx = fmaxf(mx, other_half(mx));
        const float m_loc = mx * c2;
        if (vote) {
            const bool keep_lane = qvalid && !(m_loc - m_run < tau2);
            if (__ballot(keep_lane) != 0ull && lane == 0)
                atomicOr(&keep[kt >> 5], 1u << (kt & 31));
        }

        // ---- online softmax ----
        const float m_new = fmaxf(m_run, m_loc);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        const float neg = -m_new;
        float rsum = 0.f;
        bf16x8 P[BN / 16];
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb)
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
            for (int ks = 0; ks < BN / 16; ++ks) {
                const u32x4 a = Vs[lr * (BN / 8) + ((2 * ks + g) ^ swz(lr))];
                O[eb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), P[ks], O[eb], 0, 0,
                                                                0);
            }
        }

        if (kt_next >= 0)
            store_tile(stage ^ 1);
        __syncthreads();
        kt = kt_next;
        kt_next = kt >= 0 ? it.next() : -1;
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
