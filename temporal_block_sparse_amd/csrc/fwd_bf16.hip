// Skip-masked tiled attention forward, bf16 in / bf16 out, fp32 accumulation,
// hand-written for gfx950 (CDNA4).
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
// Work decomposition
// * The work unit is a pair of adjacent q-tiles (128 queries each) of one
//   (batch, head), served by one workgroup of 8 wave64s: waves 0-3 the even
//   q-tile "A", waves 4-7 the odd q-tile "B"; each wave owns 32 queries.  Wave
//   w and wave w + 4 share a SIMD.
// * The workgroup walks the union of A's and B's live k-tiles in descending
//   order, in steps of 64 keys.  A wave computes only the steps its own q-tile
//   visits, so each q-tile sees exactly its own live tiles in its own order:
//   decisions and outputs are those of a one-q-tile kernel.  Both q-tiles
//   read the same K/V from LDS, so one copy of a step serves 256 queries.
// * Schedule: with schedule counters (two words in device memory), the grid
//   is one persistent workgroup per compute unit, and each takes the next
//   q-tile pair from an atomic ticket counter when it finishes one.  The
//   hardware hands workgroups to the XCDs round-robin and to the CUs of an XCD
//   in order; once the pairs' costs differ (sparse masks), that left whole
//   XCDs idle at the end of a launch and each CU idle between workgroups.
//   Tickets are taken in pair order, so all CUs still work on the q-tiles of
//   one or two heads at a time.  The last workgroup to finish resets the
//   counters, so they are zero again for the next launch without a memset.
//   Without counters, one workgroup per pair, in order.
// * Ping-pong: within a step, A's waves first run their MFMAs (PV of the
//   previous step, then QK^T of this one) and then the softmax of this step;
//   B's waves run the softmax of the previous step first and their MFMAs
//   after.  On every SIMD one wave then feeds the matrix core while the other
//   runs its exponentials on the vector ALU, instead of both waves competing
//   for one unit.  One barrier per step (the stage hand-over) keeps the
//   halves in step; a second one between the two halves' roles measured
//   slower.  The MFMA parts are software-pipelined by hand: the LDS reads run
//   four MFMAs ahead of their use.
//
// gfx950 layout choices
// * Both contractions are transposed, S^T = K Q^T and O^T = V^T P^T, on
//   v_mfma_f32_32x32x16_bf16.  The accumulator layout then gives every lane a
//   single query (lane % 32): its row max needs only in-register max plus one
//   v_permlane32_swap with the other half-wave, P^T feeds the second MFMA
//   straight from registers, and the O rescale uses the lane's own factor.
// * The online softmax is updated per 64-key step (exact in any grouping);
//   the QK-Skip test uses the maximum over all steps of the tile against the
//   running max taken before its first step.
// * K and V steps go global -> LDS by direct-to-LDS buffer loads
//   (buffer_load_dwordx4 ... lds): no staging registers, no LDS store
//   instructions.  Four LDS stages (128 KB at head_dim 128) and a prefetch
//   distance of two steps: while step u is computed (its K read by both
//   halves in step u, its V by both halves in step u + 1), step u + 1 is in
//   flight and A's waves issue step u + 2 among their QK^T MFMAs.  The four
//   stages' K share one LDS array and their V another, so each LDS read
//   address is a per-lane register computed once plus an immediate.  A
//   step's loads read one buffer resource (base, byte range) per tensor,
//   built in scalar registers once per step; each lane reaches its row and
//   chunk through a per-instruction offset register computed once, so a load
//   costs no vector instruction, and rows past the end of the sequence read
//   as zeros through the range check instead of being clamped.  The loads are
//   issued from asm blocks, which keeps the compiler from making LDS reads of
//   other stages wait for them; explicit vmcnt waits publish a stage at the
//   barrier that ends the step before its first use.
// * K rows sit in LDS with rows 4..7 and 8..11 of every 16 swapped, so the 8
//   scores a lane holds per 16-key MFMA step are 8 consecutive keys.  V stays
//   in natural (key x head-dim) layout and the PV A-operand (V^T) is read with
//   ds_read_b64_tr_b16, the LDS transpose read.
// * 16-byte chunks (K) and 64-byte segments (V) are XOR-swizzled per row,
//   measured free of bank conflicts for these read patterns.
// * The union walk is built once per workgroup, by all its threads, into LDS:
//   one 16-bit entry per visited tile (the k-tile and which q-tiles visit it),
//   from the mask words or from the Skip-Lists.  It is then read 64 entries
//   at a time, one per lane, and stepped with readlane: a single scalar
//   cursor, no memory round trip per tile, and few scalar registers (the
//   scalar budget is what the loop runs short of).
// * Workgroups run in plain order: at any time all XCDs work on the q-tiles of
//   one or two heads, whose K/V (39 MB per head at 75,600 tokens) then stay in
//   the 256 MB Infinity Cache, so L2 misses are served there, not by HBM.
// * The QK-Skip vote is one ballot per wave and tile; a wave that wants to
//   keep the tile sets its bit in its q-tile's LDS keep-vector with one atomic
//   OR.  Each mask row is written once, in the epilogue.
#include "lite_attn_internal.h"

#include <math.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

namespace lite_attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
#define LDS_VOID(p) ((__attribute__((address_space(3))) void *)(p))

constexpr int BM = 128;       // queries per q-tile
constexpr int NWAVES = 8;     // 4 per q-tile, 2 q-tiles per workgroup
constexpr int NT = 64 * NWAVES;
constexpr int HK = 64;        // keys per step
constexpr int MAXW = 128;     // mask words per row (Tk <= 4096)
constexpr int AHEAD = 4;      // MFMAs by which the LDS reads run ahead

// instruction classes of __builtin_amdgcn_sched_group_barrier
constexpr int SG_MFMA = 0x008, SG_VMEM = 0x010, SG_DS_READ = 0x100;

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

// LDS atomic OR whose completion is awaited in the same asm block.  Written
// out so that the compiler does not make it wait for the direct-to-LDS loads
// in flight, which never touch the keep-vector.
__device__ __forceinline__ void lds_or(uint32_t *p, uint32_t bits)
{
    const uint32_t a = (uint32_t)(size_t)LDS_VOID(p);
    asm volatile("ds_or_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" ::"v"(a), "v"(bits) : "memory");
}

// One 64-key step of the union walk (wave-uniform).
struct Step {
    int kt;    // k-tile, -1 = none
    int sub;   // 64-key step within the tile
    int fl;    // bit 0: q-tile A visits the tile, bit 1: q-tile B
    int key0;  // first key
};

// One 16-byte direct-to-LDS load: each lane's source, into LDS address
// l + 16 * lane (l is wave-uniform; it goes through M0).
// The source is a raw buffer resource (base, byte range) plus this lane's byte
// offset: an offset at or past the range reads zeros, which is how rows past
// the end of the sequence are handled.  Issued from an asm block: the compiler
// does not count these loads, so it never delays an LDS read for them; the
// kernel waits for them explicitly (vmcnt) before the barriers that publish a
// stage and before it exits.  The compiler's hazard recognizer does not look
// into the asm either: the leading s_nop is the one wait state a load to LDS
// needs after a scalar write of M0 (the rule the compiler applies to its own
// such loads).  The longer wait after a vector write of an SGPR the load
// reads (v_readlane, v_readfirstlane) is not provided: the code built here
// has no such write within that distance of any of these loads, which a test
// checks on the disassembled library over every path.
__device__ __forceinline__ void dma16(u32x4 rsrc, uint32_t off, uint32_t l)
{
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(off), "s"(rsrc), "{m0}"(l));
}

__device__ __forceinline__ const char *uniform_ptr(const char *x)
{
    // readfirstlane returns a signed int: widen through uint32_t, or an
    // address with bit 31 set would be sign-extended into the high word
    const uint64_t a = (uint64_t)x;
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
    return (const char *)(lo | (hi << 32));
}

// Raw buffer resource over [base, base + bytes): no stride, no swizzle,
// 32-bit data format (required for untyped loads).  The values are
// wave-uniform; readfirstlane makes that visible to the compiler, which must
// hold the resource in SGPRs.
__device__ __forceinline__ u32x4 buffer_rsrc(const char *base, uint32_t bytes)
{
    const uint64_t a = (uint64_t)base;
    u32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xFFFFu);
    r[2] = __builtin_amdgcn_readfirstlane(bytes);
    r[3] = 0x00020000u;
    return r;
}

// LDS layout of one 64-key step (a stage: CH chunks of K in kbuf, CH chunks
// of V in vbuf).  K and V arrive by direct-to-LDS loads
// (buffer_load_dwordx4 ... lds): each wave instruction writes 64 consecutive
// 16-byte chunks, lane i to chunk i, so the layout is any permutation of the
// step's chunks -- chosen per lane by the byte offset it loads.
// K: key x head-dim with the kperm row order; chunk c of LDS row r holds
//    head-dim chunk c ^ fk(r).  The MFMA A-operand reads (16-byte, 16 lanes
//    per LDS cycle over 32 consecutive rows) then hit 16 distinct 16-byte bank
//    groups: fk(r) = r mod 16 for 16-chunk rows, (r/2) mod 8 for 8-chunk rows.
// V: key x head-dim, natural row order; its 64-byte segments are XOR-swizzled
//    by the row so that the 4 rows touched by one ds_read_b64_tr_b16 (see the
//    PV step) land in 4 different bank groups.
template <int D>
struct Geo {
    static constexpr int CPR = D / 8;       // 16-byte chunks per row
    static constexpr int CH = HK * CPR;     // chunks of a K (or V) step
    static constexpr int IPA = CH / 64 / 4; // DMA instructions per A-wave, per tensor
    static constexpr int RPI = 256 / CPR;   // key rows covered by one instruction round of the 4 A-waves
    static_assert(CH % (64 * 4) == 0, "unsupported step geometry");
};

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

template <int D, int BN, bool LIST>
__global__ void __attribute__((amdgpu_flat_work_group_size(NT, NT), amdgpu_waves_per_eu(2, 2)))
fwd_bf16_kernel(FwdParams p, float c2, float tau2, int npairs)
{
    using G = Geo<D>;
    constexpr int SPT = BN / HK;  // steps per k-tile
    // The four pipeline stages: K of all four in one array, V in another, so
    // that every LDS read is a per-lane address register computed once plus
    // an immediate offset (stage, key block), which stays below 64 KB.
    __shared__ u32x4 kbuf[4 * G::CH];
    __shared__ u32x4 vbuf[4 * G::CH];
    __shared__ uint32_t keep[2][MAXW];
    __shared__ uint32_t wlive[2][MAXW];   // live tiles of A and B, one bit per k-tile
    __shared__ int32_t wcnt[MAXW];        // tiles of the union per mask word
    __shared__ uint16_t walk[MAXW * 32];  // the union walk: k-tile | A visits << 12 | B visits << 13
    __shared__ int32_t nwalk;
    __shared__ int s_pair;
    // Lane and wave constants, and the LDS and global byte offsets built from
    // them, are computed once for all pairs.
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
    const int half = wave >> 2;                                 // 0: q-tile A, 1: q-tile B
    const int wq = wave & 3;                                    // 32-query block in the q-tile
    const int g = lane >> 5, lq = lane & 31;
    const int rs2_0 = p.H * D * 2;  // token stride (bytes)

    // Direct-to-LDS slots of the A-waves, which load every step (fixed for the
    // kernel): DMA instruction i of A-wave wq fills LDS chunks
    // [(i*4 + wq)*64, +64) of the K (and V) step.  This lane's chunk comes from
    // key row kr0 + i*RPI (K) / vr0 + i*RPI (V) of the step -- the row pattern
    // of one instruction round repeats every RPI rows, swizzles included -- at
    // byte kc0 / vc0 within the row.
    int kr0, kc0, vr0, vc0;
    {
        const int P = wq * 64 + lane;
        const int lr = P / G::CPR, pos = P % G::CPR;
        kr0 = kperm(lr);
        kc0 = (pos ^ k_swz<D>(lr)) * 16;
        vr0 = lr;
        vc0 = (pos ^ v_swz<D>(lr)) * 16;
    }
    // LDS destinations (M0) of this wave's DMA slots, and each lane's byte
    // offsets within a step's rows of K and V, one per load instruction (held
    // in registers for the whole kernel, so that a load adds no vector work).
    const uint32_t m0_k = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)LDS_VOID(kbuf) + wq * 64 * 16);
    const uint32_t m0_v = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)LDS_VOID(vbuf) + wq * 64 * 16);
    uint32_t koff[G::IPA], voff[G::IPA];
#pragma unroll
    for (int i = 0; i < G::IPA; ++i) {
        koff[i] = (uint32_t)((kr0 + i * G::RPI) * rs2_0 + kc0);
        voff[i] = (uint32_t)((vr0 + i * G::RPI) * rs2_0 + vc0);
        asm volatile("" : "+v"(koff[i]), "+v"(voff[i]));
    }
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
    // Per-lane LDS read addresses, computed once: V^T reads of head-dim block
    // eb, and K reads of head-dim step ds; stage, key block and half offsets
    // are immediates of the reads.
    uint32_t vaddr[D / 32], kaddr[D / 16];
#pragma unroll
    for (int eb = 0; eb < D / 32; ++eb) {
        vaddr[eb] = (uint32_t)(size_t)LDS_VOID(vbuf) + vtr_row * G::CPR * 16 + vtr_col + ((eb ^ vtr_seg) * 64);
        asm volatile("" : "+v"(vaddr[eb]));
    }
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) {
        kaddr[ds] = (uint32_t)(size_t)LDS_VOID(kbuf) + (lq * G::CPR + ((2 * ds) ^ (g ^ k_swz<D>(lq)))) * 16;
        asm volatile("" : "+v"(kaddr[ds]));
    }

    int own = (int)blockIdx.x;  // without counters: this workgroup's pair, then none
    for (;;) {  // one q-tile pair per pass
        // The parameters are read through a pointer the compiler cannot prove
        // the same in every pass of this loop, so it loads them where they are
        // used instead of holding some forty of them in scalar registers for the
        // whole kernel (which spilled).  p is the first kernel argument: it sits
        // at offset 0 of the argument segment.
        typedef __attribute__((address_space(4))) const FwdParams cparams;
        cparams *pp = (cparams *)__builtin_amdgcn_kernarg_segment_ptr();
        asm volatile("" : "+s"(pp));
        cparams &prm = *pp;
        // the next q-tile pair: a ticket, or this workgroup's own pair once
        if (threadIdx.x == 0)
            s_pair = prm.sched ? (int)atomicAdd(prm.sched, 1u) : own;
        own = npairs;
        __syncthreads();
        const int pair = __builtin_amdgcn_readfirstlane(s_pair);
        if (pair >= npairs)
            break;
        const int Nq = prm.Nq, Nk = prm.Nk, H = prm.H, Tq = prm.Tq, Tk = prm.Tk, W = prm.W;
        const int Tq2 = (Tq + 1) >> 1;
        const int rs = H * D;                    // token stride (elements)
        const int rs2 = rs * 2;                  // token stride (bytes)
        const bool vote = prm.mask_out != nullptr;
        const bool ranges = prm.rg.any != 0;

        const int pq = (int)(pair % Tq2);
        const int64_t bh = pair / Tq2;
        const int h = (int)(bh % H), b = (int)(bh / H);
        const bool has_b = 2 * pq + 1 < Tq;
        const int64_t row_a = bh * Tq + 2 * pq;  // q-tile B is row_a + 1
        const int qt = 2 * pq + half;            // this wave's q-tile
        const int64_t qbase = (int64_t)b * prm.q_sb + (int64_t)h * D;
        const int64_t kvbase = (int64_t)b * prm.kv_sb + (int64_t)h * D;
        const __bf16 *Qb = (const __bf16 *)prm.q + qbase;
        const char *Kb = uniform_ptr((const char *)((const __bf16 *)prm.k + kvbase));
        const char *Vb = uniform_ptr((const char *)((const __bf16 *)prm.v + kvbase));

        // keep-vector: a clear bit marks the tile in mask_out.  Must-skip tiles are
        // never visited and never marked, so their bits start set.
        if (tid < 2 * W)
            keep[tid / W][tid % W] = ranges ? prm.rg.skip_bits[tid % W] : 0u;

        // this lane's query and its Q^T B-operand fragments
        const int qi = qt * BM + wq * 32 + lq;
        const bool qvalid = qt < Tq && qi < Nq;
        bf16x8 qf[D / 16];
#pragma unroll
        for (int ds = 0; ds < D / 16; ++ds) {
            u32x4 x = {0u, 0u, 0u, 0u};
            if (qvalid)
                x = *(const u32x4 *)(Qb + (int64_t)qi * rs + ds * 16 + 8 * g);
            qf[ds] = __builtin_bit_cast(bf16x8, x);
        }

        // The loads of one step into one LDS stage.  One buffer per tensor and
        // step starts at row key0 and spans the step's rows that exist; instruction
        // i covers rows [key0 + i*RPI, +RPI) through the lane's offsets koff[i] /
        // voff[i].  The range check applies to those offsets, so rows past the end
        // of the sequence read as zeros (their logits are set to -inf before use)
        // and no address leaves the tensors.  Building the two buffers is a few
        // scalar instructions per step; each load then needs only its M0.
        struct DmaPlan {
            u32x4 kr, vr;    // buffers over the step's rows that exist: min(Nk - key0, HK) rows
            uint32_t mk, mv; // LDS destinations of the stage's first instruction
        };
        auto plan_step = [&](int key0, int st) __attribute__((always_inline)) {
            DmaPlan d;
            const uint32_t bytes = (uint32_t)(min(Nk - key0, HK) * rs2);
            d.kr = buffer_rsrc(Kb + (int64_t)key0 * rs2, bytes);
            d.vr = buffer_rsrc(Vb + (int64_t)key0 * rs2, bytes);
            // this wave's bases, made opaque once per step so that the compiler
            // adds the stage and instruction offsets in the loop instead of
            // keeping one precomputed scalar per (stage, instruction) live
            uint32_t kb0 = m0_k, vb0 = m0_v;
            asm volatile("" : "+s"(kb0), "+s"(vb0));
            d.mk = kb0 + (uint32_t)(st * G::CH * 16);
            d.mv = vb0 + (uint32_t)(st * G::CH * 16);
            return d;
        };
        auto issue_dma = [&](const DmaPlan &d, int i) __attribute__((always_inline)) {
            dma16(d.kr, koff[i], d.mk + (uint32_t)(i * 4 * 64 * 16));
            dma16(d.vr, voff[i], d.mv + (uint32_t)(i * 4 * 64 * 16));
        };

        f32x16 O[D / 32];
#pragma unroll
        for (int eb = 0; eb < D / 32; ++eb)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                O[eb][v] = 0.f;
        float m_run = -INFINITY, l_run = 0.f;
        float m_before = -INFINITY, m_tile = -INFINITY;
        f32x16 S[HK / 32];       // raw logits of the step between QK^T and softmax
        bf16x8 P[HK / 16];       // weights of the step between softmax and PV
#pragma unroll
        for (int kb = 0; kb < HK / 32; ++kb)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                S[kb][v] = 0.f;
#pragma unroll
        for (int ks = 0; ks < HK / 16; ++ks)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                P[ks][j] = (__bf16)0.f;

        // ---- the union walk of the two q-tiles, built once into LDS ----
        // Live tiles per mask word: from the Skip-Lists (LIST) or from mask_in with
        // the token ranges applied (must-skip tiles out, must-do tiles in).  A
        // q-tile that does not exist has none.
        if (tid == 0)
            nwalk = 0;  // no mask words (no keys): an empty walk
        if (LIST) {
            if (tid < 2 * W)
                wlive[tid / W][tid % W] = 0u;
            __syncthreads();
#pragma unroll
            for (int hq = 0; hq < 2; ++hq) {
                if (hq == 1 && !has_b)
                    break;
                const int32_t *l = prm.skiplist + (row_a + hq) * (1 + Tk);
                const int c = min(max(l[0], 0), Tk);
                for (int i = tid; i < c; i += NT) {
                    const int kt = l[1 + i];
                    if (kt >= 0 && kt < Tk)
                        atomicOr(&wlive[hq][kt >> 5], 1u << (kt & 31));
                }
            }
        } else if (tid < 2 * W) {
            const int hq = tid / W, w = tid % W;
            uint32_t bits = 0u;
            if (hq == 0 || has_b) {
                bits = prm.mask_in ? ~prm.mask_in[(row_a + hq) * W + w] : 0xffffffffu;
                if (ranges)
                    bits = (bits & ~prm.rg.skip_bits[w]) | prm.rg.do_bits[w];
                if (w == W - 1 && (Tk & 31))
                    bits &= (1u << (Tk & 31)) - 1u;
            }
            wlive[hq][w] = bits;
        }
        __syncthreads();
        if (tid < W)
            wcnt[tid] = __builtin_popcount(wlive[0][tid] | wlive[1][tid]);
        __syncthreads();
        if (tid < W) {
            // descending order: the tiles of the words above this one come first
            int pos = 0;
            for (int w = W - 1; w > tid; --w)
                pos += wcnt[w];
            const uint32_t a = wlive[0][tid], bb = wlive[1][tid];
            uint32_t u = a | bb;
            while (u) {
                const int bit = 31 - __builtin_clz(u);
                u &= ~(1u << bit);
                walk[pos++] = (uint16_t)((tid * 32 + bit) | (((a >> bit) & 1u) << 12) | (((bb >> bit) & 1u) << 13));
            }
            if (tid == 0)
                nwalk = pos;
        }
        __syncthreads();

        // The walk is read 64 entries at a time, one per lane, and stepped with
        // readlane: one scalar cursor, no per-tile memory round trip.
        const int n_walk = __builtin_amdgcn_readfirstlane(nwalk);
        int g_idx = 0, g_sub = 0, g_kt = -1, g_fl = 0;
        uint32_t chunk = lane < n_walk ? walk[lane] : 0u;
        if (n_walk > 0) {
            const int e = __builtin_amdgcn_readfirstlane((int)chunk);
            g_kt = e & 0xfff;
            g_fl = e >> 12;
        }
        auto gen = [&]() __attribute__((always_inline)) {
            // wave-uniform by construction; readfirstlane lets the compiler keep
            // the step (and the load addresses built from it) in scalar registers
            Step s;
            s.kt = __builtin_amdgcn_readfirstlane(g_kt);
            s.sub = __builtin_amdgcn_readfirstlane(g_sub);
            s.fl = __builtin_amdgcn_readfirstlane(g_fl);
            s.key0 = s.kt * BN + s.sub * HK;
            if (g_kt >= 0 && ++g_sub == SPT) {
                g_sub = 0;
                if (++g_idx >= n_walk) {
                    g_kt = -1;
                } else {
                    if ((g_idx & 63) == 0)
                        chunk = g_idx + lane < n_walk ? walk[g_idx + lane] : 0u;
                    const int e = __builtin_amdgcn_readlane((int)chunk, g_idx & 63);
                    g_kt = e & 0xfff;
                    g_fl = e >> 12;
                }
            }
            return s;
        };
        auto mine = [&](const Step &s) __attribute__((always_inline)) { return s.kt >= 0 && ((s.fl >> half) & 1); };
        auto act = [&](const Step &s) __attribute__((always_inline)) { return mine(s) && s.key0 < Nk; };
        auto loadable = [&](const Step &s) __attribute__((always_inline)) { return s.kt >= 0 && s.key0 < Nk; };

        // ---- O^T += V^T P^T over one step (V in LDS stage vst) ----
        // MFMA order ks-major over the D/32 independent accumulators; each
        // transposed V read is issued AHEAD MFMAs before its use.
        auto pv_gemm = [&](int vs) __attribute__((always_inline)) {
            constexpr int NEB = D / 32, NM = NEB * (HK / 16);
            // MFMA m = ks*NEB + eb; its operand is read AHEAD MFMAs earlier
            s16x8 vf[NM];
            auto rd = [&](int m) __attribute__((always_inline)) {
                const int ks = m / NEB, eb = m % NEB;
                typedef __attribute__((address_space(3))) char lchar;
                lchar *va = (lchar *)(size_t)vaddr[eb] + vs * G::CH * 16 + 16 * ks * G::CPR * 16;
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)va);
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) s16x4 *)(va + 4 * G::CPR * 16));
                vf[m] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            };
#pragma unroll
            for (int m = 0; m < AHEAD; ++m)
                rd(m);
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                if (m + AHEAD < NM)
                    rd(m + AHEAD);
                O[m % NEB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vf[m]), P[m / NEB],
                                                                     O[m % NEB], 0, 0, 0);
            }
            __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 2 * AHEAD, 0);
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
                if (m + AHEAD < NM)
                    __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 2, 0);
            }
        };

        // ---- S^T = K Q^T over one step (K in LDS stage kst), raw logits ----
        // MFMA order ds-major over the two 32-key blocks; one K read per MFMA,
        // issued AHEAD MFMAs before its use.  With WD the loads of the next step
        // (`dma`) go out one per two MFMAs.
        auto s_gemm = [&](int ks_, const DmaPlan &dma, auto with_dma) __attribute__((always_inline)) {
            constexpr bool WD = decltype(with_dma)::value;
            constexpr int NDS = D / 16, NM = (HK / 32) * NDS;
            static_assert(NM == 4 * G::IPA, "one load pair per four MFMAs");
            // Row kb*32 + lq, chunk (2*ds + g) ^ k_swz(row) = 2*ds ^ kc: the swizzle
            // depends on the row only through lq (kaddr).
            // MFMA m = ds*2 + kb; its K fragment is read AHEAD MFMAs earlier.
            // The first MFMA of each accumulator takes a zero C operand (an inline
            // constant), so S needs no clearing moves.
            u32x4 kf[NM];
            auto rd = [&](int m) __attribute__((always_inline)) {
                const int ds = m >> 1, kb = m & 1;
                typedef __attribute__((address_space(3))) u32x4 lvec;
                kf[m] = *(lvec *)((__attribute__((address_space(3))) char *)(size_t)kaddr[ds] +
                                  (ks_ * G::CH + kb * 32 * G::CPR) * 16);
            };
#pragma unroll
            for (int m = 0; m < AHEAD; ++m)
                rd(m);
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                if (m + AHEAD < NM)
                    rd(m + AHEAD);
                const f32x16 zero = {};
                S[m & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf[m]), qf[m >> 1],
                                                                   m < 2 ? zero : S[m & 1], 0, 0, 0);
                // one (K, V) pair per four MFMAs: NM = 4 * IPA for both head dims
                if (WD && (m & 3) == 3)
                    issue_dma(dma, m >> 2);
            }
            __builtin_amdgcn_sched_group_barrier(SG_DS_READ, AHEAD, 0);
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
                if (m + AHEAD < NM)
                    __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
                if (WD && (m & 1))
                    __builtin_amdgcn_sched_group_barrier(SG_VMEM, 1, 0);
            }
        };

        // VALU part of this wave's q-tile: online softmax of step s (logits in S),
        // weights into P, then the QK-Skip vote once the whole tile has been seen.
        auto valu_part = [&](const Step &s) __attribute__((always_inline)) {
            if (mine(s) && s.sub == 0) {
                m_before = m_run;
                m_tile = -INFINITY;
            }
            if (act(s)) {
                // keys past the end of the sequence do not exist
                if (s.key0 + HK > Nk) {
#pragma unroll
                    for (int kb = 0; kb < HK / 32; ++kb)
#pragma unroll
                        for (int v = 0; v < 16; ++v)
                            if (s.key0 + kb * 32 + 16 * (v >> 3) + 8 * g + (v & 7) >= Nk)
                                S[kb][v] = -INFINITY;
                }
                // step-local max (log2 units)
                float mx = -INFINITY;
#pragma unroll
                for (int kb = 0; kb < HK / 32; ++kb)
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        mx = fmaxf(mx, S[kb][v]);
                mx = fmaxf(mx, other_half(mx));
                const float m_loc = mx * c2;
                m_tile = fmaxf(m_tile, m_loc);
                // Exponents are taken against the exact running max, so the largest
                // weight of a row is exactly 1 (exact in bf16); O and l are rescaled
                // only when some query's max moved (wave-uniform test).
                const float m_new = fmaxf(m_run, m_loc);
                const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
                const float neg = -m_new;
                float rsum = 0.f;
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
            }
            if (vote && mine(s) && s.sub == SPT - 1) {
                // a must-do tile is never marked
                const bool must_do = ranges && ((prm.rg.do_bits[s.kt >> 5] >> (s.kt & 31)) & 1u);
                const bool keep_lane = must_do || (qvalid && !(m_tile - m_before < tau2));
                if (__ballot(keep_lane) != 0ull && lane == 0)
                    lds_or(&keep[half][s.kt >> 5], 1u << (s.kt & 31));
            }
        };

        // Every A-wave issues exactly 2*IPA loads per step (real, or empty-range
        // loads that write zeros to a stage nobody reads and touch no memory), so
        // that "all but the last 2*IPA loads done" means "the step before the last
        // one has landed".
        constexpr int VM_KEEP = 2 * G::IPA;
        constexpr int WAIT_KEEP = (VM_KEEP & 15) | (7 << 4) | (15 << 8) | ((VM_KEEP >> 4) << 14);  // vmcnt only
        constexpr int WAIT_ALL = (7 << 4) | (15 << 8);  // vmcnt(0) only
        auto load_step = [&](const Step &s, int dst) __attribute__((always_inline)) {
            if (Nk <= 0)
                return;  // no key rows at all
            const DmaPlan d = plan_step(loadable(s) ? s.key0 : Nk, dst);
#pragma unroll
            for (int i = 0; i < G::IPA; ++i)
                issue_dma(d, i);
        };

        Step sp = {-1, 0, 0, 0};  // step u - 1
        Step sc = gen();          // step u
        Step sn = gen();          // step u + 1
        Step sn2 = gen();         // step u + 2
        if (half == 0) {
            load_step(sc, 0);
            load_step(sn, 1);
            __builtin_amdgcn_s_waitcnt(WAIT_KEEP);  // step 0 has landed
        }
        __syncthreads();

        // Step u, with its K in stage ST = u mod 4, step u - 1's V in stage
        // (ST + 3) mod 4, step u + 1 in flight to stage (ST + 1) mod 4 and step
        // u + 2 loading into stage (ST + 2) mod 4.  Each half runs its own copy of
        // the loop, with its two parts in its own order, so that neither path
        // carries the other's registers; both pass the same barrier once per step.
        // Returns false once both the step and the one before it are past the end.
        auto run = [&](auto half_tag) __attribute__((always_inline)) {
            constexpr int HF = decltype(half_tag)::value;
            // MFMA part: PV of step u - 1, then QK^T of step u; the A-waves load
            // step u + 2 meanwhile (spread over the QK^T MFMAs).
            auto mfma_part = [&](int vst, int kst, int lst) __attribute__((always_inline)) {
                if (act(sp))
                    pv_gemm(vst);
                if (HF == 0) {
                    if (act(sc)) {
                        s_gemm(kst, plan_step(loadable(sn2) ? sn2.key0 : Nk, lst), std::true_type{});
                    } else {
                        load_step(sn2, lst);
                    }
                } else if (act(sc)) {
                    s_gemm(kst, plan_step(0, lst), std::false_type{});
                }
            };
            auto iter = [&](auto stage_tag) __attribute__((always_inline)) -> bool {
                constexpr int ST = decltype(stage_tag)::value;
                if (sc.kt < 0 && sp.kt < 0)
                    return false;
                constexpr int kst = ST, lst = (ST + 2) & 3, vst = (ST + 3) & 3;
                // A: MFMAs, then softmax; B: softmax, then MFMAs.  No barrier in
                // between: the opposite orders alone keep one wave of each SIMD on
                // the matrix core while the other is on the vector ALU.
                if (HF == 0)
                    mfma_part(vst, kst, lst);
                else
                    valu_part(sp);
                if (HF == 0)
                    valu_part(sc);
                else
                    mfma_part(vst, kst, lst);
                // step u + 1 has landed (step u + 2 may still be in flight)
                __builtin_amdgcn_s_waitcnt(WAIT_KEEP);
                __builtin_amdgcn_s_barrier();
                asm volatile("" ::: "memory");
                sp = sc;
                sc = sn;
                sn = sn2;
                sn2 = gen();
                return true;
            };
            for (;;) {
                if (!iter(std::integral_constant<int, 0>{}))
                    break;
                if (!iter(std::integral_constant<int, 1>{}))
                    break;
                if (!iter(std::integral_constant<int, 2>{}))
                    break;
                if (!iter(std::integral_constant<int, 3>{}))
                    break;
            }
        };
        if (half == 0)
            run(std::integral_constant<int, 0>{});
        else
            run(std::integral_constant<int, 1>{});
        __builtin_amdgcn_s_waitcnt(WAIT_ALL);
        __syncthreads();  // every load landed before the next pair reuses the stages (or the LDS is released)

        // ---- epilogue ----
        const float l_tot = l_run + other_half(l_run);
        const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
        if (qvalid) {
            __bf16 *Ob = (__bf16 *)prm.out + (int64_t)b * prm.o_sb + (int64_t)h * D + (int64_t)qi * rs;
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
            if (prm.lse && g == 0)
                prm.lse[bh * Nq + qi] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
        }
        if (vote) {
            __syncthreads();
            if (tid < 2 * W) {
                const int hh = tid / W, w = tid % W;
                if (hh == 0 || has_b) {
                    const int64_t r = row_a + hh;
                    uint32_t valid = 0xffffffffu;
                    if (w == W - 1 && (Tk & 31))
                        valid = (1u << (Tk & 31)) - 1u;
                    const uint32_t in = prm.mask_in ? prm.mask_in[r * W + w] : 0u;
                    prm.mask_out[r * W + w] = (in | ~keep[hh][w]) & valid;
                }
            }
        }
    }  // pairs
    // Every workgroup has drawn its last ticket before it counts itself out
    // here, so the last one out may clear both counters for the next launch.
    if (p.sched && threadIdx.x == 0) {
        __threadfence();
        if (atomicAdd(p.sched + 1, 1u) == gridDim.x - 1) {
            atomicExch(p.sched, 0u);
            atomicExch(p.sched + 1, 0u);
        }
    }
}

template <int D, int BN>
hipError_t launch(const FwdParams &p, hipStream_t stream)
{
    const double LOG2E = 1.4426950408889634;
    const float c2 = (float)(p.scale * LOG2E);
    const float tau2 = isinf(p.tau) ? (float)p.tau : (float)(p.tau * LOG2E);
    const int64_t pairs = (int64_t)p.B * p.H * ((p.Tq + 1) / 2);
    if (pairs == 0)
        return hipSuccess;
    // with counters: one workgroup per compute unit (the LDS holds one), at
    // most one per pair
    int64_t grid = pairs;
    if (p.sched) {
        int dev = 0, ncu = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e == hipSuccess)
            e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess)
            return e;
        grid = std::min<int64_t>(pairs, std::max(ncu, 1));
    }
    if (p.skiplist)
        hipLaunchKernelGGL((fwd_bf16_kernel<D, BN, true>), dim3((unsigned)grid), dim3(NT), 0, stream, p, c2, tau2,
                           (int)pairs);
    else
        hipLaunchKernelGGL((fwd_bf16_kernel<D, BN, false>), dim3((unsigned)grid), dim3(NT), 0, stream, p, c2, tau2,
                           (int)pairs);
    return hipGetLastError();
}

}  // namespace

// Schedule counters for callers that cannot allocate (lite_attn_fwd_noalloc):
// one static array per GPU, held until the process ends.  Host code never
// uses its name as an address: each device's address comes from
// hipGetSymbolAddress, called once per device with that device current.
static __device__ __align__(256) uint32_t scratch[NOALLOC_SCHED_WORDS];

hipError_t noalloc_sched(uint32_t **ptr)
{
    constexpr int MAX_DEVICES = 64;
    static std::once_flag once[MAX_DEVICES];
    static uint32_t *addr[MAX_DEVICES];
    static hipError_t err[MAX_DEVICES];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= MAX_DEVICES)
        return hipErrorInvalidDevice;
    std::call_once(once[dev], [dev] {
        void *a = nullptr;
        err[dev] = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
        addr[dev] = static_cast<uint32_t *>(a);
    });
    if (err[dev] != hipSuccess)
        return err[dev];
    *ptr = addr[dev];
    return hipSuccess;
}

hipError_t launch_fwd_bf16(const FwdParams &p, hipStream_t stream)
{
    if (p.BM != BM || p.W > MAXW)
        return hipErrorInvalidValue;
    // byte offsets within a 64-key step are 32-bit
    if ((int64_t)p.H * p.D * 2 * HK > INT32_MAX)
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
