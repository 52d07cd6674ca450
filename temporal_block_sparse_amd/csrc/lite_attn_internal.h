// Internal interface between the C-ABI host layer (lite_attn_api.cpp) and the
// HIP kernel launchers.  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lite_attn {

constexpr int MAX_TILE_WORDS = 128;  // mask words per row: Tk <= 4096
constexpr int MAX_MERGE_PARTS = 8;

// Must-do / must-skip key ranges reduced to one bit per k-tile (the same for
// every row).  `any` = 0 when no range was given.
struct TileRanges {
    uint32_t do_bits[MAX_TILE_WORDS];    // tile holds a must-do key: always visited, never marked
    uint32_t skip_bits[MAX_TILE_WORDS];  // every key of the tile is must-skip (and it is not must-do)
    int32_t any;
};

// Everything a forward launch needs, already validated by the host layer.
struct FwdParams {
    const void *q, *k, *v;
    const uint32_t *mask_in;   // may be null: nothing skipped
    uint32_t *mask_out;        // may be null: no marking
    const int32_t *skiplist;   // may be null: walk mask_in
    void *out;
    float *lse;                // may be null
    int32_t B, Nq, Nk, H, D, BM, BN;
    int32_t Tq, Tk, W;
    int64_t q_sb, kv_sb, o_sb;  // elements between batch entries of q, of k/v and of out
    int64_t rows;              // B*H*Tq
    double tau;                // natural-log units; -inf = never mark
    double scale;              // softmax scale (> 0)
    TileRanges rg;
    uint32_t *sched;           // bf16 path: 2 schedule counters (zero at rest), or null: one workgroup per pair
};

struct MergeParams {
    const void *outs[MAX_MERGE_PARTS];
    const float *lses[MAX_MERGE_PARTS];
    void *out;
    float *lse;                // may be null
    int32_t nparts, B, N, H, D, dtype;
    int64_t q_sb, o_sb;        // batch strides of the parts and of out
};

struct ErrParams {
    const void *a, *b;
    double *sums;
    int32_t B, N, H, D, dtype;
    int64_t a_sb, b_sb;        // batch strides of a and b
};

hipError_t launch_fwd_bf16(const FwdParams &p, hipStream_t stream);
// The library's own schedule counters on the current device (lite_attn_fwd_noalloc).
constexpr int NOALLOC_SCHED_WORDS = 2;
hipError_t noalloc_sched(uint32_t **ptr);
hipError_t launch_fwd_fp32(const FwdParams &p, hipStream_t stream);
hipError_t launch_build_skiplist(const uint32_t *mask, int32_t *skiplist, int64_t rows, int32_t Tk,
                                 const TileRanges &rg, hipStream_t stream);
hipError_t launch_reset_mask(uint32_t *mask, int64_t words, hipStream_t stream);
hipError_t launch_merge(const MergeParams &p, hipStream_t stream);
hipError_t launch_error_sums(const ErrParams &p, hipStream_t stream);

}  // namespace lite_attn
