// Internal interface between the C-ABI host layer (lite_attn_api.cpp) and the
// HIP kernel launchers.  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lite_attn {

// Everything a forward launch needs, already validated by the host layer.
struct FwdParams {
    const void *q, *k, *v;
    const uint32_t *mask_in;   // may be null: nothing skipped
    uint32_t *mask_out;        // may be null: no marking
    const int32_t *skiplist;   // may be null: walk mask_in
    void *out;
    float *lse;                // may be null
    int32_t B, N, H, D, BM, BN;
    int32_t Tq, Tk, W;
    int64_t rows;              // B*H*Tq
    double tau;                // natural-log units; -inf = never mark
    double scale;              // softmax scale (> 0)
};

hipError_t launch_fwd_bf16(const FwdParams &p, hipStream_t stream);
hipError_t launch_fwd_fp32(const FwdParams &p, hipStream_t stream);
hipError_t launch_build_skiplist(const uint32_t *mask, int32_t *skiplist, int64_t rows, int32_t Tk,
                                 hipStream_t stream);
hipError_t launch_reset_mask(uint32_t *mask, int64_t words, hipStream_t stream);

}  // namespace lite_attn
