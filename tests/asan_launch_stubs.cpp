// Stand-ins for the kernel launchers, so the library's host layer (argument
// validation in lite_attn_api.cpp) can be built alone under AddressSanitizer
// and driven by the CPU ABI tests.  Every launch reports an error.
#include "lite_attn_internal.h"
namespace lite_attn {
hipError_t launch_fwd_bf16(const FwdParams &, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_fwd_fp32(const FwdParams &, hipStream_t) { return hipErrorInvalidValue; }
hipError_t noalloc_sched(uint32_t **) { return hipErrorInvalidValue; }
hipError_t launch_build_skiplist(const uint32_t *, int32_t *, int64_t, int32_t, const TileRanges &, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_reset_mask(uint32_t *, int64_t, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_merge(const MergeParams &, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_error_sums(const ErrParams &, hipStream_t) { return hipErrorInvalidValue; }
}
