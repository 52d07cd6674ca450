// Skip-Mask maintenance kernels: reset, and compaction into the Skip-List.
//
// The Skip-Mask is the persistent per-layer state of LiteAttention (README:
// "QK-Skip Algorithm"; the Python API's reset of the skip state).  The
// Skip-List is its compacted form for high sparsity (skill page "Lite
// Attention Temporal Sparse", "Architecture Overview": bitmask, or Skip-List
// for high sparsity): per row, the count of live k-tiles followed by the live
// k-tiles in the order the forward visits them (descending).  With token
// ranges (README Python API: must_do_list / must_skip_list) a must-do tile is
// live whatever the mask says and a must-skip tile never is.
#include "lite_attn_internal.h"

namespace lite_attn {
namespace {

// Plain fill kernel (not hipMemsetAsync), so a captured HIP graph replays it
// like any other kernel node.
__global__ void __launch_bounds__(256) reset_kernel(uint32_t *mask, int64_t words)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t j = i; j < words; j += stride)
        mask[j] = 0u;
}

// One wave64 per mask row.  Each pass takes 64 k-tiles from the top down:
// lane i looks at tile base - i, a ballot finds the live ones, and each live
// lane's slot is the number of live lanes below it, so the list comes out in
// descending order with no sort.
__global__ void __launch_bounds__(256) skiplist_kernel(const uint32_t *mask, int32_t *list, int64_t rows, int Tk,
                                                       TileRanges rg)
{
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows)
        return;
    const int W = (Tk + 31) >> 5;
    const uint32_t *mrow = mask ? mask + row * W : nullptr;
    int32_t *dst = list + row * (int64_t)(1 + Tk);
    int count = 0;
    for (int top = Tk - 1; top >= 0; top -= 64) {
        const int kt = top - lane;
        bool live = kt >= 0;
        if (live && mrow)
            live = ((mrow[kt >> 5] >> (kt & 31)) & 1u) == 0u;
        if (kt >= 0 && rg.any) {
            if ((rg.do_bits[kt >> 5] >> (kt & 31)) & 1u)
                live = true;
            else if ((rg.skip_bits[kt >> 5] >> (kt & 31)) & 1u)
                live = false;
        }
        const unsigned long long bal = __ballot(live);
        const int below = __popcll(bal & ((1ull << lane) - 1ull));
        if (live)
            dst[1 + count + below] = kt;
        count += __popcll(bal);
    }
    if (lane == 0)
        dst[0] = count;
}

}  // namespace

hipError_t launch_reset_mask(uint32_t *mask, int64_t words, hipStream_t stream)
{
    if (words <= 0)
        return hipSuccess;
    int64_t blocks = (words + 255) / 256;
    if (blocks > 65536)
        blocks = 65536;
    hipLaunchKernelGGL(reset_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, mask, words);
    return hipGetLastError();
}

hipError_t launch_build_skiplist(const uint32_t *mask, int32_t *skiplist, int64_t rows, int32_t Tk,
                                 const TileRanges &rg, hipStream_t stream)
{
    if (rows <= 0)
        return hipSuccess;
    const int64_t blocks = (rows + 3) / 4;
    hipLaunchKernelGGL(skiplist_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, mask, skiplist, rows, Tk, rg);
    return hipGetLastError();
}

}  // namespace lite_attn
