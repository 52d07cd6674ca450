// Support for the per-timestep threshold calibration (README "Error
// Calibration": error budgets per timestep, stricter early): the sums behind
// a relative output error, ||a - b||^2 and ||b||^2, in fp64.
//
// HBM-bound: each element of a and b is read once.  Within one batch entry
// the (n, h, d) elements of a BSHD tensor are contiguous, so the kernel walks
// the batch entries in turn and, within one, takes 8 consecutive elements per
// thread, grid-stride, at offset 8t: no index arithmetic beyond that.  Each
// block adds its partial sums into the two doubles with one atomic each.
// The element type is a template parameter: with a run-time branch on it in
// the load, the same kernel ran at 3.6 TB/s instead of 4.8 (1,024 blocks,
// same GPU); with eight blocks per CU it reaches 5.3.
#include "lite_attn_internal.h"

namespace lite_attn {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int DT>
__device__ __forceinline__ void load8(const void *base, int64_t off, float (&x)[8])
{
    if (DT == 0) {
        const u32x4 w = *(const u32x4 *)((const __bf16 *)base + off);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[2 * j] = __builtin_bit_cast(float, w[j] << 16);
            x[2 * j + 1] = __builtin_bit_cast(float, w[j] & 0xffff0000u);
        }
    } else {
        const f32x4 a = *(const f32x4 *)((const float *)base + off);
        const f32x4 b = *(const f32x4 *)((const float *)base + off + 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[j] = a[j];
            x[4 + j] = b[j];
        }
    }
}

__global__ void __launch_bounds__(256) zero2_kernel(double *sums)
{
    if (threadIdx.x < 2)
        sums[threadIdx.x] = 0.0;
}

template <int DT>
__global__ void __launch_bounds__(256) error_sums_kernel(ErrParams p)
{
    const int64_t per_b = (int64_t)p.N * p.H * (p.D / 8);  // 8-element chunks per batch entry
    const int64_t stride = (int64_t)gridDim.x * 256;
    double s0 = 0.0, s1 = 0.0;
    for (int b = 0; b < p.B; ++b) {
        const int64_t ab = (int64_t)b * p.a_sb, bb = (int64_t)b * p.b_sb;
        // four chunks per pass, all loads issued before any arithmetic, so
        // that enough bytes are in flight to cover the memory latency; chunks
        // past the end are zeros and add nothing
        for (int64_t t0 = (int64_t)blockIdx.x * 256 + threadIdx.x; t0 < per_b; t0 += 4 * stride) {
            float x[4][8], y[4][8];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int64_t t = t0 + u * stride;
                if (t < per_b) {
                    load8<DT>(p.a, ab + 8 * t, x[u]);
                    load8<DT>(p.b, bb + 8 * t, y[u]);
                } else {
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        x[u][j] = y[u][j] = 0.f;
                }
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const double d = (double)x[u][j] - (double)y[u][j];
                    s0 = fma(d, d, s0);
                    s1 = fma((double)y[u][j], (double)y[u][j], s1);
                }
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        s0 += __shfl_xor(s0, off);
        s1 += __shfl_xor(s1, off);
    }
    // the block's four waves meet in LDS: one atomic pair per block, since
    // atomics on the same two addresses serialise
    __shared__ double part[2][4];
    if ((threadIdx.x & 63) == 0) {
        part[0][threadIdx.x >> 6] = s0;
        part[1][threadIdx.x >> 6] = s1;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        atomicAdd(&p.sums[0], (part[0][0] + part[0][1]) + (part[0][2] + part[0][3]));
        atomicAdd(&p.sums[1], (part[1][0] + part[1][1]) + (part[1][2] + part[1][3]));
    }
}

}  // namespace

hipError_t launch_error_sums(const ErrParams &p, hipStream_t stream)
{
    if (p.D % 8 != 0)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(zero2_kernel, dim3(1), dim3(64), 0, stream, p.sums);
    const int64_t total = (int64_t)p.B * p.N * p.H * (p.D / 8);
    if (total <= 0)
        return hipGetLastError();
    int64_t blocks = (total + 255) / 256;
    if (blocks > 2048)
        blocks = 2048;  // eight per CU: enough loads in flight, few atomics
    if (p.dtype == 0)
        hipLaunchKernelGGL(error_sums_kernel<0>, dim3((unsigned)blocks), dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL(error_sums_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace lite_attn
