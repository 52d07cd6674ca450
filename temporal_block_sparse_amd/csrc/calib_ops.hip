// Support for the per-timestep threshold calibration (README "Error
// Calibration": error budgets per timestep, stricter early): the sums behind
// a relative output error, ||a - b||^2 and ||b||^2, in fp64.
//
// HBM-bound: each element of a and b is read once.  One thread per 8
// consecutive head-dim elements of one (b, n, h), grid-stride; each wave adds
// its partial sums into the two doubles with one atomic each.
#include "lite_attn_internal.h"

namespace lite_attn {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void load8(const void *base, int64_t off, int dtype, float (&x)[8])
{
    if (dtype == 0) {
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

__global__ void __launch_bounds__(256) error_sums_kernel(ErrParams p)
{
    const int cpq = p.D / 8;
    const int64_t total = (int64_t)p.B * p.N * p.H * cpq;
    double s0 = 0.0, s1 = 0.0;
    for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < total; t += (int64_t)gridDim.x * 256) {
        const int c = (int)(t % cpq);
        const int64_t qid = t / cpq;  // (b, n, h) in BSHD order
        const int h = (int)(qid % p.H);
        const int64_t bn = qid / p.H;
        const int n = (int)(bn % p.N), b = (int)(bn / p.N);
        const int64_t inner = ((int64_t)n * p.H + h) * p.D + 8 * c;
        float x[8], y[8];
        load8(p.a, (int64_t)b * p.a_sb + inner, p.dtype, x);
        load8(p.b, (int64_t)b * p.b_sb + inner, p.dtype, y);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const double d = (double)x[j] - (double)y[j];
            s0 = fma(d, d, s0);
            s1 = fma((double)y[j], (double)y[j], s1);
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        s0 += __shfl_xor(s0, off);
        s1 += __shfl_xor(s1, off);
    }
    if ((threadIdx.x & 63) == 0) {
        atomicAdd(&p.sums[0], s0);
        atomicAdd(&p.sums[1], s1);
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
    if (blocks > 4096)
        blocks = 4096;
    hipLaunchKernelGGL(error_sums_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace lite_attn
