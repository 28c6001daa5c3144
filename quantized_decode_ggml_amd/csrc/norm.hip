// RMSNorm ("Struct QTensorEngine" page, apply_output_norm_inplace: the final
// output_norm RMSNorm of a pre-norm model, applied in place before the
// vocabulary projection; the same normalisation precedes the attention and FFN
// products of each block).  The pages do not print the formula; the one used is
// the usual RMSNorm: out_j = x_j / sqrt(mean_j(x_j^2) + eps) * w_j.
//
// One workgroup of 256 threads per row: float4 loads, an f64 sum of squares
// per lane (no overflow for any f32 row), a shuffle fold per wave and four wave
// sums through LDS, then a second pass that scales by r = 1/sqrt(mean + eps)
// (f64, rounded once to f32).  A row is read twice (the second time from L2).
// When the normalised vector feeds a one-row Q8_0 product the norm is folded
// into that product instead (gemv_q8_0.hip) and this kernel is not launched.
#include "qdec_internal.h"

namespace qdec {

namespace {

// n % 4 == 0 and 16-byte aligned rows take the float4 path; other n the scalar one.
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* x, int64_t n, const float* __restrict__ w,
                                                      float eps, float* out, int vec4)
{
    __shared__ double wsum[4];
    const int64_t row = blockIdx.x;
    const float* xr = x + row * n;
    float* orow = out + row * n;
    const int tid = threadIdx.x;
    double ss = 0.0;
    if (vec4) {
        const float4* x4 = reinterpret_cast<const float4*>(xr);
        for (int64_t i = tid; i < n / 4; i += 256) {
            const float4 v = x4[i];
            ss = __builtin_fma((double)v.x, (double)v.x, ss);
            ss = __builtin_fma((double)v.y, (double)v.y, ss);
            ss = __builtin_fma((double)v.z, (double)v.z, ss);
            ss = __builtin_fma((double)v.w, (double)v.w, ss);
        }
    } else {
        for (int64_t i = tid; i < n; i += 256) ss = __builtin_fma((double)xr[i], (double)xr[i], ss);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
    if ((tid & 63) == 0) wsum[tid >> 6] = ss;
    __syncthreads();
    const double total = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
    const float rs = (float)(1.0 / sqrt(total / (double)n + (double)eps));
    // each thread rescales exactly the elements it summed, so out may be x
    if (vec4) {
        const float4* x4 = reinterpret_cast<const float4*>(xr);
        const float4* w4 = reinterpret_cast<const float4*>(w);
        float4* o4 = reinterpret_cast<float4*>(orow);
        for (int64_t i = tid; i < n / 4; i += 256) {
            const float4 v = x4[i], g = w4[i];
            o4[i] = make_float4(v.x * rs * g.x, v.y * rs * g.y, v.z * rs * g.z, v.w * rs * g.w);
        }
    } else {
        for (int64_t i = tid; i < n; i += 256) orow[i] = xr[i] * rs * w[i];
    }
}

}  // namespace

hipError_t launch_rmsnorm(const float* x, int64_t n, int64_t batch, const float* w, float eps, float* out,
                          hipStream_t s)
{
    const bool vec4 = n % 4 == 0 && reinterpret_cast<uintptr_t>(x) % 16 == 0 &&
                      reinterpret_cast<uintptr_t>(w) % 16 == 0 && reinterpret_cast<uintptr_t>(out) % 16 == 0;
    hipLaunchKernelGGL(rmsnorm_kernel, dim3((unsigned)batch), dim3(256), 0, s, x, n, w, eps, out, vec4 ? 1 : 0);
    count_launch();
    return hipGetLastError();
}

}  // namespace qdec
