// FP16 dynamic-range guard for the FP16 GEMM.
//
// The DeepGEMM deep-dive article (hnwysp.cn news 84236, mixed-precision
// section) guards FP16 inputs against overflow ("dynamic range-aware
// scaling"): the maxima of |A| and |B| are taken on the GPU, on the stream,
// before the GEMM; s = min(1, 65504 / (max|A| * max|B|)); A and B are each
// multiplied by sqrt(s) as they are converted to FP16, and the accumulated
// result is divided by s. Every product of the scaled operands then stays
// within the FP16 range (both operands stay finite while max|A| / max|B|
// <= 65504).
//
// Here: two amax reductions (amax_quant.hip), one single-thread launch that
// forms s, sqrt(s) and 1/s, one streaming conversion per operand (4 B read,
// 2 B written per element), and the FP16 GEMM whose epilogue multiplies the
// FP32 sum by 1/s (one FP32 factor; within a few FP32 ulps of the quotient).
#include "device_common.h"
#include "kernels.h"

namespace libgemm {

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

// s in double (the product of two floats is exact, the quotient correctly
// rounded), rounded once to FP32; 1 when the quotient is >= 1 or NaN.
// r = sqrt(s) and inv = 1 / s in FP32, correctly rounded (the library is
// built with correctly rounded FP32 divide and sqrt).
__global__ void guard_scale_kernel(const float* __restrict__ amax_a, const float* __restrict__ amax_b,
                                   float* __restrict__ scalars, float* __restrict__ scale_out) {
    const double q = 65504.0 / ((double)*amax_a * (double)*amax_b);
    const float s = q < 1.0 ? (float)q : 1.0f;
    scalars[0] = s;
    scalars[1] = __builtin_sqrtf(s);
    scalars[2] = 1.0f / s;
    if (scale_out) *scale_out = s;
}

// y = FP16(fl32(x * r)), RNE, overflow to inf (IEEE conversion). vec: x
// 16-byte aligned and y 8-byte aligned; each lane turns one 16-byte load
// into one 8-byte store.
__global__ __launch_bounds__(kThreads) void guard_to_f16_kernel(const float* __restrict__ x, int64_t n,
                                                                const float* __restrict__ scalars,
                                                                _Float16* __restrict__ y, int vec) {
    typedef _Float16 v4h __attribute__((ext_vector_type(4)));
    const float r = scalars[1];
    const int64_t tid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t nthreads = (int64_t)gridDim.x * kThreads;
    int64_t done = 0;
    if (vec) {
        const v4f* x4 = reinterpret_cast<const v4f*>(x);
        v4h* y4 = reinterpret_cast<v4h*>(y);
        const int64_t n4 = n / 4;
        for (int64_t i = tid; i < n4; i += kUnroll * nthreads) {
            v4f v[kUnroll];
#pragma unroll
            for (int j = 0; j < kUnroll; ++j)
                if (i + j * nthreads < n4) v[j] = __builtin_nontemporal_load(&x4[i + j * nthreads]);
#pragma unroll
            for (int j = 0; j < kUnroll; ++j)
                if (i + j * nthreads < n4) {
                    const v4f t = v[j] * r;
                    y4[i + j * nthreads] = v4h{(_Float16)t.x, (_Float16)t.y, (_Float16)t.z, (_Float16)t.w};
                }
        }
        done = n4 * 4;
    }
    for (int64_t i = done + tid; i < n; i += nthreads) y[i] = (_Float16)(x[i] * r);
}

int grid_for(int64_t work, int cap) {
    int64_t g = (work + kThreads - 1) / kThreads;
    if (g < 1) g = 1;
    if (g > cap) g = cap;
    return (int)g;
}

}  // namespace

hipError_t launch_guard_to_f16(const float* x, int64_t n, const float* scalars, _Float16* y, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    const int vec = (((uintptr_t)x & 15u) == 0 && ((uintptr_t)y & 7u) == 0) ? 1 : 0;
    const int grid = grid_for(vec ? (n / 4 + kUnroll - 1) / kUnroll : n, 4096);
    guard_to_f16_kernel<<<grid, kThreads, 0, stream>>>(x, n, scalars, y, vec);
    return hipGetLastError();
}

hipError_t launch_guard_scale(const float* amax_a, const float* amax_b, float* scalars, float* scale_out,
                              hipStream_t stream) {
    guard_scale_kernel<<<1, 1, 0, stream>>>(amax_a, amax_b, scalars, scale_out);
    return hipGetLastError();
}

}  // namespace libgemm
