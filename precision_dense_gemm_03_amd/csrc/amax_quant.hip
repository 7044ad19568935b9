// amax, per-tensor scale and FP8 (E4M3) quantization kernels.
//
// "DeepGEMM实战：FP8矩阵乘法与JIT编译优化指南" (sheratonhq.com news 156926):
//   §3.2  per-tensor scale = max|x| / 448, 448 being the largest E4M3 value;
//   §4.3  quantize: fp8 = clamp(round(x / scale), -448, 448).
// The DeepGEMM deep-dive (hnwysp.cn news 84236) §3.3 takes the maximum on the
// GPU, asynchronously on a stream; here the scale stays a device scalar so
// amax -> quantize -> GEMM chain on one stream without a host round trip.
//
// Both kernels are HBM-streaming: amax reads 4 B per element, quantize reads
// 4 B and writes 1 B per element. Loads are 16 B per lane, fully coalesced.
#include "device_common.h"
#include "kernels.h"

namespace libgemm {

namespace {

constexpr int kThreads = 256;

// |x| as raw bits: for non-negative floats the unsigned order of the bit
// patterns is the numeric order, and every NaN pattern lies above +inf, so an
// unsigned max over |x| bits is an exact, NaN-propagating maximum.
__device__ __forceinline__ uint32_t abs_bits(float x) { return f32_bits(x) & 0x7FFFFFFFu; }

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        uint32_t o = (uint32_t)__shfl_xor((int)v, off, 64);
        v = v > o ? v : o;
    }
    return v;
}

__global__ void amax_init_kernel(uint32_t* amax_bits) { *amax_bits = 0u; }

// Each block reduces a grid-strided share of x to one value, then merges it
// into *amax_bits with one atomic max (order-independent, hence deterministic).
__global__ __launch_bounds__(kThreads) void amax_reduce_kernel(const float* __restrict__ x, int64_t n,
                                                               uint32_t* amax_bits, int vec) {
    uint32_t m = 0u;
    const int64_t tid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t nthreads = (int64_t)gridDim.x * kThreads;
    int64_t done = 0;
    if (vec) {
        // 16 floats per thread per iteration: four 16-byte loads in flight.
        const v4u* x4 = reinterpret_cast<const v4u*>(x);
        const int64_t n16 = n / 16;
        for (int64_t i = tid; i < n16; i += nthreads) {
            v4u v[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] = __builtin_nontemporal_load(&x4[i * 4 + j]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t a = max(max(v[j].x & 0x7FFFFFFFu, v[j].y & 0x7FFFFFFFu),
                                       max(v[j].z & 0x7FFFFFFFu, v[j].w & 0x7FFFFFFFu));
                m = max(m, a);
            }
        }
        done = n16 * 16;
    }
    for (int64_t i = done + tid; i < n; i += nthreads) m = max(m, abs_bits(x[i]));

    m = wave_max_u32(m);
    __shared__ uint32_t part[kThreads / 64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) part[wave] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t b = part[0];
#pragma unroll
        for (int w = 1; w < kThreads / 64; ++w) b = max(b, part[w]);
        atomicMax(amax_bits, b);
    }
}

__global__ void amax_finalize_kernel(const uint32_t* amax_bits, float* scale) {
    if (scale) *scale = scale_from_amax(bits_f32(*amax_bits));
}

// q = E4M3(fl32(x / s)). The FP32 division is the IEEE correctly rounded one.
__global__ __launch_bounds__(kThreads) void quantize_kernel(const float* __restrict__ x, int64_t n,
                                                            const float* __restrict__ scale,
                                                            uint8_t* __restrict__ q, int vec) {
    const float s = *scale;
    const int64_t tid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t nthreads = (int64_t)gridDim.x * kThreads;
    int64_t done = 0;
    if (vec) {
        const v4f* x4 = reinterpret_cast<const v4f*>(x);
        v4u* q16 = reinterpret_cast<v4u*>(q);
        const int64_t n16 = n / 16;
        for (int64_t i = tid; i < n16; i += nthreads) {
            v4f v[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] = __builtin_nontemporal_load(&x4[i * 4 + j]);
            v4u o;
            o.x = e4m3_pack4(v[0].x / s, v[0].y / s, v[0].z / s, v[0].w / s);
            o.y = e4m3_pack4(v[1].x / s, v[1].y / s, v[1].z / s, v[1].w / s);
            o.z = e4m3_pack4(v[2].x / s, v[2].y / s, v[2].z / s, v[2].w / s);
            o.w = e4m3_pack4(v[3].x / s, v[3].y / s, v[3].z / s, v[3].w / s);
            __builtin_nontemporal_store(o, &q16[i]);
        }
        done = n16 * 16;
    }
    for (int64_t i = done + tid; i < n; i += nthreads) q[i] = e4m3_from_f32(x[i] / s);
}

__global__ __launch_bounds__(kThreads) void fill_zero_kernel(uint8_t* C, int64_t nbytes) {
    const int64_t tid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t nthreads = (int64_t)gridDim.x * kThreads;
    for (int64_t i = tid; i < nbytes; i += nthreads) C[i] = 0;
}

int grid_for(int64_t work_items, int cap) {
    int64_t g = (work_items + kThreads - 1) / kThreads;
    if (g < 1) g = 1;
    if (g > cap) g = cap;
    return (int)g;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

hipError_t launch_amax(const float* x, int64_t n, float* amax, float* scale, hipStream_t stream) {
    uint32_t* bits = reinterpret_cast<uint32_t*>(amax);
    amax_init_kernel<<<1, 1, 0, stream>>>(bits);
    if (n > 0) {
        const int vec = aligned16(x) ? 1 : 0;
        const int grid = grid_for(vec ? (n + 15) / 16 : n, 256 * 8);
        amax_reduce_kernel<<<grid, kThreads, 0, stream>>>(x, n, bits, vec);
    }
    amax_finalize_kernel<<<1, 1, 0, stream>>>(bits, scale);
    return hipGetLastError();
}

hipError_t launch_quantize(const float* x, int64_t n, const float* scale, uint8_t* q, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    const int vec = (aligned16(x) && aligned16(q)) ? 1 : 0;
    const int grid = grid_for(vec ? (n + 15) / 16 : n, 256 * 8);
    quantize_kernel<<<grid, kThreads, 0, stream>>>(x, n, scale, q, vec);
    return hipGetLastError();
}

hipError_t launch_fill_zero(void* C, int64_t count, int out_dtype, hipStream_t stream) {
    const int64_t es = out_dtype == OUT_F32 ? 4 : (out_dtype == OUT_F16 ? 2 : 1);
    const int64_t nbytes = count * es;
    if (nbytes <= 0) return hipSuccess;
    fill_zero_kernel<<<grid_for(nbytes, 256 * 8), kThreads, 0, stream>>>(reinterpret_cast<uint8_t*>(C), nbytes);
    return hipGetLastError();
}

}  // namespace libgemm
