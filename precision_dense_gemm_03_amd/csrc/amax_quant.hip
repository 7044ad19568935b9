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
// amax is a one-thread clear of the result, the reduction, and (when a scale
// is wanted) a one-thread launch that turns the maximum into the scale.
#include "device_common.h"
#include "kernels.h"
#include "quantize_tile.h"

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

// Each block reduces a grid-strided share of x (every wave instruction reads
// 1 KiB contiguous, kUnroll of them in flight per thread) to one value and
// merges it into *amax_bits with an atomic max, skipped when the running
// maximum is already at least as large (one shared word, so the atomics
// serialize; 512 blocks keep that cost small). The maximum is
// order-independent, hence deterministic. A last-block-finalizes scheme was
// measured slower here than a separate one-thread launch: the device-scope
// fence each block would need costs more than the extra launch.
constexpr int kUnroll = 4;

__global__ __launch_bounds__(kThreads) void amax_reduce_kernel(const float* __restrict__ x, int64_t n,
                                                               uint32_t* amax_bits, int vec) {
    uint32_t m = 0u;
    const int64_t tid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t nthreads = (int64_t)gridDim.x * kThreads;
    int64_t done = 0;
    if (vec) {
        const v4u* x4 = reinterpret_cast<const v4u*>(x);
        const int64_t n4 = n / 4;
        int64_t i = tid;
        for (; i + (kUnroll - 1) * nthreads < n4; i += kUnroll * nthreads) {
            v4u v[kUnroll];
#pragma unroll
            for (int j = 0; j < kUnroll; ++j) v[j] = __builtin_nontemporal_load(&x4[i + j * nthreads]);
#pragma unroll
            for (int j = 0; j < kUnroll; ++j)
                m = max(m, max(max(v[j].x & 0x7FFFFFFFu, v[j].y & 0x7FFFFFFFu),
                               max(v[j].z & 0x7FFFFFFFu, v[j].w & 0x7FFFFFFFu)));
        }
        for (; i < n4; i += nthreads) {
            const v4u v = x4[i];
            m = max(m, max(max(v.x & 0x7FFFFFFFu, v.y & 0x7FFFFFFFu), max(v.z & 0x7FFFFFFFu, v.w & 0x7FFFFFFFu)));
        }
        done = n4 * 4;
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
        if (b > __hip_atomic_load(amax_bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) atomicMax(amax_bits, b);
    }
}

__global__ void amax_finalize_kernel(const uint32_t* amax_bits, float* scale, int fmt, int pow2) {
    *scale = scale_for_format(bits_f32(*amax_bits), fmt, pow2);
}

// q = FP8(fl32(x / s)) in format FMT (E4M3 or E5M2). The FP32 division is the
// IEEE correctly rounded one.
// Each thread turns 4 floats (one 16-byte load) into one 32-bit word of codes,
// so a wave instruction reads 1 KiB and writes 256 bytes, both contiguous.
template <int FMT>
__global__ __launch_bounds__(kThreads) void quantize_kernel(const float* __restrict__ x, int64_t n,
                                                            const float* __restrict__ scale,
                                                            uint8_t* __restrict__ q, int vec) {
    const float s = *scale;
    const int64_t tid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t nthreads = (int64_t)gridDim.x * kThreads;
    int64_t done = 0;
    if (vec) {
        const v4f* x4 = reinterpret_cast<const v4f*>(x);
        uint32_t* q4 = reinterpret_cast<uint32_t*>(q);
        const int64_t n4 = n / 4;
        for (int64_t i = tid; i < n4; i += kUnroll * nthreads) {
            v4f v[kUnroll];
#pragma unroll
            for (int j = 0; j < kUnroll; ++j)
                if (i + j * nthreads < n4) v[j] = __builtin_nontemporal_load(&x4[i + j * nthreads]);
#pragma unroll
            for (int j = 0; j < kUnroll; ++j)
                if (i + j * nthreads < n4)
                    __builtin_nontemporal_store(fp8_pack4<FMT>(v[j].x / s, v[j].y / s, v[j].z / s, v[j].w / s),
                                                &q4[i + j * nthreads]);
        }
        done = n4 * 4;
    }
    for (int64_t i = done + tid; i < n; i += nthreads)
        q[i] = FMT == FMT_E5M2 ? e5m2_from_f32(x[i] / s) : e4m3_from_f32(x[i] / s);
}

// The transposed quantize (quantize_tile.h), one 128 x 64 block per workgroup.
template <int FMT>
__global__ __launch_bounds__(kThreads) void quantize_transposed_kernel(const float* __restrict__ x, int64_t rows,
                                                                       int64_t cols, const float* __restrict__ scale,
                                                                       uint8_t* __restrict__ q, int64_t tiles_c,
                                                                       int vec_in, int vec_out) {
    static_assert(kThreads == kQtThreads, "one thread count");
    __shared__ __attribute__((aligned(16))) uint8_t t[kQtCols * kQtPitch];
    quantize_transposed_tile<FMT>(x, rows, cols, *scale, q, blockIdx.x, tiles_c, vec_in, vec_out, (LDS_AS uint8_t*)t);
}

// Transpose of a row-major [rows, cols] matrix of ES-byte elements (the
// K-major packing of a weight B[K,N] into Bt[N,K]). A workgroup moves a 64 x 64
// block through LDS: each of its 4 waves reads 16 rows of the block (lane j
// takes column j, so a wave instruction reads one contiguous 64-element row
// piece) and, after the barrier, writes 16 rows of the transposed block the
// same way. The LDS row pitch of 65 elements spreads a column read over
// distinct banks. Edge blocks are predicated.
constexpr int kTrTile = 64;

template <typename T>
__global__ __launch_bounds__(kThreads) void transpose_kernel(const T* __restrict__ src, int64_t rows, int64_t cols,
                                                             T* __restrict__ dst, int64_t tiles_c) {
    __shared__ T t[kTrTile][kTrTile + 1];
    const int64_t tile = blockIdx.x;
    const int64_t r0 = (tile / tiles_c) * kTrTile, c0 = (tile % tiles_c) * kTrTile;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll 4
    for (int i = wave; i < kTrTile; i += kThreads / 64) {
        const int64_t r = r0 + i, c = c0 + lane;
        if (r < rows && c < cols) t[i][lane] = src[r * cols + c];
    }
    __syncthreads();
#pragma unroll 4
    for (int i = wave; i < kTrTile; i += kThreads / 64) {
        const int64_t orow = c0 + i, ocol = r0 + lane;  // dst[orow, ocol] = src[ocol, orow]
        if (orow < cols && ocol < rows) dst[orow * rows + ocol] = t[lane][i];
    }
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

hipError_t launch_amax(const float* x, int64_t n, float* amax, float* scale, int fmt, int pow2, hipStream_t stream) {
    uint32_t* bits = reinterpret_cast<uint32_t*>(amax);
    amax_init_kernel<<<1, 1, 0, stream>>>(bits);
    if (n > 0) {
        const int vec = aligned16(x) ? 1 : 0;
        const int grid = grid_for(vec ? (n / 4 + kUnroll - 1) / kUnroll : n, 512);
        amax_reduce_kernel<<<grid, kThreads, 0, stream>>>(x, n, bits, vec);
    }
    if (scale) amax_finalize_kernel<<<1, 1, 0, stream>>>(bits, scale, fmt, pow2);
    return hipGetLastError();
}

hipError_t launch_quantize(const float* x, int64_t n, const float* scale, uint8_t* q, int fmt, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    const int vec = (aligned16(x) && ((uintptr_t)q & 3u) == 0) ? 1 : 0;
    const int grid = grid_for(vec ? (n / 4 + kUnroll - 1) / kUnroll : n, 4096);
    if (fmt == FMT_E5M2) quantize_kernel<FMT_E5M2><<<grid, kThreads, 0, stream>>>(x, n, scale, q, vec);
    else quantize_kernel<FMT_E4M3><<<grid, kThreads, 0, stream>>>(x, n, scale, q, vec);
    return hipGetLastError();
}

hipError_t launch_quantize_transposed(const float* x, int64_t rows, int64_t cols, const float* scale, uint8_t* q,
                                      int fmt, hipStream_t stream) {
    if (rows <= 0 || cols <= 0) return hipSuccess;
    const int64_t tiles_r = (rows + kQtRows - 1) / kQtRows, tiles_c = (cols + kQtCols - 1) / kQtCols;
    const int64_t blocks = tiles_r * tiles_c;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    // 16-byte input rows need an aligned base and cols % 4 == 0; 16-byte
    // output segments an aligned base and rows % 16 == 0.
    const int vec_in = aligned16(x) && cols % 4 == 0;
    const int vec_out = aligned16(q) && rows % 16 == 0;
    if (fmt == FMT_E5M2)
        quantize_transposed_kernel<FMT_E5M2><<<(unsigned)blocks, kThreads, 0, stream>>>(x, rows, cols, scale, q,
                                                                                         tiles_c, vec_in, vec_out);
    else
        quantize_transposed_kernel<FMT_E4M3><<<(unsigned)blocks, kThreads, 0, stream>>>(x, rows, cols, scale, q,
                                                                                         tiles_c, vec_in, vec_out);
    return hipGetLastError();
}

hipError_t launch_transpose(const void* src, int64_t rows, int64_t cols, int elem_bytes, void* dst,
                            hipStream_t stream) {
    if (rows <= 0 || cols <= 0) return hipSuccess;
    const int64_t tiles_r = (rows + kTrTile - 1) / kTrTile, tiles_c = (cols + kTrTile - 1) / kTrTile;
    const int64_t blocks = tiles_r * tiles_c;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (elem_bytes == 2)
        transpose_kernel<uint16_t><<<(unsigned)blocks, kThreads, 0, stream>>>(
            reinterpret_cast<const uint16_t*>(src), rows, cols, reinterpret_cast<uint16_t*>(dst), tiles_c);
    else if (elem_bytes == 1)
        transpose_kernel<uint8_t><<<(unsigned)blocks, kThreads, 0, stream>>>(
            reinterpret_cast<const uint8_t*>(src), rows, cols, reinterpret_cast<uint8_t*>(dst), tiles_c);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_fill_zero(void* C, int64_t count, int out_dtype, hipStream_t stream) {
    const int64_t es = out_dtype == OUT_F32 ? 4 : (out_dtype == OUT_F16 ? 2 : 1);  // FP8 outputs: 1 byte
    const int64_t nbytes = count * es;
    if (nbytes <= 0) return hipSuccess;
    fill_zero_kernel<<<grid_for(nbytes, 256 * 8), kThreads, 0, stream>>>(reinterpret_cast<uint8_t*>(C), nbytes);
    return hipGetLastError();
}

}  // namespace libgemm
