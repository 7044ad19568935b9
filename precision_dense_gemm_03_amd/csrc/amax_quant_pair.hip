// Both operands of an FP8 GEMM in two launches: amax of A and of B, their
// per-tensor scales, and the FP8 codes of both.
//
// "DeepGEMM实战：FP8矩阵乘法与JIT编译优化指南" (sheratonhq.com news 156926) §3.2
// takes a per-tensor scale max|x| / 448 for each operand and §4.3 quantizes
// fp8 = clamp(round(x / scale), -448, 448); its §4.4 notes that launch
// overhead dominates small work and suggests batching. The DeepGEMM deep-dive
// (hnwysp.cn news 84236) §3.3 takes the maxima on the GPU, on a stream.
//
// Launch 1 (pair_reduce_kernel): blocks [0, PA) reduce contiguous chunks of A,
// blocks [PA, PA + PB) chunks of B, each writing the maximum of |x| bits of
// its chunk to its own slot of the workspace (no atomics, nothing to clear
// first). Launch 2 (pair_quantize_kernel): every block first reduces the PA
// and PB slots itself (at most kPairSlots words, read from L2), forms both
// scales exactly as amax_f32 / amax_scale_f32 do, block 0 stores the maxima
// and scales, and then the grid quantizes A and then B with the same
// arithmetic as quantize_fp8 (IEEE division, round to nearest even,
// saturation, NaN -> 0x7F). The maximum is order-independent, so the result
// is deterministic and bit-identical to the separate calls.
//
// HBM traffic: 4 B per element read by launch 1, 4 B read and 1 B written by
// launch 2. All of it is non-temporal. A second pass finds nothing useful in
// the caches at these sizes. Cached loads that must first evict dirty lines
// (left by whatever ran before, e.g. a GEMM's output) measured twice as slow
// (reduce of 2 x 64 MiB after a 512 MiB write: 51.8 us cached, 24.0 us
// non-temporal; back to back both about 19.5 us). Non-temporal code stores
// took the quantize of 2 x 64 MiB from 35.6 to 28.2 us back to back.
#include <algorithm>

#include "device_common.h"
#include "kernels.h"
#include "quantize_tile.h"

namespace libgemm {

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 16;      // 16-byte loads in flight per thread, reduce (2 x 64 MiB: 55.7 us against 56.4 with 4)
constexpr int kQuantUnroll = 2;  // the same, quantize (measured: 28.2 us for 2 x 64 MiB against 29.8 with 4)

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const uint32_t o = (uint32_t)__shfl_xor((int)v, off, 64);
        v = v > o ? v : o;
    }
    return v;
}

__device__ __forceinline__ uint32_t max_abs_bits4(v4u v) {
    return max(max(v.x & 0x7FFFFFFFu, v.y & 0x7FFFFFFFu), max(v.z & 0x7FFFFFFFu, v.w & 0x7FFFFFFFu));
}

// Block-wide maximum of one value per thread (every thread gets it).
__device__ __forceinline__ uint32_t block_max(uint32_t m, uint32_t* red) {
    m = wave_max_u32(m);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) red[wave] = m;
    __syncthreads();
    uint32_t b = red[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) b = max(b, red[w]);
    return b;
}

// Maximum of |x| bits over elements [lo, hi) of x; vec: x is 16-byte aligned
// and lo is a multiple of 4.
__device__ __forceinline__ uint32_t range_max(const float* __restrict__ x, int64_t lo, int64_t hi, bool vec) {
    uint32_t m = 0u;
    int64_t done = lo;
    if (vec) {
        const v4u* x4 = reinterpret_cast<const v4u*>(x);
        const int64_t v0 = lo / 4, v1 = hi / 4;
        int64_t i = v0 + threadIdx.x;
        for (; i + (kUnroll - 1) * kThreads < v1; i += kUnroll * kThreads) {
            v4u v[kUnroll];
#pragma unroll
            for (int j = 0; j < kUnroll; ++j) v[j] = __builtin_nontemporal_load(&x4[i + j * kThreads]);
#pragma unroll
            for (int j = 0; j < kUnroll; ++j) m = max(m, max_abs_bits4(v[j]));
        }
        for (; i < v1; i += kThreads) m = max(m, max_abs_bits4(__builtin_nontemporal_load(&x4[i])));
        done = v1 * 4;
    }
    for (int64_t i = done + threadIdx.x; i < hi; i += kThreads) m = max(m, f32_bits(x[i]) & 0x7FFFFFFFu);
    return m;
}

__global__ __launch_bounds__(kThreads) void pair_reduce_kernel(const float* __restrict__ xa, int64_t na,
                                                               const float* __restrict__ xb, int64_t nb, int pa,
                                                               int pb, int64_t chunk_a, int64_t chunk_b, int vec_a,
                                                               int vec_b, uint32_t* __restrict__ slots) {
    __shared__ uint32_t red[kThreads / 64];
    const int b = blockIdx.x;
    const bool is_a = b < pa;
    const float* x = is_a ? xa : xb;
    const int64_t n = is_a ? na : nb, chunk = is_a ? chunk_a : chunk_b;
    const int64_t lo = min((int64_t)(is_a ? b : b - pa) * chunk, n), hi = min(lo + chunk, n);
    const uint32_t m = block_max(range_max(x, lo, hi, is_a ? vec_a : vec_b), red);
    if (threadIdx.x == 0) slots[b] = m;
}

// Quantize x[0, n) into q by blocks [0, nblk) of the grid (this is block bid).
template <int FMT>
__device__ __forceinline__ void quantize_range(const float* __restrict__ x, int64_t n, float s,
                                               uint8_t* __restrict__ q, bool vec, int bid, int nblk) {
    const int64_t tid = (int64_t)bid * kThreads + threadIdx.x;
    const int64_t nthreads = (int64_t)nblk * kThreads;
    int64_t done = 0;
    if (vec) {
        const v4f* x4 = reinterpret_cast<const v4f*>(x);
        uint32_t* q4 = reinterpret_cast<uint32_t*>(q);
        const int64_t n4 = n / 4;
        for (int64_t i = tid; i < n4; i += kQuantUnroll * nthreads) {
            v4f v[kQuantUnroll];
#pragma unroll
            for (int j = 0; j < kQuantUnroll; ++j)
                if (i + j * nthreads < n4) v[j] = __builtin_nontemporal_load(&x4[i + j * nthreads]);
#pragma unroll
            for (int j = 0; j < kQuantUnroll; ++j)
                if (i + j * nthreads < n4)
                    __builtin_nontemporal_store(fp8_pack4<FMT>(v[j].x / s, v[j].y / s, v[j].z / s, v[j].w / s),
                                                &q4[i + j * nthreads]);
        }
        done = n4 * 4;
    }
    for (int64_t i = done + tid; i < n; i += nthreads)
        q[i] = FMT == FMT_E5M2 ? e5m2_from_f32(x[i] / s) : e4m3_from_f32(x[i] / s);
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void pair_quantize_kernel(const float* __restrict__ xa, int64_t na,
                                                                 const float* __restrict__ xb, int64_t nb, int pa,
                                                                 int pb, const uint32_t* __restrict__ slots,
                                                                 int pow2, float* __restrict__ amax,
                                                                 float* __restrict__ scale, uint8_t* __restrict__ qa,
                                                                 uint8_t* __restrict__ qb, int vec_a, int vec_b) {
    __shared__ uint32_t red[kThreads / 64];
    uint32_t ma = 0u, mb = 0u;
    for (int i = threadIdx.x; i < pa; i += kThreads) ma = max(ma, slots[i]);
    for (int i = threadIdx.x; i < pb; i += kThreads) mb = max(mb, slots[pa + i]);
    ma = block_max(ma, red);
    mb = block_max(mb, red);
    const float amax_a = bits_f32(ma), amax_b = bits_f32(mb);
    const float sa = scale_for_format(amax_a, FMT, pow2), sb = scale_for_format(amax_b, FMT, pow2);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        amax[0] = amax_a;
        scale[0] = sa;
        if (pb > 0) {
            amax[1] = amax_b;
            scale[1] = sb;
        }
    }
    quantize_range<FMT>(xa, na, sa, qa, vec_a, blockIdx.x, gridDim.x);
    if (pb > 0) quantize_range<FMT>(xb, nb, sb, qb, vec_b, blockIdx.x, gridDim.x);
}

// The maxima of the slots, both scales, and (block 0) amax[0..1], scale[0..1].
template <int FMT>
__device__ __forceinline__ void pair_scales(int pa, int pb, const uint32_t* __restrict__ slots, int pow2,
                                            float* __restrict__ amax, float* __restrict__ scale, uint32_t* red,
                                            float& sa, float& sb) {
    uint32_t ma = 0u, mb = 0u;
    for (int i = threadIdx.x; i < pa; i += kThreads) ma = max(ma, slots[i]);
    for (int i = threadIdx.x; i < pb; i += kThreads) mb = max(mb, slots[pa + i]);
    ma = block_max(ma, red);
    mb = block_max(mb, red);
    const float amax_a = bits_f32(ma), amax_b = bits_f32(mb);
    sa = scale_for_format(amax_a, FMT, pow2);
    sb = scale_for_format(amax_b, FMT, pow2);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        amax[0] = amax_a;
        scale[0] = sa;
        amax[1] = amax_b;
        scale[1] = sb;
    }
}

// Launch 2 with B's codes written K-major: blocks [0, ga) quantize A as
// pair_quantize_kernel does, blocks [ga, ga + tiles) one 128 x 64 block of
// B[K, N] each into Bt[N, K] (quantize_tile.h), with the same arithmetic.
template <int FMT>
__global__ __launch_bounds__(kThreads) void pair_quantize_bt_kernel(
    const float* __restrict__ xa, int64_t na, const float* __restrict__ xb, int64_t K, int64_t N, int pa, int pb,
    const uint32_t* __restrict__ slots, int pow2, float* __restrict__ amax, float* __restrict__ scale,
    uint8_t* __restrict__ qa, uint8_t* __restrict__ qbt, int vec_a, int ga, int64_t tiles_c, int vec_in_b,
    int vec_out_b) {
    static_assert(kThreads == kQtThreads, "one thread count");
    __shared__ uint32_t red[kThreads / 64];
    __shared__ __attribute__((aligned(16))) uint8_t t[kQtCols * kQtPitch];
    float sa, sb;
    pair_scales<FMT>(pa, pb, slots, pow2, amax, scale, red, sa, sb);
    if ((int)blockIdx.x < ga) quantize_range<FMT>(xa, na, sa, qa, vec_a, blockIdx.x, ga);
    else quantize_transposed_tile<FMT>(xb, K, N, sb, qbt, blockIdx.x - ga, tiles_c, vec_in_b, vec_out_b,
                                       (LDS_AS uint8_t*)t);
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

// Slots: PA + PB <= kPairSlots, split in proportion to the sizes (at least one
// each for a non-empty tensor); each block's chunk is a multiple of 1024
// elements so that vector loads stay aligned.
hipError_t launch_amax_quantize_pair(const float* xa, int64_t na, const float* xb, int64_t nb, int fmt, int pow2,
                                     float* amax, float* scale, uint8_t* qa, uint8_t* qb, uint32_t* slots,
                                     hipStream_t stream) {
    const int64_t total = na + nb;
    int pa = 1, pb = nb > 0 ? 1 : 0;
    if (total > 0) {
        const int64_t want = std::min<int64_t>(kPairSlots, (total + 16383) / 16384);  // ~64 KiB of input per block
        pa = (int)std::max<int64_t>(1, want * na / total);
        if (nb > 0) pb = (int)std::max<int64_t>(1, want - pa);
        if (pa + pb > kPairSlots) pa = kPairSlots - pb;
    }
    auto chunk_of = [](int64_t n, int p) -> int64_t {
        const int64_t c = (n + p - 1) / p;
        return (c + 1023) / 1024 * 1024;
    };
    const int64_t ca = chunk_of(na, pa), cb = nb > 0 ? chunk_of(nb, pb) : 1024;
    const int vec_a = aligned16(xa), vec_b = nb > 0 && aligned16(xb);
    pair_reduce_kernel<<<pa + pb, kThreads, 0, stream>>>(xa, na, xb, nb, pa, pb, ca, cb, vec_a, vec_b, slots);
    const int qvec_a = vec_a && ((uintptr_t)qa & 3u) == 0;
    const int qvec_b = vec_b && ((uintptr_t)qb & 3u) == 0;
    const int64_t work = (na + nb) / 4 / kQuantUnroll;
    const int grid = (int)std::min<int64_t>(4096, std::max<int64_t>(1, (work + kThreads - 1) / kThreads));
    if (fmt == FMT_E5M2)
        pair_quantize_kernel<FMT_E5M2><<<grid, kThreads, 0, stream>>>(xa, na, xb, nb, pa, pb, slots, pow2, amax, scale,
                                                                      qa, qb, qvec_a, qvec_b);
    else
        pair_quantize_kernel<FMT_E4M3><<<grid, kThreads, 0, stream>>>(xa, na, xb, nb, pa, pb, slots, pow2, amax, scale,
                                                                      qa, qb, qvec_a, qvec_b);
    return hipGetLastError();
}

// As launch_amax_quantize_pair with B = xb[K, N] row-major and its codes
// written K-major into qbt[N, K]. Launch 1 is the same reduce; in launch 2
// A's blocks take 8192 elements each (the size of one B block), at most 4096.
hipError_t launch_amax_quantize_pair_bt(const float* xa, int64_t na, const float* xb, int64_t K, int64_t N, int fmt,
                                        int pow2, float* amax, float* scale, uint8_t* qa, uint8_t* qbt,
                                        uint32_t* slots, hipStream_t stream) {
    const int64_t nb = K * N;
    if (nb == 0) return launch_amax_quantize_pair(xa, na, xb, 0, fmt, pow2, amax, scale, qa, qbt, slots, stream);
    const int64_t total = na + nb;
    const int64_t want = std::min<int64_t>(kPairSlots, (total + 16383) / 16384);
    int pa = (int)std::max<int64_t>(1, want * na / total);
    int pb = (int)std::max<int64_t>(1, want - pa);
    if (pa + pb > kPairSlots) pa = kPairSlots - pb;
    auto chunk_of = [](int64_t n, int p) -> int64_t {
        const int64_t c = (n + p - 1) / p;
        return (c + 1023) / 1024 * 1024;
    };
    const int64_t ca = chunk_of(na, pa), cb = chunk_of(nb, pb);
    const int vec_a = aligned16(xa), vec_b = aligned16(xb);
    pair_reduce_kernel<<<pa + pb, kThreads, 0, stream>>>(xa, na, xb, nb, pa, pb, ca, cb, vec_a, vec_b, slots);
    const int qvec_a = vec_a && ((uintptr_t)qa & 3u) == 0;
    const int64_t tiles_r = (K + kQtRows - 1) / kQtRows, tiles_c = (N + kQtCols - 1) / kQtCols;
    const int64_t tiles = tiles_r * tiles_c;
    const int ga = (int)std::min<int64_t>(4096, std::max<int64_t>(1, (na + 8191) / 8192));
    if (tiles + ga > 0x7FFFFFFF) return hipErrorInvalidValue;
    // 16-byte input rows: an aligned base and N % 4 == 0; 16-byte output
    // pieces: an aligned base and K % 16 == 0.
    const int vec_in = vec_b && N % 4 == 0;
    const int vec_out = aligned16(qbt) && K % 16 == 0;
    const unsigned grid = (unsigned)(ga + tiles);
    if (fmt == FMT_E5M2)
        pair_quantize_bt_kernel<FMT_E5M2><<<grid, kThreads, 0, stream>>>(xa, na, xb, K, N, pa, pb, slots, pow2, amax,
                                                                         scale, qa, qbt, qvec_a, ga, tiles_c, vec_in,
                                                                         vec_out);
    else
        pair_quantize_bt_kernel<FMT_E4M3><<<grid, kThreads, 0, stream>>>(xa, na, xb, K, N, pa, pb, slots, pow2, amax,
                                                                         scale, qa, qbt, qvec_a, ga, tiles_c, vec_in,
                                                                         vec_out);
    return hipGetLastError();
}

}  // namespace libgemm
