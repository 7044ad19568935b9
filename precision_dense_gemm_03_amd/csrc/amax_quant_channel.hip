// Per-channel amax, scale and FP8 quantization kernels.
//
// "DeepGEMM实战：FP8矩阵乘法与JIT编译优化指南" (sheratonhq.com news 156926)
// §2.1 and §3.2 name per-channel scaling as the finer alternative to one scale
// per tensor. A scale has to be constant along K to be applied to the
// accumulator at write-back (§3.2), so the channels are the rows of A[M,K]
// and the columns of B[K,N]: axis 0 gives one value per row of a row-major
// x[rows, cols], axis 1 one value per column. Each channel's scale is the
// per-tensor rule (§3.2, or the power-of-two rule of §2.1) applied to that
// channel's max|x|, and quantization divides by the channel's scale (§4.3).
//
// All four kernels stream x once from HBM (4 B per element; quantize also
// writes 1 B per element) with 16-byte loads per lane:
//   axis 0  one wave per row: lanes walk the row, so every wave instruction
//           reads 1 KiB of one row; the wave reduces with cross-lane max and
//           lane 0 writes the row's amax and scale. No atomics, one launch.
//   axis 1  a block covers 256 columns (64 lanes x 4 columns) and a chunk of
//           rows; its 4 waves take interleaved rows of the chunk, so every
//           wave instruction reads 1 KiB of one row. The waves' maxima meet
//           in LDS and one atomic max per column and chunk merges the chunks
//           (amax is zeroed first and turned into scales by a last launch).
#include "device_common.h"
#include "kernels.h"

namespace libgemm {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kColsPerBlock = 256;   // axis 1: 64 lanes x 4 columns
constexpr int kRowChunk = 128;       // axis 1: rows per block and chunk
constexpr int kUnroll = 4;

__device__ __forceinline__ uint32_t abs_bits(float x) { return f32_bits(x) & 0x7FFFFFFFu; }

__device__ __forceinline__ uint32_t max4(v4u v) {
    return max(max(v.x & 0x7FFFFFFFu, v.y & 0x7FFFFFFFu), max(v.z & 0x7FFFFFFFu, v.w & 0x7FFFFFFFu));
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        uint32_t o = (uint32_t)__shfl_xor((int)v, off, 64);
        v = v > o ? v : o;
    }
    return v;
}

// ---------------------------------------------------------------- axis 0

// vec: x 16-byte aligned and cols % 4 == 0, so every row starts aligned.
__global__ __launch_bounds__(kThreads) void amax_rows_kernel(const float* __restrict__ x, int64_t rows, int64_t cols,
                                                             float* __restrict__ amax, float* __restrict__ scale,
                                                             int fmt, int pow2, int vec) {
    const int lane = threadIdx.x & 63;
    const int64_t nwaves = (int64_t)gridDim.x * kWaves;
    for (int64_t r = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6); r < rows; r += nwaves) {
        const float* xr = x + r * cols;
        uint32_t m = 0u;
        if (vec) {
            const v4u* x4 = reinterpret_cast<const v4u*>(xr);
            const int64_t n4 = cols / 4;
            int64_t i = lane;
            for (; i + (kUnroll - 1) * 64 < n4; i += kUnroll * 64) {
                v4u v[kUnroll];
#pragma unroll
                for (int j = 0; j < kUnroll; ++j) v[j] = __builtin_nontemporal_load(&x4[i + j * 64]);
#pragma unroll
                for (int j = 0; j < kUnroll; ++j) m = max(m, max4(v[j]));
            }
            for (; i < n4; i += 64) m = max(m, max4(x4[i]));
        } else {
            for (int64_t i = lane; i < cols; i += 64) m = max(m, abs_bits(xr[i]));
        }
        m = wave_max_u32(m);
        if (lane == 0) {
            const float a = bits_f32(m);
            amax[r] = a;
            if (scale) scale[r] = scale_for_format(a, fmt, pow2);
        }
    }
}

// q[r, :] = FP8(fl32(x[r, :] / scale[r])), one wave per row. vec: x 16-byte
// aligned, q 4-byte aligned and cols % 4 == 0.
template <int FMT>
__global__ __launch_bounds__(kThreads) void quantize_rows_kernel(const float* __restrict__ x, int64_t rows,
                                                                 int64_t cols, const float* __restrict__ scale,
                                                                 uint8_t* __restrict__ q, int vec) {
    const int lane = threadIdx.x & 63;
    const int64_t nwaves = (int64_t)gridDim.x * kWaves;
    for (int64_t r = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6); r < rows; r += nwaves) {
        const float s = scale[r];
        const float* xr = x + r * cols;
        uint8_t* qr = q + r * cols;
        if (vec) {
            const v4f* x4 = reinterpret_cast<const v4f*>(xr);
            uint32_t* q4 = reinterpret_cast<uint32_t*>(qr);
            const int64_t n4 = cols / 4;
            for (int64_t i = lane; i < n4; i += kUnroll * 64) {
                v4f v[kUnroll];
#pragma unroll
                for (int j = 0; j < kUnroll; ++j)
                    if (i + j * 64 < n4) v[j] = __builtin_nontemporal_load(&x4[i + j * 64]);
#pragma unroll
                for (int j = 0; j < kUnroll; ++j)
                    if (i + j * 64 < n4)
                        __builtin_nontemporal_store(fp8_pack4<FMT>(v[j].x / s, v[j].y / s, v[j].z / s, v[j].w / s),
                                                    &q4[i + j * 64]);
            }
        } else {
            for (int64_t i = lane; i < cols; i += 64)
                qr[i] = FMT == FMT_E5M2 ? e5m2_from_f32(xr[i] / s) : e4m3_from_f32(xr[i] / s);
        }
    }
}

// ---------------------------------------------------------------- axis 1

__global__ void fill_u32_kernel(uint32_t* p, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) p[i] = 0u;
}

// Block b covers columns [cb * 256, cb * 256 + 256), cb = b % col_blocks, and
// the row chunks b / col_blocks, + chunk_stride, ...; lane l owns the four
// columns cb * 256 + 4l .. + 3 and wave w the rows w, w + 4, ... of a chunk.
__global__ __launch_bounds__(kThreads) void amax_cols_kernel(const float* __restrict__ x, int64_t rows, int64_t cols,
                                                             uint32_t* __restrict__ amax_bits, int64_t col_blocks,
                                                             int64_t chunk_stride, int vec) {
    __shared__ v4u part[kWaves][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t cb = blockIdx.x % col_blocks;
    const int64_t c0 = cb * kColsPerBlock + 4 * lane;
    const int64_t nchunks = (rows + kRowChunk - 1) / kRowChunk;
    const bool full = vec && c0 + 3 < cols;
    for (int64_t ch = blockIdx.x / col_blocks; ch < nchunks; ch += chunk_stride) {
        const int64_t r0 = ch * kRowChunk;
        const int64_t r1 = min(rows, r0 + kRowChunk);
        v4u m = {0u, 0u, 0u, 0u};
        if (full) {
            int64_t r = r0 + wave;
            for (; r + (kUnroll - 1) * kWaves < r1; r += kUnroll * kWaves) {
                v4u v[kUnroll];
#pragma unroll
                for (int j = 0; j < kUnroll; ++j)
                    v[j] = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(x + (r + j * kWaves) * cols + c0));
#pragma unroll
                for (int j = 0; j < kUnroll; ++j) {
                    m.x = max(m.x, v[j].x & 0x7FFFFFFFu);
                    m.y = max(m.y, v[j].y & 0x7FFFFFFFu);
                    m.z = max(m.z, v[j].z & 0x7FFFFFFFu);
                    m.w = max(m.w, v[j].w & 0x7FFFFFFFu);
                }
            }
            for (; r < r1; r += kWaves) {
                const v4u v = *reinterpret_cast<const v4u*>(x + r * cols + c0);
                m.x = max(m.x, v.x & 0x7FFFFFFFu);
                m.y = max(m.y, v.y & 0x7FFFFFFFu);
                m.z = max(m.z, v.z & 0x7FFFFFFFu);
                m.w = max(m.w, v.w & 0x7FFFFFFFu);
            }
        } else {
            for (int64_t r = r0 + wave; r < r1; r += kWaves) {
                const float* xr = x + r * cols;
                if (c0 < cols) m.x = max(m.x, abs_bits(xr[c0]));
                if (c0 + 1 < cols) m.y = max(m.y, abs_bits(xr[c0 + 1]));
                if (c0 + 2 < cols) m.z = max(m.z, abs_bits(xr[c0 + 2]));
                if (c0 + 3 < cols) m.w = max(m.w, abs_bits(xr[c0 + 3]));
            }
        }
        part[wave][lane] = m;
        __syncthreads();
        if (wave == 0) {
#pragma unroll
            for (int w = 1; w < kWaves; ++w) {
                const v4u o = part[w][lane];
                m.x = max(m.x, o.x);
                m.y = max(m.y, o.y);
                m.z = max(m.z, o.z);
                m.w = max(m.w, o.w);
            }
            const uint32_t mv[4] = {m.x, m.y, m.z, m.w};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                uint32_t* dst = amax_bits + c0 + c;
                if (c0 + c < cols && mv[c] > __hip_atomic_load(dst, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
                    atomicMax(dst, mv[c]);
            }
        }
        __syncthreads();   // part is rewritten by the next chunk
    }
}

__global__ void scale_cols_kernel(const float* __restrict__ amax, int64_t n, float* __restrict__ scale, int fmt,
                                  int pow2) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride)
        scale[i] = scale_for_format(amax[i], fmt, pow2);
}

// q[r, c] = FP8(fl32(x[r, c] / scale[c])), with the block layout of
// amax_cols_kernel; each lane loads its four column scales once.
template <int FMT>
__global__ __launch_bounds__(kThreads) void quantize_cols_kernel(const float* __restrict__ x, int64_t rows,
                                                                 int64_t cols, const float* __restrict__ scale,
                                                                 uint8_t* __restrict__ q, int64_t col_blocks,
                                                                 int64_t chunk_stride, int vec) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t cb = blockIdx.x % col_blocks;
    const int64_t c0 = cb * kColsPerBlock + 4 * lane;
    if (c0 >= cols) return;   // no barrier below: idle lanes may leave
    const int64_t nchunks = (rows + kRowChunk - 1) / kRowChunk;
    const bool full = vec && c0 + 3 < cols;
    float s[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) s[c] = c0 + c < cols ? scale[c0 + c] : 1.0f;
    for (int64_t ch = blockIdx.x / col_blocks; ch < nchunks; ch += chunk_stride) {
        const int64_t r0 = ch * kRowChunk;
        const int64_t r1 = min(rows, r0 + kRowChunk);
        if (full) {
            for (int64_t r = r0 + wave; r < r1; r += kUnroll * kWaves) {
                v4f v[kUnroll];
#pragma unroll
                for (int j = 0; j < kUnroll; ++j)
                    if (r + j * kWaves < r1)
                        v[j] = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(x + (r + j * kWaves) * cols + c0));
#pragma unroll
                for (int j = 0; j < kUnroll; ++j)
                    if (r + j * kWaves < r1)
                        __builtin_nontemporal_store(
                            fp8_pack4<FMT>(v[j].x / s[0], v[j].y / s[1], v[j].z / s[2], v[j].w / s[3]),
                            reinterpret_cast<uint32_t*>(q + (r + j * kWaves) * cols + c0));
            }
        } else {
            for (int64_t r = r0 + wave; r < r1; r += kWaves) {
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    if (c0 + c < cols) {
                        const float y = x[r * cols + c0 + c] / s[c];
                        q[r * cols + c0 + c] = FMT == FMT_E5M2 ? e5m2_from_f32(y) : e4m3_from_f32(y);
                    }
            }
        }
    }
}

int64_t blocks_for(int64_t work, int64_t per_block, int64_t cap) {
    int64_t g = (work + per_block - 1) / per_block;
    if (g < 1) g = 1;
    return g < cap ? g : cap;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Axis-1 launch shape: every column block, and as many row chunks per column
// block as keep the launch near 2048 blocks (the rest loop).
void cols_grid(int64_t rows, int64_t cols, int64_t* col_blocks, int64_t* chunk_stride, int64_t* blocks) {
    *col_blocks = (cols + kColsPerBlock - 1) / kColsPerBlock;
    const int64_t nchunks = (rows + kRowChunk - 1) / kRowChunk;
    int64_t want = 2048 / *col_blocks;
    if (want < 1) want = 1;
    *chunk_stride = nchunks < want ? nchunks : want;
    if (*chunk_stride < 1) *chunk_stride = 1;
    *blocks = *col_blocks * *chunk_stride;
}

}  // namespace

hipError_t launch_amax_channel(const float* x, int64_t rows, int64_t cols, int axis, float* amax, float* scale,
                               int fmt, int pow2, hipStream_t stream) {
    if (axis == 0) {
        if (rows <= 0) return hipSuccess;
        const int vec = (aligned(x, 16) && cols % 4 == 0) ? 1 : 0;
        const int64_t grid = blocks_for(rows, kWaves, 4096);
        amax_rows_kernel<<<(unsigned)grid, kThreads, 0, stream>>>(x, rows, cols, amax, scale, fmt, pow2, vec);
        return hipGetLastError();
    }
    if (cols <= 0) return hipSuccess;
    uint32_t* bits = reinterpret_cast<uint32_t*>(amax);
    fill_u32_kernel<<<(unsigned)blocks_for(cols, kThreads, 1024), kThreads, 0, stream>>>(bits, cols);
    if (rows > 0) {
        int64_t col_blocks, chunk_stride, blocks;
        cols_grid(rows, cols, &col_blocks, &chunk_stride, &blocks);
        const int vec = (aligned(x, 16) && cols % 4 == 0) ? 1 : 0;
        amax_cols_kernel<<<(unsigned)blocks, kThreads, 0, stream>>>(x, rows, cols, bits, col_blocks, chunk_stride,
                                                                    vec);
    }
    if (scale)
        scale_cols_kernel<<<(unsigned)blocks_for(cols, kThreads, 1024), kThreads, 0, stream>>>(amax, cols, scale, fmt,
                                                                                              pow2);
    return hipGetLastError();
}

hipError_t launch_quantize_channel(const float* x, int64_t rows, int64_t cols, int axis, const float* scale,
                                   uint8_t* q, int fmt, hipStream_t stream) {
    if (rows <= 0 || cols <= 0) return hipSuccess;
    const int vec = (aligned(x, 16) && aligned(q, 4) && cols % 4 == 0) ? 1 : 0;
    if (axis == 0) {
        const unsigned grid = (unsigned)blocks_for(rows, kWaves, 4096);
        if (fmt == FMT_E5M2)
            quantize_rows_kernel<FMT_E5M2><<<grid, kThreads, 0, stream>>>(x, rows, cols, scale, q, vec);
        else
            quantize_rows_kernel<FMT_E4M3><<<grid, kThreads, 0, stream>>>(x, rows, cols, scale, q, vec);
        return hipGetLastError();
    }
    int64_t col_blocks, chunk_stride, blocks;
    cols_grid(rows, cols, &col_blocks, &chunk_stride, &blocks);
    if (fmt == FMT_E5M2)
        quantize_cols_kernel<FMT_E5M2><<<(unsigned)blocks, kThreads, 0, stream>>>(x, rows, cols, scale, q, col_blocks,
                                                                                 chunk_stride, vec);
    else
        quantize_cols_kernel<FMT_E4M3><<<(unsigned)blocks, kThreads, 0, stream>>>(x, rows, cols, scale, q, col_blocks,
                                                                                 chunk_stride, vec);
    return hipGetLastError();
}

}  // namespace libgemm
