// Split-K reduction and epilogue.
//
// When the output tiles alone cannot fill 256 compute units (decode and
// mid-M shapes, where B streams from HBM once and the grid has a few dozen
// workgroups), the K dimension is cut into ranges and each range is summed
// by its own workgroups into an FP32 slice ws[s][M][N] of a caller-provided
// workspace. This kernel adds the slices in slice order (so the result does
// not depend on scheduling) and applies the epilogue of the
// "DeepGEMM实战：FP8矩阵乘法与JIT编译优化指南" (sheratonhq.com news 156926) §3.2: the
// FP32 sum times sA*sB (per tensor, or sA[i]*sB[j] per channel), divided by
// the output scale for an FP8 output, converted once at the very end (the
// rounding to FP16/FP8 has to follow the full sum). The same step splits K
// across devices in "HGEMM优化" (jsqmd.com news 710660) §6.
//
// HBM/L2-streaming: each lane reads 16 B from every slice and writes 4
// output elements; the slices were written just before, so they are mostly
// served from the last-level caches.
#include "device_common.h"
#include "kernels.h"

namespace libgemm {

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;   // slices in flight per lane

template <int OUT>
__device__ __forceinline__ void store4(void* C, int64_t idx, v4f y, int eflags) {
    if constexpr (OUT == OUT_F32) {
        *reinterpret_cast<v4f*>(reinterpret_cast<float*>(C) + idx) = y;
    } else if constexpr (OUT == OUT_F16) {
        typedef _Float16 v4h __attribute__((ext_vector_type(4)));
        *reinterpret_cast<v4h*>(reinterpret_cast<_Float16*>(C) + idx) =
            v4h{(_Float16)y.x, (_Float16)y.y, (_Float16)y.z, (_Float16)y.w};
    } else {
        const uint32_t w = (eflags & EPI_E5M2) ? fp8_pack4<FMT_E5M2>(y.x, y.y, y.z, y.w)
                                               : fp8_pack4<FMT_E4M3>(y.x, y.y, y.z, y.w);
        *reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(C) + idx) = w;
    }
}

template <int OUT>
__device__ __forceinline__ void store1(void* C, int64_t idx, float y, int eflags) {
    if constexpr (OUT == OUT_F32) {
        reinterpret_cast<float*>(C)[idx] = y;
    } else if constexpr (OUT == OUT_F16) {
        reinterpret_cast<_Float16*>(C)[idx] = (_Float16)y;
    } else {
        reinterpret_cast<uint8_t*>(C)[idx] = (eflags & EPI_E5M2) ? e5m2_from_f32(y) : e4m3_from_f32(y);
    }
}

// vec: N % 4 == 0 and ws, C aligned for 16-byte slice loads and 4-element
// stores, so each group of 4 elements lies in one row.
template <int OUT>
__global__ __launch_bounds__(kThreads) void splitk_reduce_kernel(const float* __restrict__ ws, int splits, int64_t M,
                                                                 int64_t N, void* __restrict__ C,
                                                                 const float* __restrict__ sA,
                                                                 const float* __restrict__ sB,
                                                                 const float* __restrict__ sOut, int eflags, int vec) {
    const bool chan = (eflags & EPI_CHANNEL) != 0;
    const float scale = epilogue_base(sA, sB, sOut, OUT == OUT_E4M3, chan);  // both FP8 outputs
    const int64_t mn = M * N;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    const int64_t tid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (vec) {
        const int64_t nq = mn / 4;
        const v4f* w4 = reinterpret_cast<const v4f*>(ws);
        for (int64_t q = tid; q < nq; q += stride) {
            // The slices are loaded kUnroll at a time (independent loads in
            // flight) and added in slice order.
            v4f s = __builtin_nontemporal_load(&w4[q]);
            int sp = 1;
            for (; sp + kUnroll <= splits; sp += kUnroll) {
                v4f t[kUnroll];
#pragma unroll
                for (int j = 0; j < kUnroll; ++j) t[j] = __builtin_nontemporal_load(&w4[(int64_t)(sp + j) * nq + q]);
#pragma unroll
                for (int j = 0; j < kUnroll; ++j) s += t[j];
            }
            if (sp < splits) {  // the last < kUnroll slices, loaded together, added in order
                v4f t[kUnroll - 1];
#pragma unroll
                for (int j = 0; j < kUnroll - 1; ++j)
                    if (sp + j < splits) t[j] = __builtin_nontemporal_load(&w4[(int64_t)(sp + j) * nq + q]);
#pragma unroll
                for (int j = 0; j < kUnroll - 1; ++j)
                    if (sp + j < splits) s += t[j];
            }
            v4f y = s * scale;
            const int64_t idx = 4 * q;
            if (chan) {
                const int64_t row = idx / N, col = idx - row * N;
                const float a = sA[row];
                y.x *= a * sB[col];
                y.y *= a * sB[col + 1];
                y.z *= a * sB[col + 2];
                y.w *= a * sB[col + 3];
            }
            store4<OUT>(C, idx, y, eflags);
        }
    } else {
        for (int64_t i = tid; i < mn; i += stride) {
            float s = ws[i];
            int sp = 1;
            for (; sp + kUnroll <= splits; sp += kUnroll) {
                float t[kUnroll];
#pragma unroll
                for (int j = 0; j < kUnroll; ++j) t[j] = ws[(int64_t)(sp + j) * mn + i];
#pragma unroll
                for (int j = 0; j < kUnroll; ++j) s += t[j];
            }
            if (sp < splits) {
                float t[kUnroll - 1];
#pragma unroll
                for (int j = 0; j < kUnroll - 1; ++j)
                    if (sp + j < splits) t[j] = ws[(int64_t)(sp + j) * mn + i];
#pragma unroll
                for (int j = 0; j < kUnroll - 1; ++j)
                    if (sp + j < splits) s += t[j];
            }
            float y = s * scale;
            if (chan) {
                const int64_t row = i / N;
                y *= sA[row] * sB[i - row * N];
            }
            store1<OUT>(C, i, y, eflags);
        }
    }
}

}  // namespace

hipError_t launch_splitk_reduce(const GemmArgs& a) {
    const int64_t mn = a.M * a.N;
    if (mn <= 0) return hipSuccess;
    if (a.splits < 1 || !a.ws) return hipErrorInvalidValue;
    const int es = a.out_dtype == OUT_F32 ? 4 : (a.out_dtype == OUT_F16 ? 2 : 1);
    const int vec = (a.N % 4 == 0) && ((uintptr_t)a.ws % 16 == 0) && ((uintptr_t)a.C % (4 * es) == 0);
    int64_t g = ((vec ? mn / 4 : mn) + kThreads - 1) / kThreads;
    if (g > 4096) g = 4096;
    if (g < 1) g = 1;
    const int eflags = (a.out_dtype == OUT_E5M2 ? EPI_E5M2 : 0) | (a.channel ? EPI_CHANNEL : 0);
    switch (a.out_dtype) {
        case OUT_F32:
            splitk_reduce_kernel<OUT_F32><<<(unsigned)g, kThreads, 0, a.stream>>>(a.ws, a.splits, a.M, a.N, a.C, a.sA,
                                                                                 a.sB, a.sOut, eflags, vec);
            break;
        case OUT_F16:
            splitk_reduce_kernel<OUT_F16><<<(unsigned)g, kThreads, 0, a.stream>>>(a.ws, a.splits, a.M, a.N, a.C, a.sA,
                                                                                 a.sB, a.sOut, eflags, vec);
            break;
        default:
            splitk_reduce_kernel<OUT_E4M3><<<(unsigned)g, kThreads, 0, a.stream>>>(a.ws, a.splits, a.M, a.N, a.C,
                                                                                  a.sA, a.sB, a.sOut, eflags, vec);
    }
    return hipGetLastError();
}

}  // namespace libgemm
