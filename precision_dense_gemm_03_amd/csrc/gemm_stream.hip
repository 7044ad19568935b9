// HBM-streaming GEMM for decode shapes, M <= 16: C[M,N] = (sA*A[M,K]) (sB*B[K,N]).
//
// At M = 1 the [1,4096] x [4096,12288] projection of the DeepGEMM deep-dive
// article (hnwysp.cn news 84236, §2.1 "weight-aware tiling", §4.1) reads each
// weight once and does 1 flop per byte, so it is bound by HBM bandwidth, not
// by the matrix units. The article keeps B out of shared memory and
// broadcasts the A row to every worker; this kernel does the same on gfx950:
//   - every lane owns one 16-byte column chunk of B (8 fp16 / 16 fp8 columns)
//     and a slice of K; B is read exactly once with 16-byte loads, U rows in
//     flight per lane, so a wave reads full 128-byte row segments;
//   - the A values a lane needs (M rows x U consecutive k) are vector loads
//     shared by all lanes of the wave (an L1 broadcast);
//   - products accumulate in FP32 (fma), one partial sum per (m, column) per
//     K slice; slices are reduced inside the wave with cross-lane shuffles and
//     across waves through LDS in a fixed order (deterministic), then the
//     epilogue applies sA*sB and converts (FP8 guide §3.2).
#include "device_common.h"
#include "kernels.h"

namespace libgemm {

namespace {

// Two FP8 codes (the low or high half HI of a 32-bit word) to floats, in format F.
template <int F, bool HI>
__device__ __forceinline__ auto fp8x2_to_f32(uint32_t w) {
    if constexpr (F == FMT_E5M2) return __builtin_amdgcn_cvt_pk_f32_bf8((int)w, HI);
    else return __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
}

template <int ES, int F>
__device__ __forceinline__ void decode16(const v4u& v, float (&out)[16 / ES]) {
    if constexpr (ES == 2) {
        const v8h h = __builtin_bit_cast(v8h, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) out[e] = (float)h[e];
    } else {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            auto lo = fp8x2_to_f32<F, false>(w[q]);
            auto hi = fp8x2_to_f32<F, true>(w[q]);
            out[4 * q + 0] = lo[0];
            out[4 * q + 1] = lo[1];
            out[4 * q + 2] = hi[0];
            out[4 * q + 3] = hi[1];
        }
    }
}

template <int ES, int F>
__device__ __forceinline__ float decode1(const uint8_t* p, int64_t idx) {
    if constexpr (ES == 2) {
        return (float)reinterpret_cast<const _Float16*>(p)[idx];
    } else {
        auto v = fp8x2_to_f32<F, false>((uint32_t)p[idx]);
        return v[0];
    }
}

// NT threads; each owns a 16-byte column chunk (VE columns) and a K slice.
// CX = COLS / VE chunks across, KY = NT / CX slices down. Lane order inside a
// wave is cx fastest, so one wave covers (64 / CX) slices of a full
// COLS-wide row segment.
template <int ES, int MMAX, int COLS, int NT, int U, int FA, int FB>
__global__ __launch_bounds__(NT) void gemm_stream_kernel(const uint8_t* __restrict__ A,
                                                         const uint8_t* __restrict__ B, void* __restrict__ C,
                                                         int64_t M, int64_t N, int64_t K,
                                                         const float* __restrict__ sA, const float* __restrict__ sB,
                                                         const float* __restrict__ sOut, int out_dtype, int a_vec,
                                                         int b_vec, int eflags, int64_t kchunk) {
    constexpr int VE = 16 / ES;
    constexpr int CX = COLS / VE;
    constexpr int KY = NT / CX;
    constexpr int NW = NT / 64;
    constexpr int SLW = 64 / CX;  // K slices per wave
    static_assert(COLS % VE == 0 && NT % CX == 0 && 64 % CX == 0, "bad stream shape");

    const int tid = threadIdx.x;
    const int cx = tid % CX;
    const int ky = tid / CX;
    const int64_t n0 = (int64_t)blockIdx.x * COLS;
    const int64_t ncol = n0 + (int64_t)cx * VE;  // first column of this lane's chunk
    // Split-K: workgroup row blockIdx.y sums K range [kbeg, kend) (all of K
    // when the launch is not split); kbeg is a multiple of KY * U.
    const int64_t kbeg = (int64_t)blockIdx.y * kchunk;
    const int64_t kend = min(K, kbeg + kchunk);

    float acc[MMAX][VE];
#pragma unroll
    for (int m = 0; m < MMAX; ++m)
#pragma unroll
        for (int e = 0; e < VE; ++e) acc[m][e] = 0.0f;

    const bool chunk_full = b_vec && (ncol + VE <= N);
    for (int64_t kb = kbeg + (int64_t)ky * U; kb < kend; kb += (int64_t)KY * U) {
        // B rows kb .. kb+U-1 of this lane's chunk (zero beyond K / N).
        v4u braw[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t k = kb + u;
            if (chunk_full && k < kend) {
                braw[u] = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(B + (k * N + ncol) * ES));
            } else {
                union {
                    v4u v;
                    uint8_t b[16];
                    uint16_t h[8];
                } t;
                t.v = v4u{0u, 0u, 0u, 0u};
                if (k < kend) {
#pragma unroll
                    for (int e = 0; e < VE; ++e) {
                        if (ncol + e < N) {
                            if (ES == 2) t.h[e] = reinterpret_cast<const uint16_t*>(B)[k * N + ncol + e];
                            else t.b[e] = B[k * N + ncol + e];
                        }
                    }
                }
                braw[u] = t.v;
            }
        }
        // A[m][kb .. kb+U-1] as floats (zero beyond M / K).
        float a[MMAX][U];
#pragma unroll
        for (int m = 0; m < MMAX; ++m) {
            if (m < M) {
                if (a_vec && kb + U <= kend) {
                    static_assert(U % 8 == 0, "A vector loads cover 8 elements");
#pragma unroll
                    for (int g8 = 0; g8 < U / 8; ++g8) {
                        if constexpr (ES == 2) {
                            const v8h h = __builtin_bit_cast(
                                v8h, *reinterpret_cast<const v4u*>(A + (m * K + kb + 8 * g8) * 2));
#pragma unroll
                            for (int u = 0; u < 8; ++u) a[m][8 * g8 + u] = (float)h[u];
                        } else {
                            const uint2 w = *reinterpret_cast<const uint2*>(A + m * K + kb + 8 * g8);
                            const uint32_t ww[2] = {w.x, w.y};
#pragma unroll
                            for (int q = 0; q < 2; ++q) {
                                auto lo = fp8x2_to_f32<FA, false>(ww[q]);
                                auto hi = fp8x2_to_f32<FA, true>(ww[q]);
                                a[m][8 * g8 + 4 * q + 0] = lo[0];
                                a[m][8 * g8 + 4 * q + 1] = lo[1];
                                a[m][8 * g8 + 4 * q + 2] = hi[0];
                                a[m][8 * g8 + 4 * q + 3] = hi[1];
                            }
                        }
                    }
                } else {
#pragma unroll
                    for (int u = 0; u < U; ++u) a[m][u] = (kb + u < kend) ? decode1<ES, FA>(A, m * K + kb + u) : 0.0f;
                }
            } else {
#pragma unroll
                for (int u = 0; u < U; ++u) a[m][u] = 0.0f;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float b[VE];
            decode16<ES, FB>(braw[u], b);
#pragma unroll
            for (int m = 0; m < MMAX; ++m)
#pragma unroll
                for (int e = 0; e < VE; ++e) acc[m][e] = fmaf(a[m][u], b[e], acc[m][e]);
        }
    }

    // Reduce the K slices inside the wave: lanes cx + CX*s (s = 0..SLW-1).
#pragma unroll
    for (int off = CX; off < 64; off <<= 1) {
#pragma unroll
        for (int m = 0; m < MMAX; ++m)
#pragma unroll
            for (int e = 0; e < VE; ++e) acc[m][e] += __shfl_xor(acc[m][e], off, 64);
    }
    // Across waves through LDS, in wave order.
    __shared__ float red[NW][MMAX][COLS];
    const int lane = tid & 63, wave = tid >> 6;
    if (lane < CX) {
#pragma unroll
        for (int m = 0; m < MMAX; ++m)
#pragma unroll
            for (int e = 0; e < VE; ++e) red[wave][m][lane * VE + e] = acc[m][e];
    }
    __syncthreads();
    // per-channel scales (sA[M], sB[N]) are applied per stored element; a
    // split-K partial (EPI_PARTIAL) stores the raw FP32 sum into its split's
    // [M, N] slice of the workspace C
    const bool partial = (eflags & EPI_PARTIAL) != 0;
    if (partial) {
        C = reinterpret_cast<float*>(C) + (int64_t)blockIdx.y * M * N;
        out_dtype = OUT_F32;
    }
    const bool channel = !partial && (eflags & EPI_CHANNEL) != 0;
    const float scale = partial ? 1.0f
                                : epilogue_base(sA, sB, sOut, out_dtype == OUT_E4M3 || out_dtype == OUT_E5M2, channel);

    for (int o = tid; o < MMAX * COLS; o += NT) {
        const int m = o / COLS, c = o % COLS;
        float s = red[0][m][c];
#pragma unroll
        for (int w = 1; w < NW; ++w) s += red[w][m][c];
        const int64_t col = n0 + c;
        if (m < M && col < N) {
            float y = s * scale;
            if (channel) y *= sA[m] * sB[col];
            store_out(C, (int64_t)m * N + col, y, out_dtype);
        }
    }
    (void)SLW;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// K rows one pass of a workgroup covers: the split-K granularity.
template <int ES, int COLS, int NT, int U>
constexpr int stream_kgran() {
    return NT / (COLS / (16 / ES)) * U;
}

template <int ES, int MMAX, int COLS, int NT, int U, int FA = 0, int FB = 0>
hipError_t launch_stream(const GemmArgs& a) {
    const int64_t blocks = (a.N + COLS - 1) / COLS;
    if (blocks <= 0 || a.M <= 0) return hipSuccess;
    if (blocks > 0x7FFFFFFF || a.M > MMAX) return hipErrorInvalidValue;
    const int splits = a.splits > 1 ? a.splits : 1;
    constexpr int kgran = stream_kgran<ES, COLS, NT, U>();
    if (splits > 1 && (a.k_chunk % kgran != 0 || a.k_chunk <= 0 || (int64_t)(splits - 1) * a.k_chunk >= a.K ||
                       splits > 65535 || !a.ws))
        return hipErrorInvalidValue;
    const int a_vec = aligned16(a.A) && ((a.K * ES) % 16 == 0);
    const int b_vec = aligned16(a.B) && ((a.N * ES) % 16 == 0);
    const int eflags = splits > 1 ? EPI_PARTIAL : (a.channel ? EPI_CHANNEL : 0);
    const dim3 grid((unsigned)blocks, (unsigned)splits);
    gemm_stream_kernel<ES, MMAX, COLS, NT, U, FA, FB><<<grid, NT, 0, a.stream>>>(
        reinterpret_cast<const uint8_t*>(a.A), reinterpret_cast<const uint8_t*>(a.B), splits > 1 ? a.ws : a.C, a.M,
        a.N, a.K, a.sA, a.sB, a.sOut, a.out_dtype, a_vec, b_vec, eflags, splits > 1 ? a.k_chunk : a.K);
    return hipGetLastError();
}

// FP8 operand-format dispatch.
template <int MMAX, int COLS, int NT, int U>
hipError_t launch_stream_fp8_any(const GemmArgs& a) {
    switch (a.fmt_a * 2 + a.fmt_b) {
        case 0: return launch_stream<1, MMAX, COLS, NT, U, 0, 0>(a);
        case 1: return launch_stream<1, MMAX, COLS, NT, U, 0, 1>(a);
        case 2: return launch_stream<1, MMAX, COLS, NT, U, 1, 0>(a);
        default: return launch_stream<1, MMAX, COLS, NT, U, 1, 1>(a);
    }
}

}  // namespace

// bm = largest M served, bn = columns per workgroup, bk = threads per workgroup.
// The table lives in a host function so that the kernels it names are
// instantiated for the device while the table itself stays host data.
const GemmConfig* stream_configs(int* count) {
    // The last field is the split-K granularity (K rows per workgroup pass).
    // For one bound M the first entry is the plain choice; the split-K plan
    // takes the one with the smallest granularity (fewer threads, so a K
    // range of a few hundred rows still keeps every lane busy).
    static const GemmConfig table[] = {
    {"stream_f16_m1_c64_t512", KIND_F16, 1, 1, 64, 512, launch_stream<2, 1, 64, 512, 8>, 0,
     stream_kgran<2, 64, 512, 8>()},
    {"stream_f16_m1_c64_t1024", KIND_F16, 1, 1, 64, 1024, launch_stream<2, 1, 64, 1024, 8>, 0,
     stream_kgran<2, 64, 1024, 8>()},
    {"stream_f16_m4_c64_t512", KIND_F16, 1, 4, 64, 512, launch_stream<2, 4, 64, 512, 8>, 0,
     stream_kgran<2, 64, 512, 8>()},
    {"stream_f16_m8_c64_t256", KIND_F16, 1, 8, 64, 256, launch_stream<2, 8, 64, 256, 8>, 0,
     stream_kgran<2, 64, 256, 8>()},
    {"stream_f16_m16_c64_t256", KIND_F16, 1, 16, 64, 256, launch_stream<2, 16, 64, 256, 8>, 0,
     stream_kgran<2, 64, 256, 8>()},
    {"stream_fp8_m1_c64_t1024", KIND_FP8, 1, 1, 64, 1024, launch_stream_fp8_any<1, 64, 1024, 8>, kAllFp8Pairs,
     stream_kgran<1, 64, 1024, 8>()},
    {"stream_fp8_m4_c64_t512", KIND_FP8, 1, 4, 64, 512, launch_stream_fp8_any<4, 64, 512, 8>, kAllFp8Pairs,
     stream_kgran<1, 64, 512, 8>()},
    {"stream_f16_m1_c64_t256", KIND_F16, 1, 1, 64, 256, launch_stream<2, 1, 64, 256, 8>, 0,
     stream_kgran<2, 64, 256, 8>()},

    {"stream_fp8_m1_c128_t256", KIND_FP8, 1, 1, 128, 256, launch_stream_fp8_any<1, 128, 256, 8>, kAllFp8Pairs,
     stream_kgran<1, 128, 256, 8>()},
    {"stream_fp8_m4_c128_t256", KIND_FP8, 1, 4, 128, 256, launch_stream_fp8_any<4, 128, 256, 8>, kAllFp8Pairs,
     stream_kgran<1, 128, 256, 8>()},
    };
    *count = (int)(sizeof(table) / sizeof(table[0]));
    return table;
}
}  // namespace libgemm
