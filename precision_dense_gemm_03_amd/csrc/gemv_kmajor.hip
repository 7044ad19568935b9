// Decode GEMM with a K-major weight, M <= 8:
//   C[M,N] = (sA*A[M,K]) (sB*B)  with B given as Bt[N,K] row-major,
// the layout in which a linear layer keeps its weight (element (k, n) of B at
// n*K + k).
//
// The [1,4096] x [4096,12288] projection of the DeepGEMM deep-dive article
// (hnwysp.cn news 84236, §2.1 "weight-aware tiling", §4.1) does about one
// flop per weight byte, so it is bound by HBM bandwidth. The article also
// stores the weight in a layout chosen for the kernel instead of plain
// row-major (§3.2, "Data Layout"); with B K-major every output element is one
// dot product over a contiguous weight row, so:
//   - each wave owns R consecutive weight rows (output columns) and its 64
//     lanes walk K in 16-byte chunks (lane l takes chunks l, l+64, ...): every
//     wave load instruction reads 1 KiB of one row, U of them per row in
//     flight, and no lane exchanges data until the end;
//   - the M activation rows are 16-byte vector loads shared by all waves (L1
//     and L2 hits);
//   - FP16 products are summed by v_dot2_f32_f16 (FP32 sum of two exact
//     products), FP8 codes are widened to FP32 and summed by FMA; each chunk
//     is summed on its own and then added to the lane's running sum;
//   - the 64 lane sums of each (m, row) are combined by a butterfly of
//     cross-lane shuffles in a fixed order (deterministic), then the epilogue
//     applies sA*sB (or the per-channel scales) and converts (FP8 guide §3.2).
// A second, cooperative kernel gives each workgroup R weight rows read by all
// of its W waves together (each workgroup load instruction covers W KiB of one
// row); the waves' sums meet in LDS. It streams the FP16 M = 1 weight fastest.
// No workgroup shares work with another, so there is no second launch and no
// cross-workgroup reduction.
#include "device_common.h"
#include "kernels.h"

namespace libgemm {

namespace {

typedef _Float16 v2h __attribute__((ext_vector_type(2)));

// Two FP8 codes (the low or high half HI of a 32-bit word) as floats, format F.
template <int F, bool HI>
__device__ __forceinline__ auto fp8x2(uint32_t w) {
    if constexpr (F == FMT_E5M2) return __builtin_amdgcn_cvt_pk_f32_bf8((int)w, HI);
    else return __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
}

// Sum over the 8 (FP16) or 16 (FP8, formats FA and FB) products of two
// 16-byte chunks, in FP32.
template <int ES, int FA, int FB>
__device__ __forceinline__ float chunk_dot(const v4u& a, const v4u& b) {
    const uint32_t wa[4] = {a.x, a.y, a.z, a.w};
    const uint32_t wb[4] = {b.x, b.y, b.z, b.w};
    float s = 0.0f;
    if constexpr (ES == 2) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            s = __builtin_amdgcn_fdot2(__builtin_bit_cast(v2h, wa[q]), __builtin_bit_cast(v2h, wb[q]), s, false);
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const auto alo = fp8x2<FA, false>(wa[q]);
            const auto ahi = fp8x2<FA, true>(wa[q]);
            const auto blo = fp8x2<FB, false>(wb[q]);
            const auto bhi = fp8x2<FB, true>(wb[q]);
            s = fmaf(alo[0], blo[0], s);
            s = fmaf(alo[1], blo[1], s);
            s = fmaf(ahi[0], bhi[0], s);
            s = fmaf(ahi[1], bhi[1], s);
        }
    }
    return s;
}

// One element (FP16 value, or FP8 code of format F) as a float.
template <int ES, int F>
__device__ __forceinline__ float elem(const uint8_t* p, int64_t idx) {
    if constexpr (ES == 2) return (float)reinterpret_cast<const _Float16*>(p)[idx];
    else return fp8x2<F, false>((uint32_t)p[idx])[0];
}

// ES: element bytes (2 FP16, 1 FP8). MMAX: largest M served. R: weight rows
// per wave. U: 16-byte chunks of each row in flight per lane. NT: threads per
// workgroup. FA, FB: FP8 formats of A and B (0 for FP16).
template <int ES, int MMAX, int R, int U, int NT, int FA, int FB>
__global__ __launch_bounds__(NT) void gemv_kmajor_kernel(const uint8_t* __restrict__ A,
                                                               const uint8_t* __restrict__ B, void* __restrict__ C,
                                                               int M, int N, int64_t K, const float* __restrict__ sA,
                                                               const float* __restrict__ sB,
                                                               const float* __restrict__ sOut, int out_dtype,
                                                               int vec, int eflags) {
    constexpr int VE = 16 / ES;
    const int lane = threadIdx.x & 63;
    const int64_t n0l = ((int64_t)blockIdx.x * (NT / 64) + (threadIdx.x >> 6)) * R;
    if (n0l >= N) return;  // the whole wave leaves together
    const int n0 = (int)n0l;

    float acc[MMAX][R];
#pragma unroll
    for (int m = 0; m < MMAX; ++m)
#pragma unroll
        for (int r = 0; r < R; ++r) acc[m][r] = 0.0f;

    // Rows past N re-read row N-1 (valid addresses; never stored).
    const uint8_t* brow[R];
#pragma unroll
    for (int r = 0; r < R; ++r) brow[r] = B + min((int64_t)n0 + r, (int64_t)N - 1) * K * ES;

    // Whole 16-byte chunks of a row (vector path: aligned bases, K*ES % 16 == 0).
    const int64_t nchunks = vec ? K / VE : 0;
    int64_t c = lane;
    for (; c + (U - 1) * 64 < nchunks; c += U * 64) {
        v4u bv[U][R];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int r = 0; r < R; ++r)
                bv[u][r] = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(brow[r] + (c + u * 64) * 16));
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int m = 0; m < MMAX; ++m) {
                if (m < M) {
                    const v4u av = *reinterpret_cast<const v4u*>(A + ((int64_t)m * K + (c + u * 64) * VE) * ES);
#pragma unroll
                    for (int r = 0; r < R; ++r) acc[m][r] += chunk_dot<ES, FA, FB>(av, bv[u][r]);
                }
            }
    }
    for (; c < nchunks; c += 64) {
#pragma unroll
        for (int m = 0; m < MMAX; ++m) {
            if (m < M) {
                const v4u av = *reinterpret_cast<const v4u*>(A + ((int64_t)m * K + c * VE) * ES);
#pragma unroll
                for (int r = 0; r < R; ++r)
                    acc[m][r] += chunk_dot<ES, FA, FB>(av, *reinterpret_cast<const v4u*>(brow[r] + c * 16));
            }
        }
    }
    // Elements after the whole chunks (all of K on the unaligned path).
    for (int64_t k = nchunks * VE + lane; k < K; k += 64) {
#pragma unroll
        for (int m = 0; m < MMAX; ++m) {
            if (m < M) {
                const float a = elem<ES, FA>(A, (int64_t)m * K + k);
#pragma unroll
                for (int r = 0; r < R; ++r) acc[m][r] = fmaf(a, elem<ES, FB>(brow[r], k), acc[m][r]);
            }
        }
    }

    // Butterfly over the 64 lanes: afterwards every lane holds every total.
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
#pragma unroll
        for (int m = 0; m < MMAX; ++m)
#pragma unroll
            for (int r = 0; r < R; ++r) acc[m][r] += __shfl_xor(acc[m][r], off, 64);

    const bool channel = (eflags & EPI_CHANNEL) != 0;
    const float scale = epilogue_base(sA, sB, sOut, out_dtype == OUT_E4M3 || out_dtype == OUT_E5M2, channel);
#pragma unroll
    for (int m = 0; m < MMAX; ++m)
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int64_t n = (int64_t)n0 + r;
            if (lane == m * R + r && m < M && n < N) {
                float y = acc[m][r] * scale;
                if (channel) y *= sA[m] * sB[n];
                store_out(C, (int64_t)m * N + n, y, out_dtype);
            }
        }
}

// Workgroup-cooperative variant: the W waves of a workgroup read the same R
// weight rows together (wave w takes chunks w*64 + lane + i*64*W), so each
// workgroup load instruction covers W KiB of one row; the per-wave sums meet
// in LDS, added in wave order.
template <int ES, int MMAX, int R, int W, int FA, int FB>
__global__ __launch_bounds__(64 * W) void gemv_kmajor_coop_kernel(const uint8_t* __restrict__ A,
                                                                  const uint8_t* __restrict__ B,
                                                                  void* __restrict__ C, int M, int N, int64_t K,
                                                                  const float* __restrict__ sA,
                                                                  const float* __restrict__ sB,
                                                                  const float* __restrict__ sOut, int out_dtype,
                                                                  int vec, int eflags) {
    constexpr int VE = 16 / ES;
    __shared__ float red[W][MMAX * R];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n0 = (int)((int64_t)blockIdx.x * R);  // < N: the grid has ceil(N / R) blocks

    float acc[MMAX][R];
#pragma unroll
    for (int m = 0; m < MMAX; ++m)
#pragma unroll
        for (int r = 0; r < R; ++r) acc[m][r] = 0.0f;
    const uint8_t* brow[R];
#pragma unroll
    for (int r = 0; r < R; ++r) brow[r] = B + min((int64_t)n0 + r, (int64_t)N - 1) * K * ES;

    const int64_t nchunks = vec ? K / VE : 0;
    for (int64_t c = wave * 64 + lane; c < nchunks; c += 64 * W) {
        v4u bv[R];
#pragma unroll
        for (int r = 0; r < R; ++r) bv[r] = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(brow[r] + c * 16));
#pragma unroll
        for (int m = 0; m < MMAX; ++m) {
            if (m < M) {
                const v4u av = *reinterpret_cast<const v4u*>(A + ((int64_t)m * K + c * VE) * ES);
#pragma unroll
                for (int r = 0; r < R; ++r) acc[m][r] += chunk_dot<ES, FA, FB>(av, bv[r]);
            }
        }
    }
    for (int64_t k = nchunks * VE + wave * 64 + lane; k < K; k += 64 * W) {
#pragma unroll
        for (int m = 0; m < MMAX; ++m) {
            if (m < M) {
                const float a = elem<ES, FA>(A, (int64_t)m * K + k);
#pragma unroll
                for (int r = 0; r < R; ++r) acc[m][r] = fmaf(a, elem<ES, FB>(brow[r], k), acc[m][r]);
            }
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
#pragma unroll
        for (int m = 0; m < MMAX; ++m)
#pragma unroll
            for (int r = 0; r < R; ++r) acc[m][r] += __shfl_xor(acc[m][r], off, 64);
    if (lane == 0) {
#pragma unroll
        for (int m = 0; m < MMAX; ++m)
#pragma unroll
            for (int r = 0; r < R; ++r) red[wave][m * R + r] = acc[m][r];
    }
    __syncthreads();
    const bool channel = (eflags & EPI_CHANNEL) != 0;
    const float scale = epilogue_base(sA, sB, sOut, out_dtype == OUT_E4M3 || out_dtype == OUT_E5M2, channel);
    for (int o = threadIdx.x; o < MMAX * R; o += 64 * W) {
        const int m = o / R, r = o % R;
        const int64_t n = (int64_t)n0 + r;
        float sum = red[0][o];
#pragma unroll
        for (int w = 1; w < W; ++w) sum += red[w][o];
        if (m < M && n < N) {
            float y = sum * scale;
            if (channel) y *= sA[m] * sB[n];
            store_out(C, (int64_t)m * N + n, y, out_dtype);
        }
    }
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

template <int ES, int MMAX, int R, int W, int FA = 0, int FB = 0>
hipError_t launch_gemv_kmajor_coop(const GemmArgs& a) {
    if (a.M <= 0 || a.N <= 0) return hipSuccess;
    if (a.M > MMAX || !a.b_kmajor || a.splits > 1) return hipErrorInvalidValue;
    if (ES == 1 && (a.fmt_a != FA || a.fmt_b != FB)) return hipErrorInvalidValue;
    const int64_t blocks = (a.N + R - 1) / R;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    const int vec = aligned16(a.A) && aligned16(a.B) && ((a.K * ES) % 16 == 0);
    const int eflags = a.channel ? EPI_CHANNEL : 0;
    gemv_kmajor_coop_kernel<ES, MMAX, R, W, FA, FB><<<(unsigned)blocks, 64 * W, 0, a.stream>>>(
        reinterpret_cast<const uint8_t*>(a.A), reinterpret_cast<const uint8_t*>(a.B), a.C, (int)a.M, (int)a.N, a.K,
        a.sA, a.sB, a.sOut, a.out_dtype, vec, eflags);
    return hipGetLastError();
}

template <int ES, int MMAX, int R, int U, int NT = 256, int FA = 0, int FB = 0>
hipError_t launch_gemv_kmajor(const GemmArgs& a) {
    static_assert(MMAX * R <= 64, "one lane stores each output");
    if (a.M <= 0 || a.N <= 0) return hipSuccess;
    if (a.M > MMAX || !a.b_kmajor || a.splits > 1) return hipErrorInvalidValue;
    if (ES == 1 && (a.fmt_a != FA || a.fmt_b != FB)) return hipErrorInvalidValue;
    constexpr int rows_per_block = (NT / 64) * R;
    const int64_t blocks = (a.N + rows_per_block - 1) / rows_per_block;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    const int vec = aligned16(a.A) && aligned16(a.B) && ((a.K * ES) % 16 == 0);
    const int eflags = a.channel ? EPI_CHANNEL : 0;
    gemv_kmajor_kernel<ES, MMAX, R, U, NT, FA, FB><<<(unsigned)blocks, NT, 0, a.stream>>>(
        reinterpret_cast<const uint8_t*>(a.A), reinterpret_cast<const uint8_t*>(a.B), a.C, (int)a.M, (int)a.N, a.K,
        a.sA, a.sB, a.sOut, a.out_dtype, vec, eflags);
    return hipGetLastError();
}

// FP8 operand-format dispatch (every pair of E4M3 / E5M2).
template <int MMAX, int R, int U>
hipError_t launch_gemv_kmajor_fp8(const GemmArgs& a) {
    switch (a.fmt_a * 2 + a.fmt_b) {
        case 0: return launch_gemv_kmajor<1, MMAX, R, U, 256, 0, 0>(a);
        case 1: return launch_gemv_kmajor<1, MMAX, R, U, 256, 0, 1>(a);
        case 2: return launch_gemv_kmajor<1, MMAX, R, U, 256, 1, 0>(a);
        default: return launch_gemv_kmajor<1, MMAX, R, U, 256, 1, 1>(a);
    }
}

template <int MMAX, int R, int W>
hipError_t launch_gemv_kmajor_coop_fp8(const GemmArgs& a) {
    switch (a.fmt_a * 2 + a.fmt_b) {
        case 0: return launch_gemv_kmajor_coop<1, MMAX, R, W, 0, 0>(a);
        case 1: return launch_gemv_kmajor_coop<1, MMAX, R, W, 0, 1>(a);
        case 2: return launch_gemv_kmajor_coop<1, MMAX, R, W, 1, 0>(a);
        default: return launch_gemv_kmajor_coop<1, MMAX, R, W, 1, 1>(a);
    }
}

}  // namespace

// bm = largest M served, bn = weight rows per workgroup, bk = chunks in flight
// per lane and row (per-wave kernel) or waves per workgroup (cooperative
// kernel). For each bound M the first entry is the selector's choice.
// Measured on MI355X (weights rotated over enough copies to miss the 256 MB
// Infinity Cache; us): FP16 [M,4096] x [4096,12288]: M = 1 cooperative 4 rows
// x 8 waves 16.1-16.5 (6.2 TB/s) vs per-wave 4 rows x 4 chunks 18.3, 3 x 4
// 17.5, cooperative 16 waves 21.1; M = 4 per-wave 2 rows x 4 chunks 24.7, 4 x
// 2 26.6, 4 x 4 25.5, 8 x 2 35.6, cooperative 31.1; M = 8 per-wave 4 x 2 35.7,
// 2 x 2 37.5, cooperative 56.1, the 64x64 MFMA tile 53.4. At M = 16 every
// variant tried (57-87) lost to the 64x64 tile (53.4) and to split-K over it
// (22.9), so decode kernels stop at M = 8.
// E4M3 [M,4096] x [4096,4096]: M = 1 10.0 for every variant tried (launch and
// latency bound at 16 MB); M = 4 cooperative 10.4 vs per-wave 14.8; M = 8
// cooperative 14.7 vs per-wave 16.5 and the 64x64 tile 28.9.
// The table lives in a host function so that the kernels it names are
// instantiated for the device while the table itself stays host data.
const GemmConfig* gemv_kmajor_configs(int* count) {
    static const GemmConfig table[] = {
        {"gemv_coop_f16_m1_r4_w8", KIND_F16, 3, 1, 4, 8, launch_gemv_kmajor_coop<2, 1, 4, 8>, 0, 0, 1},
        {"gemv_bt_f16_m1_r4_u4", KIND_F16, 3, 1, 16, 4, launch_gemv_kmajor<2, 1, 4, 4>, 0, 0, 1},
        {"gemv_bt_f16_m4_r2_u4", KIND_F16, 3, 4, 8, 4, launch_gemv_kmajor<2, 4, 2, 4>, 0, 0, 1},
        {"gemv_bt_f16_m4_r4_u2", KIND_F16, 3, 4, 16, 2, launch_gemv_kmajor<2, 4, 4, 2>, 0, 0, 1},
        {"gemv_coop_f16_m4_r2_w8", KIND_F16, 3, 4, 2, 8, launch_gemv_kmajor_coop<2, 4, 2, 8>, 0, 0, 1},
        {"gemv_bt_f16_m8_r4_u2", KIND_F16, 3, 8, 16, 2, launch_gemv_kmajor<2, 8, 4, 2>, 0, 0, 1},
        {"gemv_bt_f16_m8_r2_u2", KIND_F16, 3, 8, 8, 2, launch_gemv_kmajor<2, 8, 2, 2>, 0, 0, 1},
        // E4M3 M = 1, N = K = 4096, rotated cold weights: one row per wave
        // (1024 workgroups) 11.05 us, two 11.15, four 12.12
        {"gemv_bt_fp8_m1_r1_u4", KIND_FP8, 3, 1, 4, 4, launch_gemv_kmajor_fp8<1, 1, 4>, kAllFp8Pairs, 0, 1},
        {"gemv_bt_fp8_m1_r2_u4", KIND_FP8, 3, 1, 8, 4, launch_gemv_kmajor_fp8<1, 2, 4>, kAllFp8Pairs, 0, 1},
        {"gemv_bt_fp8_m1_r4_u4", KIND_FP8, 3, 1, 16, 4, launch_gemv_kmajor_fp8<1, 4, 4>, kAllFp8Pairs, 0, 1},
        {"gemv_coop_fp8_m1_r4_w4", KIND_FP8, 3, 1, 4, 4, launch_gemv_kmajor_coop_fp8<1, 4, 4>, kAllFp8Pairs, 0, 1},
        {"gemv_coop_fp8_m4_r4_w4", KIND_FP8, 3, 4, 4, 4, launch_gemv_kmajor_coop_fp8<4, 4, 4>, kAllFp8Pairs, 0, 1},
        {"gemv_bt_fp8_m4_r4_u2", KIND_FP8, 3, 4, 16, 2, launch_gemv_kmajor_fp8<4, 4, 2>, kAllFp8Pairs, 0, 1},
        {"gemv_coop_fp8_m8_r2_w4", KIND_FP8, 3, 8, 2, 4, launch_gemv_kmajor_coop_fp8<8, 2, 4>, kAllFp8Pairs, 0, 1},
        {"gemv_bt_fp8_m8_r2_u2", KIND_FP8, 3, 8, 8, 2, launch_gemv_kmajor_fp8<8, 2, 2>, kAllFp8Pairs, 0, 1},
    };
    *count = (int)(sizeof(table) / sizeof(table[0]));
    return table;
}

}  // namespace libgemm
