// MFMA tile GEMM for gfx950: C[M,N] = (sA*A[M,K]) (sB*B[K,N]), all row-major.
//
// Operands are FP16 (v_mfma_f32_16x16x32_f16) or OCP E4M3 codes
// (v_mfma_scale_f32_16x16x128_f8f6f4 with neutral block scales), always with
// FP32 accumulation ("DeepGEMM实战：FP8矩阵乘法与JIT编译优化指南" §2.1;
// "HGEMM优化：深度学习中的矩阵乘法性能提升策略" §1.3).
//
// Data flow per workgroup (one BM x BN output tile):
//   HBM/L2 --16-byte coalesced loads--> registers --ds_write_b128--> LDS
//   (two stages: the next K tile is fetched while the current one is consumed;
//   FP8 guide §2.3 "double buffering", HGEMM §3.2/§3.3)
//   LDS --ds_read_b128 (A) / ds_read_b64_tr_b16|b8 (B)--> MFMA operands
// A is row-major [M,K]: its K-contiguous rows are exactly the MFMA A operand.
// B is row-major [K,N]: N is contiguous, so the B operand (8 or 32 consecutive
// k for one column per lane) is produced by gfx950's LDS transpose reads
// instead of a transposing copy. LDS rows are padded (A: +16 B, B: +16/32 B)
// so that the lanes served together by one LDS pass hit distinct banks
// (DeepGEMM deep-dive article §3.2 motivates the bank-aware layout).
//
// Edges (FP8 guide §3.3): rows >= M and columns >= N are neither loaded nor
// stored (predicated), the K tail is zero-filled in the staged tile, so one
// kernel serves every shape. The epilogue multiplies by sA*sB once and
// converts to FP32 / FP16 / E4M3 (FP8 guide §3.2, scales applied at write-back).
#include "device_common.h"
#include "kernels.h"

namespace libgemm {

namespace {

template <int ES, int BM, int BN, int BK, int WM, int WN>
struct Tile {
    static constexpr int NT = 64 * WM * WN;           // threads per workgroup
    static constexpr int KPI = ES == 2 ? 32 : 128;    // k per MFMA instruction
    static constexpr int OPB = ES == 2 ? 16 : 32;     // operand bytes per lane
    static constexpr int VE = 16 / ES;                // elements per 16-byte chunk
    static constexpr int BKB = BK * ES;               // bytes of one A tile row
    static constexpr int BNB = BN * ES;               // bytes of one B tile row
    static constexpr int SA = BKB + 16;               // padded LDS row strides
    static constexpr int SB = BNB + (ES == 2 ? 32 : 16);
    static constexpr int A_BYTES = BM * SA;
    static constexpr int B_BYTES = BK * SB;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int A_CPR = BKB / 16;            // 16-byte chunks per A row
    static constexpr int B_CPR = BNB / 16;
    static constexpr int CA = BM * A_CPR / NT;        // A chunks per thread
    static constexpr int CB = BK * B_CPR / NT;
    static constexpr int WTM = BM / WM, WTN = BN / WN;
    static constexpr int TM = WTM / 16, TN = WTN / 16;
    static constexpr int KS = BK / KPI;
    static_assert(BK % KPI == 0, "BK must be a multiple of the MFMA depth");
    static_assert((BM * A_CPR) % NT == 0 && (BK * B_CPR) % NT == 0, "tile chunks must divide evenly");
    static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile must be whole 16x16 blocks");
    static_assert(2 * STAGE <= 160 * 1024, "two stages must fit in LDS");
};

// Loads one 16-byte chunk of `ES`-byte elements starting at element `col` of a
// row, zero-filling elements at or beyond `limit`, and the whole chunk when the
// row is out of range. Used only on edges and for unaligned operands.
template <int ES>
__device__ __forceinline__ v4u load_chunk_guarded(const uint8_t* row_ptr, bool row_ok, int64_t col, int64_t limit) {
    union {
        v4u v;
        uint8_t b[16];
        uint16_t h[8];
    } u;
    u.v = v4u{0u, 0u, 0u, 0u};
    if (row_ok) {
        if (ES == 1) {
#pragma unroll
            for (int e = 0; e < 16; ++e)
                if (col + e < limit) u.b[e] = row_ptr[col + e];
        } else {
            const uint16_t* p = reinterpret_cast<const uint16_t*>(row_ptr);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (col + e < limit) u.h[e] = p[col + e];
        }
    }
    return u.v;
}

template <int ES, int BM, int BN, int BK, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN) void gemm_tile_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ B, void* __restrict__ C,
    int64_t M, int64_t N, int64_t K, const float* __restrict__ sA, const float* __restrict__ sB,
    const float* __restrict__ sOut, int out_dtype, int a_vec, int b_vec, int tiles_n) {
    using T = Tile<ES, BM, BN, BK, WM, WN>;
    __shared__ __attribute__((aligned(16))) uint8_t smem_raw[2 * T::STAGE];
    LDS_AS uint8_t* smem = (LDS_AS uint8_t*)smem_raw;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;

    const int64_t tile_m = blockIdx.x / tiles_n;
    const int64_t tile_n = blockIdx.x % tiles_n;
    const int64_t m0 = tile_m * BM;
    const int64_t n0 = tile_n * BN;

    v4u ra[T::CA];
    v4u rb[T::CB];

    // global -> registers for the K tile starting at k0
    auto gload = [&](int64_t k0) {
#pragma unroll
        for (int i = 0; i < T::CA; ++i) {
            const int c = tid + T::NT * i;
            const int row = c / T::A_CPR, col = c % T::A_CPR;
            const int64_t gm = m0 + row;
            const int64_t gk = k0 + (int64_t)col * T::VE;
            const uint8_t* rp = A + gm * K * ES;
            if (a_vec && gm < M && gk + T::VE <= K)
                ra[i] = *reinterpret_cast<const v4u*>(rp + gk * ES);
            else
                ra[i] = load_chunk_guarded<ES>(rp, gm < M, gk, K);
        }
#pragma unroll
        for (int i = 0; i < T::CB; ++i) {
            const int c = tid + T::NT * i;
            const int row = c / T::B_CPR, col = c % T::B_CPR;
            const int64_t gk = k0 + row;
            const int64_t gn = n0 + (int64_t)col * T::VE;
            const uint8_t* rp = B + gk * N * ES;
            if (b_vec && gk < K && gn + T::VE <= N)
                rb[i] = *reinterpret_cast<const v4u*>(rp + gn * ES);
            else
                rb[i] = load_chunk_guarded<ES>(rp, gk < K, gn, N);
        }
    };
    // registers -> LDS stage `buf`
    auto sstore = [&](int buf) {
        LDS_AS uint8_t* As = smem + buf * T::STAGE;
        LDS_AS uint8_t* Bs = As + T::A_BYTES;
#pragma unroll
        for (int i = 0; i < T::CA; ++i) {
            const int c = tid + T::NT * i;
            const int row = c / T::A_CPR, col = c % T::A_CPR;
            *(LDS_AS v4u*)(As + row * T::SA + col * 16) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < T::CB; ++i) {
            const int c = tid + T::NT * i;
            const int row = c / T::B_CPR, col = c % T::B_CPR;
            *(LDS_AS v4u*)(Bs + row * T::SB + col * 16) = rb[i];
        }
    };

    v4f acc[T::TM][T::TN];
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int j = 0; j < T::TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    // Per-lane LDS offsets that do not depend on the k step.
    const int g = lane >> 4;   // 16-lane group: selects the k sub-range of the operand
    const int j16 = lane & 15; // lane within its group
    const int a_row0 = wm * T::WTM + j16;
    // B transpose-read address pattern (see the lane maps measured for
    // ds_read_b64_tr_b16 / _b8: lane i of a 16-lane group receives element
    // i % E of lanes (16/E)*e + i/E, E = elements per 64 bits).
    const int b_row_in = (ES == 2) ? (j16 >> 2) : (j16 >> 1);
    const int b_col_in = (ES == 2) ? 4 * (j16 & 3) : 8 * (j16 & 1);

    auto compute = [&](int buf) {
        const LDS_AS uint8_t* As = smem + buf * T::STAGE;
        const LDS_AS uint8_t* Bs = As + T::A_BYTES;
#pragma unroll
        for (int ks = 0; ks < T::KS; ++ks) {
            if constexpr (ES == 2) {
                v8h bop[T::TN];
#pragma unroll
                for (int tn = 0; tn < T::TN; ++tn) {
                    const int col = wn * T::WTN + tn * 16 + b_col_in;
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int row = ks * T::KPI + 8 * g + 4 * h + b_row_in;
                        v4s t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (LDS_AS v4s*)(Bs + row * T::SB + col * 2));
                        v4s* dst = reinterpret_cast<v4s*>(&bop[tn]) + h;
                        *dst = t;
                    }
                }
#pragma unroll
                for (int tm = 0; tm < T::TM; ++tm) {
                    const int row = a_row0 + tm * 16;
                    v8h aop = __builtin_bit_cast(v8h, *(const LDS_AS v4u*)(As + row * T::SA + ks * T::KPI * 2 + g * 16));
#pragma unroll
                    for (int tn = 0; tn < T::TN; ++tn)
                        acc[tm][tn] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, bop[tn], acc[tm][tn], 0, 0, 0);
                }
            } else {
                v8i bop[T::TN];
#pragma unroll
                for (int tn = 0; tn < T::TN; ++tn) {
                    const int col = wn * T::WTN + tn * 16 + b_col_in;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int row = ks * T::KPI + 32 * g + 8 * r + b_row_in;
                        v2i t = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS v2i*)(Bs + row * T::SB + col));
                        bop[tn][2 * r] = t[0];
                        bop[tn][2 * r + 1] = t[1];
                    }
                }
#pragma unroll
                for (int tm = 0; tm < T::TM; ++tm) {
                    const int row = a_row0 + tm * 16;
                    const LDS_AS uint8_t* ap = As + row * T::SA + ks * T::KPI + g * 32;
                    v4u lo = *(const LDS_AS v4u*)ap;
                    v4u hi = *(const LDS_AS v4u*)(ap + 16);
                    v8i aop = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
#pragma unroll
                    for (int tn = 0; tn < T::TN; ++tn)
                        acc[tm][tn] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aop, bop[tn], acc[tm][tn], 0, 0,
                                                                                      0, 127, 0, 127);
                }
            }
        }
    };

    const int64_t nk = (K + BK - 1) / BK;
    if (nk > 0) {
        gload(0);
        sstore(0);
        __syncthreads();
        for (int64_t kt = 0; kt < nk; ++kt) {
            const bool more = kt + 1 < nk;
            if (more) gload((kt + 1) * BK);
            compute((int)(kt & 1));
            if (more) sstore((int)((kt + 1) & 1));
            __syncthreads();
        }
    }

    // Epilogue: y = acc * (sA*sB), converted and stored with M/N predication.
    const float scale = (sA ? *sA : 1.0f) * (sB ? *sB : 1.0f);
    const float s_out = (out_dtype == OUT_E4M3) ? *sOut : 1.0f;
#pragma unroll
    for (int tm = 0; tm < T::TM; ++tm) {
#pragma unroll
        for (int tn = 0; tn < T::TN; ++tn) {
            const int64_t col = n0 + wn * T::WTN + tn * 16 + j16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t row = m0 + wm * T::WTM + tm * 16 + 4 * g + r;
                if (row < M && col < N) store_out(C, row * N + col, acc[tm][tn][r] * scale, out_dtype, s_out);
            }
        }
    }
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

template <int ES, int BM, int BN, int BK, int WM, int WN>
hipError_t launch_tile(const GemmArgs& a) {
    const int64_t tiles_m = (a.M + BM - 1) / BM;
    const int64_t tiles_n = (a.N + BN - 1) / BN;
    const int64_t blocks = tiles_m * tiles_n;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7FFFFFFF || tiles_n > 0x7FFFFFFF) return hipErrorInvalidValue;
    const int a_vec = aligned16(a.A) && ((a.K * ES) % 16 == 0);
    const int b_vec = aligned16(a.B) && ((a.N * ES) % 16 == 0);
    gemm_tile_kernel<ES, BM, BN, BK, WM, WN><<<(unsigned)blocks, 64 * WM * WN, 0, a.stream>>>(
        reinterpret_cast<const uint8_t*>(a.A), reinterpret_cast<const uint8_t*>(a.B), a.C, a.M, a.N, a.K, a.sA,
        a.sB, a.sOut, a.out_dtype, a_vec, b_vec, (int)tiles_n);
    return hipGetLastError();
}

}  // namespace

// The table lives in a host function so that the kernels it names are
// instantiated for the device while the table itself stays host data.
const GemmConfig* tile_configs(int* count) {
    static const GemmConfig table[] = {
    {"tile_f16_64x64x64_w2x2", KIND_F16, 0, 64, 64, 64, launch_tile<2, 64, 64, 64, 2, 2>},
    {"tile_f16_128x128x64_w2x2", KIND_F16, 0, 128, 128, 64, launch_tile<2, 128, 128, 64, 2, 2>},
    {"tile_f16_256x256x64_w2x2", KIND_F16, 0, 256, 256, 64, launch_tile<2, 256, 256, 64, 2, 2>},
    {"tile_fp8_64x64x128_w2x2", KIND_FP8, 0, 64, 64, 128, launch_tile<1, 64, 64, 128, 2, 2>},
    {"tile_fp8_128x128x128_w2x2", KIND_FP8, 0, 128, 128, 128, launch_tile<1, 128, 128, 128, 2, 2>},
    {"tile_fp8_256x256x128_w2x2", KIND_FP8, 0, 256, 256, 128, launch_tile<1, 256, 256, 128, 2, 2>},
    };
    *count = (int)(sizeof(table) / sizeof(table[0]));
    return table;
}
}  // namespace libgemm
