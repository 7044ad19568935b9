// MFMA tile GEMM for gfx950: C[M,N] = (sA*A[M,K]) (sB*B[K,N]), all row-major.
//
// Operands are FP16 (v_mfma_f32_16x16x32_f16) or OCP E4M3 codes
// (v_mfma_scale_f32_16x16x128_f8f6f4 with neutral block scales), always with
// FP32 accumulation ("DeepGEMM实战：FP8矩阵乘法与JIT编译优化指南" §2.1;
// "HGEMM优化：深度学习中的矩阵乘法性能提升策略" §1.3).
//
// Data flow per workgroup (one BM x BN output tile, 4 waves in a 2 x 2 grid):
//   HBM/L2 --16-byte coalesced loads--> registers --ds_write_b128--> LDS
//   (two LDS stages plus one register stage: tile k+2 is in flight while
//   tile k is multiplied; FP8 guide §2.3 "double buffering", HGEMM §3.2/§3.3
//   on prefetch depth)
//   LDS --ds_read_b128 (A) / ds_read_b64_tr_b16|b8 (B)--> MFMA operands
// A is row-major [M,K]: its K-contiguous rows are exactly the MFMA A operand.
// B is row-major [K,N]: N is contiguous, so the B operand (8 or 32 consecutive
// k for one column per lane) comes from gfx950's LDS transpose reads instead of
// a transposing copy. LDS rows are padded (A: +16 B, B: +16/32 B) so that the
// lanes served by one LDS pass hit distinct banks (the bank-aware layout the
// DeepGEMM deep-dive article, §3.2, argues for).
//
// Edges (FP8 guide §3.3): rows >= M and columns >= N are neither loaded nor
// stored, the K tail is zero-filled in the staged tile, so one kernel serves
// every shape. Interior tiles take a branch-free path; only edge tiles (and
// unaligned operands) run the guarded element loads. The epilogue multiplies
// by sA*sB once and converts to the output type, which is a template
// parameter so that every accumulator index is a compile-time constant and
// the accumulators stay in registers.
//
// Tile order: consecutive workgroups are dispatched round-robin over the 8
// XCDs, each with its own L2. Workgroup ids are remapped so that every XCD
// receives a compact block of tiles (shared A row-blocks and B column-blocks
// stay in one L2), walked in groups of 4 tile rows.
#include "device_common.h"
#include "kernels.h"

namespace libgemm {

namespace {

constexpr int kXcds = 8;
constexpr int kGroupM = 4;

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
    static constexpr int A_RPP = NT / A_CPR;          // A rows covered per pass of all threads
    static constexpr int B_RPP = NT / B_CPR;
    static constexpr int CA = BM / A_RPP;             // A chunks per thread
    static constexpr int CB = BK / B_RPP;
    static constexpr int WTM = BM / WM, WTN = BN / WN;
    static constexpr int TM = WTM / 16, TN = WTN / 16;
    static constexpr int KS = BK / KPI;
    static_assert(BK % KPI == 0, "BK must be a multiple of the MFMA depth");
    static_assert(NT % A_CPR == 0 && NT % B_CPR == 0, "chunk rows must tile the workgroup");
    static_assert(BM % A_RPP == 0 && BK % B_RPP == 0, "tile chunks must divide evenly");
    static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile must be whole 16x16 blocks");
    static_assert(2 * STAGE <= 160 * 1024, "two stages must fit in LDS");
};

// One 16-byte chunk of `ES`-byte elements starting at element `col` of a row,
// zero beyond `limit` and for rows out of range (edges and unaligned operands).
template <int ES>
__device__ __forceinline__ v4u load_chunk_guarded(const uint8_t* row_ptr, bool row_ok, int64_t col, int64_t limit) {
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    if (row_ok) {
#pragma unroll
        for (int e = 0; e < 16 / ES; ++e) {
            if (col + e < limit) {
                uint32_t v = (ES == 1) ? (uint32_t)row_ptr[col + e]
                                       : (uint32_t)reinterpret_cast<const uint16_t*>(row_ptr)[col + e];
                const int bit = e * ES * 8;
                w[bit >> 5] |= v << (bit & 31);
            }
        }
    }
    return v4u{w[0], w[1], w[2], w[3]};
}

template <int OUT>
__device__ __forceinline__ void store_one(void* C, int64_t idx, float y, float s_out) {
    if constexpr (OUT == OUT_F32) {
        reinterpret_cast<float*>(C)[idx] = y;
    } else if constexpr (OUT == OUT_F16) {
        reinterpret_cast<_Float16*>(C)[idx] = (_Float16)y;
    } else {
        reinterpret_cast<uint8_t*>(C)[idx] = e4m3_from_f32(y / s_out);
    }
}

// Workgroup id -> (tile row, tile column), XCD-compact and grouped by kGroupM rows.
__device__ __forceinline__ void tile_coords(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
    const int total = tiles_m * tiles_n;
    const int full = total - total % kXcds;
    int id = bid;
    if (bid < full) id = (bid % kXcds) * (full / kXcds) + bid / kXcds;  // XCD x owns ids [x*per, (x+1)*per)
    const int group_span = kGroupM * tiles_n;
    const int group = id / group_span;
    const int first_m = group * kGroupM;
    const int rows = min(tiles_m - first_m, kGroupM);
    const int in_group = id - group * group_span;
    tm = first_m + in_group % rows;
    tn = in_group / rows;
}

template <int ES, int OUT, int BM, int BN, int BK, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN) void gemm_tile_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ B, void* __restrict__ C, int M, int N, int K,
    const float* __restrict__ sA, const float* __restrict__ sB, const float* __restrict__ sOut, int tiles_m,
    int tiles_n, int aligned) {
    using T = Tile<ES, BM, BN, BK, WM, WN>;
    __shared__ __attribute__((aligned(16))) uint8_t smem_raw[2 * T::STAGE];
    LDS_AS uint8_t* smem = (LDS_AS uint8_t*)smem_raw;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;

    int tile_m, tile_n;
    tile_coords(blockIdx.x, tiles_m, tiles_n, tile_m, tile_n);
    const int m0 = tile_m * BM;
    const int n0 = tile_n * BN;
    const bool interior_mn = aligned && (m0 + BM <= M) && (n0 + BN <= N);

    // This thread's chunk coordinates inside a staged tile.
    const int a_row = tid / T::A_CPR, a_col = tid % T::A_CPR;  // + i * A_RPP rows
    const int b_row = tid / T::B_CPR, b_col = tid % T::B_CPR;  // + i * B_RPP rows
    const uint8_t* a_base = A + ((int64_t)(m0 + a_row) * K + a_col * T::VE) * ES;
    const uint8_t* b_base = B + ((int64_t)b_row * N + n0 + b_col * T::VE) * ES;
    const int64_t a_step = (int64_t)T::A_RPP * K * ES;  // bytes between this thread's A chunks
    const int64_t b_step = (int64_t)T::B_RPP * N * ES;

    v4u ra[T::CA];
    v4u rb[T::CB];

    v4f acc[T::TM][T::TN];
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int j = 0; j < T::TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    const int g = lane >> 4;    // 16-lane group: selects the k sub-range of an operand
    const int j16 = lane & 15;  // lane within its group
    // B transpose-read pattern (lane maps measured for ds_read_b64_tr_b16 /
    // _b8: lane i of a 16-lane group receives element i % E of lanes
    // (16/E)*e + i/E, E = elements per 64 bits).
    const int b_row_in = (ES == 2) ? (j16 >> 2) : (j16 >> 1);
    const int b_col_in = (ES == 2) ? 4 * (j16 & 3) : 8 * (j16 & 1);
    const int a_lds = (wm * T::WTM + j16) * T::SA + g * T::OPB;                    // + tm*16*SA + ks*KPI*ES
    const int b_lds = T::A_BYTES + (8 * (ES == 2 ? 1 : 4) * g + b_row_in) * T::SB  // + ks*KPI*SB + ...
                      + (wn * T::WTN + b_col_in) * ES;

    const int nk = (K + BK - 1) / BK;

    auto load_tile = [&](int kt) __attribute__((always_inline)) {
        const int k0 = kt * BK;
        if (interior_mn && k0 + BK <= K) {
            const uint8_t* pa = a_base + (int64_t)k0 * ES;
            const uint8_t* pb = b_base + (int64_t)k0 * N * ES;
#pragma unroll
            for (int i = 0; i < T::CA; ++i) ra[i] = *reinterpret_cast<const v4u*>(pa + i * a_step);
#pragma unroll
            for (int i = 0; i < T::CB; ++i) rb[i] = *reinterpret_cast<const v4u*>(pb + i * b_step);
        } else {
#pragma unroll
            for (int i = 0; i < T::CA; ++i) {
                const int gm = m0 + a_row + i * T::A_RPP;
                const int64_t gk = (int64_t)k0 + a_col * T::VE;
                const uint8_t* rp = A + (int64_t)gm * K * ES;
                if (aligned && gm < M && gk + T::VE <= K)
                    ra[i] = *reinterpret_cast<const v4u*>(rp + gk * ES);
                else
                    ra[i] = load_chunk_guarded<ES>(rp, gm < M, gk, K);
            }
#pragma unroll
            for (int i = 0; i < T::CB; ++i) {
                const int gk = k0 + b_row + i * T::B_RPP;
                const int64_t gn = (int64_t)n0 + b_col * T::VE;
                const uint8_t* rp = B + (int64_t)gk * N * ES;
                if (aligned && gk < K && gn + T::VE <= N)
                    rb[i] = *reinterpret_cast<const v4u*>(rp + gn * ES);
                else
                    rb[i] = load_chunk_guarded<ES>(rp, gk < K, gn, N);
            }
        }
    };

    auto store_tile = [&](int buf) __attribute__((always_inline)) {
        LDS_AS uint8_t* As = smem + buf * T::STAGE;
#pragma unroll
        for (int i = 0; i < T::CA; ++i)
            *(LDS_AS v4u*)(As + (a_row + i * T::A_RPP) * T::SA + a_col * 16) = ra[i];
#pragma unroll
        for (int i = 0; i < T::CB; ++i)
            *(LDS_AS v4u*)(As + T::A_BYTES + (b_row + i * T::B_RPP) * T::SB + b_col * 16) = rb[i];
    };

    auto compute = [&](int buf) __attribute__((always_inline)) {
        const LDS_AS uint8_t* base = smem + buf * T::STAGE;
#pragma unroll
        for (int ks = 0; ks < T::KS; ++ks) {
            if constexpr (ES == 2) {
                v8h bop[T::TN];
#pragma unroll
                for (int tn = 0; tn < T::TN; ++tn) {
                    // two transpose reads give k = 8g + 0..3 and 8g + 4..7 of column n
                    const LDS_AS uint8_t* p = base + b_lds + ks * T::KPI * T::SB + tn * 16 * ES;
                    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4s*)p);
                    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4s*)(p + 4 * T::SB));
                    bop[tn] = __builtin_bit_cast(v8h, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                }
#pragma unroll
                for (int tm = 0; tm < T::TM; ++tm) {
                    const v4u a = *(const LDS_AS v4u*)(base + a_lds + tm * 16 * T::SA + ks * T::KPI * ES);
                    const v8h aop = __builtin_bit_cast(v8h, a);
#pragma unroll
                    for (int tn = 0; tn < T::TN; ++tn)
                        acc[tm][tn] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, bop[tn], acc[tm][tn], 0, 0, 0);
                }
            } else {
                v8i bop[T::TN];
#pragma unroll
                for (int tn = 0; tn < T::TN; ++tn) {
                    // four transpose reads give k = 32g + 0..7, 8..15, 16..23, 24..31 of column n
                    const LDS_AS uint8_t* p = base + b_lds + ks * T::KPI * T::SB + tn * 16;
                    const v2i t0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS v2i*)p);
                    const v2i t1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS v2i*)(p + 8 * T::SB));
                    const v2i t2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS v2i*)(p + 16 * T::SB));
                    const v2i t3 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS v2i*)(p + 24 * T::SB));
                    const v4i t01 = __builtin_shufflevector(t0, t1, 0, 1, 2, 3);
                    const v4i t23 = __builtin_shufflevector(t2, t3, 0, 1, 2, 3);
                    bop[tn] = __builtin_shufflevector(t01, t23, 0, 1, 2, 3, 4, 5, 6, 7);
                }
#pragma unroll
                for (int tm = 0; tm < T::TM; ++tm) {
                    const LDS_AS uint8_t* ap = base + a_lds + tm * 16 * T::SA + ks * T::KPI;
                    const v4i lo = *(const LDS_AS v4i*)ap;
                    const v4i hi = *(const LDS_AS v4i*)(ap + 16);
                    const v8i aop = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
                    for (int tn = 0; tn < T::TN; ++tn)
                        acc[tm][tn] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aop, bop[tn], acc[tm][tn],
                                                                                      0, 0, 0, 127, 0, 127);
                }
            }
        }
    };

    // Pipeline: iteration kt first writes tile kt+1 (fetched into registers
    // one iteration earlier, so its loads have had a whole iteration to land)
    // to the stage that iteration kt-1 finished reading, issues the fetch of
    // tile kt+2, and then multiplies tile kt out of the other stage. One
    // barrier per iteration separates the readers of a stage from its next
    // writers.
    if (nk > 0) {
        load_tile(0);
        store_tile(0);
        if (nk > 1) load_tile(1);
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            if (kt + 1 < nk) store_tile((kt + 1) & 1);
            if (kt + 2 < nk) load_tile(kt + 2);
            compute(kt & 1);
            __syncthreads();
        }
    }

    // Epilogue: y = acc * (sA*sB), converted, stored with M/N predication on edge tiles.
    const float scale = (sA ? *sA : 1.0f) * (sB ? *sB : 1.0f);
    const float s_out = (OUT == OUT_E4M3) ? *sOut : 1.0f;
    const int row0 = m0 + wm * T::WTM + 4 * g;
    const int col0 = n0 + wn * T::WTN + j16;
    if (interior_mn) {
#pragma unroll
        for (int tm = 0; tm < T::TM; ++tm)
#pragma unroll
            for (int tn = 0; tn < T::TN; ++tn)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    store_one<OUT>(C, (int64_t)(row0 + tm * 16 + r) * N + col0 + tn * 16, acc[tm][tn][r] * scale,
                                   s_out);
    } else {
#pragma unroll
        for (int tm = 0; tm < T::TM; ++tm)
#pragma unroll
            for (int tn = 0; tn < T::TN; ++tn)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = row0 + tm * 16 + r, col = col0 + tn * 16;
                    if (row < M && col < N)
                        store_one<OUT>(C, (int64_t)row * N + col, acc[tm][tn][r] * scale, s_out);
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
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    const int aligned = aligned16(a.A) && aligned16(a.B) && ((a.K * ES) % 16 == 0) && ((a.N * ES) % 16 == 0);
    const uint8_t* A = reinterpret_cast<const uint8_t*>(a.A);
    const uint8_t* B = reinterpret_cast<const uint8_t*>(a.B);
    const int M = (int)a.M, N = (int)a.N, K = (int)a.K;
    const dim3 grid((unsigned)blocks), block(64 * WM * WN);
    switch (a.out_dtype) {
        case OUT_F32:
            gemm_tile_kernel<ES, OUT_F32, BM, BN, BK, WM, WN><<<grid, block, 0, a.stream>>>(
                A, B, a.C, M, N, K, a.sA, a.sB, a.sOut, (int)tiles_m, (int)tiles_n, aligned);
            break;
        case OUT_F16:
            gemm_tile_kernel<ES, OUT_F16, BM, BN, BK, WM, WN><<<grid, block, 0, a.stream>>>(
                A, B, a.C, M, N, K, a.sA, a.sB, a.sOut, (int)tiles_m, (int)tiles_n, aligned);
            break;
        default:
            if constexpr (ES == 1) {
                gemm_tile_kernel<ES, OUT_E4M3, BM, BN, BK, WM, WN><<<grid, block, 0, a.stream>>>(
                    A, B, a.C, M, N, K, a.sA, a.sB, a.sOut, (int)tiles_m, (int)tiles_n, aligned);
            } else {
                return hipErrorInvalidValue;
            }
    }
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
