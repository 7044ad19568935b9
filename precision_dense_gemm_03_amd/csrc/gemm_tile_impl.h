// Register-staged MFMA tile GEMM for gfx950: kernel and launcher templates,
// shared by gemm_tile.hip (configuration table, E4M3 x E4M3 and FP16
// instantiations) and gemm_tile_mixed.hip (the other FP8 operand pairs).
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

#pragma once

#include "device_common.h"
#include "kernels.h"
#include "tile_order.h"

namespace libgemm {
namespace tile {

// 8-wave kernels with K-major B: read the next A operand before the current
// row block's MFMAs (one more operand register set) and raise the wave's issue
// priority while it issues MFMAs. Measured on one MI355X (us, K-major B):
// E4M3 4096^3 80.2-81.5 -> 78.3, E4M3 16384x12288x4096 822-827 -> 785, FP16
// 4096^3 158-161 -> 151; the same change slowed the row-major kernels (83 ->
// 86, 832 -> 887), whose B operands come from transpose reads, so it is
// applied with K-major B only.
template <bool BT>
constexpr bool kPrefetchA = BT;
template <bool BT>
constexpr bool kMfmaPrio = BT;
// K-major kernels keep A and B rows unpadded (128 bytes) with chunk c of row r
// in slot c ^ ((r >> 1) & 7): the 16 lanes an LDS pass serves (16 consecutive
// rows at one chunk for operand reads, two rows of 8 chunks for the stores)
// then cover all 16 four-bank groups of the 64 banks. Counters on MI355X, per
// 4096^3 launch: FP16 bank-conflict cycles 12.6 M -> 0 (LDS-active 33.6 M ->
// 21.0 M, run time about 1 % lower); FP8, with each lane's operand split over
// chunks g and g + 4 (rd below), 6.3 M -> 0 (LDS-active 16.8 M -> 10.5 M, run
// time 1-2 % lower).
constexpr bool kSwizzleBT = true;

// BT: B is stored K-major, as Bt[N,K] row-major (the layout of a linear
// layer's weight); its tile is then staged and read exactly like A's.
template <int ES, int BM, int BN, int BK, int WM, int WN, bool BT = false>
struct Tile {
    static constexpr int NT = 64 * WM * WN;           // threads per workgroup
    static constexpr int KPI = ES == 2 ? 32 : 128;    // k per MFMA instruction
    static constexpr int OPB = ES == 2 ? 16 : 32;     // operand bytes per lane
    static constexpr int VE = 16 / ES;                // elements per 16-byte chunk
    static constexpr int BKB = BK * ES;               // bytes of one A tile row
    static constexpr int BNB = BN * ES;               // bytes of one B tile row
    static constexpr bool SWZ = BT && kSwizzleBT;     // XOR-swizzled rows (A, and B when K-major)
    static constexpr int SA = SWZ ? BKB : BKB + 16;   // LDS row strides (padded unless swizzled)
    static constexpr int SB = BNB + (ES == 2 ? 32 : 16);
    // B rows come in groups of RB (the rows one 16-lane group of a transpose
    // read spans: 32 for FP8, 8 for FP16) and each group starts 128 bytes
    // further: without that, the row stride times RB is a multiple of the 64
    // banks' 256 bytes and the lane groups that LDS serves together (groups
    // g and g+1 start RB rows apart) read the same 32 banks.
    static constexpr int RB = ES == 2 ? 8 : 32;
    static constexpr int A_BYTES = BM * SA;
    static constexpr int B_BYTES = BT ? BN * SA : BK * SB + (BK / RB) * 128;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int A_CPR = BKB / 16;            // 16-byte chunks per A row
    static constexpr int B_CPR = BT ? BKB / 16 : BNB / 16;
    static constexpr int A_RPP = NT / A_CPR;          // A rows covered per pass of all threads
    static constexpr int B_RPP = NT / B_CPR;
    static constexpr int CA = BM / A_RPP;             // A chunks per thread
    static constexpr int CB = (BT ? BN : BK) / B_RPP;  // B chunks per thread
    static constexpr int WTM = BM / WM, WTN = BN / WN;
    static constexpr int TM = WTM / 16, TN = WTN / 16;
    static constexpr int KS = BK / KPI;
    static_assert(BK % KPI == 0, "BK must be a multiple of the MFMA depth");
    static_assert(NT % A_CPR == 0 && NT % B_CPR == 0, "chunk rows must tile the workgroup");
    static_assert(BM % A_RPP == 0 && (BT ? BN : BK) % B_RPP == 0, "tile chunks must divide evenly");
    static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile must be whole 16x16 blocks");
    static_assert(2 * STAGE <= 160 * 1024, "two stages must fit in LDS");
    static_assert(!SWZ || (A_CPR == 8 && B_CPR == 8 && A_RPP % 16 == 0 && B_RPP % 16 == 0),
                  "the row swizzle assumes 8 chunks per row and row passes of whole 16-row groups");
    // Byte offset of 16-byte chunk c in LDS row r.
    static __device__ __forceinline__ int chunk(int r, int c) { return (SWZ ? (c ^ ((r >> 1) & 7)) : c) * 16; }
    // LDS map: A stage 0, A stage 1, B stage 0, B stage 1
    static constexpr int a_stage(int s) { return s * A_BYTES; }
    static constexpr int b_stage(int s) { return 2 * A_BYTES + s * B_BYTES; }
    // LDS byte offset of staged B row r (a k row, or for BT an n row)
    static __device__ __forceinline__ int b_row(int r) { return BT ? r * SA : r * SB + (r / RB) * 128; }
};

// MFMA operand type, LDS operand reads and the multiply for each element size.
template <int ES>
struct Operand;

template <>
struct Operand<2> {  // FP16: v_mfma_f32_16x16x32_f16, 8 halves per lane
    typedef v8h type;
    template <int FA, int FB>
    static __device__ __forceinline__ v4f mma(v8h a, v8h b, v4f c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ v8h read_a(const LDS_AS uint8_t* p) {
        return __builtin_bit_cast(v8h, *(const LDS_AS v4u*)p);
    }
    // two transpose reads give k = 8g + 0..3 and 8g + 4..7 of one column
    static __device__ __forceinline__ v8h read_b(const LDS_AS uint8_t* p, int sb) {
        const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4s*)p);
        const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4s*)(p + 4 * sb));
        return __builtin_bit_cast(v8h, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
};

template <>
struct Operand<1> {  // FP8: v_mfma_scale_f32_16x16x128_f8f6f4 (neutral scales), 32 codes per lane
    typedef v8i type;
    static __device__ __forceinline__ v8i read_a(const LDS_AS uint8_t* p) {
        const v4i lo = *(const LDS_AS v4i*)p;
        const v4i hi = *(const LDS_AS v4i*)(p + 16);
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    // four transpose reads give k = 32g + 0..7, 8..15, 16..23, 24..31 of one column
    static __device__ __forceinline__ v8i read_b(const LDS_AS uint8_t* p, int sb) {
        const v2i t0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS v2i*)p);
        const v2i t1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS v2i*)(p + 8 * sb));
        const v2i t2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS v2i*)(p + 16 * sb));
        const v2i t3 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS v2i*)(p + 24 * sb));
        const v4i t01 = __builtin_shufflevector(t0, t1, 0, 1, 2, 3);
        const v4i t23 = __builtin_shufflevector(t2, t3, 0, 1, 2, 3);
        return __builtin_shufflevector(t01, t23, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    // FA, FB: operand formats (0 = E4M3, 1 = E5M2), the instruction's A and B
    // format selectors.
    template <int FA, int FB>
    static __device__ __forceinline__ v4f mma(v8i a, v8i b, v4f c) {
        return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FA, FB, 0, 127, 0, 127);
    }
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

// Eight FP8 codes starting at element col of a row, zero beyond limit and for
// rows out of range.
__device__ __forceinline__ v2i load_codes8_guarded(const uint8_t* row_ptr, bool row_ok, int64_t col, int64_t limit) {
    uint32_t w[2] = {0u, 0u};
    if (row_ok) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (col + e < limit) w[e >> 2] |= (uint32_t)row_ptr[col + e] << (8 * (e & 3));
    }
    return v2i{(int)w[0], (int)w[1]};
}

// OUT_E4M3 stands for both FP8 outputs; EPI_E5M2 in eflags (uniform) picks the
// format.
template <int OUT>
__device__ __forceinline__ void store_one(void* C, int64_t idx, float y, int eflags) {
    if constexpr (OUT == OUT_F32) {
        reinterpret_cast<float*>(C)[idx] = y;
    } else if constexpr (OUT == OUT_F16) {
        reinterpret_cast<_Float16*>(C)[idx] = (_Float16)y;
    } else {
        reinterpret_cast<uint8_t*>(C)[idx] = (eflags & EPI_E5M2) ? e5m2_from_f32(y) : e4m3_from_f32(y);
    }
}

// GES: bytes per element of A and B in global memory. GES == ES except for
// the exact FP8 mode (ES = 2, GES = 1): FP8 codes are widened to FP16 as they
// are staged (eflags EPI_A_E5M2 / EPI_B_E5M2 give the operand formats) and
// summed on the FP16 matrix cores.
template <int ES, int OUT, int BM, int BN, int BK, int WM, int WN, int FA, int FB, bool BT, int GES = ES>
__global__ __launch_bounds__(64 * WM * WN) void gemm_tile_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ B, void* __restrict__ C, int M, int N, int K,
    const float* __restrict__ sA, const float* __restrict__ sB, const float* __restrict__ sOut, int tiles_m,
    int tiles_n, int aligned, int eflags, int kchunk) {
    using T = Tile<ES, BM, BN, BK, WM, WN, BT>;
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
    // Split-K: workgroup row blockIdx.y sums K range [kbeg, kend) (the whole
    // of K when the launch is not split). kbeg is a multiple of BK.
    const int split = blockIdx.y;
    const int kbeg = split * kchunk;
    const int klen = min(K - kbeg, kchunk);
    const int kend = kbeg + klen;

    // This thread's chunk coordinates inside a staged tile.
    const int a_row = tid / T::A_CPR, a_col = tid % T::A_CPR;  // + i * A_RPP rows
    const int b_row = tid / T::B_CPR, b_col = tid % T::B_CPR;  // + i * B_RPP rows

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
    // Operand reads: row of this lane (+ stage + tm*16*SA) and byte offset in
    // the row (g*OPB + ks*KPI*ES, through rd below).
    const int a_lds = (wm * T::WTM + j16) * T::SA;
    const int goff = g * T::OPB;
    // BT: row of this lane + stage + tn*16*SA, offsets as for A
    const int b_lds = BT ? (wn * T::WTN + j16) * T::SA
                         : T::b_row(8 * (ES == 2 ? 1 : 4) * g + b_row_in)  // + stage + b_row(ks*KPI) + tn*16*ES
                               + (wn * T::WTN + b_col_in) * ES;

    const int nk = (klen + BK - 1) / BK;
    typedef typename Operand<ES>::type Op;

    // ---- global <-> registers <-> LDS (A and B have separate stages) ----
    // Fast-path loads: a wave-uniform base (kept in SGPRs) plus a 32-bit
    // per-lane offset, so the 16 loads of a tile need no 64-bit VGPR addresses.
    // Valid while one tile row block spans less than 2^31 bytes (checked below).
    const uint8_t* a_tile = A + ((int64_t)m0 * K + kbeg) * GES;
    const uint8_t* b_tile = BT ? B + ((int64_t)n0 * K + kbeg) * GES : B + ((int64_t)kbeg * N + n0) * GES;
    constexpr bool kWiden = GES != ES;
    const bool a_e5m2 = (eflags & EPI_A_E5M2) != 0, b_e5m2 = (eflags & EPI_B_E5M2) != 0;
    // One staged 16-byte chunk from global memory at p (VE elements).
    auto gload = [&](const uint8_t* p, bool e5m2) __attribute__((always_inline)) -> v4u {
        if constexpr (kWiden) {
            const v2i w = *reinterpret_cast<const v2i*>(p);
            return widen8_fp8((uint32_t)w.x, (uint32_t)w.y, e5m2);
        } else {
            return *reinterpret_cast<const v4u*>(p);
        }
    };
    auto gload_guarded = [&](const uint8_t* row_ptr, bool row_ok, int64_t col, int64_t limit, bool e5m2)
        __attribute__((always_inline)) -> v4u {
        if constexpr (kWiden) {
            const v2i w = load_codes8_guarded(row_ptr, row_ok, col, limit);
            return widen8_fp8((uint32_t)w.x, (uint32_t)w.y, e5m2);
        } else {
            return load_chunk_guarded<ES>(row_ptr, row_ok, col, limit);
        }
    };
    // Edge tiles (aligned operands) use the same unguarded loads with the
    // addresses clamped into the matrix: A rows past M re-read row M-1 and B
    // column chunks past N re-read the last chunk. Those values only reach
    // output rows/columns that are never stored, and every address is valid.
    uint32_t a_offs[T::CA], b_offs[T::CB];
#pragma unroll
    for (int i = 0; i < T::CA; ++i) {
        const int r = min(m0 + a_row + i * T::A_RPP, M - 1) - m0;
        a_offs[i] = (uint32_t)((r * K + a_col * T::VE) * GES);
    }
#pragma unroll
    for (int i = 0; i < T::CB; ++i) {
        if constexpr (BT) {
            const int r = min(n0 + b_row + i * T::B_RPP, N - 1) - n0;
            b_offs[i] = (uint32_t)((r * K + b_col * T::VE) * GES);
        } else {
            const int c = min(n0 + b_col * T::VE, N - T::VE) - n0;
            b_offs[i] = (uint32_t)(((b_row + i * T::B_RPP) * N + c) * GES);
        }
    }
    auto load_a = [&](int kt) __attribute__((always_inline)) {
        const uint8_t* pa = a_tile + (int64_t)kt * BK * GES;
#pragma unroll
        for (int i = 0; i < T::CA; ++i) ra[i] = gload(pa + a_offs[i], a_e5m2);
    };
    auto load_b = [&](int kt) __attribute__((always_inline)) {
        const uint8_t* pb = b_tile + (BT ? (int64_t)kt * BK * GES : (int64_t)kt * BK * N * GES);
#pragma unroll
        for (int i = 0; i < T::CB; ++i) rb[i] = gload(pb + b_offs[i], b_e5m2);
    };
    auto store_a = [&](int stage) __attribute__((always_inline)) {
        LDS_AS uint8_t* As = smem + T::a_stage(stage);
#pragma unroll
        for (int i = 0; i < T::CA; ++i)
            *(LDS_AS v4u*)(As + (a_row + i * T::A_RPP) * T::SA + T::chunk(a_row, a_col)) = ra[i];
    };
    auto store_b = [&](int stage) __attribute__((always_inline)) {
        LDS_AS uint8_t* Bs = smem + T::b_stage(stage);
#pragma unroll
        for (int i = 0; i < T::CB; ++i)
            *(LDS_AS v4u*)(Bs + T::b_row(b_row + i * T::B_RPP) + T::chunk(b_row, b_col)) = rb[i];
    };
    // Edge tiles, the K tail and unaligned operands: each 16-byte chunk is
    // loaded with per-element guards and written straight to LDS (no register
    // staging, and a rolled loop, so this path costs almost no registers).
    auto guarded_to_lds = [&](int kt, int stage) __attribute__((always_inline)) {
        const int k0 = kbeg + kt * BK;
        LDS_AS uint8_t* As = smem + T::a_stage(stage);
        LDS_AS uint8_t* Bs = smem + T::b_stage(stage);
#pragma unroll 1
        for (int i = 0; i < T::CA; ++i) {
            const int gm = m0 + a_row + i * T::A_RPP;
            const int64_t gk = (int64_t)k0 + a_col * T::VE;
            const uint8_t* rp = A + (int64_t)gm * K * GES;
            v4u v;
            if (aligned && gm < M && gk + T::VE <= kend)
                v = gload(rp + gk * GES, a_e5m2);
            else
                v = gload_guarded(rp, gm < M, gk, kend, a_e5m2);
            *(LDS_AS v4u*)(As + (a_row + i * T::A_RPP) * T::SA + T::chunk(a_row, a_col)) = v;
        }
#pragma unroll 1
        for (int i = 0; i < T::CB; ++i) {
            if constexpr (BT) {
                const int gn = n0 + b_row + i * T::B_RPP;
                const int64_t gk = (int64_t)k0 + b_col * T::VE;
                const uint8_t* rp = B + (int64_t)gn * K * GES;
                v4u v;
                if (aligned && gn < N && gk + T::VE <= kend)
                    v = gload(rp + gk * GES, b_e5m2);
                else
                    v = gload_guarded(rp, gn < N, gk, kend, b_e5m2);
                *(LDS_AS v4u*)(Bs + T::b_row(b_row + i * T::B_RPP) + T::chunk(b_row, b_col)) = v;
                continue;
            }
            const int gk = k0 + b_row + i * T::B_RPP;
            const int64_t gn = (int64_t)n0 + b_col * T::VE;
            const uint8_t* rp = B + (int64_t)gk * N * GES;
            v4u v;
            if (aligned && gk < kend && gn + T::VE <= N)
                v = gload(rp + gn * GES, b_e5m2);
            else
                v = gload_guarded(rp, gk < kend, gn, N, b_e5m2);
            *(LDS_AS v4u*)(Bs + T::b_row(b_row + i * T::B_RPP) + T::chunk(b_row, b_col)) = v;
        }
    };

    // ---- LDS -> MFMA operands ----
    // One operand (OPB bytes) at byte offset off of an LDS row; rows of a row
    // block start at multiples of 16, so the swizzle of this lane's row is j16/2.
    const int rsw = j16 >> 1;
    auto rd = [&](const LDS_AS uint8_t* rowp, int off) __attribute__((always_inline)) -> Op {
        if constexpr (T::SWZ) {
            const int q = off >> 4;
            if constexpr (ES == 1) {
                // The 32 codes of k-group g are chunks g and g + 4 of the row
                // (A and B alike, so the sum over k is unchanged; every aligned
                // group of 8 k the FP8 matrix cores add together is still 8
                // consecutive k). Two adjacent chunks per lane left about 3
                // bank-conflict cycles per LDS read; this split leaves none.
                const int q0 = q >> 1;
                const v4i lo = *(const LDS_AS v4i*)(rowp + ((q0 ^ rsw) << 4));
                const v4i hi = *(const LDS_AS v4i*)(rowp + (((q0 + 4) ^ rsw) << 4));
                return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            } else {
                return __builtin_bit_cast(v8h, *(const LDS_AS v4u*)(rowp + ((q ^ rsw) << 4)));
            }
        } else {
            return Operand<ES>::read_a(rowp + off);
        }
    };
    auto read_b = [&](int stage, Op (&bop)[T::KS][T::TN]) __attribute__((always_inline)) {
        const LDS_AS uint8_t* base = smem + T::b_stage(stage) + b_lds;
#pragma unroll
        for (int ks = 0; ks < T::KS; ++ks)
#pragma unroll
            for (int tn = 0; tn < T::TN; ++tn) {
                if constexpr (BT)
                    bop[ks][tn] = rd(base + tn * 16 * T::SA, goff + ks * T::KPI * ES);
                else
                    bop[ks][tn] = Operand<ES>::read_b(base + T::b_row(ks * T::KPI) + tn * 16 * ES, T::SB);
            }
    };
    auto mma_tile = [&](int stage, const Op (&bop)[T::KS][T::TN]) __attribute__((always_inline)) {
        const LDS_AS uint8_t* base = smem + T::a_stage(stage) + a_lds;
        if constexpr (kPrefetchA<BT> && T::NT > 256) {
            // Row blocks in (ks, tm) order; the A operand of the next block is
            // read before this block's MFMAs, so its LDS latency runs under them.
            constexpr int NB = T::KS * T::TM;
            auto a_read = [&](int b) { return rd(base + (b % T::TM) * 16 * T::SA, goff + (b / T::TM) * T::KPI * ES); };
            Op acur = a_read(0);
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const int ks = b / T::TM, tm = b % T::TM;
                const Op anext = a_read(b + 1 < NB ? b + 1 : b);
                if constexpr (kMfmaPrio<BT>) __builtin_amdgcn_s_setprio(1);
#pragma unroll
                for (int tn = 0; tn < T::TN; ++tn)
                    acc[tm][tn] = Operand<ES>::template mma<FA, FB>(acur, bop[ks][tn], acc[tm][tn]);
                if constexpr (kMfmaPrio<BT>) __builtin_amdgcn_s_setprio(0);
#pragma unroll
                for (int tn = 0; tn < T::TN; ++tn) asm volatile("" : "+v"(acc[tm][tn])::"memory");
                acur = anext;
            }
            return;
        }
#pragma unroll
        for (int ks = 0; ks < T::KS; ++ks)
#pragma unroll
            for (int tm = 0; tm < T::TM; ++tm) {
                const Op aop = rd(base + tm * 16 * T::SA, goff + ks * T::KPI * ES);
                if constexpr (kMfmaPrio<BT> && T::NT > 256) __builtin_amdgcn_s_setprio(1);
#pragma unroll
                for (int tn = 0; tn < T::TN; ++tn) acc[tm][tn] = Operand<ES>::template mma<FA, FB>(aop, bop[ks][tn], acc[tm][tn]);
                if constexpr (kMfmaPrio<BT> && T::NT > 256) __builtin_amdgcn_s_setprio(0);
                // With two waves per SIMD the other wave hides the A read
                // latency. Pinning this row block's products here (an empty
                // asm that reads and rewrites its accumulators, after which no
                // LDS read may be hoisted) keeps one A operand live at a time
                // instead of letting the compiler sink every MFMA to the loop
                // end and hold all A operands.
                if constexpr (T::NT > 256) {
#pragma unroll
                    for (int tn = 0; tn < T::TN; ++tn) asm volatile("" : "+v"(acc[tm][tn])::"memory");
                }
            }
    };

    const bool offsets_fit = (int64_t)BM * K * GES < (1ll << 31) &&
                             (BT ? (int64_t)BN * K * GES : (int64_t)BK * N * GES) < (1ll << 31);
    if (nk > 0) {
        Op bop[T::KS][T::TN];
        // Tile kt+1 is fetched into registers while tile kt is multiplied;
        // the K tail and unaligned operands load each chunk with element
        // guards straight into LDS.
        auto fast = [&](int kt) __attribute__((always_inline)) {
            return aligned && offsets_fit && (kt + 1) * BK <= klen;
        };
        if (fast(0)) {
            load_a(0);
            load_b(0);
            store_a(0);
            store_b(0);
        } else {
            guarded_to_lds(0, 0);
        }
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            const bool more = kt + 1 < nk;
            const bool fast_next = more && fast(kt + 1);
            if (fast_next) {
                load_a(kt + 1);
                load_b(kt + 1);
            }
            read_b(kt & 1, bop);
            mma_tile(kt & 1, bop);
            if (fast_next) {
                store_a((kt + 1) & 1);
                store_b((kt + 1) & 1);
            } else if (more) {
                guarded_to_lds(kt + 1, (kt + 1) & 1);
            }
            __syncthreads();
        }
    }

    // Epilogue: y = acc * (sA*sB), converted, stored with M/N predication on edge tiles.
    // Per-tensor: y = acc * sA*sB (/ sOut). Per-channel (EPI_CHANNEL, sA[M] and
    // sB[N]): y = acc * (1/sOut) * sA[row] * sB[col], loaded only for stored
    // elements.
    // A split-K partial (EPI_PARTIAL, OUT_F32) stores the raw sum into the
    // split's [M, N] slice of the workspace C.
    const bool partial = (eflags & EPI_PARTIAL) != 0;
    if (partial) C = reinterpret_cast<float*>(C) + (int64_t)split * M * N;
    const bool chan = !partial && (eflags & EPI_CHANNEL) != 0;
    const float scale = partial ? 1.0f : epilogue_base(sA, sB, sOut, OUT == OUT_E4M3, chan);  // both FP8 outputs
    const int row0 = m0 + wm * T::WTM + 4 * g;
    const int col0 = n0 + wn * T::WTN + j16;
    if (interior_mn) {
#pragma unroll
        for (int tm = 0; tm < T::TM; ++tm)
#pragma unroll
            for (int tn = 0; tn < T::TN; ++tn)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = row0 + tm * 16 + r, col = col0 + tn * 16;
                    float y = acc[tm][tn][r] * scale;
                    if (chan) y *= sA[row] * sB[col];
                    store_one<OUT>(C, (int64_t)row * N + col, y, eflags);
                }
    } else {
#pragma unroll
        for (int tm = 0; tm < T::TM; ++tm)
#pragma unroll
            for (int tn = 0; tn < T::TN; ++tn)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = row0 + tm * 16 + r, col = col0 + tn * 16;
                    if (row < M && col < N) {
                        float y = acc[tm][tn][r] * scale;
                        if (chan) y *= sA[row] * sB[col];
                        store_one<OUT>(C, (int64_t)row * N + col, y, eflags);
                    }
                }
    }
}

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Launches one configuration for operand formats FA, FB (FP8 only; FP16 uses
// 0, 0). Defined here for every translation unit that instantiates it.
template <int ES, int BM, int BN, int BK, int WM, int WN, int FA, int FB, bool BT = false, int GES = ES>
hipError_t launch_tile(const GemmArgs& a) {
    const int64_t tiles_m = (a.M + BM - 1) / BM;
    const int64_t tiles_n = (a.N + BN - 1) / BN;
    const int64_t blocks = tiles_m * tiles_n;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    const int splits = a.splits > 1 ? a.splits : 1;
    if (splits > 1 && (a.k_chunk % BK != 0 || a.k_chunk <= 0 || (int64_t)(splits - 1) * a.k_chunk >= a.K ||
                       splits > 65535 || !a.ws))
        return hipErrorInvalidValue;
    const int kchunk = splits > 1 ? (int)a.k_chunk : (int)a.K;
    if (BT != (a.b_kmajor != 0)) return hipErrorInvalidValue;
    // Vector loads need 16-byte aligned bases and row pitches (for BT, B's
    // rows are K long like A's, so N needs no alignment).
    // Vector loads read 16 / ES elements: 16 bytes, or 8 bytes of codes when
    // widening.
    const int64_t lb = 16 / ES * GES;
    const bool al = ((uintptr_t)a.A % lb) == 0 && ((uintptr_t)a.B % lb) == 0;
    const int aligned = al && ((a.K * GES) % lb == 0) && (BT || (a.N * GES) % lb == 0);
    const uint8_t* A = reinterpret_cast<const uint8_t*>(a.A);
    const uint8_t* B = reinterpret_cast<const uint8_t*>(a.B);
    const int M = (int)a.M, N = (int)a.N, K = (int)a.K;
    const dim3 grid((unsigned)blocks, (unsigned)splits), block(64 * WM * WN);
    if (splits > 1) {   // FP32 partial sums into the workspace
        const int pflags = EPI_PARTIAL | (GES != ES && a.fmt_a == FMT_E5M2 ? EPI_A_E5M2 : 0) |
                           (GES != ES && a.fmt_b == FMT_E5M2 ? EPI_B_E5M2 : 0);
        gemm_tile_kernel<ES, OUT_F32, BM, BN, BK, WM, WN, FA, FB, BT, GES><<<grid, block, 0, a.stream>>>(
            A, B, a.ws, M, N, K, nullptr, nullptr, nullptr, (int)tiles_m, (int)tiles_n, aligned, pflags, kchunk);
        return hipGetLastError();
    }
    const int eflags = (a.out_dtype == OUT_E5M2 ? EPI_E5M2 : 0) | (a.channel ? EPI_CHANNEL : 0) |
                       (GES != ES && a.fmt_a == FMT_E5M2 ? EPI_A_E5M2 : 0) |
                       (GES != ES && a.fmt_b == FMT_E5M2 ? EPI_B_E5M2 : 0);
    switch (a.out_dtype) {
        case OUT_F32:
            gemm_tile_kernel<ES, OUT_F32, BM, BN, BK, WM, WN, FA, FB, BT, GES><<<grid, block, 0, a.stream>>>(
                A, B, a.C, M, N, K, a.sA, a.sB, a.sOut, (int)tiles_m, (int)tiles_n, aligned, eflags, kchunk);
            break;
        case OUT_F16:
            gemm_tile_kernel<ES, OUT_F16, BM, BN, BK, WM, WN, FA, FB, BT, GES><<<grid, block, 0, a.stream>>>(
                A, B, a.C, M, N, K, a.sA, a.sB, a.sOut, (int)tiles_m, (int)tiles_n, aligned, eflags, kchunk);
            break;
        default:
            if constexpr (GES == 1) {
                gemm_tile_kernel<ES, OUT_E4M3, BM, BN, BK, WM, WN, FA, FB, BT, GES><<<grid, block, 0, a.stream>>>(
                    A, B, a.C, M, N, K, a.sA, a.sB, a.sOut, (int)tiles_m, (int)tiles_n, aligned,
                    eflags, kchunk);
            } else {
                return hipErrorInvalidValue;
            }
    }
    return hipGetLastError();
}

// Operand-format dispatch for configurations compiled for every FP8 pair; the
// pairs other than E4M3 x E4M3 are instantiated in gemm_tile_mixed.hip.
template <int BM, int BN, int BK, int WM, int WN, bool BT = false>
hipError_t launch_tile_fp8_any(const GemmArgs& a) {
    switch (a.fmt_a * 2 + a.fmt_b) {
        case 0: return launch_tile<1, BM, BN, BK, WM, WN, 0, 0, BT>(a);
        case 1: return launch_tile<1, BM, BN, BK, WM, WN, 0, 1, BT>(a);
        case 2: return launch_tile<1, BM, BN, BK, WM, WN, 1, 0, BT>(a);
        default: return launch_tile<1, BM, BN, BK, WM, WN, 1, 1, BT>(a);
    }
}

// The exact-accumulation FP8 mode: FP8 codes in global memory, FP16 in LDS and
// on the matrix cores (formats from the arguments at run time).
template <int BM, int BN, int BK, int WM, int WN, bool BT = false>
hipError_t launch_tile_fp8_exact(const GemmArgs& a) {
    return launch_tile<2, BM, BN, BK, WM, WN, 0, 0, BT, 1>(a);
}

#define LIBGEMM_TILE_MIXED_CONFIGS(X) \
    X(64, 64, 128, 2, 2, false)       \
    X(128, 128, 128, 2, 2, false)     \
    X(256, 256, 128, 2, 4, false)     \
    X(64, 64, 128, 2, 2, true)        \
    X(128, 128, 128, 2, 2, true)      \
    X(256, 256, 128, 2, 4, true)

}  // namespace tile
}  // namespace libgemm
