// Ping-pong MFMA tile GEMM for gfx950: kernel and launcher templates, shared by
// gemm_pp.hip (configuration table, E4M3 x E4M3 and FP16 instantiations) and
// gemm_pp_mixed.hip (the other FP8 operand pairs).
//
// C[M,N] = (sA*A[M,K]) (sB*B[K,N]) with FP32 accumulation on the matrix cores
// ("DeepGEMM实战：FP8矩阵乘法与JIT编译优化指南" §2.1: FP8 in, FP32 accumulate, scales
// applied at write-back, §3.2; "HGEMM优化：深度学习中的矩阵乘法性能提升策略" §1.3 for
// FP16 with an FP32 accumulator). B is row-major B[K,N] or K-major Bt[N,K].
//
// One workgroup computes a 256 x 256 output tile (or 192 x 256, see Pp) with 8
// waves, two per SIMD. The waves form two groups of four (one wave of each
// group per SIMD): group G owns output rows [128 G, 128 G + 128), and wave j
// of a group the columns [64 j, 64 j + 64), i.e. a 128 x 64 wave tile held as
// 4 x 2 accumulators of the 32x32 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4 with
// neutral block scales for FP8, v_mfma_f32_32x32x16_f16 for FP16): 128
// registers per lane. With 192-row tiles a group owns 96 rows, 3 x 2 blocks.
//
// K advances in tiles of 64 bytes of every A row (64 FP8 or 32 FP16 values).
// Each K tile runs as two phases per group, and the groups are offset by one
// phase, so that on every SIMD one wave issues MFMAs while the other moves
// data:
//   MEM(t): read this wave's operands of tile t from LDS into registers; issue
//           this group's share of the direct loads (group 0: at odd t, A's
//           tiles t+3 and t+4; group 1: B's tile t+3); wait until this wave's
//           loads of tile t+1 have landed and its LDS reads are done; barrier.
//   MMA(t): the 8 (FP8) or 16 (FP16) MFMAs of tile t, at raised issue
//           priority; barrier.
// Group 1 enters the loop one barrier later than group 0, so the barrier that
// ends one group's MMA phase ends the other group's MEM phase. The staging
// (the double buffering of the FP8 guide §2.3, deepened as the HGEMM article
// §3.2/§3.3 discusses) is two rings filled by direct buffer->LDS loads:
//   A: three regions of BM rows x 128 bytes, each holding two K tiles, so that
//      every load reads whole 128-byte pieces of A's rows (a 64-byte piece
//      costs the L1 a whole line as well); pairs are loaded two or three
//      tiles before their first tile is read;
//   B: four stages of one K tile (64 k-rows x 256 n, or 256 Bt rows x 64
//      bytes), loaded three tiles ahead.
// 160 KiB of LDS in all (136 KiB with 192-row tiles). Every region and stage
// is its own LDS object, so the compiler can tell the in-flight direct loads
// from the 16-byte operand reads of the others and inserts no waits of its
// own for them; the transpose reads of row-major B are asm groups
// (device_common.h), since before a transpose-read builtin it would wait for
// every load in flight. The loads take 32-bit per-lane offsets and uniform
// ones through buffer resources, which keeps the address registers few.
//
// LDS layouts are bank-conflict free for the 16-lane passes of 16-byte reads
// (the DeepGEMM deep-dive §3.2 argues for a bank-aware layout; here it is an
// XOR permutation, since a direct load fixes each lane's LDS slot):
//   A region rows (128 bytes = 8 chunks of 16): chunk c of row r lives in
//   slot c ^ swz8(r), so 16 consecutive rows read at one chunk cover all 16
//   four-bank groups of two rows' 256 bytes;
//   Bt rows (64 bytes = 4 chunks of 16): chunk c of row r lives in slot
//   c ^ ((r >> 2) & 3), so 16 consecutive rows read at one chunk cover all 16
//   four-bank groups;
//   row-major B rows (256 or 512 bytes): chunk c of k-row r lives in slot
//   c ^ swz_b(r), so the rows and chunks of one transpose-read pass land in
//   distinct bank groups.
// Row-major B reaches the MFMA's K-contiguous operand layout through gfx950's
// LDS transpose reads (ds_read_b64_tr_b8 / _b16); a lane of a 16-lane group
// receives element (lane % E) of lanes (16 / E) e + lane / E of the group.
//
// The MFMAs take B's operand first and A's second, so each lane's 16
// accumulator values of a 32 x 32 block are one output row (lane % 32) and
// four runs of four consecutive columns. The epilogue multiplies by the scale
// product (sA*sB, or sA*sB/sOut for an FP8 output; per-channel sA[i]*sB[j]),
// converts, and for FP8 and FP16 outputs stages the wave's 128 x 64 block in
// LDS so that every lane stores 16-byte pieces of output rows.
//
// Edges (FP8 guide §3.3): rows of A (and Bt) past M (N) are loaded from the
// last valid row and column chunks of row-major B past N from the last valid
// chunk (valid addresses, never stored); a partial last K tile is loaded with
// guarded vector loads and zero fill; edge tiles store element by element with
// predicates. Operands that are not 16-byte aligned, or row blocks beyond
// 32-bit offsets, go to the register-staged tile kernel.
#pragma once

#include <cstring>

#include "device_common.h"
#include "kernels.h"
#include "tile_order.h"

namespace libgemm {
namespace pp {

// BM_: tile rows, 256 or 192 (three 32-row blocks per wave instead of four:
// 3000 x 4096 is 16 x 16 tiles of 192 x 256 on 256 CUs, against 12 x 16 tiles
// of 256 x 256 that leave a quarter of them idle).
template <int ES, int BM_ = 256>
struct Pp {
    static constexpr int BM = BM_, BN = 256;
    static_assert(BM == 256 || BM == 192, "tile rows: 256 or 192");
    static constexpr int NT = 512;                  // 8 waves
    static constexpr int S = 4;                     // B: LDS ring stages, one K tile each
    static constexpr int AP = 3;                    // A: LDS regions, two K tiles each
    static constexpr int ROWB = 64;                 // bytes of every A row per K tile
    static constexpr int BK = ROWB / ES;            // k per K tile (64 FP8, 32 FP16)
    static constexpr int VE = 16 / ES;              // elements per 16-byte chunk
    static constexpr int MR = BM / 2;               // A rows of one group
    static constexpr int MI = BM / 64;              // 32-row blocks per wave
    static constexpr int A_STAGE = BM * ROWB;       // A of one K tile: BM rows x 64 B
    static constexpr int A_PAIR = 2 * A_STAGE;      // A region: BM rows x 128 B (two K tiles)
    static constexpr int B_STAGE = 16384;           // B: 64 B of k x 256 n
    static constexpr int A_RPW = BM / 4;            // A rows one wave of group 0 loads
    static constexpr int BNB = BN * ES;             // row-major B: bytes of one k-row of the tile
    static constexpr int B_CPR = BNB / 16;          // chunks per row-major B row
    static constexpr int B_RPB = 1024 / BNB;        // row-major B rows per 1 KiB direct load
    static constexpr int LAP = A_RPW / 8;           // direct loads per wave per A region, group 0
    static constexpr int LB = B_STAGE / 4096;       // direct loads per wave per B stage, group 1
    static constexpr int KSUB = ES == 1 ? 1 : 2;    // MFMA k-steps per K tile (64 or 2 x 16 values)
    static_assert(AP * A_PAIR + S * B_STAGE <= 160 * 1024, "the LDS rings must fit in 160 KiB");
};

// s_waitcnt vmcnt(NA) for a wave of group 0, vmcnt(NB) for group 1 (their
// direct loads per K tile differ when BM < 256); LDS count LGKM.
template <int NA, int NB, int LGKM = 0>
__device__ __forceinline__ void wait_vm(bool group0) {
    if (NA == NB || !group0) __builtin_amdgcn_s_waitcnt(waitcnt_imm(NB, LGKM));
    else __builtin_amdgcn_s_waitcnt(waitcnt_imm(NA, LGKM));
}

__device__ __forceinline__ int swz_a(int r) { return (r >> 2) & 3; }

// A region rows (128 bytes, 8 chunks): chunk c of row r lives in slot
// c ^ swz8(r). Any 8 consecutive rows from a multiple of 8, and the even and
// the odd rows of 16 from a multiple of 16, take 8 distinct values.
__device__ __forceinline__ int swz8(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// Row-major B: k-row r's chunk c lives in slot c ^ swz_b(r). FP8 passes read 8
// rows x 2 adjacent chunks, FP16 passes 4 rows x 4 adjacent chunks; the values
// below differ in the bits those chunk pairs/quads do not cover.
template <int ES>
__device__ __forceinline__ int swz_b(int r) {
    return ES == 1 ? ((2 * (r & 7)) | ((r >> 2) & 1)) : (2 * (r & 3) + 8 * (r & 1));
}

template <int ES>
struct Mfma;

template <>
struct Mfma<1> {
    typedef v8i op;
    // FA, FB: operand formats (0 = E4M3, 1 = E5M2) of the instruction's first
    // and second operand.
    template <int FA, int FB>
    static __device__ __forceinline__ v16f mma(v8i a, v8i b, v16f c) {
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA, FB, 0, 127, 0, 127);
    }
};

template <>
struct Mfma<2> {
    typedef v8h op;
    template <int FA, int FB>
    static __device__ __forceinline__ v16f mma(v8h a, v8h b, v16f c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};

// OUT_E4M3 stands for both FP8 outputs; EPI_E5M2 in eflags picks the format.
template <int OUT>
__device__ __forceinline__ void store_elem(void* C, int64_t idx, float y, int eflags) {
    if constexpr (OUT == OUT_F32) {
        reinterpret_cast<float*>(C)[idx] = y;
    } else if constexpr (OUT == OUT_F16) {
        reinterpret_cast<_Float16*>(C)[idx] = (_Float16)y;
    } else {
        reinterpret_cast<uint8_t*>(C)[idx] = (eflags & EPI_E5M2) ? e5m2_from_f32(y) : e4m3_from_f32(y);
    }
}

// EX (FP8 only): exact accumulation. The FP8 codes are staged and read as in
// the FP8 kernel, then each 64-k operand is widened in registers to FP16 (every
// E4M3 and E5M2 value is an FP16 value) and multiplied as four k-steps of the
// FP16 MFMA (v_mfma_f32_32x32x16_f16), whose products and sums are exact in
// FP32. A lane's 32 codes cover k = 32 h .. 32 h + 31; k-step s takes codes
// 8 s .. 8 s + 7 of both operands, so every product pairs the same k.
template <int ES, int OUT, int FA, int FB, bool BT, bool EX = false, int BM = 256>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_pp_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ B, void* __restrict__ C, int M, int N, int K,
    const float* __restrict__ sA, const float* __restrict__ sB, const float* __restrict__ sOut, int tiles_m,
    int tiles_n, int eflags, int vec_out) {
    using T = Pp<ES, BM>;
    using Op = typename Mfma<ES>::op;
    __shared__ __attribute__((aligned(1024))) uint8_t a0[T::A_PAIR], a1[T::A_PAIR], a2[T::A_PAIR];
    __shared__ __attribute__((aligned(1024))) uint8_t b0[T::B_STAGE], b1[T::B_STAGE], b2[T::B_STAGE], b3[T::B_STAGE];
    // Region and stage selection; the index is a compile-time constant wherever
    // it matters (the main loop is unrolled by the ring periods).
    auto region_a = [&](int r) __attribute__((always_inline)) -> LDS_AS uint8_t* {
        switch (r) {
            case 0: return (LDS_AS uint8_t*)a0;
            case 1: return (LDS_AS uint8_t*)a1;
            default: return (LDS_AS uint8_t*)a2;
        }
    };
    auto stage_b = [&](int st) __attribute__((always_inline)) -> LDS_AS uint8_t* {
        switch (st) {
            case 0: return (LDS_AS uint8_t*)b0;
            case 1: return (LDS_AS uint8_t*)b1;
            case 2: return (LDS_AS uint8_t*)b2;
            default: return (LDS_AS uint8_t*)b3;
        }
    };

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int G = wave >> 2, wj = wave & 3;
    int tile_m, tile_n;
    tile_coords(blockIdx.x, tiles_m, tiles_n, tile_m, tile_n);
    const int m0 = tile_m * T::BM, n0 = tile_n * T::BN;
    const int nk = (K + T::BK - 1) / T::BK;
    const int nk_full = K / T::BK;
    // the epilogue's multiplier, loaded now (see epilogue_base_early)
    const bool chan = (eflags & EPI_CHANNEL) != 0;
    const float scale = epilogue_base_early(sA, sB, sOut, OUT == OUT_E4M3, chan);
    const int npf = nk_full / 2;            // K tile pairs whose two tiles are full
    const int KE = K * ES;                  // bytes of one A (or Bt) row

    // ---- group 0: A in pairs of K tiles, as whole 128-byte row pieces ----
    // Load i (< LAP) of wave j fills 1 KiB of a pair region: rows
    // A_RPW j + 8 i + lane / 8, slot lane % 8, which holds chunk slot ^ swz8(row)
    // of the row's 128 bytes (rows past M read the last row). The loads are
    // buffer loads: a 32-bit per-lane offset (two values, for even and odd i,
    // in interior tiles) and a uniform one.
    const uint8_t* srcA = A + (int64_t)m0 * KE;
    const int64_t a_end = (int64_t)M * KE, b_end = (int64_t)K * N * ES;
    const int arow = T::A_RPW * wj + (lane >> 3);
    const int cb_even = 16 * ((lane & 7) ^ (lane >> 3));   // chunk bytes where (row >> 3) is even
    const int par0 = (T::A_RPW * wj / 8) & 1;             // parity of the wave's first 8-row block
    const int mlast = M - 1 - m0;
    const bool a_inner = m0 + T::BM <= M;
    auto a_cb = [&](int i) __attribute__((always_inline)) -> int {
        return ((i + par0) & 1) ? (cb_even ^ 16) : cb_even;
    };
    auto a_off = [&](int i) __attribute__((always_inline)) -> uint32_t {
        return __umul24((uint32_t)min(arow + 8 * i, mlast), (uint32_t)KE) + (uint32_t)a_cb(i);
    };
    const uint32_t va[2] = {a_off(0), a_off(1)};          // interior tiles: rows arow, arow + 8
    // One resource for the tile's rows of A; the pair's K offset is uniform.
    const auto rsA = buffer_rsrc(srcA, a_end - (int64_t)m0 * KE);
    auto issue_a_pair = [&](int p, int reg) __attribute__((always_inline)) {
        const uint32_t kofs = (uint32_t)p * (2 * T::ROWB);
        LDS_AS uint8_t* dst = region_a(reg) + T::A_RPW * wj * (2 * T::ROWB);
        if (a_inner) {
#pragma unroll
            for (int i = 0; i < T::LAP; ++i)
                buffer_load_lds16(rsA, (LDS_AS void*)(dst + i * 1024), va[i & 1],
                                  kofs + (uint32_t)(16 * (i >> 1)) * (uint32_t)KE);
        } else {
#pragma unroll
            for (int i = 0; i < T::LAP; ++i) buffer_load_lds16(rsA, (LDS_AS void*)(dst + i * 1024), a_off(i), kofs);
        }
    };
    // A pair with a partial or missing tile: guarded vector loads, zero beyond
    // K, ordinary LDS stores (waiting for them also waits for every direct load
    // this wave has in flight).
    auto issue_a_pair_guarded = [&](int p, int reg) __attribute__((always_inline)) {
        const uint8_t* base = srcA + (int64_t)p * (2 * T::ROWB);
        LDS_AS uint8_t* dst = region_a(reg) + T::A_RPW * wj * (2 * T::ROWB);
#pragma unroll 1
        for (int i = 0; i < T::LAP; ++i) {
            const int k8 = (((i + par0) & 1) ? (cb_even ^ 16) : cb_even) >> 4;
            v4u v = v4u{0u, 0u, 0u, 0u};
            if ((p * 2 * T::ROWB + 16 * k8) / ES < K) v = *reinterpret_cast<const v4u*>(base + a_off(i));
            *(LDS_AS v4u*)(dst + i * 1024 + lane * 16) = v;
        }
    };

    // ---- group 1: B, one K tile per stage ----
    // Load i of wave j fills 1 KiB of a B stage: Bt rows 64 j + 16 i + lane / 4
    // (slot lane % 4), or row-major B rows B_RPB (4 j + i) + lane / B_CPR (slot
    // lane % B_CPR). goff: the byte offset of load i within the K tile.
    const uint8_t* srcB = BT ? B + (int64_t)n0 * KE : B + (int64_t)n0 * ES;
    auto b_off = [&](int i) __attribute__((always_inline)) -> uint32_t {
        if (BT) {
            const int r = 64 * wj + 16 * i + (lane >> 2);
            const int c = (lane & 3) ^ swz_a(r);
            const int rr = min(n0 + r, N - 1) - n0;
            return (uint32_t)(rr * KE + c * 16);
        } else {
            const int r = T::B_RPB * (4 * wj + i) + lane / T::B_CPR;
            const int c = (lane % T::B_CPR) ^ swz_b<ES>(r);
            const int col = min(n0 + c * T::VE, N - T::VE) - n0;
            return (uint32_t)(r * N * ES + col * ES);
        }
    };
    uint32_t goff[T::LB];
#pragma unroll
    for (int i = 0; i < T::LB; ++i) goff[i] = b_off(i);
    // The same as a per-lane part (even or odd i) and a uniform one, where
    // that holds: row-major B always, Bt in interior tiles.
    const bool b_split = !BT || n0 + T::BN <= N;
    const uint32_t vb[2] = {goff[0], goff[1]};
    auto b_uni = [&](int i) __attribute__((always_inline)) -> uint32_t {
        return BT ? (uint32_t)(16 * (i & ~1)) * (uint32_t)KE : (uint32_t)(T::B_RPB * (i & ~1)) * (uint32_t)(N * ES);
    };
    const int64_t kstep_b = BT ? (int64_t)T::ROWB : (int64_t)T::BK * N * ES;
    // Loads of B tile kt into stage st through resource rs, whose base is
    // kb K tiles before tile kt (kb <= 15; the offsets stay below 2^31, see
    // pp_fits).
    auto issue_b_via = [&](__amdgpu_buffer_rsrc_t rs, int kb, int st) __attribute__((always_inline)) {
        const uint32_t kofs = (uint32_t)kb * (uint32_t)kstep_b;
        LDS_AS uint8_t* dst = stage_b(st) + wj * 4096;
        if (b_split) {
#pragma unroll
            for (int i = 0; i < T::LB; ++i)
                buffer_load_lds16(rs, (LDS_AS void*)(dst + i * 1024), vb[i & 1], kofs + b_uni(i));
        } else {
#pragma unroll
            for (int i = 0; i < T::LB; ++i) buffer_load_lds16(rs, (LDS_AS void*)(dst + i * 1024), goff[i], kofs);
        }
    };
    // B from K tile kt on (a resource per block of the main loop, or per tile).
    auto rsrc_b = [&](int kt) __attribute__((always_inline)) {
        const uint8_t* p = srcB + (int64_t)kt * kstep_b;
        return buffer_rsrc(p, b_end - (p - B));
    };
    auto issue_b = [&](int kt, int st) __attribute__((always_inline)) { issue_b_via(rsrc_b(kt), 0, st); };
    auto issue_b_partial = [&](int kt, int st) __attribute__((always_inline)) {
        const uint8_t* p = srcB + (int64_t)kt * kstep_b;
        const int k0 = kt * T::BK;
        LDS_AS uint8_t* dst = stage_b(st) + wj * 4096;
#pragma unroll 1
        for (int i = 0; i < T::LB; ++i) {
            v4u v = v4u{0u, 0u, 0u, 0u};
            if (BT) {
                const int r = 64 * wj + 16 * i + (lane >> 2);
                const int c = (lane & 3) ^ swz_a(r);
                if (k0 + c * T::VE < K) v = *reinterpret_cast<const v4u*>(p + goff[i]);
            } else {
                const int r = T::B_RPB * (4 * wj + i) + lane / T::B_CPR;
                if (k0 + r < K) v = *reinterpret_cast<const v4u*>(p + goff[i]);
            }
            *(LDS_AS v4u*)(dst + i * 1024 + lane * 16) = v;
        }
    };

    // ---- operand reads ----
    // A: rows MR G + 32 i + lane % 32 of the pair region; tile t is chunks
    // 4 (t % 2) .. + 3 of the row; FP8 takes chunks 2h, 2h + 1 of the tile
    // (k = 32 h .. 32 h + 31), FP16 k-step u takes chunk 2u + h (h = lane / 32).
    // The row's swizzle is that of lane % 32 (row blocks start at multiples of 16).
    const int lr = lane & 31, h = lane >> 5;
    const int sw8 = swz8(lr);
    const int sw = swz_a(lr);
    const int j16 = lane & 15, half = (lane >> 4) & 1;
    auto rd_a = [&](const LDS_AS uint8_t* rowp, int u, int par) __attribute__((always_inline)) -> Op {
        if constexpr (ES == 1) {
            const v4i lo = *(const LDS_AS v4i*)(rowp + (((4 * par + 2 * h) ^ sw8) << 4));
            const v4i hi = *(const LDS_AS v4i*)(rowp + (((4 * par + 2 * h + 1) ^ sw8) << 4));
            return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        } else {
            return __builtin_bit_cast(v8h, *(const LDS_AS v4u*)(rowp + (((4 * par + 2 * u + h) ^ sw8) << 4)));
        }
    };
    // Bt rows of a B stage (64 bytes, 4 chunks, swizzle swz_a).
    auto rd_bt = [&](const LDS_AS uint8_t* rowp, int u) __attribute__((always_inline)) -> Op {
        if constexpr (ES == 1) {
            const v4i lo = *(const LDS_AS v4i*)(rowp + (((2 * h) ^ sw) << 4));
            const v4i hi = *(const LDS_AS v4i*)(rowp + (((2 * h + 1) ^ sw) << 4));
            return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        } else {
            return __builtin_bit_cast(v8h, *(const LDS_AS v4u*)(rowp + (((2 * u + h) ^ sw) << 4)));
        }
    };
    // Row-major B: all of this wave's operands of one K tile, ob[u][jb] for
    // column block jb (64 wj + 32 jb + 0..31), as eight transpose reads with
    // one wait.
    // FP8: 16-lane group (h, half) reads columns 64 wj + 32 jb + 16 half +
    // 0..15; read q: lane j16 addresses k-row 32 h + 8 q + j16 / 2, bytes
    // 8 (j16 % 2) of the column chunk; k-row % 8 = j16 / 2.
    // FP16, k-step u: lane j16 addresses k-row 16 u + 8 h + 4 q + j16 / 4,
    // columns 64 wj + 32 jb + 16 half + 4 (j16 % 4) .. + 3; k-row % 4 = j16 / 4.
    auto rd_b_rowmajor_all = [&](const LDS_AS uint8_t* sb, typename Mfma<ES>::op (&ob)[T::KSUB][2])
        __attribute__((always_inline)) {
        uint32_t ad[8];
        if constexpr (ES == 1) {
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) {
                const int chunk = (4 * wj + 2 * jb + half) ^ swz_b<1>(j16 >> 1);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int k = 32 * h + 8 * q + (j16 >> 1);
                    ad[4 * jb + q] = lds_addr(sb + k * T::BNB + chunk * 16 + 8 * (j16 & 1));
                }
            }
            v2i t[8];
            lds_tr8_x8(t, ad);
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) {
                const v4i t01 = __builtin_shufflevector(t[4 * jb], t[4 * jb + 1], 0, 1, 2, 3);
                const v4i t23 = __builtin_shufflevector(t[4 * jb + 2], t[4 * jb + 3], 0, 1, 2, 3);
                ob[0][jb] = __builtin_shufflevector(t01, t23, 0, 1, 2, 3, 4, 5, 6, 7);
            }
        } else {
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int jb = 0; jb < 2; ++jb) {
                    const int chunk = (8 * wj + 4 * jb + 2 * half + ((j16 & 3) >> 1)) ^ swz_b<2>(j16 >> 2);
#pragma unroll
                    for (int q = 0; q < 2; ++q) {
                        const int k = 16 * u + 8 * h + 4 * q + (j16 >> 2);
                        ad[4 * u + 2 * jb + q] = lds_addr(sb + k * T::BNB + chunk * 16 + 8 * (j16 & 1));
                    }
                }
            v4s t[8];
            lds_tr16_x8(t, ad);
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int jb = 0; jb < 2; ++jb)
                    ob[u][jb] = __builtin_bit_cast(
                        v8h, __builtin_shufflevector(t[4 * u + 2 * jb], t[4 * u + 2 * jb + 1], 0, 1, 2, 3, 4, 5, 6, 7));
        }
    };

    v16f acc[T::MI][2];
#pragma unroll
    for (int i = 0; i < T::MI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;


    Op opa[T::KSUB][T::MI], opb[T::KSUB][2];
    // vmcnt immediate for at most n of this wave's loads in flight, n known at
    // run time: the largest count used here that is not above n (waiting for
    // fewer is always safe).
    auto wait_rt = [&](int n) __attribute__((always_inline)) {
        if (n >= 8) __builtin_amdgcn_s_waitcnt(waitcnt_imm(8, 0));
        else if (n >= 6) __builtin_amdgcn_s_waitcnt(waitcnt_imm(6, 0));
        else if (n >= 4) __builtin_amdgcn_s_waitcnt(waitcnt_imm(4, 0));
        else __builtin_amdgcn_s_waitcnt(0);
    };
    // This wave's loads that may stay in flight once K tile t+1 has landed,
    // after the loads of step t were issued (t = -1: the prologue).
    // Group 0: pairs issued after the pair of tile t+1 (at most one), unless
    // a guarded pair load has drained them. Group 1: B tiles issued after t+1
    // (at most two), likewise.
    auto younger = [&](int t) __attribute__((always_inline)) -> int {
        if (G == 0) {
            const int sched = (t & 1) ? (t + 3) / 2 : (t + 2) / 2;  // last pair issued by now
            if (2 * npf < nk && sched >= npf) return 0;
            return max(0, min(sched, npf - 1) - (t + 1) / 2) * T::LAP;
        }
        if (nk > nk_full && t + 3 >= nk_full) return 0;
        return max(0, min(t + 3, nk_full - 1) - (t + 1)) * T::LB;
    };
    // Loads of step t (odd t: group 0 the A pair (t+3)/2; every t: group 1
    // B tile t+3), choosing full, guarded or none at run time.
    auto issue_rt = [&](int t) __attribute__((always_inline)) {
        if (G == 0) {
            if (t & 1) {
                const int p = (t + 3) / 2;
                if (p < npf) issue_a_pair(p, p % T::AP);
                else if (2 * p < nk) issue_a_pair_guarded(p, p % T::AP);
            }
        } else {
            const int nt = t + 3;
            if (nt < nk_full) issue_b(nt, nt % T::S);
            else if (nt < nk) issue_b_partial(nt, nt % T::S);
        }
    };
    // One K tile: MEM(t) then MMA(t). steady: every tile step t loads exists
    // and is full, and the LDS indices are compile-time constants (t is
    // congruent to tm modulo 12); otherwise everything is chosen at run time.
    __amdgpu_buffer_rsrc_t rs_blk;  // B from the first K tile of the main-loop block
    auto step = [&](int t, int tm, bool steady) __attribute__((always_inline)) {
        const int ar = steady ? (tm / 2) % T::AP : (t / 2) % T::AP;
        const int par = steady ? (tm & 1) : (t & 1);
        const int bs = steady ? tm % T::S : t % T::S;
        // MEM(t)
        const LDS_AS uint8_t* sa = region_a(ar) + (T::MR * G + lr) * (2 * T::ROWB);
#pragma unroll
        for (int u = 0; u < T::KSUB; ++u)
#pragma unroll
            for (int i = 0; i < T::MI; ++i) opa[u][i] = rd_a(sa + 32 * i * (2 * T::ROWB), u, par);
        if constexpr (BT) {
            const LDS_AS uint8_t* sbt = stage_b(bs) + (64 * wj + lr) * T::ROWB;
#pragma unroll
            for (int u = 0; u < T::KSUB; ++u)
#pragma unroll
                for (int j = 0; j < 2; ++j) opb[u][j] = rd_bt(sbt + 32 * j * T::ROWB, u);
        } else {
            rd_b_rowmajor_all(stage_b(bs), opb);
        }
        if (steady) {
            if (G == 0) {
                if (tm & 1) issue_a_pair((t + 3) / 2, ((tm + 3) / 2) % T::AP);
            } else {
                issue_b_via(rs_blk, tm + 3, (tm + 3) % T::S);
            }
            wait_vm<T::LAP, 2 * T::LB>(G == 0);
        } else {
            issue_rt(t);
            wait_rt(t + 1 < nk ? younger(t) : 0);
        }
        asm volatile("s_barrier" ::: "memory");
        // MMA(t): operands pinned after the barrier, products before the next one
#pragma unroll
        for (int u = 0; u < T::KSUB; ++u) {
#pragma unroll
            for (int i = 0; i < T::MI; ++i) asm volatile("" : "+v"(opa[u][i]));
#pragma unroll
            for (int j = 0; j < 2; ++j) asm volatile("" : "+v"(opb[u][j]));
        }
        __builtin_amdgcn_s_setprio(1);
        if constexpr (EX) {
            static_assert(ES == 1, "exact accumulation widens FP8 codes");
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                // B's two operands widened once per k-step, A's one at a time
                // (fewer live registers)
                v8h wb[2];
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    wb[j] = __builtin_bit_cast(
                        v8h, widen8_fp8((uint32_t)opb[0][j][2 * ks], (uint32_t)opb[0][j][2 * ks + 1], FB == 1));
#pragma unroll
                for (int i = 0; i < T::MI; ++i) {
                    const v8h wa = __builtin_bit_cast(
                        v8h, widen8_fp8((uint32_t)opa[0][i][2 * ks], (uint32_t)opa[0][i][2 * ks + 1], FA == 1));
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wb[j], wa, acc[i][j], 0, 0, 0);
                }
            }
        } else {
#pragma unroll
            for (int u = 0; u < T::KSUB; ++u)
#pragma unroll
                for (int i = 0; i < T::MI; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        acc[i][j] = Mfma<ES>::template mma<FB, FA>(opb[u][j], opa[u][i], acc[i][j]);
        }
#pragma unroll
        for (int i = 0; i < T::MI; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) asm volatile("" : "+v"(acc[i][j]));
        __builtin_amdgcn_s_setprio(0);
        asm volatile("s_barrier" ::: "memory");
    };

    // ---- prologue: A pairs 0 and 1 (tiles 0-3), B tiles 0-2; wait for tile 0 ----
    if (G == 0) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            if (p < npf) issue_a_pair(p, p);
            else if (2 * p < nk) issue_a_pair_guarded(p, p);
        }
    } else {
#pragma unroll
        for (int kt = 0; kt < 3; ++kt) {
            if (kt < nk_full) issue_b(kt, kt);
            else if (kt < nk) issue_b_partial(kt, kt);
        }
    }
    wait_rt(younger(-1));
    asm volatile("s_barrier" ::: "memory");
    if (G == 1) asm volatile("s_barrier" ::: "memory");

    // Main loop, unrolled by 12 (the A regions repeat every 6 tiles, the B
    // stages every 4) so that every region and stage is a fixed LDS object; it
    // runs while the tiles it loads (up to t + 15) are full tiles.
    int t = 0;
    for (; t + 16 <= nk_full; t += 12) {
        rs_blk = rsrc_b(t);
        step(t, 0, true);
        step(t + 1, 1, true);
        step(t + 2, 2, true);
        step(t + 3, 3, true);
        step(t + 4, 4, true);
        step(t + 5, 5, true);
        step(t + 6, 6, true);
        step(t + 7, 7, true);
        step(t + 8, 8, true);
        step(t + 9, 9, true);
        step(t + 10, 10, true);
        step(t + 11, 11, true);
    }
#pragma unroll 1
    for (; t < nk; ++t) step(t, 0, false);
    if (G == 0) asm volatile("s_barrier" ::: "memory");

    // ---- epilogue ----
    // Block (i, j), element 4q + e: row MR G + 32 i + lr, column
    // 64 wj + 32 j + 8 q + 4 h + e of the tile.
    const int row_t = T::MR * G + lr;          // + 32 i
    const int col_t = 64 * wj + 4 * h;         // + 32 j + 8 q
    // Vector stores need a 16-byte aligned C with 16-byte row pitches (vec_out).
    const bool interior = vec_out && (m0 + T::BM <= M) && (n0 + T::BN <= N);
    if (!interior) {
#pragma unroll
        for (int i = 0; i < T::MI; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = m0 + row_t + 32 * i, col = n0 + col_t + 32 * j + 8 * (r >> 2) + (r & 3);
                    if (row < M && col < N) {
                        float y = acc[i][j][r] * scale;
                        if (chan) y *= sA[row] * sB[col];
                        store_elem<OUT>(C, (int64_t)row * N + col, y, eflags);
                    }
                }
        return;
    }
    // Interior tile: the scaled values of one run of four columns.
    auto run4 = [&](int i, int j, int q) __attribute__((always_inline)) -> v4f {
        v4f y;
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = acc[i][j][4 * q + e] * scale;
        if (chan) {
            const float sr = sA[m0 + row_t + 32 * i];
            const int col = n0 + col_t + 32 * j + 8 * q;
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] *= sr * sB[col + e];
        }
        return y;
    };
    // The same without per-channel factors (the per-tensor case, decided once
    // for the whole block rather than per run).
    auto plain4 = [&](int i, int j, int q) __attribute__((always_inline)) -> v4f {
        v4f y;
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = acc[i][j][4 * q + e] * scale;
        return y;
    };
    if constexpr (OUT == OUT_F32) {
        float* Cf = reinterpret_cast<float*>(C);
        auto store_all = [&](auto val4) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < T::MI; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        *reinterpret_cast<v4f*>(Cf + (int64_t)(m0 + row_t + 32 * i) * N + n0 + col_t + 32 * j +
                                                8 * q) = val4(i, j, q);
        };
        if (chan) store_all(run4);
        else store_all(plain4);
        return;
    }
    // FP8 / FP16: the wave's 32 MI x 64 block goes to its own LDS stage array
    // (row pitch 64 ES bytes), then each lane stores 16-byte row pieces. Every
    // wave has finished its last operand read (the final barrier above).
    // The 16-byte chunk c of block row r sits at slot c ^ esw(r): a write
    // instruction puts 32 rows at one column, and with plain row pitches of
    // 64 / 128 bytes every fourth / second row would hit the same banks
    // (8-way conflicts; measured at about 7700 conflict cycles per FP8 tile).
    constexpr int RB = 64 * (OUT == OUT_F16 ? 2 : 1);  // bytes of one block row
    auto esw = [](int r) __attribute__((always_inline)) -> int {
        return OUT == OUT_F16 ? ((r >> 1) & 7) : ((r >> 2) & 3);
    };
    static_assert(32 * T::MI * RB <= T::A_STAGE, "a wave's staged block fits in one LDS stage");
    LDS_AS uint8_t* ep = wave < 4 ? stage_b(wave) : region_a((wave - 4) >> 1) + ((wave - 4) & 1) * T::A_STAGE;
    auto slot = [&](int i, int j, int q) __attribute__((always_inline)) -> int {
        const int r = 32 * i + lr, cb = (32 * j + 8 * q + 4 * h) * (RB / 64);
        return r * RB + ((((cb >> 4) ^ esw(r)) << 4) | (cb & 15));
    };
    if constexpr (OUT == OUT_F16) {
        auto stage_all = [&](auto val4) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < T::MI; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const v4f y = val4(i, j, q);
                        typedef _Float16 v4hh __attribute__((ext_vector_type(4)));
                        const v4hh hv = {(_Float16)y[0], (_Float16)y[1], (_Float16)y[2], (_Float16)y[3]};
                        *(LDS_AS v2i*)(ep + slot(i, j, q)) = __builtin_bit_cast(v2i, hv);
                    }
        };
        if (chan) stage_all(run4);
        else stage_all(plain4);
    } else {
        // FP8 codes. Per-tensor blocks take a short path: the clamp to the
        // format's largest finite value is one median-of-three (as the
        // fmin/fmax pair of the code functions, for every value but NaN), and
        // NaN is only detected, one unordered compare per pair; a wave that
        // met one writes its block again with the code functions, which map
        // NaN to 0x7F. Per-channel blocks take the code functions directly.
        bool exact = chan;
        if (!chan) {
            bool nan = false;
            auto stage_fast = [&](auto fmt) __attribute__((always_inline)) {
                constexpr bool E5 = decltype(fmt)::value;
                constexpr float hi = E5 ? 57344.0f : 448.0f;
#pragma unroll
                for (int i = 0; i < T::MI; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const v4f y = plain4(i, j, q);
                            nan |= __builtin_isunordered(y[0], y[1]) | __builtin_isunordered(y[2], y[3]);
                            float c[4];
#pragma unroll
                            for (int e = 0; e < 4; ++e) c[e] = __builtin_amdgcn_fmed3f(y[e], -hi, hi);
                            // the first conversion's upper half is overwritten by
                            // the second, so any register serves as its old value
                            uint32_t w = __builtin_bit_cast(uint32_t, c[3]);
                            if constexpr (E5) {
                                w = (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(c[0], c[1], (int)w, false);
                                w = (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(c[2], c[3], (int)w, true);
                            } else {
                                w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], (int)w, false);
                                w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], (int)w, true);
                            }
                            *(LDS_AS uint32_t*)(ep + slot(i, j, q)) = w;
                        }
            };
            if (eflags & EPI_E5M2) stage_fast(BoolC<true>{});
            else stage_fast(BoolC<false>{});
            exact = __builtin_amdgcn_ballot_w64(nan) != 0;
        }
        if (exact) {
#pragma unroll
            for (int i = 0; i < T::MI; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const v4f y = run4(i, j, q);
                        const uint32_t w = (eflags & EPI_E5M2) ? e5m2_pack4(y[0], y[1], y[2], y[3])
                                                              : e4m3_pack4(y[0], y[1], y[2], y[3]);
                        *(LDS_AS uint32_t*)(ep + slot(i, j, q)) = w;
                    }
        }
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
    constexpr int LPR = RB / 16;             // lanes per block row
    constexpr int RPI = 64 / LPR;            // block rows per store instruction
    uint8_t* Cb = reinterpret_cast<uint8_t*>(C);
    const int es_out = RB / 64;
#pragma unroll
    for (int p = 0; p < 32 * T::MI / RPI; ++p) {
        const int r = RPI * p + lane / LPR, seg = lane % LPR;
        const v4i v = *(const LDS_AS v4i*)(ep + r * RB + 16 * (seg ^ esw(r)));
        *reinterpret_cast<v4i*>(Cb + ((int64_t)(m0 + T::MR * G + r) * N + n0 + 64 * wj) * es_out + 16 * seg) = v;
    }
}

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Whether the ping-pong kernel can take the request: 16-byte aligned operands
// and row pitches, and 32-bit offsets within a tile's row block.
template <int ES, bool BT, int BM = 256>
inline bool pp_fits(const GemmArgs& a) {
    using T = Pp<ES, BM>;
    const bool aligned = aligned16(a.A) && aligned16(a.B) && (a.K * ES) % 16 == 0 && (BT || (a.N * ES) % 16 == 0);
    const bool fits = (int64_t)T::BM * a.K * ES < (1ll << 31) &&
                      (BT ? (int64_t)T::BN * a.K * ES : (int64_t)16 * T::BK * a.N * ES) < (1ll << 31);
    return aligned && fits;
}

// The register-staged 256 x 256 kernel, for requests the ping-pong kernel
// cannot take.
inline hipError_t fallback(int kind, const GemmArgs& a, bool exact = false) {
    const char* name = exact ? (a.b_kmajor ? "exact_fp8_256x256x64_w2x4_bt" : "exact_fp8_256x256x64_w2x4")
                     : a.b_kmajor ? (kind == KIND_FP8 ? "tile_fp8_256x256x128_w2x4_bt" : "tile_f16_256x256x64_w2x4_bt")
                                  : (kind == KIND_FP8 ? "tile_fp8_256x256x128_w2x4" : "tile_f16_256x256x64_w2x4");
    int nt = 0;
    const GemmConfig* tt = exact ? exact_configs(&nt) : tile_configs(&nt);
    for (int i = 0; i < nt; ++i)
        if (std::strcmp(tt[i].name, name) == 0) return tt[i].launch(a);
    return hipErrorInvalidValue;
}

template <int ES, int FA, int FB, bool BT, bool EX = false, int BM = 256>
hipError_t launch_pp(const GemmArgs& a) {
    using T = Pp<ES, BM>;
    if (a.splits > 1) return hipErrorInvalidValue;  // no split-K (kgran 0 in the table)
    if (BT != (a.b_kmajor != 0)) return hipErrorInvalidValue;
    const int64_t tiles_m = (a.M + T::BM - 1) / T::BM;
    const int64_t tiles_n = (a.N + T::BN - 1) / T::BN;
    const int64_t blocks = tiles_m * tiles_n;
    if (blocks <= 0) return hipSuccess;
    if (!pp_fits<ES, BT, BM>(a) || blocks > 0x7FFFFFFF) return fallback(ES == 1 ? KIND_FP8 : KIND_F16, a, EX);
    const uint8_t* A = reinterpret_cast<const uint8_t*>(a.A);
    const uint8_t* B = reinterpret_cast<const uint8_t*>(a.B);
    const int M = (int)a.M, N = (int)a.N, K = (int)a.K;
    const dim3 grid((unsigned)blocks), block(T::NT);
    const int eflags = (a.out_dtype == OUT_E5M2 ? EPI_E5M2 : 0) | (a.channel ? EPI_CHANNEL : 0);
    const int64_t out_es = a.out_dtype == OUT_F32 ? 4 : (a.out_dtype == OUT_F16 ? 2 : 1);
    const int vec_out = aligned16(a.C) && (a.N * out_es) % 16 == 0;
    switch (a.out_dtype) {
        case OUT_F32:
            gemm_pp_kernel<ES, OUT_F32, FA, FB, BT, EX, BM><<<grid, block, 0, a.stream>>>(
                A, B, a.C, M, N, K, a.sA, a.sB, a.sOut, (int)tiles_m, (int)tiles_n, eflags, vec_out);
            break;
        case OUT_F16:
            gemm_pp_kernel<ES, OUT_F16, FA, FB, BT, EX, BM><<<grid, block, 0, a.stream>>>(
                A, B, a.C, M, N, K, a.sA, a.sB, a.sOut, (int)tiles_m, (int)tiles_n, eflags, vec_out);
            break;
        default:
            if constexpr (ES == 1) {
                gemm_pp_kernel<ES, OUT_E4M3, FA, FB, BT, EX, BM><<<grid, block, 0, a.stream>>>(
                    A, B, a.C, M, N, K, a.sA, a.sB, a.sOut, (int)tiles_m, (int)tiles_n, eflags, vec_out);
            } else {
                return hipErrorInvalidValue;
            }
    }
    return hipGetLastError();
}

// Operand-format dispatch; the pairs other than E4M3 x E4M3 are instantiated
// in gemm_pp_mixed.hip.
template <bool BT, int BM = 256>
hipError_t launch_pp_fp8_any(const GemmArgs& a) {
    switch (a.fmt_a * 2 + a.fmt_b) {
        case 0: return launch_pp<1, 0, 0, BT, false, BM>(a);
        case 1: return launch_pp<1, 0, 1, BT, false, BM>(a);
        case 2: return launch_pp<1, 1, 0, BT, false, BM>(a);
        default: return launch_pp<1, 1, 1, BT, false, BM>(a);
    }
}

// Exact accumulation (gemm_pp_exact.hip instantiates it).
template <bool BT>
hipError_t launch_pp_fp8_exact(const GemmArgs& a) {
    switch (a.fmt_a * 2 + a.fmt_b) {
        case 0: return launch_pp<1, 0, 0, BT, true>(a);
        case 1: return launch_pp<1, 0, 1, BT, true>(a);
        case 2: return launch_pp<1, 1, 0, BT, true>(a);
        default: return launch_pp<1, 1, 1, BT, true>(a);
    }
}

}  // namespace pp
}  // namespace libgemm
