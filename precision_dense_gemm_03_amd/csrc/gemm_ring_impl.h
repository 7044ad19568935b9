// Deep-ring MFMA tile GEMM for skinny shapes (M <= 256) on gfx950: kernel and
// launcher templates, shared by gemm_ring.hip (configuration table, E4M3 x
// E4M3 and FP16 instantiations) and gemm_ring_mixed.hip (the other FP8
// operand pairs).
//
// C[M,N] = (sA*A[M,K]) (sB*B[K,N]), FP32 accumulation on the matrix cores
// ("DeepGEMM实战：FP8矩阵乘法与JIT编译优化指南" §2.1, §3.2; "HGEMM优化：深度学习中的矩阵乘法性能
// 提升策略" §1.3). B is row-major B[K,N] or K-major Bt[N,K].
//
// With M a few dozen rows the product is bound by moving B (and A, which every
// workgroup re-reads from L2) into the compute units, not by the matrix cores
// (the FP8 guide §3.3 picks a smaller tile when an edge tile would be mostly
// padding; the HGEMM article §3.1 sizes tiles by shape). On MI355X one compute
// unit streams at most about 50 GB/s from HBM, so the tile is chosen small
// enough (BM x BN, BM and BN from 16 to 64) that the grid covers every compute
// unit, and each workgroup's loads run far ahead: a ring of S LDS stages (8,
// or as many as fit in 144 KiB), each holding 128 bytes of every A row and
// the matching 128 BN bytes of B, is filled by direct global->LDS loads S-1 K
// tiles ahead (the HGEMM article §3.2/§3.3 on prefetch depth). One barrier per
// K tile: each wave waits for its own loads of tile t, the barrier makes
// everyone's visible (and retires tile t-1's stage), the wave refills that
// stage with tile t+S-1 and multiplies tile t. B's loads carry the
// non-temporal hint (B streams through once; measured faster for both layouts,
// most for row-major B, whose cached loads evict more dirty lines).
//
// Four waves. The tile's 16x16 MFMA blocks (v_mfma_scale_f32_16x16x128_f8f6f4
// with neutral scales for FP8, v_mfma_f32_16x16x32_f16 for FP16) are spread
// over the waves; a tile with fewer than four blocks gives each block to
// KW = 4 / blocks waves, which take turns over the K tiles (wave group g
// multiplies the tiles t with t % KW == g) and add their partial sums through
// LDS at the end, in group order. The MFMA takes B's operand first, so a
// lane's four accumulator values are four consecutive columns of one output
// row, stored as one vector.
//
// LDS layouts (XOR permutations chosen so that the lanes of one LDS pass hit
// distinct bank groups; a direct load fixes each lane's LDS slot, so the
// permutation goes into which chunk a lane fetches, the deep-dive's §3.2 idea
// of a bank-aware layout):
//   A and Bt rows (128 bytes = 8 chunks): chunk c of row r in slot c ^ ((r >> 1) & 7);
//   row-major FP8 B (BN-byte k-rows): c ^ ((((r >> 2) & 1) | ((r >> 4) & 2)) & (BN / 16 - 1));
//   row-major FP16 B (2 BN-byte k-rows): c ^ ((2 * ((r >> 1) & 1) + 4 * ((r >> 3) & 1)) & (BN / 8 - 1)).
// Row-major B reaches the MFMA's K-contiguous operand through gfx950's LDS
// transpose reads (ds_read_b64_tr_b8 / _b16, in asm groups: device_common.h).
//
// Edges: A rows past M and Bt rows / B column chunks past N are loaded from
// clamped (valid) addresses and never stored. A partial last K tile is loaded
// like the others, its chunks past K from clamped addresses; once it has
// landed, each wave writes zeros over the chunks it fetched past K before the
// tile is multiplied. Edge tiles store element by element.
#pragma once

#include <cstring>

#include "device_common.h"
#include "kernels.h"
#include "tile_order.h"

namespace libgemm {
namespace ring {

template <int ES, int BM, int BN, bool BT>
struct Ring {
    static constexpr int NT = 256;
    static constexpr int ROWB = 128;                          // bytes of every A row per K tile
    static constexpr int BK = ROWB / ES;                      // k per K tile (128 FP8, 64 FP16)
    static constexpr int VE = 16 / ES;                        // elements per 16-byte chunk
    static constexpr int A_BYTES = BM * ROWB;
    static constexpr int B_BYTES = BN * ROWB;                 // BN n x 128 bytes, or BK k-rows x BN ES bytes
    static constexpr int BNB = BN * ES;                       // row-major B: bytes of one k-row of the tile
    static constexpr int CPR = BNB / 16;                      // row-major B: 16-byte chunks per k-row
    static constexpr int STAGE = A_BYTES + B_BYTES;
    // LDS ring stages: 8, or as many as fit in 144 KiB (deeper rings measured
    // no faster: the stream is then bound by the memory system, not the
    // number of loads in flight)
    static constexpr int S = (144 * 1024 / STAGE) < 8 ? (144 * 1024 / STAGE) : 8;
    static constexpr int A_INST = A_BYTES / 1024;             // 1 KiB direct loads per stage
    static constexpr int INST = A_INST + B_BYTES / 1024;
    static constexpr int MAX_PER_WAVE = (INST + 3) / 4;       // loads of one wave per stage
    static constexpr int BLOCKS = (BM / 16) * (BN / 16);      // 16x16 MFMA blocks per tile
    static constexpr int KW = BLOCKS >= 4 ? 1 : 4 / BLOCKS;   // wave groups taking turns over K tiles
    static constexpr int WPK = 4 / KW;                        // waves per group
    static constexpr int WROWS = BM / 16;                     // a group's waves along M
    static constexpr int WCOLS = WPK / WROWS;                 // ... and along N
    static constexpr int TN = BN / 16 / WCOLS;                // 16-column blocks per wave
    static constexpr int KSUB = ES == 1 ? 1 : 2;              // MFMA k-steps per K tile
    static_assert(BM == 16 || BM == 32 || BM == 64, "BM is 16, 32 or 64");
    static_assert(BN == 16 || BN == 32 || BN == 64, "BN is 16, 32 or 64");
    static_assert(WROWS <= WPK && WCOLS * WROWS == WPK && TN * WCOLS * 16 == BN, "wave layout");
    static_assert(INST >= 4, "every wave issues at least one load per stage");
    static_assert(S >= 4 && S * STAGE <= 144 * 1024, "the LDS ring must fit in 144 KiB");
};

// Loads of wave w per stage: the 1 KiB loads j = w, w + 4, ... < INST.
template <int INST>
constexpr int loads_of(int w) {
    return (INST - w + 3) / 4;
}

__device__ __forceinline__ int swz_row(int r) { return (r >> 1) & 7; }

// One K-step's operand reads of every column block in one asm group with one
// LDS wait (A's operand first, then the column blocks' reads in order): the
// wave pays one LDS round trip per k-step instead of one per column block
// (row-major FP8 B; FP16 takes both of its k-steps in one group).
// The outputs are early-clobber and the wait is inside the block, for the
// reasons given with the groups in device_common.h.
__device__ __forceinline__ void ring_b128x2_tr16x4(v4i (&r)[2], v4s (&t)[4], const uint32_t (&a)[6]) {
    asm volatile(
        "ds_read_b128 %0, %6\n\t"
        "ds_read_b128 %1, %7\n\t"
        "ds_read_b64_tr_b16 %2, %8\n\t"
        "ds_read_b64_tr_b16 %3, %9\n\t"
        "ds_read_b64_tr_b16 %4, %10\n\t"
        "ds_read_b64_tr_b16 %5, %11\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5])
        : "memory");
}

__device__ __forceinline__ void ring_b128x2_tr16x8(v4i (&r)[2], v4s (&t)[8], const uint32_t (&a)[10]) {
    asm volatile(
        "ds_read_b128 %0, %10\n\t"
        "ds_read_b128 %1, %11\n\t"
        "ds_read_b64_tr_b16 %2, %12\n\t"
        "ds_read_b64_tr_b16 %3, %13\n\t"
        "ds_read_b64_tr_b16 %4, %14\n\t"
        "ds_read_b64_tr_b16 %5, %15\n\t"
        "ds_read_b64_tr_b16 %6, %16\n\t"
        "ds_read_b64_tr_b16 %7, %17\n\t"
        "ds_read_b64_tr_b16 %8, %18\n\t"
        "ds_read_b64_tr_b16 %9, %19\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3]), "=&v"(t[4]), "=&v"(t[5]), "=&v"(t[6]), "=&v"(t[7])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]), "v"(a[8]), "v"(a[9])
        : "memory");
}

__device__ __forceinline__ void ring_b128x2_tr16x16(v4i (&r)[2], v4s (&t)[16], const uint32_t (&a)[18]) {
    asm volatile(
        "ds_read_b128 %0, %18\n\t"
        "ds_read_b128 %1, %19\n\t"
        "ds_read_b64_tr_b16 %2, %20\n\t"
        "ds_read_b64_tr_b16 %3, %21\n\t"
        "ds_read_b64_tr_b16 %4, %22\n\t"
        "ds_read_b64_tr_b16 %5, %23\n\t"
        "ds_read_b64_tr_b16 %6, %24\n\t"
        "ds_read_b64_tr_b16 %7, %25\n\t"
        "ds_read_b64_tr_b16 %8, %26\n\t"
        "ds_read_b64_tr_b16 %9, %27\n\t"
        "ds_read_b64_tr_b16 %10, %28\n\t"
        "ds_read_b64_tr_b16 %11, %29\n\t"
        "ds_read_b64_tr_b16 %12, %30\n\t"
        "ds_read_b64_tr_b16 %13, %31\n\t"
        "ds_read_b64_tr_b16 %14, %32\n\t"
        "ds_read_b64_tr_b16 %15, %33\n\t"
        "ds_read_b64_tr_b16 %16, %34\n\t"
        "ds_read_b64_tr_b16 %17, %35\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3]), "=&v"(t[4]), "=&v"(t[5]), "=&v"(t[6]), "=&v"(t[7]), "=&v"(t[8]), "=&v"(t[9]), "=&v"(t[10]), "=&v"(t[11]), "=&v"(t[12]), "=&v"(t[13]), "=&v"(t[14]), "=&v"(t[15])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]), "v"(a[8]), "v"(a[9]), "v"(a[10]), "v"(a[11]), "v"(a[12]), "v"(a[13]), "v"(a[14]), "v"(a[15]), "v"(a[16]), "v"(a[17])
        : "memory");
}

__device__ __forceinline__ void ring_b128x6(v4i (&r)[6], const uint32_t (&a)[6]) {
    asm volatile(
        "ds_read_b128 %0, %6\n\t"
        "ds_read_b128 %1, %7\n\t"
        "ds_read_b128 %2, %8\n\t"
        "ds_read_b128 %3, %9\n\t"
        "ds_read_b128 %4, %10\n\t"
        "ds_read_b128 %5, %11\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5])
        : "memory");
}

__device__ __forceinline__ void ring_b128x10(v4i (&r)[10], const uint32_t (&a)[10]) {
    asm volatile(
        "ds_read_b128 %0, %10\n\t"
        "ds_read_b128 %1, %11\n\t"
        "ds_read_b128 %2, %12\n\t"
        "ds_read_b128 %3, %13\n\t"
        "ds_read_b128 %4, %14\n\t"
        "ds_read_b128 %5, %15\n\t"
        "ds_read_b128 %6, %16\n\t"
        "ds_read_b128 %7, %17\n\t"
        "ds_read_b128 %8, %18\n\t"
        "ds_read_b128 %9, %19\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7]), "=&v"(r[8]), "=&v"(r[9])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]), "v"(a[8]), "v"(a[9])
        : "memory");
}

__device__ __forceinline__ void ring_b128x2_tr8x8(v4i (&r)[2], v2i (&t)[8], const uint32_t (&a)[10]) {
    asm volatile(
        "ds_read_b128 %0, %10\n\t"
        "ds_read_b128 %1, %11\n\t"
        "ds_read_b64_tr_b8 %2, %12\n\t"
        "ds_read_b64_tr_b8 %3, %13\n\t"
        "ds_read_b64_tr_b8 %4, %14\n\t"
        "ds_read_b64_tr_b8 %5, %15\n\t"
        "ds_read_b64_tr_b8 %6, %16\n\t"
        "ds_read_b64_tr_b8 %7, %17\n\t"
        "ds_read_b64_tr_b8 %8, %18\n\t"
        "ds_read_b64_tr_b8 %9, %19\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3]), "=&v"(t[4]), "=&v"(t[5]), "=&v"(t[6]), "=&v"(t[7])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]), "v"(a[8]), "v"(a[9])
        : "memory");
}

__device__ __forceinline__ void ring_b128x2_tr8x16(v4i (&r)[2], v2i (&t)[16], const uint32_t (&a)[18]) {
    asm volatile(
        "ds_read_b128 %0, %18\n\t"
        "ds_read_b128 %1, %19\n\t"
        "ds_read_b64_tr_b8 %2, %20\n\t"
        "ds_read_b64_tr_b8 %3, %21\n\t"
        "ds_read_b64_tr_b8 %4, %22\n\t"
        "ds_read_b64_tr_b8 %5, %23\n\t"
        "ds_read_b64_tr_b8 %6, %24\n\t"
        "ds_read_b64_tr_b8 %7, %25\n\t"
        "ds_read_b64_tr_b8 %8, %26\n\t"
        "ds_read_b64_tr_b8 %9, %27\n\t"
        "ds_read_b64_tr_b8 %10, %28\n\t"
        "ds_read_b64_tr_b8 %11, %29\n\t"
        "ds_read_b64_tr_b8 %12, %30\n\t"
        "ds_read_b64_tr_b8 %13, %31\n\t"
        "ds_read_b64_tr_b8 %14, %32\n\t"
        "ds_read_b64_tr_b8 %15, %33\n\t"
        "ds_read_b64_tr_b8 %16, %34\n\t"
        "ds_read_b64_tr_b8 %17, %35\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3]), "=&v"(t[4]), "=&v"(t[5]), "=&v"(t[6]), "=&v"(t[7]), "=&v"(t[8]), "=&v"(t[9]), "=&v"(t[10]), "=&v"(t[11]), "=&v"(t[12]), "=&v"(t[13]), "=&v"(t[14]), "=&v"(t[15])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]), "v"(a[8]), "v"(a[9]), "v"(a[10]), "v"(a[11]), "v"(a[12]), "v"(a[13]), "v"(a[14]), "v"(a[15]), "v"(a[16]), "v"(a[17])
        : "memory");
}

template <int ES, int CPR>
__device__ __forceinline__ int swz_b(int r) {
    return (ES == 1 ? (((r >> 2) & 1) | ((r >> 4) & 2)) : (2 * ((r >> 1) & 1) + 4 * ((r >> 3) & 1))) & (CPR - 1);
}


// Wait until at most L * n of this wave's loads are outstanding (0 <= n <= N)
// and its LDS operations have completed (the count is an immediate, so one
// branch per possible n).
template <int L, int N>
__device__ __forceinline__ void wait_loads(int n) {
    if constexpr (N == 0) {
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
    } else {
        static_assert(L * N < 64, "vmcnt holds at most 63");
        if (n >= N) __builtin_amdgcn_s_waitcnt(waitcnt_imm(L * N, 0));
        else wait_loads<L, N - 1>(n);
    }
}

template <int ES>
struct Op16;

template <>
struct Op16<1> {  // FP8: 32 codes per lane
    typedef v8i type;
    template <int FA, int FB>
    static __device__ __forceinline__ v4f mma(v8i a, v8i b, v4f c) {
        return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FA, FB, 0, 127, 0, 127);
    }
};

template <>
struct Op16<2> {  // FP16: 8 halves per lane
    typedef v8h type;
    template <int FA, int FB>
    static __device__ __forceinline__ v4f mma(v8h a, v8h b, v4f c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
};

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

template <int ES, int BM, int BN, int OUT, int FA, int FB, bool BT>
__global__ __launch_bounds__(256) void gemm_ring_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ B,
                                                        void* __restrict__ C, int M, int N, int K,
                                                        const float* __restrict__ sA, const float* __restrict__ sB,
                                                        const float* __restrict__ sOut, int tiles_m, int tiles_n,
                                                        int eflags, int vec_out) {
    using T = Ring<ES, BM, BN, BT>;
    using Op = typename Op16<ES>::type;
    // The ring: stage st at ring + st * STAGE. Every read of it is an asm group
    // (device_common.h), so the compiler does not need to tell stages apart.
    __shared__ __attribute__((aligned(1024))) uint8_t ring[T::S * T::STAGE];
    // partial sums of wave groups 1 .. KW-1 (one slot when KW == 1, unused)
    __shared__ v4f red[(T::KW > 1 ? (T::KW - 1) * T::WPK : 1) * 64 * T::TN];
    auto stage = [&](int st) __attribute__((always_inline)) -> LDS_AS uint8_t* {
        return (LDS_AS uint8_t*)ring + st * T::STAGE;
    };

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int tile_m, tile_n;
    tile_coords(blockIdx.x, tiles_m, tiles_n, tile_m, tile_n);
    const int m0 = tile_m * BM, n0 = tile_n * BN;
    const int nk = (K + T::BK - 1) / T::BK, nk_full = K / T::BK;
    // the epilogue's multiplier, loaded now (see epilogue_base_early)
    const bool chan = (eflags & EPI_CHANNEL) != 0;
    const float scale = epilogue_base_early(sA, sB, sOut, OUT == OUT_E4M3, chan);
    const int k0p = nk_full * T::BK;                 // first k of the partial tile (when nk > nk_full)

    // ---- this wave's direct loads: 1 KiB load j = wave + 4 i of every stage ----
    //   j <  A_INST: A rows 8 j + lane / 8, slot lane % 8
    //   j >= A_INST: Bt rows 8 j' + lane / 8 (slot lane % 8), or row-major B
    //                k-rows (1024 / BNB) j' + lane / CPR, slot lane % CPR
    // goff: offset within the K tile; goffp: the same for the partial tile with
    // chunks past K redirected to valid bytes; dead: the chunk lies past K.
    constexpr int NL = T::MAX_PER_WAVE;
    uint32_t goff[NL], goffp[NL];
    bool is_a[NL], dead[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        const int j = wave + 4 * i;
        is_a[i] = j < T::A_INST;
        goff[i] = goffp[i] = 0;
        dead[i] = false;
        if (j >= T::INST) continue;
        if (j < T::A_INST || BT) {
            const int jj = j < T::A_INST ? j : j - T::A_INST;
            const int r = 8 * jj + (lane >> 3);
            const int c = (lane & 7) ^ swz_row(r);
            const int rr = j < T::A_INST ? min(m0 + r, M - 1) - m0 : min(n0 + r, N - 1) - n0;
            goff[i] = (uint32_t)(rr * K * ES + c * 16);
            dead[i] = k0p + c * T::VE >= K;
            goffp[i] = dead[i] ? (uint32_t)(rr * K * ES) : goff[i];
        } else {
            const int r = (1024 / T::BNB) * (j - T::A_INST) + lane / T::CPR;
            const int c = (lane % T::CPR) ^ swz_b<ES, T::CPR>(r);
            const int col = min(n0 + c * T::VE, N - T::VE) - n0;
            goff[i] = (uint32_t)(r * N * ES + col * ES);
            dead[i] = k0p + r >= K;
            goffp[i] = dead[i] ? (uint32_t)((K - 1 - k0p) * N * ES + col * ES) : goff[i];
        }
    }
    const uint8_t* a_src = A + (int64_t)m0 * K * ES;
    const uint8_t* b_src = BT ? B + (int64_t)n0 * K * ES : B + (int64_t)n0 * ES;
    const int64_t b_step = BT ? (int64_t)T::ROWB : (int64_t)T::BK * N * ES;

    auto issue = [&](int kt, int st, bool partial) __attribute__((always_inline)) {
        LDS_AS uint8_t* base = stage(st);
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int j = wave + 4 * i;
            if (j >= T::INST) break;
            const uint32_t off = partial ? goffp[i] : goff[i];
            if (is_a[i])
                __builtin_amdgcn_global_load_lds((const void*)(a_src + (int64_t)kt * T::ROWB + off),
                                                 (LDS_AS void*)(base + j * 1024), 16, 0, 0);
            else  // non-temporal: B is streamed once through the chip
                __builtin_amdgcn_global_load_lds((const void*)(b_src + (int64_t)kt * b_step + off),
                                                 (LDS_AS void*)(base + j * 1024), 16, 0, 2);
        }
    };
    // After the partial tile has landed: zeros over this wave's chunks past K.
    auto zero_dead = [&](int st) __attribute__((always_inline)) {
        LDS_AS uint8_t* base = stage(st);
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int j = wave + 4 * i;
            if (j >= T::INST) break;
            if (dead[i]) *(LDS_AS v4u*)(base + j * 1024 + lane * 16) = v4u{0u, 0u, 0u, 0u};
        }
    };

    // ---- operands ----
    // Wave layout: group kg = wave / WPK; within the group, row block
    // wr = w % WROWS and columns [16 TN wc, 16 TN wc + 16 TN), wc = w / WROWS.
    const int kg = wave / T::WPK, wg = wave % T::WPK;
    const int wr = wg % T::WROWS, wc = wg / T::WROWS;
    const int j16 = lane & 15, g = lane >> 4;
    const int ar = 16 * wr + j16;                    // A row of this lane (within the tile)
    const int asw = swz_row(ar);
    // FP8: chunks 2g, 2g+1 (k = 32 g .. 32 g + 31); FP16 k-step u: chunk 4u + g (k = 32u + 8g .. + 7).
    // Addresses of the 16-byte chunks a lane reads from a 128-byte row.
    auto row_lo = [&](const LDS_AS uint8_t* rowp, int sw, int u) __attribute__((always_inline)) -> uint32_t {
        return lds_addr(rowp + ((ES == 1 ? (2 * g) ^ sw : (4 * u + g) ^ sw) << 4));
    };
    auto row_hi = [&](const LDS_AS uint8_t* rowp, int sw) __attribute__((always_inline)) -> uint32_t {
        return lds_addr(rowp + (((2 * g + 1) ^ sw) << 4));
    };
    auto as_op2 = [](v4i lo, v4i hi) __attribute__((always_inline)) -> Op {
        if constexpr (ES == 1) return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        else return __builtin_bit_cast(v8h, lo);
    };
    // Row-major B, column block tn of this wave (16 columns), k-step u: the
    // LDS addresses of its transpose reads (4 FP8, 2 FP16) and the operand
    // they form.
    auto b_rm_addrs = [&](const LDS_AS uint8_t* sb, int tn, int u, uint32_t (&ad)[4]) __attribute__((always_inline)) {
        const int nb = 16 * (T::TN * wc + tn);           // first column of the block (within the tile)
        if constexpr (ES == 1) {
            // read q: lane j16 addresses k-row 32 g + 8 q + j16 / 2, bytes 8 (j16 % 2) of column chunk nb / 16
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int k = 32 * g + 8 * q + (j16 >> 1);
                const int slot = (nb >> 4) ^ swz_b<1, T::CPR>(k);
                ad[q] = lds_addr(sb + k * T::BNB + slot * 16 + 8 * (j16 & 1));
            }
        } else {
            // read q: lane j16 addresses k-row 32 u + 8 g + 4 q + j16 / 4, columns nb + 4 (j16 % 4) .. + 3
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int k = 32 * u + 8 * g + 4 * q + (j16 >> 2);
                const int cb = (nb + 4 * (j16 & 3)) * 2;   // byte offset of the 4 halves in the k-row
                const int slot = (cb >> 4) ^ swz_b<2, T::CPR>(k);
                ad[q] = lds_addr(sb + k * T::BNB + slot * 16 + (cb & 15));
            }
            ad[2] = ad[3] = 0u;
        }
    };
    auto op_tr8 = [](const v2i (&t)[4]) __attribute__((always_inline)) -> v8i {
        const v4i t01 = __builtin_shufflevector(t[0], t[1], 0, 1, 2, 3);
        const v4i t23 = __builtin_shufflevector(t[2], t[3], 0, 1, 2, 3);
        return __builtin_shufflevector(t01, t23, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    auto op_tr16 = [](const v4s (&t)[2]) __attribute__((always_inline)) -> v8h {
        return __builtin_bit_cast(v8h, __builtin_shufflevector(t[0], t[1], 0, 1, 2, 3, 4, 5, 6, 7));
    };

    v4f acc[T::TN];
#pragma unroll
    for (int tn = 0; tn < T::TN; ++tn) acc[tn] = v4f{0.f, 0.f, 0.f, 0.f};

    // One K tile: per k-step, A's operand and every column block's operand
    // in one LDS read group with one wait (asm groups, see device_common.h),
    // then the column blocks' MFMAs.
    auto compute = [&](int st) __attribute__((always_inline)) {
        const LDS_AS uint8_t* base = stage(st);
        const LDS_AS uint8_t* arow = base + ar * T::ROWB;
#pragma unroll
        for (int u = 0; u < T::KSUB; ++u) {
            Op a, b[T::TN];
            if constexpr (BT && ES == 1) {
                // K-major FP8: A's operand with the first column block, then
                // one group per further block, each followed by its MFMA (two
                // 16-byte reads per block are cheap enough that overlapping
                // them with the previous block's MFMA pays more than one wait:
                // 64x64 tiles measured 17.7 us against 18.3 us merged)
#pragma unroll
                for (int tn = 0; tn < T::TN; ++tn) {
                    const int br = 16 * (T::TN * wc + tn) + j16;
                    const LDS_AS uint8_t* brow = base + T::A_BYTES + br * T::ROWB;
                    const int bsw = swz_row(br);
                    if (tn == 0) {
                        v4i r[4];
                        lds_b128_x4(r, row_lo(arow, asw, u), row_hi(arow, asw), row_lo(brow, bsw, u),
                                    row_hi(brow, bsw));
                        a = as_op2(r[0], r[1]);
                        b[0] = as_op2(r[2], r[3]);
                    } else {
                        v4i r[2];
                        lds_b128_x2(r, row_lo(brow, bsw, u), row_hi(brow, bsw));
                        b[tn] = as_op2(r[0], r[1]);
                    }
                    acc[tn] = Op16<ES>::template mma<FB, FA>(b[tn], a, acc[tn]);
                }
                continue;
            } else if constexpr (BT) {
                // FP16: both k-steps' reads (A's operand, then the column
                // blocks', per k-step) in one group, then both k-steps' MFMAs
                if (u > 0) break;
                uint32_t ad[2 * (1 + T::TN)];
#pragma unroll
                for (int uu = 0; uu < 2; ++uu) {
                    ad[uu * (1 + T::TN)] = row_lo(arow, asw, uu);
#pragma unroll
                    for (int tn = 0; tn < T::TN; ++tn) {
                        const int br = 16 * (T::TN * wc + tn) + j16;
                        ad[uu * (1 + T::TN) + 1 + tn] = row_lo(base + T::A_BYTES + br * T::ROWB, swz_row(br), uu);
                    }
                }
                v4i r[2 * (1 + T::TN)];
                if constexpr (T::TN == 1) lds_b128_x4(r, ad[0], ad[1], ad[2], ad[3]);
                else if constexpr (T::TN == 2) ring_b128x6(r, ad);
                else ring_b128x10(r, ad);
#pragma unroll
                for (int uu = 0; uu < 2; ++uu) {
                    const Op au = as_op2(r[uu * (1 + T::TN)], r[uu * (1 + T::TN)]);
#pragma unroll
                    for (int tn = 0; tn < T::TN; ++tn) {
                        const v4i rb = r[uu * (1 + T::TN) + 1 + tn];
                        acc[tn] = Op16<ES>::template mma<FB, FA>(as_op2(rb, rb), au, acc[tn]);
                    }
                }
                break;
            } else if constexpr (ES == 1) {
                uint32_t ad[2 + 4 * T::TN];
                ad[0] = row_lo(arow, asw, u);
                ad[1] = row_hi(arow, asw);
#pragma unroll
                for (int tn = 0; tn < T::TN; ++tn) {
                    uint32_t q4[4];
                    b_rm_addrs(base + T::A_BYTES, tn, u, q4);
#pragma unroll
                    for (int q = 0; q < 4; ++q) ad[2 + 4 * tn + q] = q4[q];
                }
                v4i r[2];
                v2i t[4 * T::TN];
                if constexpr (T::TN == 1) {
                    v2i t4[4];
                    lds_b128x2_tr8x4(r, t4, ad[0], ad[1], ad[2], ad[3], ad[4], ad[5]);
#pragma unroll
                    for (int q = 0; q < 4; ++q) t[q] = t4[q];
                } else if constexpr (T::TN == 2) {
                    ring_b128x2_tr8x8(r, t, ad);
                } else {
                    ring_b128x2_tr8x16(r, t, ad);
                }
                a = as_op2(r[0], r[1]);
#pragma unroll
                for (int tn = 0; tn < T::TN; ++tn) {
                    const v2i tt[4] = {t[4 * tn], t[4 * tn + 1], t[4 * tn + 2], t[4 * tn + 3]};
                    b[tn] = op_tr8(tt);
                }
            } else {
                // FP16, row-major B: both k-steps in one group, as above
                if (u > 0) break;
                uint32_t ad[2 + 4 * T::TN];
                ad[0] = row_lo(arow, asw, 0);
                ad[1] = row_lo(arow, asw, 1);
#pragma unroll
                for (int uu = 0; uu < 2; ++uu)
#pragma unroll
                    for (int tn = 0; tn < T::TN; ++tn) {
                        uint32_t q4[4];
                        b_rm_addrs(base + T::A_BYTES, tn, uu, q4);
                        ad[2 + 2 * (uu * T::TN + tn)] = q4[0];
                        ad[3 + 2 * (uu * T::TN + tn)] = q4[1];
                    }
                v4i r[2];
                v4s t[4 * T::TN];
                if constexpr (T::TN == 1) ring_b128x2_tr16x4(r, t, ad);
                else if constexpr (T::TN == 2) ring_b128x2_tr16x8(r, t, ad);
                else ring_b128x2_tr16x16(r, t, ad);
#pragma unroll
                for (int uu = 0; uu < 2; ++uu) {
                    const Op au = as_op2(r[uu], r[uu]);
#pragma unroll
                    for (int tn = 0; tn < T::TN; ++tn) {
                        const v4s tt[2] = {t[2 * (uu * T::TN + tn)], t[2 * (uu * T::TN + tn) + 1]};
                        acc[tn] = Op16<ES>::template mma<FB, FA>(op_tr16(tt), au, acc[tn]);
                    }
                }
                break;
            }
#pragma unroll
            for (int tn = 0; tn < T::TN; ++tn) acc[tn] = Op16<ES>::template mma<FB, FA>(b[tn], a, acc[tn]);
        }
    };

    // this wave's loads per stage (MAX_PER_WAVE or one fewer)
    const bool full_share = loads_of<T::INST>(wave) == T::MAX_PER_WAVE;

    // ---- prologue: tiles 0 .. S-2 ----
#pragma unroll
    for (int p = 0; p < T::S - 1; ++p)
        if (p < nk) issue(p, p, p >= nk_full);

    // ---- main loop: unrolled by the ring size so that every stage is a fixed
    // LDS object; step t waits until only tiles t+1 .. min(t+S-2, nk-1) can
    // still be in flight ----
    for (int t0 = 0; t0 < nk; t0 += T::S) {
#pragma unroll
        for (int u = 0; u < T::S; ++u) {
            const int t = t0 + u;
            if (t >= nk) break;
            const int after = min(T::S - 2, nk - 1 - t);
            if (full_share) wait_loads<T::MAX_PER_WAVE, T::S - 2>(after);
            else wait_loads<(T::MAX_PER_WAVE > 1 ? T::MAX_PER_WAVE - 1 : 1), T::S - 2>(after);
            asm volatile("s_barrier" ::: "memory");
            if (t == nk_full) {  // the partial last tile: clear what was fetched past K
                zero_dead(u);
                __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
                asm volatile("s_barrier" ::: "memory");
            }
            const int nt = t + T::S - 1;
            if (nt < nk) issue(nt, (u + T::S - 1) % T::S, nt >= nk_full);
            if (T::KW == 1 || t % T::KW == kg) compute(u);
        }
    }

    // ---- wave groups 1 .. KW-1 hand their partial sums to group 0 ----
    if constexpr (T::KW > 1) {
        if (kg > 0) {
#pragma unroll
            for (int tn = 0; tn < T::TN; ++tn) red[(((kg - 1) * T::WPK + wg) * T::TN + tn) * 64 + lane] = acc[tn];
        }
        __syncthreads();
        if (kg > 0) return;
#pragma unroll
        for (int q = 1; q < T::KW; ++q)
#pragma unroll
            for (int tn = 0; tn < T::TN; ++tn) acc[tn] += red[(((q - 1) * T::WPK + wg) * T::TN + tn) * 64 + lane];
    }

    // ---- epilogue: lane holds row 16 wr + j16 and columns 16 (TN wc + tn) + 4 g + 0..3 ----
    const int row = m0 + 16 * wr + j16;
    const bool interior = vec_out && (m0 + BM <= M) && (n0 + BN <= N);
#pragma unroll
    for (int tn = 0; tn < T::TN; ++tn) {
        const int col = n0 + 16 * (T::TN * wc + tn) + 4 * g;
        v4f y;
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = acc[tn][e] * scale;
        if (interior) {
            if (chan) {
                const float sr = sA[row];
#pragma unroll
                for (int e = 0; e < 4; ++e) y[e] *= sr * sB[col + e];
            }
            const int64_t idx = (int64_t)row * N + col;
            if constexpr (OUT == OUT_F32) {
                *reinterpret_cast<v4f*>(reinterpret_cast<float*>(C) + idx) = y;
            } else if constexpr (OUT == OUT_F16) {
                typedef _Float16 v4hh __attribute__((ext_vector_type(4)));
                const v4hh hv = {(_Float16)y[0], (_Float16)y[1], (_Float16)y[2], (_Float16)y[3]};
                *reinterpret_cast<v4hh*>(reinterpret_cast<_Float16*>(C) + idx) = hv;
            } else {
                *reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(C) + idx) =
                    (eflags & EPI_E5M2) ? e5m2_pack4(y[0], y[1], y[2], y[3]) : e4m3_pack4(y[0], y[1], y[2], y[3]);
            }
        } else if (row < M) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (col + e < N) {
                    float v = y[e];
                    if (chan) v *= sA[row] * sB[col + e];
                    store_elem<OUT>(C, (int64_t)row * N + col + e, v, eflags);
                }
        }
    }
}

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

template <int ES, int BN, bool BT>
inline bool ring_fits(const GemmArgs& a, int bm) {
    const bool aligned = aligned16(a.A) && aligned16(a.B) && (a.K * ES) % 16 == 0 && (BT || (a.N * ES) % 16 == 0);
    const bool fits = (int64_t)bm * a.K * ES < (1ll << 31) &&
                      (BT ? (int64_t)BN * a.K * ES : (int64_t)(128 / ES) * a.N * ES) < (1ll << 31);
    return aligned && fits;
}

// The register-staged 64x64 kernel, for requests the ring kernel cannot take.
inline hipError_t fallback(int kind, const GemmArgs& a) {
    const char* name = a.b_kmajor ? (kind == KIND_FP8 ? "tile_fp8_64x64x128_w2x2_bt" : "tile_f16_64x64x64_w2x2_bt")
                                  : (kind == KIND_FP8 ? "tile_fp8_64x64x128_w2x2" : "tile_f16_64x64x64_w2x2");
    int nt = 0;
    const GemmConfig* tt = tile_configs(&nt);
    for (int i = 0; i < nt; ++i)
        if (std::strcmp(tt[i].name, name) == 0) return tt[i].launch(a);
    return hipErrorInvalidValue;
}

template <int ES, int BM, int BN, int FA, int FB, bool BT>
hipError_t launch_ring(const GemmArgs& a) {
    if (a.splits > 1) return hipErrorInvalidValue;  // no split-K (kgran 0 in the table)
    if (BT != (a.b_kmajor != 0)) return hipErrorInvalidValue;
    const int64_t tiles_m = (a.M + BM - 1) / BM;
    const int64_t tiles_n = (a.N + BN - 1) / BN;
    const int64_t blocks = tiles_m * tiles_n;
    if (blocks <= 0) return hipSuccess;
    if (!ring_fits<ES, BN, BT>(a, BM) || blocks > 0x7FFFFFFF) return fallback(ES == 1 ? KIND_FP8 : KIND_F16, a);
    const uint8_t* A = reinterpret_cast<const uint8_t*>(a.A);
    const uint8_t* B = reinterpret_cast<const uint8_t*>(a.B);
    const int M = (int)a.M, N = (int)a.N, K = (int)a.K;
    const int eflags = (a.out_dtype == OUT_E5M2 ? EPI_E5M2 : 0) | (a.channel ? EPI_CHANNEL : 0);
    const int64_t out_es = a.out_dtype == OUT_F32 ? 4 : (a.out_dtype == OUT_F16 ? 2 : 1);
    const int vec_out = ((uintptr_t)a.C % (4 * out_es)) == 0 && (a.N % 4) == 0;
    const dim3 grid((unsigned)blocks), block(256);
    switch (a.out_dtype) {
        case OUT_F32:
            gemm_ring_kernel<ES, BM, BN, OUT_F32, FA, FB, BT><<<grid, block, 0, a.stream>>>(
                A, B, a.C, M, N, K, a.sA, a.sB, a.sOut, (int)tiles_m, (int)tiles_n, eflags, vec_out);
            break;
        case OUT_F16:
            gemm_ring_kernel<ES, BM, BN, OUT_F16, FA, FB, BT><<<grid, block, 0, a.stream>>>(
                A, B, a.C, M, N, K, a.sA, a.sB, a.sOut, (int)tiles_m, (int)tiles_n, eflags, vec_out);
            break;
        default:
            if constexpr (ES == 1) {
                gemm_ring_kernel<ES, BM, BN, OUT_E4M3, FA, FB, BT><<<grid, block, 0, a.stream>>>(
                    A, B, a.C, M, N, K, a.sA, a.sB, a.sOut, (int)tiles_m, (int)tiles_n, eflags, vec_out);
            } else {
                return hipErrorInvalidValue;
            }
    }
    return hipGetLastError();
}

template <int BM, int BN, bool BT>
hipError_t launch_ring_fp8_any(const GemmArgs& a) {
    switch (a.fmt_a * 2 + a.fmt_b) {
        case 0: return launch_ring<1, BM, BN, 0, 0, BT>(a);
        case 1: return launch_ring<1, BM, BN, 0, 1, BT>(a);
        case 2: return launch_ring<1, BM, BN, 1, 0, BT>(a);
        default: return launch_ring<1, BM, BN, 1, 1, BT>(a);
    }
}

// (BM, BN, B K-major) of every configuration
#define LIBGEMM_RING_CONFIGS(X) \
    X(16, 16, false)            \
    X(16, 32, false)            \
    X(16, 64, false)            \
    X(32, 32, false)            \
    X(32, 64, false)            \
    X(64, 64, false)            \
    X(16, 16, true)             \
    X(16, 32, true)             \
    X(16, 64, true)             \
    X(32, 32, true)             \
    X(32, 64, true)             \
    X(64, 64, true)

}  // namespace ring
}  // namespace libgemm
