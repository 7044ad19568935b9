// Direct-to-LDS MFMA tile GEMM for gfx950: kernel and launcher templates,
// shared by gemm_dma.hip (configuration table, E4M3 x E4M3 and FP16
// instantiations) and gemm_dma_mixed.hip (the other FP8 operand pairs).
// Large-tile MFMA GEMM for gfx950 with direct global->LDS loads.
// C[M,N] = (sA*A[M,K]) (sB*B[K,N]), all row-major, FP32 accumulation
// ("DeepGEMM实战：FP8矩阵乘法与JIT编译优化指南" §2.1 for the scaled FP8 product,
// "HGEMM优化：深度学习中的矩阵乘法性能提升策略" §1.3 for FP16 with FP32 accumulation).
//
// One workgroup computes a 256 x 256 output tile with 4 waves, one per SIMD,
// each owning a 128 x 128 block held in 16 32x32 MFMA accumulators (256
// registers per lane). A wave tile that large halves the LDS reads per MFMA
// relative to a 128 x 64 wave tile, which is what bounds the smaller-wave
// kernels on this chip.
//
// Staging (the "double buffering" of the FP8 guide §2.3, deepened as the HGEMM
// article §3.2 and §3.3 discuss):
//   HBM/L2 --global_load_lds_dwordx4--> LDS ring of STAGES tiles
//   (no staging registers; tile k+STAGES-1 is in flight while tile k is
//   multiplied)
//   LDS --ds_read_b128 (A) / ds_read_b64_tr_b8|b16 (B)--> operand registers,
//   double-buffered: the operands of tile k+1 are read while the MFMAs of
//   tile k run.
// A direct LDS load places lane i's 16 bytes at a fixed 16*i offset, so LDS
// rows cannot be padded; instead each lane fetches the chunk that belongs at
// its slot under an XOR swizzle that spreads the lanes of every LDS read over
// distinct banks (the bank-conflict-free layout of the DeepGEMM deep-dive,
// §3.2, reached by permutation instead of padding). gfx950 serves 16 lanes of
// a 16-byte read, or 32 lanes of an 8-byte (transpose) read, per LDS pass over
// 64 four-byte banks; the swizzles below leave every such pass (and every
// 8- or 16-lane pass over 32 banks) free of conflicts:
//   A row r (64 bytes = 4 chunks): chunk c lives in slot c ^ swz_a(r),
//     swz_a(r) = ((r >> 1) ^ (r >> 3)) & 3, so 16 consecutive rows read at one
//     chunk cover all 16 bank groups;
//   B row k (BN*ES bytes): chunk c lives in slot c ^ swz_b(k); for FP8 the 8
//     rows x 2 chunks of a transpose-read pass, for FP16 its 4 rows x 4
//     chunks, land in 16 different bank groups.

// K-major B (BT, B given as Bt[N,K] row-major, the layout a linear layer keeps
// its weight in): B's tile is 256 rows of 64 bytes exactly like A's, loaded,
// swizzled (swz_a) and read (ds_read_b128) the same way, so no transpose read
// is needed; the LDS bytes read per MFMA stay the same but every read is a
// full-width one.
//
// Edges: rows past M and column chunks past N are loaded from clamped (valid)
// addresses and never stored; a partial last K tile is loaded by guarded
// vector loads with zero fill. Operands that are not 16-byte aligned, or whose
// row blocks exceed 32-bit offsets, go to the register-staged tile kernel.

#pragma once

#include <cstring>

#include "device_common.h"
#include "kernels.h"
#include "tile_order.h"

namespace libgemm {
namespace dma {

template <int ES, int STAGES>
struct Dma {
    static constexpr int BM = 256, BN = 256;
    static constexpr int NT = 256;                   // 4 waves, 2 x 2
    static constexpr int BK = ES == 1 ? 64 : 32;     // k per staged tile: 64 bytes of every A row
    static constexpr int VE = 16 / ES;               // elements per 16-byte chunk
    static constexpr int ROWB = BK * ES;             // A row bytes per tile (64)
    static constexpr int BNB = BN * ES;              // B row bytes per tile
    static constexpr int A_BYTES = BM * ROWB;        // 16 KiB
    static constexpr int B_BYTES = BK * BNB;         // 16 KiB
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int A_BLOCKS = A_BYTES / 1024;  // 1 KiB per wave-wide direct load
    static constexpr int B_BLOCKS = B_BYTES / 1024;
    static constexpr int A_PER_WAVE = A_BLOCKS / 4;
    static constexpr int B_PER_WAVE = B_BLOCKS / 4;
    static constexpr int LOADS_PER_TILE = A_PER_WAVE + B_PER_WAVE;  // per wave
    static constexpr int B_RPB = 1024 / BNB;         // B rows per 1 KiB block
    static constexpr int B_CPR = BNB / 16;           // chunks per B row
    static constexpr int KSUB = ES == 1 ? 1 : 2;     // MFMA k-steps per tile (64 / 16 k each)
    static_assert(STAGES >= 2 && STAGES * STAGE <= 160 * 1024, "LDS ring must fit in 160 KiB");
    static_assert(A_PER_WAVE == 4 && B_PER_WAVE == 4, "dma_tile issues 4 A and 4 B blocks per wave");
};

__device__ __forceinline__ int swz_a(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }

// FP8: k%8 -> {0, 2, 4, 6, 9, 11, 13, 15} (distinct in bits 0-2 and in bits 1-3);
// FP16: k%4 -> {0, 10, 4, 14} (distinct in bits 1-2 and in bits 2-3).
template <int ES>
__device__ __forceinline__ int swz_b(int k) {
    return ES == 1 ? ((2 * (k & 7)) | ((k >> 2) & 1)) : (2 * (k & 3) + 8 * (k & 1));
}

// Operands of the 32x32 MFMAs.
//   FP8:  v_mfma_scale_f32_32x32x64_f8f6f4 (neutral scales): lane l holds 32
//         codes, k = 32*(l/32) + 0..31, of row (A) or column (B) l % 32.
//   FP16: v_mfma_f32_32x32x16_f16: lane l holds 8 halves, k = 8*(l/32) + 0..7.
template <int ES>
struct Mfma32;

template <>
struct Mfma32<1> {
    typedef v8i op;
    // FA, FB: operand formats (0 = E4M3, 1 = E5M2), the instruction's A and B
    // format selectors.
    template <int FA, int FB>
    static __device__ __forceinline__ v16f mma(v8i a, v8i b, v16f c) {
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA, FB, 0, 127, 0, 127);
    }
};

template <>
struct Mfma32<2> {
    typedef v8h op;
    template <int FA, int FB>
    static __device__ __forceinline__ v16f mma(v8h a, v8h b, v16f c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};

// The direct loads of one staged tile: 4 A blocks and 4 B blocks of 1 KiB,
// each lane moving 16 bytes from base + off into LDS at lds + 16 * lane (the
// wave-uniform LDS block address goes through M0). Written as one inline asm
// block so that the compiler does not treat every later LDS read as possibly
// aliasing the in-flight loads and wait for all of them; the kernel orders
// these loads itself with wait_vm_then_barrier. Because the compiler's hazard
// checks cannot see the memory instructions inside the block, the block
// provides the wait states itself: s_nop 4 first (a VALU write of an SGPR,
// such as a v_readlane restoring a spilled base pointer, needs 5 before a
// vector memory instruction reads that SGPR) and s_nop 0 between each M0
// write and the load that reads M0. Nothing else in these kernels keeps a
// value in M0.
__device__ __forceinline__ void dma_tile(const uint8_t* pa, const uint8_t* pb, uint32_t la, uint32_t lb,
                                         const uint32_t (&ao)[4], const uint32_t (&bo)[4]) {
    asm volatile(
        "s_nop 4\n\t"
        "s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %10, %8\n\t"
        "s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %11, %8\n\t"
        "s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %12, %8\n\t"
        "s_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %13, %8\n\t"
        "s_mov_b32 m0, %4\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %14, %9\n\t"
        "s_mov_b32 m0, %5\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %15, %9\n\t"
        "s_mov_b32 m0, %6\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %16, %9\n\t"
        "s_mov_b32 m0, %7\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %17, %9" ::"s"(la),
        "s"(la + 1024), "s"(la + 2048), "s"(la + 3072), "s"(lb), "s"(lb + 1024), "s"(lb + 2048), "s"(lb + 3072),
        "s"(pa), "s"(pb), "v"(ao[0]), "v"(ao[1]), "v"(ao[2]), "v"(ao[3]), "v"(bo[0]), "v"(bo[1]), "v"(bo[2]),
        "v"(bo[3])
        : "memory", "m0");
}

// s_waitcnt with vmcnt(n) and lgkmcnt(0), then the workgroup barrier. The
// memory clobber keeps the compiler from moving LDS accesses across it.
template <int N>
__device__ __forceinline__ void wait_vm_then_barrier() {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_outstanding_tiles(int tiles) {
    // tiles is 0 .. 3; each in-flight tile is N direct loads per wave.
    if (tiles >= 3) wait_vm_then_barrier<3 * N>();
    else if (tiles == 2) wait_vm_then_barrier<2 * N>();
    else if (tiles == 1) wait_vm_then_barrier<N>();
    else wait_vm_then_barrier<0>();
}

// Scheduling pattern for one iteration: 24 LDS operand reads spread between
// the MFMAs (16 of 32x32x64 for FP8, 32 of 32x32x16 for FP16), so the matrix
// core has work queued while the reads are issued.
template <int ES, bool BT>
__device__ __forceinline__ void interleave_reads_with_mfma() {
    constexpr int kMfma = ES == 1 ? 16 : 32;
    constexpr int kReads = BT ? 16 : 24;  // K-major B: 8 A and 8 B ds_read_b128
    constexpr int kPer = (kReads + kMfma - 1) / kMfma;  // reads after each MFMA
#pragma unroll
    for (int i = 0; i < kMfma; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // one MFMA
        if (i * kPer < kReads) __builtin_amdgcn_sched_group_barrier(0x100, kPer, 0);  // then LDS reads
    }
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

template <int ES, int OUT, int STAGES, int FA, int FB, bool BT>
__global__ __launch_bounds__(256) void gemm_dma_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ B,
                                                       void* __restrict__ C, int M, int N, int K,
                                                       const float* __restrict__ sA, const float* __restrict__ sB,
                                                       const float* __restrict__ sOut, int tiles_m, int tiles_n,
                                                       int eflags) {
    using T = Dma<ES, STAGES>;
    using Op = typename Mfma32<ES>::op;
    static_assert(STAGES - 2 <= 3, "wait_outstanding_tiles covers at most three tiles in flight");
    __shared__ __attribute__((aligned(1024))) uint8_t smem_raw[STAGES * T::STAGE];
    LDS_AS uint8_t* smem = (LDS_AS uint8_t*)smem_raw;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const uint32_t lds_base = (uint32_t)(uintptr_t)smem;

    int tile_m, tile_n;
    tile_coords(blockIdx.x, tiles_m, tiles_n, tile_m, tile_n);
    const int m0 = tile_m * T::BM;
    const int n0 = tile_n * T::BN;
    const int nk = (K + T::BK - 1) / T::BK;
    const int nk_full = K / T::BK;

    // ---- direct loads: this lane's global offsets for its A and B slots ----
    // A block q (16 rows) = A_PER_WAVE blocks per wave; lane -> row 16q + lane/4,
    // slot lane%4 holding chunk slot ^ swz_a(row). Rows past M re-read M-1.
    const uint8_t* a_tile = A + (int64_t)m0 * K * ES;
    const uint8_t* b_tile = BT ? B + (int64_t)n0 * K * ES : B + (int64_t)n0 * ES;
    uint32_t a_off[T::A_PER_WAVE], b_off[T::B_PER_WAVE];
#pragma unroll
    for (int i = 0; i < T::A_PER_WAVE; ++i) {
        const int r = 16 * (wave * T::A_PER_WAVE + i) + (lane >> 2);
        const int c = (lane & 3) ^ swz_a(r);
        const int rr = min(m0 + r, M - 1) - m0;
        a_off[i] = (uint32_t)(rr * K * ES + c * 16);
    }
    // B block q = B_RPB rows; lane -> row B_RPB*q + lane/B_CPR, slot lane%B_CPR
    // holding chunk slot ^ swz_b(row). Column chunks past N re-read the last
    // chunk of the row.
#pragma unroll
    for (int i = 0; i < T::B_PER_WAVE; ++i) {
        if constexpr (BT) {  // as A: rows of Bt past N re-read row N-1
            const int r = 16 * (wave * T::B_PER_WAVE + i) + (lane >> 2);
            const int c = (lane & 3) ^ swz_a(r);
            const int rr = min(n0 + r, N - 1) - n0;
            b_off[i] = (uint32_t)(rr * K * ES + c * 16);
        } else {
            const int r = T::B_RPB * (wave * T::B_PER_WAVE + i) + lane / T::B_CPR;
            const int c = (lane % T::B_CPR) ^ swz_b<ES>(r);
            const int col = min(n0 + c * T::VE, N - T::VE) - n0;
            b_off[i] = (uint32_t)(r * N * ES + col * ES);
        }
    }

    auto issue_tile = [&](int kt) __attribute__((always_inline)) {
        LDS_AS uint8_t* st = smem + (kt % STAGES) * T::STAGE;
        if (kt < nk_full) {
            const uint8_t* pa = a_tile + (int64_t)kt * T::ROWB;
            const uint8_t* pb = b_tile + (BT ? (int64_t)kt * T::ROWB : (int64_t)kt * T::BK * N * ES);
            const uint32_t la = lds_base + (kt % STAGES) * T::STAGE + wave * T::A_PER_WAVE * 1024;
            const uint32_t lb = lds_base + (kt % STAGES) * T::STAGE + T::A_BYTES + wave * T::B_PER_WAVE * 1024;
            dma_tile(pa, pb, la, lb, a_off, b_off);
        } else {
            // Partial last tile: the same slots, loaded with guards, zero past K.
            const int k0 = kt * T::BK;
#pragma unroll 1
            for (int i = 0; i < T::A_PER_WAVE; ++i) {
                const int r = 16 * (wave * T::A_PER_WAVE + i) + (lane >> 2);
                const int c = (lane & 3) ^ swz_a(r);
                v4u v = v4u{0u, 0u, 0u, 0u};
                if (k0 + c * T::VE < K) v = *reinterpret_cast<const v4u*>(a_tile + (int64_t)k0 * ES + a_off[i]);
                *(LDS_AS v4u*)(st + (wave * T::A_PER_WAVE + i) * 1024 + lane * 16) = v;
            }
#pragma unroll 1
            for (int i = 0; i < T::B_PER_WAVE; ++i) {
                v4u v = v4u{0u, 0u, 0u, 0u};
                if constexpr (BT) {
                    const int r = 16 * (wave * T::B_PER_WAVE + i) + (lane >> 2);
                    const int c = (lane & 3) ^ swz_a(r);
                    if (k0 + c * T::VE < K) v = *reinterpret_cast<const v4u*>(b_tile + (int64_t)k0 * ES + b_off[i]);
                } else {
                    const int r = T::B_RPB * (wave * T::B_PER_WAVE + i) + lane / T::B_CPR;
                    if (k0 + r < K) v = *reinterpret_cast<const v4u*>(b_tile + (int64_t)k0 * N * ES + b_off[i]);
                }
                *(LDS_AS v4u*)(st + T::A_BYTES + (wave * T::B_PER_WAVE + i) * 1024 + lane * 16) = v;
            }
        }
    };

    // ---- LDS -> operand registers ----
    // A: row r = 128 wm + 32 tm + lane%32; FP8 reads chunks 2h, 2h+1 (h = lane/32),
    // FP16 k-step u reads chunk 2u + h.
    const int ar = wm * 128 + (lane & 31);
    const int a_sw = swz_a(ar);  // swizzle of rows ar + 32 tm (same for every tm)
    const int br = wn * 128 + (lane & 31);  // K-major B: Bt row br + 32 tn
    const int b_sw = swz_a(br);
    const int h = lane >> 5;
    const int j16 = lane & 15, half = (lane >> 4) & 1;
    Op ra0[T::KSUB][4], rb0[T::KSUB][4], ra1[T::KSUB][4], rb1[T::KSUB][4];

    auto read_ops = [&](int kt, Op (&ra)[T::KSUB][4], Op (&rb)[T::KSUB][4]) __attribute__((always_inline)) {
        const LDS_AS uint8_t* st = smem + (kt % STAGES) * T::STAGE;
        const LDS_AS uint8_t* sa = st + ar * T::ROWB;
        const LDS_AS uint8_t* sb = st + T::A_BYTES;
        const LDS_AS uint8_t* sbt = sb + br * T::ROWB;  // K-major B: this lane's row
        if constexpr (ES == 1) {
#pragma unroll
            for (int tm = 0; tm < 4; ++tm) {
                const v4i lo = *(const LDS_AS v4i*)(sa + tm * 32 * T::ROWB + ((2 * h) ^ a_sw) * 16);
                const v4i hi = *(const LDS_AS v4i*)(sa + tm * 32 * T::ROWB + ((2 * h + 1) ^ a_sw) * 16);
                ra[0][tm] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            }
            if constexpr (BT) {  // as A: Bt row 128 wn + 32 tn + lane%32, chunks 2h, 2h+1
#pragma unroll
                for (int tn = 0; tn < 4; ++tn) {
                    const LDS_AS uint8_t* p = sbt + tn * 32 * T::ROWB;
                    const v4i lo = *(const LDS_AS v4i*)(p + ((2 * h) ^ b_sw) * 16);
                    const v4i hi = *(const LDS_AS v4i*)(p + ((2 * h + 1) ^ b_sw) * 16);
                    rb[0][tn] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                }
                return;
            }
            // B: 16-lane group (h, half) covers columns 128 wn + 32 tn + 16 half + 0..15;
            // lane j16 addresses row 32h + 8t + j16/2, bytes 8*(j16%2) of that chunk.
#pragma unroll
            for (int tn = 0; tn < 4; ++tn) {
                const int chunk = (wn * 8 + tn * 2 + half) ^ swz_b<1>(j16 >> 1);  // row % 8 = j16 / 2
                v2i t[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int k = 32 * h + 8 * q + (j16 >> 1);
                    t[q] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                        (LDS_AS v2i*)(sb + k * T::BNB + chunk * 16 + 8 * (j16 & 1)));
                }
                const v4i t01 = __builtin_shufflevector(t[0], t[1], 0, 1, 2, 3);
                const v4i t23 = __builtin_shufflevector(t[2], t[3], 0, 1, 2, 3);
                rb[0][tn] = __builtin_shufflevector(t01, t23, 0, 1, 2, 3, 4, 5, 6, 7);
            }
        } else {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
#pragma unroll
                for (int tm = 0; tm < 4; ++tm)
                    ra[u][tm] = __builtin_bit_cast(
                        v8h, *(const LDS_AS v4u*)(sa + tm * 32 * T::ROWB + ((2 * u + h) ^ a_sw) * 16));
                if constexpr (BT) {
#pragma unroll
                    for (int tn = 0; tn < 4; ++tn)
                        rb[u][tn] = __builtin_bit_cast(
                            v8h, *(const LDS_AS v4u*)(sbt + tn * 32 * T::ROWB + ((2 * u + h) ^ b_sw) * 16));
                    continue;
                }
                // B: lane j16 addresses row 16u + 8h + 4t + j16/4, columns
                // 128 wn + 32 tn + 16 half + 4 (j16%4) .. +3.
#pragma unroll
                for (int tn = 0; tn < 4; ++tn) {
                    const int chunk = (wn * 16 + tn * 4 + half * 2 + ((j16 & 3) >> 1)) ^ swz_b<2>(j16 >> 2);  // row % 4 = j16 / 4
                    v4s t[2];
#pragma unroll
                    for (int q = 0; q < 2; ++q) {
                        const int k = 16 * u + 8 * h + 4 * q + (j16 >> 2);
                        t[q] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (LDS_AS v4s*)(sb + k * T::BNB + chunk * 16 + 8 * (j16 & 1)));
                    }
                    rb[u][tn] = __builtin_bit_cast(v8h, __builtin_shufflevector(t[0], t[1], 0, 1, 2, 3, 4, 5, 6, 7));
                }
            }
        }
    };

    v16f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    auto mma = [&](const Op (&ra)[T::KSUB][4], const Op (&rb)[T::KSUB][4]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < T::KSUB; ++u)
#pragma unroll
            for (int tm = 0; tm < 4; ++tm)
#pragma unroll
                for (int tn = 0; tn < 4; ++tn) acc[tm][tn] = Mfma32<ES>::template mma<FA, FB>(ra[u][tm], rb[u][tn], acc[tm][tn]);
    };

    // ---- main loop ----
    // Tile kt lives in stage kt % STAGES. Entering iteration kt the operands of
    // tile kt are in registers and tiles up to kt+STAGES-2 have been issued.
    // The iteration waits for tile kt+1 (its own direct loads, then the
    // barrier for everyone else's), refills the stage that tile kt-1 used
    // (its reads all finished before the previous barrier), reads the
    // operands of tile kt+1 and multiplies tile kt.
    constexpr int D = STAGES - 1;
    if (nk > 0) {
#pragma unroll
        for (int t = 0; t < D; ++t)
            if (t < nk) issue_tile(t);
        wait_outstanding_tiles<T::LOADS_PER_TILE>(min(D, nk) - 1);
        read_ops(0, ra0, rb0);
        // The operand read of the last iteration (tile nk, never multiplied)
        // is kept unconditional so that both register sets are always
        // written; it reads stale but valid LDS. Within an iteration the
        // operand reads are interleaved with the MFMAs (which use the other
        // register set), the accumulators are then pinned so that no MFMA
        // sinks past the next barrier, and the refill of the freed stage is
        // issued while the last MFMAs drain.
        auto body = [&](int kt, const Op (&ca)[T::KSUB][4], const Op (&cb)[T::KSUB][4], Op (&na)[T::KSUB][4],
                        Op (&nb)[T::KSUB][4]) __attribute__((always_inline)) {
            wait_outstanding_tiles<T::LOADS_PER_TILE>(max(min(kt + D - 1, nk - 1) - (kt + 1), 0));
            read_ops(kt + 1, na, nb);
            mma(ca, cb);
            interleave_reads_with_mfma<ES, BT>();
#pragma unroll
            for (int tm = 0; tm < 4; ++tm)
#pragma unroll
                for (int tn = 0; tn < 4; ++tn) asm volatile("" : "+a"(acc[tm][tn]));
            if (kt + D < nk) issue_tile(kt + D);
        };
        int kt = 0;
        for (; kt + 1 < nk; kt += 2) {
            body(kt, ra0, rb0, ra1, rb1);
            body(kt + 1, ra1, rb1, ra0, rb0);
        }
        if (kt < nk) body(kt, ra0, rb0, ra1, rb1);
    }

    // ---- epilogue: y = acc * (sA*sB), converted; rows/columns past M/N are not stored ----
    // 32x32 accumulator element r of lane l: row 8*(r/4) + 4*(l/32) + r%4, column l%32.
    // Per-tensor: y = acc * sA*sB (/ sOut). Per-channel (EPI_CHANNEL, sA[M] and
    // sB[N]): y = acc * (1/sOut) * sA[row] * sB[col], loaded only for stored
    // elements.
    const bool chan = (eflags & EPI_CHANNEL) != 0;
    const float scale = epilogue_base(sA, sB, sOut, OUT == OUT_E4M3, chan);
    const int row0 = m0 + wm * 128 + 4 * h;
    const int col0 = n0 + wn * 128 + (lane & 31);
    const bool interior = (m0 + T::BM <= M) && (n0 + T::BN <= N);
#pragma unroll
    for (int tm = 0; tm < 4; ++tm)
#pragma unroll
        for (int tn = 0; tn < 4; ++tn)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = row0 + tm * 32 + 8 * (r >> 2) + (r & 3);
                const int col = col0 + tn * 32;
                if (interior || (row < M && col < N)) {
                    float y = acc[tm][tn][r] * scale;
                    if (chan) y *= sA[row] * sB[col];
                    store_one<OUT>(C, (int64_t)row * N + col, y, eflags);
                }
            }
}

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Falls back to the register-staged 256x256 kernel when the direct-load
// kernel's preconditions (16-byte aligned rows, 32-bit tile offsets) fail.
inline hipError_t fallback(int kind, const GemmArgs& a) {
    const char* name = a.b_kmajor ? (kind == KIND_FP8 ? "tile_fp8_256x256x128_w2x4_bt" : "tile_f16_256x256x64_w2x4_bt")
                                  : (kind == KIND_FP8 ? "tile_fp8_256x256x128_w2x4" : "tile_f16_256x256x64_w2x4");
    int nt = 0;
    const GemmConfig* tt = tile_configs(&nt);
    for (int i = 0; i < nt; ++i)
        if (std::strcmp(tt[i].name, name) == 0) return tt[i].launch(a);
    return hipErrorInvalidValue;
}

template <int ES, int STAGES, int FA, int FB, bool BT = false>
hipError_t launch_dma(const GemmArgs& a) {
    using T = Dma<ES, STAGES>;
    if (a.splits > 1) return hipErrorInvalidValue;   // no split-K here (kgran 0 in the table)
    if (BT != (a.b_kmajor != 0)) return hipErrorInvalidValue;
    const int64_t tiles_m = (a.M + T::BM - 1) / T::BM;
    const int64_t tiles_n = (a.N + T::BN - 1) / T::BN;
    const int64_t blocks = tiles_m * tiles_n;
    if (blocks <= 0) return hipSuccess;
    const bool aligned = aligned16(a.A) && aligned16(a.B) && (a.K * ES) % 16 == 0 && (BT || (a.N * ES) % 16 == 0);
    const bool fits = (int64_t)T::BM * a.K * ES < (1ll << 31) &&
                      (BT ? (int64_t)T::BN * a.K * ES : (int64_t)T::BK * a.N * ES) < (1ll << 31) &&
                      blocks <= 0x7FFFFFFF;
    if (!aligned || !fits) return fallback(ES == 1 ? KIND_FP8 : KIND_F16, a);
    const uint8_t* A = reinterpret_cast<const uint8_t*>(a.A);
    const uint8_t* B = reinterpret_cast<const uint8_t*>(a.B);
    const int M = (int)a.M, N = (int)a.N, K = (int)a.K;
    const dim3 grid((unsigned)blocks), block(T::NT);
    const int eflags = (a.out_dtype == OUT_E5M2 ? EPI_E5M2 : 0) | (a.channel ? EPI_CHANNEL : 0);
    switch (a.out_dtype) {
        case OUT_F32:
            gemm_dma_kernel<ES, OUT_F32, STAGES, FA, FB, BT><<<grid, block, 0, a.stream>>>(
                A, B, a.C, M, N, K, a.sA, a.sB, a.sOut, (int)tiles_m, (int)tiles_n, eflags);
            break;
        case OUT_F16:
            gemm_dma_kernel<ES, OUT_F16, STAGES, FA, FB, BT><<<grid, block, 0, a.stream>>>(
                A, B, a.C, M, N, K, a.sA, a.sB, a.sOut, (int)tiles_m, (int)tiles_n, eflags);
            break;
        default:
            if constexpr (ES == 1) {
                gemm_dma_kernel<ES, OUT_E4M3, STAGES, FA, FB, BT><<<grid, block, 0, a.stream>>>(
                    A, B, a.C, M, N, K, a.sA, a.sB, a.sOut, (int)tiles_m, (int)tiles_n,
                    eflags);
            } else {
                return hipErrorInvalidValue;
            }
    }
    return hipGetLastError();
}

// Operand-format dispatch; the pairs other than E4M3 x E4M3 are instantiated
// in gemm_dma_mixed.hip.
template <int STAGES>
hipError_t launch_dma_fp8_any(const GemmArgs& a) {
    switch (a.fmt_a * 2 + a.fmt_b) {
        case 0: return launch_dma<1, STAGES, 0, 0>(a);
        case 1: return launch_dma<1, STAGES, 0, 1>(a);
        case 2: return launch_dma<1, STAGES, 1, 0>(a);
        default: return launch_dma<1, STAGES, 1, 1>(a);
    }
}

}  // namespace dma
}  // namespace libgemm
