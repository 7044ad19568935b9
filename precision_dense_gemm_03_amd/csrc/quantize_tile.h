// The transposed quantize tile, shared by quantize_fp8_transposed and the
// paired quantize that writes B K-major.
#pragma once

#include "device_common.h"

namespace libgemm {

// Quantize with a transposed output (a K-major B from a row-major FP32 B):
// q[c * rows + r] = code(fl32(x[r * cols + c] / s)). A workgroup takes a
// 128-row x 64-column block of x: each thread loads two 4 x 4 sub-blocks (four
// 16-byte row loads each; a wave reads 256-byte row segments), encodes them,
// transposes each 4 x 4 block of codes in registers and writes four 32-bit
// words into an LDS block held transposed (row pitch 132 bytes: the 64 lanes'
// words land in 64 distinct banks); then each thread writes two 16-byte pieces
// of output rows, a wave writing whole 128-byte rows.
constexpr int kQtRows = 128, kQtCols = 64;
// The write-out loop covers all kQtCols x (kQtRows / 16) pieces only when the
// pieces per output row divide the thread count (kQtRows 64, 128 or 256).
constexpr int kQtThreads = 256;
static_assert(kQtRows % 64 == 0 && kQtRows <= 256 && kQtThreads % (kQtRows / 16) == 0,
              "a thread takes kQtRows / 64 row blocks and the write-out covers every piece");
constexpr int kQtPitch = kQtRows + 4;

// One 128 x 64 block (tile) of the transposed quantize, by a workgroup of
// kQtThreads threads; t: kQtCols * kQtPitch bytes of LDS, 16-byte aligned.
template <int FMT>
__device__ __forceinline__ void quantize_transposed_tile(const float* __restrict__ x, int64_t rows, int64_t cols,
                                                         float s, uint8_t* __restrict__ q, int64_t tile,
                                                         int64_t tiles_c, int vec_in, int vec_out,
                                                         LDS_AS uint8_t* t) {
    const int64_t r0 = (tile / tiles_c) * kQtRows, c0 = (tile % tiles_c) * kQtCols;
    const int tc = threadIdx.x % 16, tr = threadIdx.x / 16;  // 4 x 4 block (tr + 16 h, tc)
    const bool interior = r0 + kQtRows <= rows && c0 + kQtCols <= cols;

#pragma unroll
    for (int h = 0; h < kQtRows / 64; ++h) {
        const int rb = tr + 16 * h;  // row block: rows 4 rb .. 4 rb + 3 of the tile
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t r = r0 + 4 * rb + i, c = c0 + 4 * tc;
            v4f v;
            if (interior && vec_in) {
                v = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(x + r * cols + c));
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) v[j] = (r < rows && c + j < cols) ? x[r * cols + c + j] : 0.0f;
            }
            w[i] = fp8_pack4<FMT>(v.x / s, v.y / s, v.z / s, v.w / s);  // byte j = column c + j
        }
        // 4 x 4 byte transpose: word j holds column c + j of the block's 4 rows.
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t o = ((w[0] >> (8 * j)) & 0xFFu) | (((w[1] >> (8 * j)) & 0xFFu) << 8) |
                               (((w[2] >> (8 * j)) & 0xFFu) << 16) | (((w[3] >> (8 * j)) & 0xFFu) << 24);
            *reinterpret_cast<LDS_AS uint32_t*>(&t[(4 * tc + j) * kQtPitch + 4 * rb]) = o;
        }
    }
    __syncthreads();

    constexpr int kSegs = kQtRows / 16;  // 16-code pieces per output row
#pragma unroll
    for (int h = 0; h < kQtRows / 64; ++h) {
        const int oc = threadIdx.x / kSegs + (kQtThreads / kSegs) * h, seg = threadIdx.x % kSegs;  // row c0 + oc
        const int64_t orow = c0 + oc, ocol = r0 + 16 * seg;
        const LDS_AS uint32_t* src = reinterpret_cast<const LDS_AS uint32_t*>(&t[oc * kQtPitch + 16 * seg]);
        if (interior && vec_out) {
            const v4u v = {src[0], src[1], src[2], src[3]};
            __builtin_nontemporal_store(v, reinterpret_cast<v4u*>(q + orow * rows + ocol));
        } else if (orow < cols) {
#pragma unroll
            for (int e = 0; e < 16; ++e)
                if (ocol + e < rows) q[orow * rows + ocol + e] = (uint8_t)(src[e / 4] >> (8 * (e % 4)));
        }
    }
}

}  // namespace libgemm
