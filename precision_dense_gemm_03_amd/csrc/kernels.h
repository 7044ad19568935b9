// Internal interface between the C-ABI layer, the shape selector and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace libgemm {

enum OperandKind { KIND_F16 = 0, KIND_FP8 = 1 };

// Arguments every GEMM launcher receives (validated by the C-ABI layer).
struct GemmArgs {
    const void* A;
    const void* B;
    void* C;
    const float* sA;   // device scalars (per-channel: sA[M], sB[N]); NULL for FP16
    const float* sB;
    const float* sOut; // device scalar; only read for FP8 outputs
    int out_dtype;
    int64_t M, N, K;
    hipStream_t stream;
    int fmt_a = 0;     // FP8 operand formats (Fp8Format: 0 = E4M3, 1 = E5M2); 0 for FP16
    int fmt_b = 0;
    int channel = 0;   // 1: sA holds M per-row scales and sB N per-column scales
    // Split-K: with splits > 1 the launch covers K in ranges of k_chunk and
    // writes FP32 partial sums to ws[split][M][N] instead of C; the reduce
    // launch (launch_splitk_reduce) then writes C.
    float* ws = nullptr;
    int splits = 1;
    int64_t k_chunk = 0;
    // 1: B is stored K-major, as Bt[N,K] row-major (element (k, n) at n*K + k)
    int b_kmajor = 0;
};

typedef hipError_t (*GemmLauncher)(const GemmArgs&);

// One entry of the compiled-in configuration table.
struct GemmConfig {
    const char* name;   // e.g. "tile_fp8_256x256x128_w2x2"
    int kind;           // OperandKind
    int family;         // 0 = MFMA tile kernel, 1 = M<=16 streaming kernel, 2 = direct-load tile kernel,
                        // 3 = K-major decode kernel, 4 = ping-pong tile kernel,
                        // 5 = exact-accumulation FP8 tile kernel, 6 = deep-ring skinny kernel
    int bm, bn, bk;     // tile (stream: bm = max M, bn = columns per block, bk = k-slices)
    GemmLauncher launch;
    int fmt_mask = 0;   // FP8 operand pairs served: bit (2*fmt_a + fmt_b); 0 means E4M3 x E4M3 only
    int kgran = 0;      // split-K: K ranges are multiples of kgran; 0 = this config does not split
    int b_kmajor = 0;   // B layout served: 0 row-major B[K,N], 1 K-major Bt[N,K]
};

constexpr int kAllFp8Pairs = 15;

// Whether configuration c serves FP8 operand formats (fa, fb).
inline bool serves_formats(const GemmConfig& c, int fa, int fb) {
    const int mask = c.fmt_mask ? c.fmt_mask : 1;
    return (mask >> (2 * fa + fb)) & 1;
}

// Configuration tables, defined next to their kernels.
const GemmConfig* tile_configs(int* count);
const GemmConfig* stream_configs(int* count);
const GemmConfig* dma_configs(int* count);
const GemmConfig* gemv_kmajor_configs(int* count);
const GemmConfig* pp_configs(int* count);
const GemmConfig* exact_configs(int* count);
// exact-accumulation ping-pong launchers (gemm_pp_exact.hip), row-major / K-major B
hipError_t launch_pp_exact_rm(const GemmArgs& a);
hipError_t launch_pp_exact_bt(const GemmArgs& a);
const GemmConfig* ring_configs(int* count);

// Shape (and FP8 operand formats) -> configuration (host only, no HIP calls).
// Returns NULL if none fits.
const GemmConfig* select_config(int kind, int out_dtype, int64_t M, int64_t N, int64_t K, int fmt_a = 0,
                                int fmt_b = 0, int b_kmajor = 0);

// Split-K plan for the workspace entry points: the configuration, the number
// of K ranges and their length (splits == 1: no split, the plain launch).
struct SplitPlan {
    const GemmConfig* cfg;
    int splits;
    int64_t k_chunk;
};
// The exact-accumulation FP8 mode: the FP32-FMA streaming (row-major B,
// M <= 4) and decode (K-major B, M <= 8) kernels, whose products are exact and
// whose sums are FP32 additions, else the widening tile kernels by the tile
// rules. NULL if none fits.
const GemmConfig* select_config_exact(int out_dtype, int64_t M, int64_t N, int64_t K, int fmt_a, int fmt_b,
                                      int b_kmajor);

SplitPlan plan_splitk(int kind, int out_dtype, int64_t M, int64_t N, int64_t K, int fmt_a = 0, int fmt_b = 0,
                      int b_kmajor = 0);

// C = epilogue(sum over a.splits slices of a.ws), in slice order.
hipError_t launch_splitk_reduce(const GemmArgs& a);

// amax / quantize launchers.
// amax and (scale != NULL) the scale for FP8 format fmt, pow2 != 0 for a
// power-of-two scale.
hipError_t launch_amax(const float* x, int64_t n, float* amax, float* scale, int fmt, int pow2, hipStream_t stream);
hipError_t launch_quantize(const float* x, int64_t n, const float* scale, uint8_t* q, int fmt, hipStream_t stream);
// amax, scale and quantize of two tensors in two launches (A, and B when
// nb > 0): amax[0..1], scale[0..1], qa, qb. slots: kPairSlots words of device
// scratch for the per-block maxima.
constexpr int kPairSlots = 1024;
hipError_t launch_amax_quantize_pair(const float* xa, int64_t na, const float* xb, int64_t nb, int fmt, int pow2,
                                     float* amax, float* scale, uint8_t* qa, uint8_t* qb, uint32_t* slots,
                                     hipStream_t stream);
// The same with B = xb[K, N] row-major and its codes written K-major, qbt[N, K].
hipError_t launch_amax_quantize_pair_bt(const float* xa, int64_t na, const float* xb, int64_t K, int64_t N, int fmt,
                                        int pow2, float* amax, float* scale, uint8_t* qa, uint8_t* qbt,
                                        uint32_t* slots, hipStream_t stream);
// Quantize with a transposed output: q[c * rows + r] = code(x[r * cols + c] / scale).
hipError_t launch_quantize_transposed(const float* x, int64_t rows, int64_t cols, const float* scale, uint8_t* q,
                                      int fmt, hipStream_t stream);
// Per-channel amax / scale / quantize over a row-major x[rows, cols]: axis 0
// one channel per row, axis 1 one per column. For axis 1, amax doubles as the
// running maximum while the launches run.
hipError_t launch_amax_channel(const float* x, int64_t rows, int64_t cols, int axis, float* amax, float* scale,
                               int fmt, int pow2, hipStream_t stream);
hipError_t launch_quantize_channel(const float* x, int64_t rows, int64_t cols, int axis, const float* scale,
                                   uint8_t* q, int fmt, hipStream_t stream);
// FP16 dynamic-range guard: scalars[0..2] = s, sqrt(s), 1/s from the two
// maxima (scale_out, if not NULL, receives s); y = FP16(fl32(x * sqrt(s))).
hipError_t launch_guard_scale(const float* amax_a, const float* amax_b, float* scalars, float* scale_out,
                              hipStream_t stream);
hipError_t launch_guard_to_f16(const float* x, int64_t n, const float* scalars, _Float16* y, hipStream_t stream);
// dst[c * rows + r] = src[r * cols + c] for 1- or 2-byte elements.
hipError_t launch_transpose(const void* src, int64_t rows, int64_t cols, int elem_bytes, void* dst,
                            hipStream_t stream);
// Writes zeros to an [M,N] output of the given dtype (the K = 0 empty sum).
hipError_t launch_fill_zero(void* C, int64_t count, int out_dtype, hipStream_t stream);

}  // namespace libgemm
