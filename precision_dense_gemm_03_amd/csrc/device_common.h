// Device-side helpers shared by the libgemm kernels (gfx950 only).
//
// Number formats follow the FP8 GEMM guide "DeepGEMM实战：FP8矩阵乘法与JIT编译优化指南"
// (sheratonhq.com news 156926): E4M3 = 4 exponent / 3 mantissa bits, largest value
// 448 (§2.1, §3.2), quantization clamps to [-448, 448] (§4.3).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace libgemm {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

#define LDS_AS __attribute__((address_space(3)))

enum OutDtype { OUT_F32 = 0, OUT_F16 = 1, OUT_E4M3 = 2 };

// E4M3 (OCP "FN" variant) code of an FP32 value: round to nearest, ties to the
// even code; |w| >= 448 and +-inf saturate to +-448 (0x7E / 0xFE); NaN -> 0x7F.
// gfx950's v_cvt_pk_fp8_f32 rounds to nearest-even in this format but turns
// out-of-range values into NaN, so the value is clamped first; the NaN test
// comes before the clamp because fmin/fmax would turn NaN into a bound.
__device__ __forceinline__ uint32_t e4m3_pack2(float a, float b) {
    float ca = fminf(fmaxf(a, -448.0f), 448.0f);
    float cb = fminf(fmaxf(b, -448.0f), 448.0f);
    uint32_t pk = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, 0, false) & 0xFFFFu;
    if (a != a) pk = (pk & 0xFF00u) | 0x7Fu;
    if (b != b) pk = (pk & 0x00FFu) | 0x7F00u;
    return pk;
}

__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
    return e4m3_pack2(a, b) | (e4m3_pack2(c, d) << 16);
}

__device__ __forceinline__ uint8_t e4m3_from_f32(float w) { return (uint8_t)(e4m3_pack2(w, 0.0f) & 0xFFu); }

// Per-tensor scale from amax: fl32(amax / 448), and 1 when that is zero.
// Division is IEEE correctly rounded (the library is built without fast-math
// and with correctly rounded FP32 divide).
__device__ __forceinline__ float scale_from_amax(float a) {
    float s = a / 448.0f;
    return (s == 0.0f) ? 1.0f : s;
}

__device__ __forceinline__ uint32_t f32_bits(float x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ float bits_f32(uint32_t u) { return __builtin_bit_cast(float, u); }

// Multiplier applied to the FP32 accumulator in every epilogue: sA*sB, and
// for E4M3 output sA*sB / sOut, so that the result is y = acc * m. Folding
// the output scale into one factor instead of dividing every element by sOut
// changes y by at most a few FP32 ulps, well inside the one-code-step
// tolerance of an E4M3 output.
__device__ __forceinline__ float epilogue_multiplier(const float* sA, const float* sB, const float* sOut,
                                                     bool e4m3_out) {
    const float s = (sA ? *sA : 1.0f) * (sB ? *sB : 1.0f);
    return e4m3_out ? s / *sOut : s;
}

// Stores one output element of the final value y (already multiplied by the
// epilogue multiplier).
__device__ __forceinline__ void store_out(void* C, int64_t idx, float y, int out_dtype) {
    if (out_dtype == OUT_F32) {
        reinterpret_cast<float*>(C)[idx] = y;
    } else if (out_dtype == OUT_F16) {
        reinterpret_cast<_Float16*>(C)[idx] = (_Float16)y;
    } else {
        reinterpret_cast<uint8_t*>(C)[idx] = e4m3_from_f32(y);
    }
}

}  // namespace libgemm
