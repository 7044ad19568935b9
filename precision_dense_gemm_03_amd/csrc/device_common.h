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

enum OutDtype { OUT_F32 = 0, OUT_F16 = 1, OUT_E4M3 = 2, OUT_E5M2 = 3 };

// A compile-time flag passed as a value (for generic lambdas).
template <bool B>
struct BoolC {
    static constexpr bool value = B;
};

// FP8 element formats (operands and quantize): OCP E4M3 ("FN") and OCP E5M2.
enum Fp8Format { FMT_E4M3 = 0, FMT_E5M2 = 1 };

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

// E5M2 code of an FP32 value: round to nearest, ties to the even code;
// |w| >= 57344 and +-inf saturate to +-57344 (0x7B / 0xFB); NaN -> 0x7F. The
// value is clamped before v_cvt_pk_bf8_f32 (which would otherwise round large
// values to inf); the NaN test comes first, as for E4M3.
__device__ __forceinline__ uint32_t e5m2_pack2(float a, float b) {
    float ca = fminf(fmaxf(a, -57344.0f), 57344.0f);
    float cb = fminf(fmaxf(b, -57344.0f), 57344.0f);
    uint32_t pk = (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(ca, cb, 0, false) & 0xFFFFu;
    if (a != a) pk = (pk & 0xFF00u) | 0x7Fu;
    if (b != b) pk = (pk & 0x00FFu) | 0x7F00u;
    return pk;
}

__device__ __forceinline__ uint32_t e5m2_pack4(float a, float b, float c, float d) {
    return e5m2_pack2(a, b) | (e5m2_pack2(c, d) << 16);
}

__device__ __forceinline__ uint8_t e5m2_from_f32(float w) { return (uint8_t)(e5m2_pack2(w, 0.0f) & 0xFFu); }

template <int FMT>
__device__ __forceinline__ uint32_t fp8_pack4(float a, float b, float c, float d) {
    return FMT == FMT_E5M2 ? e5m2_pack4(a, b, c, d) : e4m3_pack4(a, b, c, d);
}

// Largest finite value of an FP8 format (E4M3 448, E5M2 57344).
__device__ __forceinline__ float fp8_max(int fmt) { return fmt == FMT_E5M2 ? 57344.0f : 448.0f; }

// Per-tensor scale from amax: fl32(amax / 448), and 1 when that is zero.
// Division is IEEE correctly rounded (the library is built without fast-math
// and with correctly rounded FP32 divide).
__device__ __forceinline__ float scale_from_amax(float a) {
    float s = a / 448.0f;
    return (s == 0.0f) ? 1.0f : s;
}

// Scale of amax a for an FP8 format. pow2 == 0: fl32(a / fmax), 1 when that is
// 0. pow2 != 0: the smallest power of two s with a / s <= fmax, not below
// 2^-149; 0 -> 1, inf -> inf, NaN -> NaN. With a = ma * 2^ea and fmax =
// mf * 2^ef (mantissas in [0.5, 1)), a / fmax lies in (2^(ea-ef-1), 2^(ea-ef)]
// when ma <= mf and in (2^(ea-ef), 2^(ea-ef+1)) otherwise; both comparisons
// and the exponent arithmetic are exact.
__device__ __forceinline__ float scale_for_format(float a, int fmt, int pow2) {
    const float fmax = fp8_max(fmt);
    if (!pow2) {
        const float s = a / fmax;
        return (s == 0.0f) ? 1.0f : s;
    }
    if (a != a) return a;
    if (a == 0.0f) return 1.0f;
    if (__builtin_isinf(a)) return a;
    int ea, ef;
    const float ma = __builtin_frexpf(a, &ea);
    const float mf = __builtin_frexpf(fmax, &ef);
    int e = ea - ef + (ma > mf ? 1 : 0);
    if (e < -149) e = -149;
    return __builtin_ldexpf(1.0f, e);
}

__device__ __forceinline__ uint32_t f32_bits(float x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ float bits_f32(uint32_t u) { return __builtin_bit_cast(float, u); }

// Multiplier applied to the FP32 accumulator in every epilogue: sA*sB, and
// for FP8 output sA*sB / sOut, so that the result is y = acc * m. Folding
// the output scale into one factor instead of dividing every element by sOut
// changes y by at most a few FP32 ulps, well inside the one-code-step
// tolerance of an FP8 output.
__device__ __forceinline__ float epilogue_multiplier(const float* sA, const float* sB, const float* sOut,
                                                     bool fp8_out) {
    const float s = (sA ? *sA : 1.0f) * (sB ? *sB : 1.0f);
    return fp8_out ? s / *sOut : s;
}

// Epilogue options passed to the kernels as one uniform integer. EPI_PARTIAL:
// the workgroup stores the raw FP32 sum over its K range (no scale, no
// conversion) into its split's [M, N] slice of the workspace; a reduce kernel
// then applies the epilogue to the sum of the slices.
// EPI_A_E5M2 / EPI_B_E5M2: operand formats of the exact-accumulation FP8
// mode, whose kernels widen the codes to FP16 as they stage them.
enum EpilogueFlags { EPI_E5M2 = 1, EPI_CHANNEL = 2, EPI_PARTIAL = 4, EPI_A_E5M2 = 8, EPI_B_E5M2 = 16 };

// Per-tensor multiplier, or with per-channel scales (sA[M], sB[N]) the part
// common to every element: 1 / sOut for an FP8 output, else 1; the element
// (i, j) is then multiplied by sA[i] * sB[j] as it is stored.
__device__ __forceinline__ float epilogue_base(const float* sA, const float* sB, const float* sOut, bool fp8_out,
                                               bool channel) {
    if (channel) return fp8_out ? 1.0f / *sOut : 1.0f;
    return epilogue_multiplier(sA, sB, sOut, fp8_out);
}

// The same, taken at a kernel's start and held in a scalar register: its
// loads then wait under the prologue instead of after the main loop, where
// their two round trips to memory stood between the last MFMA and the
// stores.
__device__ __forceinline__ float epilogue_base_early(const float* sA, const float* sB, const float* sOut,
                                                     bool fp8_out, bool channel) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, epilogue_base(sA, sB, sOut, fp8_out, channel))));
}

// Stores one output element of the final value y (already multiplied by the
// epilogue multiplier).
__device__ __forceinline__ void store_out(void* C, int64_t idx, float y, int out_dtype) {
    if (out_dtype == OUT_F32) {
        reinterpret_cast<float*>(C)[idx] = y;
    } else if (out_dtype == OUT_F16) {
        reinterpret_cast<_Float16*>(C)[idx] = (_Float16)y;
    } else if (out_dtype == OUT_E5M2) {
        reinterpret_cast<uint8_t*>(C)[idx] = e5m2_from_f32(y);
    } else {
        reinterpret_cast<uint8_t*>(C)[idx] = e4m3_from_f32(y);
    }
}

// s_waitcnt immediate (gfx9 encoding): at most `vm` vector-memory and `lgkm`
// LDS operations of this wave outstanding.
constexpr int waitcnt_imm(int vm, int lgkm) { return (vm & 0xF) | ((vm >> 4) << 14) | (7 << 4) | ((lgkm & 0xF) << 8); }

// Exact widening of 8 FP8 codes (two words, code e in byte e % 4 of word e / 4)
// to 8 FP16 values for the exact-accumulation mode. Every E4M3 and E5M2 value
// is an FP16 value: E5M2 codes are the upper byte of the FP16 encoding (inf and
// NaN included), E4M3 codes go through gfx950's FP8 -> FP16 conversion with a
// unit scale (the E4M3 range, 2^-9 .. 448, lies inside FP16's normal range;
// 0x7F / 0xFF stay NaN).
__device__ __forceinline__ v4u widen8_fp8(uint32_t w0, uint32_t w1, bool e5m2) {
    if (e5m2) {
        auto two = [](uint32_t w, int hi) -> uint32_t {
            const uint32_t b = hi ? (w >> 16) : w;
            return ((b & 0xFFu) << 8) | ((b & 0xFF00u) << 16);
        };
        return v4u{two(w0, 0), two(w0, 1), two(w1, 0), two(w1, 1)};
    }
    typedef _Float16 v2hh __attribute__((ext_vector_type(2)));
    const v2hh a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false);
    const v2hh b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true);
    const v2hh c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false);
    const v2hh d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true);
    return v4u{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, c),
               __builtin_bit_cast(uint32_t, d)};
}

// LDS reads issued as a group and waited for inside the same asm block, so
// the results are complete when the block ends. Written in asm for kernels
// that fill LDS with direct global->LDS loads and wait for them explicitly:
// where the compiler cannot tell which LDS object a read touches (always for
// the transpose-read builtins, and at some loop heads for plain loads) it
// waits for every outstanding global->LDS load before the read, which drains
// the prefetch ring. The outputs are early-
// clobber (a result must not land in a register that a later address of the
// group still needs). Arguments are LDS byte addresses.
__device__ __forceinline__ void lds_tr8_x4(v2i (&t)[4], uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3) {
    asm volatile(
        "ds_read_b64_tr_b8 %0, %4\n\t"
        "ds_read_b64_tr_b8 %1, %5\n\t"
        "ds_read_b64_tr_b8 %2, %6\n\t"
        "ds_read_b64_tr_b8 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3])
        : "v"(a0), "v"(a1), "v"(a2), "v"(a3)
        : "memory");
}

__device__ __forceinline__ void lds_tr16_x2(v4s (&t)[2], uint32_t a0, uint32_t a1) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %2\n\t"
        "ds_read_b64_tr_b16 %1, %3\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(t[0]), "=&v"(t[1])
        : "v"(a0), "v"(a1)
        : "memory");
}

// Eight transpose reads with one wait: every operand read of a MEM phase
// waits for the LDS once, not once per group of four.
__device__ __forceinline__ void lds_tr8_x8(v2i (&t)[8], const uint32_t (&a)[8]) {
    asm volatile(
        "ds_read_b64_tr_b8 %0, %8\n\t"
        "ds_read_b64_tr_b8 %1, %9\n\t"
        "ds_read_b64_tr_b8 %2, %10\n\t"
        "ds_read_b64_tr_b8 %3, %11\n\t"
        "ds_read_b64_tr_b8 %4, %12\n\t"
        "ds_read_b64_tr_b8 %5, %13\n\t"
        "ds_read_b64_tr_b8 %6, %14\n\t"
        "ds_read_b64_tr_b8 %7, %15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3]), "=&v"(t[4]), "=&v"(t[5]), "=&v"(t[6]), "=&v"(t[7])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
        : "memory");
}

__device__ __forceinline__ void lds_tr16_x8(v4s (&t)[8], const uint32_t (&a)[8]) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8\n\t"
        "ds_read_b64_tr_b16 %1, %9\n\t"
        "ds_read_b64_tr_b16 %2, %10\n\t"
        "ds_read_b64_tr_b16 %3, %11\n\t"
        "ds_read_b64_tr_b16 %4, %12\n\t"
        "ds_read_b64_tr_b16 %5, %13\n\t"
        "ds_read_b64_tr_b16 %6, %14\n\t"
        "ds_read_b64_tr_b16 %7, %15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3]), "=&v"(t[4]), "=&v"(t[5]), "=&v"(t[6]), "=&v"(t[7])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
        : "memory");
}

// 16-byte LDS reads in one asm block with their wait, for the same reason.
__device__ __forceinline__ void lds_b128_x1(v4i& t, uint32_t a0) {
    asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(t) : "v"(a0) : "memory");
}

__device__ __forceinline__ void lds_b128_x2(v4i (&t)[2], uint32_t a0, uint32_t a1) {
    asm volatile(
        "ds_read_b128 %0, %2\n\t"
        "ds_read_b128 %1, %3\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(t[0]), "=&v"(t[1])
        : "v"(a0), "v"(a1)
        : "memory");
}

__device__ __forceinline__ void lds_b128_x4(v4i (&t)[4], uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3) {
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %5\n\t"
        "ds_read_b128 %2, %6\n\t"
        "ds_read_b128 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3])
        : "v"(a0), "v"(a1), "v"(a2), "v"(a3)
        : "memory");
}

// Mixed groups: two 16-byte reads and four 8-bit transpose reads, or one
// 16-byte read and two 16-bit transpose reads, with one wait.
__device__ __forceinline__ void lds_b128x2_tr8x4(v4i (&a)[2], v2i (&t)[4], uint32_t a0, uint32_t a1, uint32_t t0,
                                                 uint32_t t1, uint32_t t2, uint32_t t3) {
    asm volatile(
        "ds_read_b128 %0, %6\n\t"
        "ds_read_b128 %1, %7\n\t"
        "ds_read_b64_tr_b8 %2, %8\n\t"
        "ds_read_b64_tr_b8 %3, %9\n\t"
        "ds_read_b64_tr_b8 %4, %10\n\t"
        "ds_read_b64_tr_b8 %5, %11\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(a[0]), "=&v"(a[1]), "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3])
        : "v"(a0), "v"(a1), "v"(t0), "v"(t1), "v"(t2), "v"(t3)
        : "memory");
}

__device__ __forceinline__ void lds_b128x1_tr16x2(v4i& a, v4s (&t)[2], uint32_t a0, uint32_t t0, uint32_t t1) {
    asm volatile(
        "ds_read_b128 %0, %3\n\t"
        "ds_read_b64_tr_b16 %1, %4\n\t"
        "ds_read_b64_tr_b16 %2, %5\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(a), "=&v"(t[0]), "=&v"(t[1])
        : "v"(a0), "v"(t0), "v"(t1)
        : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const LDS_AS void* p) { return (uint32_t)(uintptr_t)p; }

// Raw buffer resource over `bytes` bytes from p (clamped to 2^31 - 1): 32-bit
// per-lane and uniform offsets, and loads at or past the end read zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, int64_t bytes) {
    const int n = (int)(bytes < 0 ? 0 : (bytes > 0x7FFFFFFF ? 0x7FFFFFFF : bytes));
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, n, 0x00020000);
}

// 16-byte buffer load of each lane straight into LDS (lane i's bytes land at
// dst + 16 i); voff per lane, soff uniform. (A plain function, so that kernel
// templates never name the builtin with dependent arguments.)
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t rs, LDS_AS void* dst, uint32_t voff,
                                                  uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, voff, soff, 0, 0);
}

}  // namespace libgemm
