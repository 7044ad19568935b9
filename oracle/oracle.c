/*
 * Reference oracle for the FP8 (E4M3) per-tensor-scaled GEMM and the FP16 GEMM.
 *
 * TEST INFRASTRUCTURE ONLY. Plain, slow, obviously correct host C in double
 * precision. Only the test suite, the package smoke check and the CPU-baseline
 * leg of the benchmark may load this library; the product path never does.
 * It shares no code, header, table or constant generator with the HIP library.
 *
 * Sources (the pages this follows; "P1/P2/P3" below):
 *   P1  DeepGEMM deep-dive article (hnwysp.cn, news 84236), sections 3.3 and 4.1
 *   P2  "DeepGEMM实战：FP8矩阵乘法与JIT编译优化指南" (sheratonhq.com, news 156926)
 *   P3  "HGEMM优化：深度学习中的矩阵乘法性能提升策略" (jsqmd.com, news 710660)
 *
 * What is computed, and where it is stated:
 *   - E4M3 is the 8-bit format with 4 exponent and 3 mantissa bits whose largest
 *     finite value is 448 (P2 §2.1, §3.2). That maximum identifies the OCP
 *     "E4M3FN" variant: bias 7, subnormals, no infinities, S.1111.111 is NaN.
 *   - Inputs are FP8, products accumulate in a wide accumulator, never in FP8
 *     (P2 §2.1). The oracle accumulates in double: every E4M3 x E4M3 product is
 *     exact in double, and so is every partial sum while K <= 171196 (all E4M3
 *     values are multiples of 2^-9 below 2^9), so for FP8 operands the result
 *     is the exact sum in any order.
 *   - Per-tensor scale = max|x| / 448 (P2 §3.2); quantize q = clamp(round(x/s),
 *     -448, 448) (P2 §4.3), read as: divide in FP32 (correctly rounded), round
 *     to the nearest E4M3 value, ties to the even code, saturate at +-448.
 *   - The accumulator is multiplied by sA*sB at write-back and, for an FP8
 *     output, divided by the output scale (P2 §3.2); FP8 output needs its own
 *     output scale (P2 §4.3).
 *   - FP16 GEMM with a 32-bit (here: wider) accumulator (P3 §1.3).
 *   - E5M2 is the other FP8 format: 5 exponent and 2 mantissa bits, wider
 *     range, less precision (P2 §2.1); its quantization clamps at 57344
 *     (P2 §4.3). That maximum identifies the OCP E5M2 variant (IEEE-like:
 *     bias 15, subnormals, S.11111.00 = inf, S.11111.mm (mm != 0) = NaN).
 *   - A scale may be a power of two just above the calibrated maximum, so
 *     that scaling is exponent arithmetic (P2 §2.1). Read as: the smallest
 *     2^e with max|x| / 2^e <= the format's largest value.
 *   - FP16 dynamic-range guard (P1, mixed-precision section): with max|A|
 *     and max|B| taken on the GPU before the GEMM, s = min(1, 65504 /
 *     (max|A| max|B|)); A and B are multiplied by sqrt(s) before they enter
 *     the FP16 GEMM and the result is divided by s, so that no product of
 *     the scaled FP16 operands exceeds the FP16 range.
 *   - Per-channel scaling is the named alternative to per-tensor scales
 *     (P2 §2.1, §3.2): one scale per row of A and per column of B, the
 *     per-tensor rule applied to each channel; the write-back multiplies the
 *     accumulator by sA[i] * sB[j].
 *
 * Readings where the pages are silent (each is listed with its reason in the
 * design notes): a NaN always encodes to the canonical code 0x7F (both
 * formats); +-inf and anything of magnitude >= 448 (E4M3) or >= 57344 (E5M2)
 * saturate to the largest finite value; amax == 0 (or a scale that
 * underflows to 0) gives scale 1; NaN propagates through amax; signed zeros
 * keep their sign; FP16 output overflows to +-inf as IEEE rounding does.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_API __attribute__((visibility("default")))

/* ---------------------------------------------------------------- E4M3 --- */

/* Decode one E4M3 code: s eeee mmm, bias 7. e == 0: m * 2^-9 (subnormal);
 * otherwise (1 + m/8) * 2^(e-7); e == 15 with m == 7 is NaN (no infinity). */
ORC_API double orc_e4m3_decode(uint8_t code) {
    int s = (code >> 7) & 1;
    int e = (code >> 3) & 15;
    int m = code & 7;
    double mag;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        mag = ldexp((double)m, -9);
    else
        mag = ldexp(8.0 + (double)m, e - 10); /* (1 + m/8) * 2^(e-7) */
    return s ? -mag : mag;
}

/* Non-negative E4M3 magnitudes in code order 0x00..0x7E (strictly increasing),
 * tabulated once from the decoder when the library is loaded. */
static double e4m3_mag_table[127];

__attribute__((constructor)) static void e4m3_mag_init(void) {
    for (int c = 0; c < 127; ++c) e4m3_mag_table[c] = orc_e4m3_decode((uint8_t)c);
}

static double e4m3_mag(int c) { return e4m3_mag_table[c]; }

/* Encode a real value to E4M3: nearest representable magnitude, ties to the
 * code with even last bit (round-to-nearest-even), saturate at 448, NaN -> 0x7F.
 * Plain bisection over the 127 sorted magnitudes, then a comparison with the
 * exact midpoint of the bracketing pair. */
ORC_API uint8_t orc_e4m3_encode(double v) {
    uint8_t sign;
    double a, mid;
    int lo, hi;
    if (isnan(v)) return 0x7F;
    sign = signbit(v) ? 0x80 : 0x00;
    a = fabs(v);
    if (a >= 448.0) return (uint8_t)(sign | 0x7E);
    /* largest lo with mag(lo) <= a; mag(0) = 0 <= a always */
    lo = 0;
    hi = 126;
    while (hi - lo > 1) {
        int m = (lo + hi) / 2;
        if (e4m3_mag(m) <= a) lo = m; else hi = m;
    }
    /* now hi == lo + 1 and mag(lo) <= a < mag(hi) */
    if (e4m3_mag(lo) == a) return (uint8_t)(sign | lo);
    mid = 0.5 * (e4m3_mag(lo) + e4m3_mag(hi)); /* exact: dyadic with one more bit */
    if (a < mid) return (uint8_t)(sign | lo);
    if (a > mid) return (uint8_t)(sign | hi);
    return (uint8_t)(sign | ((lo & 1) == 0 ? lo : hi));
}

ORC_API void orc_e4m3_decode_n(const uint8_t* c, int64_t n, double* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_decode(c[i]);
}

ORC_API void orc_e4m3_encode_n(const double* v, int64_t n, uint8_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_encode(v[i]);
}

/* Encode every FP32 value given as raw bits (used for exhaustive checks). */
ORC_API void orc_e4m3_encode_f32bits(const uint32_t* bits, int64_t n, uint8_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        float f;
        memcpy(&f, &bits[i], 4);
        out[i] = orc_e4m3_encode((double)f);
    }
}

/* ---------------------------------------------------------------- E5M2 --- */

/* Decode one E5M2 code: s eeeee mm, bias 15. e == 0: m * 2^-16 (subnormal);
 * 1 <= e <= 30: (1 + m/4) * 2^(e-15); e == 31: inf (m == 0) or NaN. */
ORC_API double orc_e5m2_decode(uint8_t code) {
    int s = (code >> 7) & 1;
    int e = (code >> 2) & 31;
    int m = code & 3;
    double mag;
    if (e == 31) mag = (m == 0) ? INFINITY : NAN;
    else if (e == 0) mag = ldexp((double)m, -16);
    else mag = ldexp(4.0 + (double)m, e - 17); /* (1 + m/4) * 2^(e-15) */
    return s ? -mag : mag;
}

/* Finite non-negative E5M2 magnitudes, codes 0x00..0x7B (0x7B = 57344). */
static double e5m2_mag_table[124];

__attribute__((constructor)) static void e5m2_mag_init(void) {
    for (int c = 0; c < 124; ++c) e5m2_mag_table[c] = orc_e5m2_decode((uint8_t)c);
}

/* Encode a real value to E5M2: nearest finite magnitude, ties to the code with
 * even last bit, saturate at 57344 (inf included), NaN -> 0x7F. Bisection over
 * the 124 sorted magnitudes and the exact midpoint, as for E4M3. */
ORC_API uint8_t orc_e5m2_encode(double v) {
    uint8_t sign;
    double a, mid;
    int lo, hi;
    if (isnan(v)) return 0x7F;
    sign = signbit(v) ? 0x80 : 0x00;
    a = fabs(v);
    if (a >= 57344.0) return (uint8_t)(sign | 0x7B);
    lo = 0;
    hi = 123;
    while (hi - lo > 1) {
        int m = (lo + hi) / 2;
        if (e5m2_mag_table[m] <= a) lo = m; else hi = m;
    }
    if (e5m2_mag_table[lo] == a) return (uint8_t)(sign | lo);
    mid = 0.5 * (e5m2_mag_table[lo] + e5m2_mag_table[hi]);
    if (a < mid) return (uint8_t)(sign | lo);
    if (a > mid) return (uint8_t)(sign | hi);
    return (uint8_t)(sign | ((lo & 1) == 0 ? lo : hi));
}

ORC_API void orc_e5m2_decode_n(const uint8_t* c, int64_t n, double* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e5m2_decode(c[i]);
}

ORC_API void orc_e5m2_encode_n(const double* v, int64_t n, uint8_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e5m2_encode(v[i]);
}

ORC_API void orc_e5m2_encode_f32bits(const uint32_t* bits, int64_t n, uint8_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        float f;
        memcpy(&f, &bits[i], 4);
        out[i] = orc_e5m2_encode((double)f);
    }
}

/* FP8 formats by number: 0 = E4M3, 2 = E5M2 (1 is FP16 in the GEMM below). */
enum { ORC_FMT_E4M3 = 0, ORC_FMT_F16 = 1, ORC_FMT_E5M2 = 2 };

static double fp8_decode(int fmt, uint8_t c) { return fmt == ORC_FMT_E5M2 ? orc_e5m2_decode(c) : orc_e4m3_decode(c); }
static uint8_t fp8_encode(int fmt, double v) { return fmt == ORC_FMT_E5M2 ? orc_e5m2_encode(v) : orc_e4m3_encode(v); }
static double fp8_max(int fmt) { return fmt == ORC_FMT_E5M2 ? 57344.0 : 448.0; }

/* ---------------------------------------------------------------- FP16 --- */

/* Decode IEEE binary16: s eeeee mmmmmmmmmm, bias 15. */
ORC_API double orc_f16_decode(uint16_t h) {
    int s = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int m = h & 1023;
    double mag;
    if (e == 31) mag = (m == 0) ? INFINITY : NAN;
    else if (e == 0) mag = ldexp((double)m, -24);
    else mag = ldexp(1024.0 + (double)m, e - 25);
    return s ? -mag : mag;
}

/* Round a double to binary16, round-to-nearest-even, overflow to +-inf,
 * NaN -> 0x7E00. The value is scaled by the ulp of its binade (an exact power
 * of two), rounded to an integer with rint (nearest-even in the default mode),
 * and the bits are rebuilt; a carry into the next binade falls out naturally. */
ORC_API uint16_t orc_f16_round(double v) {
    uint16_t sign;
    double a, r;
    int E;
    if (isnan(v)) return 0x7E00;
    sign = signbit(v) ? 0x8000 : 0;
    a = fabs(v);
    if (a >= 65520.0) return (uint16_t)(sign | 0x7C00); /* >= max + ulp/2 (tie goes up: 65504 is odd) */
    if (a < ldexp(1.0, -14)) {
        r = rint(ldexp(a, 24)); /* subnormal grid 2^-24; r <= 1024 (1024 = min normal) */
        return (uint16_t)(sign | (uint16_t)r);
    }
    frexp(a, &E); /* a = f * 2^E, f in [0.5, 1): binade exponent is E-1 */
    r = rint(ldexp(a, 10 - (E - 1))); /* in [1024, 2048] */
    return (uint16_t)(sign | (uint16_t)(((E - 1 + 15) << 10) + ((int)r - 1024)));
}

ORC_API void orc_f16_decode_n(const uint16_t* h, int64_t n, double* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_f16_decode(h[i]);
}

ORC_API void orc_f16_round_n(const double* v, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = orc_f16_round(v[i]);
}

/* -------------------------------------------------- amax, scale, quantize --- */

/* max_i |x_i| over FP32 values, exact; any NaN makes the result NaN. */
ORC_API float orc_amax(const float* x, int64_t n) {
    float m = 0.0f;
    int saw_nan = 0;
    for (int64_t i = 0; i < n; ++i) {
        float a = fabsf(x[i]);
        if (isnan(a)) saw_nan = 1;
        else if (a > m) m = a;
    }
    return saw_nan ? NAN : m;
}

/* Per-tensor scale max|x| / 448 (P2 §3.2), an IEEE FP32 quotient: the double
 * quotient rounded to float is the correctly rounded FP32 quotient (double
 * rounding is innocuous for division since 53 >= 2*24 + 2). A zero amax, or a
 * quotient that underflows to zero, gives 1 so the later division is defined. */
ORC_API float orc_scale_from_amax(float a) {
    float s = (float)((double)a / 448.0);
    if (s == 0.0f) return 1.0f;
    return s;
}

/* Scale for format fmt from amax a. pow2 == 0: fl32(a / fmax), 1 when that
 * is 0 (P2 §3.2). pow2 != 0: the smallest power of two s with a / s <= fmax
 * (P2 §2.1), found by exact doubling/halving in double, not below 2^-149 (the
 * smallest FP32 power of two); a == 0 gives 1, inf gives inf, NaN gives NaN. */
ORC_API float orc_scale(float a, int fmt, int pow2) {
    const double fmax = fp8_max(fmt);
    double s;
    if (!pow2) {
        float q = (float)((double)a / fmax);
        return q == 0.0f ? 1.0f : q;
    }
    if (isnan(a)) return NAN;
    if (isinf(a)) return INFINITY;
    if (a == 0.0f) return 1.0f;
    s = 1.0;
    while ((double)a / s > fmax) s *= 2.0;          /* exact: powers of two */
    while (s > ldexp(1.0, -149) && (double)a / (s * 0.5) <= fmax) s *= 0.5;
    return (float)s;
}

/* q_i = FP8_fmt(fl32(x_i / s)) (P2 §4.3) for either format. */
ORC_API void orc_quantize_fmt(const float* x, int64_t n, float s, int fmt, uint8_t* q) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        float t = (float)((double)x[i] / (double)s);
        q[i] = fp8_encode(fmt, (double)t);
    }
}

/* Per-channel scaling, named in P2 §2.1 and §3.2 as the finer alternative to
 * one scale per tensor. Read as: a scale must be constant along K to be
 * applied to the accumulator at write-back (P2 §3.2), so A[M,K] gets one scale
 * per row and B[K,N] one per column; each channel's scale is the per-tensor
 * rule applied to that channel's max|x|. axis 0: one value per row of the
 * row-major x[rows, cols]; axis 1: one value per column. */
ORC_API void orc_amax_channel(const float* x, int64_t rows, int64_t cols, int axis, float* out) {
    if (axis == 0) {
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < rows; ++i) out[i] = orc_amax(x + i * cols, cols);
        return;
    }
    for (int64_t j = 0; j < cols; ++j) {
        float m = 0.0f;
        int saw_nan = 0;
        for (int64_t i = 0; i < rows; ++i) {
            float a = fabsf(x[i * cols + j]);
            if (isnan(a)) saw_nan = 1;
            else if (a > m) m = a;
        }
        out[j] = saw_nan ? NAN : m;
    }
}

/* out_c = the scale of channel c from its amax a_c (orc_scale, per channel). */
ORC_API void orc_scale_n(const float* a, int64_t n, int fmt, int pow2, float* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_scale(a[i], fmt, pow2);
}

/* q[i,j] = FP8_fmt(fl32(x[i,j] / s_c)) with c = i (axis 0) or c = j (axis 1). */
ORC_API void orc_quantize_channel(const float* x, int64_t rows, int64_t cols, int axis, const float* s, int fmt,
                                  uint8_t* q) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; ++i)
        for (int64_t j = 0; j < cols; ++j) {
            double sc = (double)s[axis == 0 ? i : j];
            float t = (float)((double)x[i * cols + j] / sc);
            q[i * cols + j] = fp8_encode(fmt, (double)t);
        }
}

/* q_i = E4M3(fl32(x_i / s)) (P2 §4.3), fl32 being correctly rounded division. */
ORC_API void orc_quantize(const float* x, int64_t n, float s, uint8_t* q) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        float t = (float)((double)x[i] / (double)s);
        q[i] = orc_e4m3_encode((double)t);
    }
}

/* --------------------------------------------- FP16 dynamic-range guard --- */

/* s = min(1, 65504 / (aA * aB)) (P1, mixed-precision section). Read as: the
 * product and the quotient in double (exact product of two floats; the
 * quotient correctly rounded), the result rounded once to FP32. aA * aB == 0
 * gives 65504/0 = inf, so s = 1; a NaN maximum also gives 1 (the NaN
 * element poisons the GEMM by itself); a product so large that s rounds to 0
 * in FP32 (inputs holding inf included) gives 0. */
ORC_API float orc_guard_scale(float aA, float aB) {
    const double q = 65504.0 / ((double)aA * (double)aB);
    return q < 1.0 ? (float)q : 1.0f;
}

/* binary16 bits of fl32(x_i * fl32(sqrt(s))): the operand scaled by the
 * square root of the guard scale in FP32, then rounded to FP16 (RNE, IEEE
 * overflow to inf). sqrt and the product are formed in double and rounded to
 * FP32 once, which is the correctly rounded FP32 result for both. */
ORC_API void orc_guard_to_f16(const float* x, int64_t n, float s, uint16_t* out) {
    const float r = (float)sqrt((double)s);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        const float t = (float)((double)x[i] * (double)r);
        out[i] = orc_f16_round((double)t);
    }
}

/* -------------------------------------------------------------- GEMM ---- */

static double* decode_matrix(int fmt, const void* p, int64_t n) {
    double* d = (double*)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    if (!d) return NULL;
    if (fmt != ORC_FMT_F16) {
        const uint8_t* c = (const uint8_t*)p;
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < n; ++i) d[i] = fp8_decode(fmt, c[i]);
    } else {
        const uint16_t* h = (const uint16_t*)p;
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < n; ++i) d[i] = orc_f16_decode(h[i]);
    }
    return d;
}

/* Row-major A[M,K] (format fa) and B[K,N] (format fb), unscaled products
 * summed in double in ascending k:  R[r,j] = sum_k a[i,k] b[k,j],
 *                                   S[r,j] = sum_k |a[i,k] b[k,j]|,
 * for the rows i = rows[r] (rows == NULL: every row, r == i). R and S are
 * [nrows, N] row-major. E4M3 x E4M3 sums are exact (see above); E5M2 spans a
 * wider range, so its sums are the double-rounded sequential sum. FP16 pairs
 * only with FP16. Returns 0, or -1 when out of memory. */
ORC_API int orc_gemm_mixed(int fa, int fb, const void* A, const void* B, int64_t M, int64_t N, int64_t K,
                           const int64_t* rows, int64_t nrows, double* R, double* S) {
    const uint8_t* a8 = (const uint8_t*)A;
    const uint16_t* a16 = (const uint16_t*)A;
    double* Bd;
    if (rows == NULL) nrows = M;
    Bd = decode_matrix(fb, B, K * N);
    if (!Bd) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t i = rows ? rows[r] : r;
        double* restrict Rr = R + r * N;
        double* restrict Sr = S + r * N;
        for (int64_t j = 0; j < N; ++j) { Rr[j] = 0.0; Sr[j] = 0.0; }
        for (int64_t k = 0; k < K; ++k) {
            double a = (fa == ORC_FMT_F16) ? orc_f16_decode(a16[i * K + k]) : fp8_decode(fa, a8[i * K + k]);
            const double* restrict Bk = Bd + k * N;
            for (int64_t j = 0; j < N; ++j) {
                double p = a * Bk[j];
                Rr[j] += p;
                Sr[j] += fabs(p);
            }
        }
    }
    free(Bd);
    (void)M;
    return 0;
}

/* Both operands in the same format fmt. */
ORC_API int orc_gemm(int fmt, const void* A, const void* B, int64_t M, int64_t N, int64_t K,
                     const int64_t* rows, int64_t nrows, double* R, double* S) {
    return orc_gemm_mixed(fmt, fmt, A, B, M, N, K, rows, nrows, R, S);
}

/* Output rounding of the scaled result V (P2 §3.2, §4.3). */
ORC_API void orc_out_f16(const double* V, int64_t n, uint16_t* out) { orc_f16_round_n(V, n, out); }

ORC_API void orc_out_e4m3(const double* V, int64_t n, double sOut, uint8_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_encode(V[i] / sOut);
}

ORC_API void orc_out_fp8(const double* V, int64_t n, double sOut, int fmt, uint8_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = fp8_encode(fmt, V[i] / sOut);
}

ORC_API int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
