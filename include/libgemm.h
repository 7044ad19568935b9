/*
 * libgemm — FP8 (E4M3 / E5M2) per-tensor-scaled GEMM and FP16 GEMM for AMD
 * Instinct MI355X (gfx950), with the amax and FP8 quantize steps that feed it.
 *
 * Sources that define the operations (cited per entry point below):
 *   P1  DeepGEMM deep-dive article (hnwysp.cn, news 84236)
 *   P2  "DeepGEMM实战：FP8矩阵乘法与JIT编译优化指南" (sheratonhq.com, news 156926)
 *   P3  "HGEMM优化：深度学习中的矩阵乘法性能提升策略" (jsqmd.com, news 710660)
 *
 * Common conventions
 *   - Every matrix is row-major and densely packed: A[M,K], B[K,N], C[M,N]
 *     (leading dimensions K, N and N). Element (i,j) of C is at C + i*N + j.
 *   - Every data pointer is a device pointer (memory the current HIP device
 *     can read or write). Scale arguments are device pointers to ONE float.
 *   - The caller owns every buffer. The library allocates no device memory and
 *     keeps no per-call state; entry points are reentrant and thread-safe.
 *   - Each call validates its arguments on the host first; on any error it
 *     returns a negative status and enqueues nothing. On success the work is
 *     enqueued on `stream` (NULL = the null stream) and the call returns
 *     without synchronising; faults during execution surface at the caller's
 *     next synchronisation, as for any HIP kernel.
 *   - Outputs must not overlap inputs.
 *   - Results never depend on pointer alignment; 16-byte aligned pointers and
 *     row lengths that are multiples of 16 bytes take the fastest kernels.
 *   - Dimensions are int64_t; each must be in [0, 2^31 - 1].
 */
#ifndef LIBGEMM_H
#define LIBGEMM_H

#include <stdint.h>

#include <hip/hip_runtime_api.h> /* hipStream_t */

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------ statuses */
#define GEMM_OK 0
#define GEMM_ERR_NULL (-1)        /* a required pointer is NULL                          */
#define GEMM_ERR_DIM (-2)         /* a dimension is negative or above 2^31 - 1, or an      */
                                  /* operand or output would span 2^62 bytes or more      */
#define GEMM_ERR_DTYPE (-3)       /* unknown out_dtype, or one the entry point cannot write */
#define GEMM_ERR_SCALE (-4)       /* sOut is NULL while out_dtype is an FP8 output         */
#define GEMM_ERR_LAUNCH (-5)      /* the HIP runtime rejected a kernel launch              */
#define GEMM_ERR_UNSUPPORTED (-6) /* no kernel for this request                            */
#define GEMM_ERR_DEVICE (-7)      /* no current HIP device, or it is not gfx950            */
#define GEMM_ERR_ALIAS (-8)       /* the output overlaps an input                          */
#define GEMM_ERR_WORKSPACE (-9)   /* a split-K workspace too small or not 16-byte aligned   */

/* ------------------------------------------------------- output types */
#define GEMM_OUT_F32 0  /* float                                                  */
#define GEMM_OUT_F16 1  /* IEEE binary16, round to nearest even, overflow to inf   */
#define GEMM_OUT_E4M3 2 /* OCP E4M3 code (uint8), nearest even, saturate at +-448 */
#define GEMM_OUT_E5M2 3 /* OCP E5M2 code (uint8), nearest even, saturate at +-57344 */

/* ----------------------------------------------------- FP8 formats */
/* P2 §2.1: E4M3 (4 exponent, 3 mantissa bits; largest value 448) and E5M2
 * (5 exponent, 2 mantissa bits; wider range, less precision; largest 57344,
 * P2 §4.3). Both are the OCP variants: E4M3 without infinities, E5M2 IEEE-like. */
#define GEMM_FMT_E4M3 0
#define GEMM_FMT_E5M2 1

/*
 * gemm_f16 — C = A·B for FP16 operands with FP32 accumulation.
 * P3 §1.3 (half-precision GEMM with a 32-bit accumulator) and P1 §4.1 (the
 * [1,4096]x[4096,12288] projection as the M = 1 case).
 *   A          device, _Float16[M*K], row-major
 *   B          device, _Float16[K*N], row-major
 *   C          device, float[M*N] (out_dtype GEMM_OUT_F32) or _Float16[M*N]
 *              (GEMM_OUT_F16); written, never read
 *   out_dtype  GEMM_OUT_F32 or GEMM_OUT_F16 (anything else: GEMM_ERR_DTYPE)
 *   M, N, K    M = 0 or N = 0 is a no-op; K = 0 writes zeros (the empty sum)
 * M <= 4 runs an HBM-streaming kernel, larger M an MFMA tile kernel; the
 * choice never changes which outputs are written.
 */
int gemm_f16(const void* A, const void* B, void* C, int out_dtype,
             int64_t M, int64_t N, int64_t K, hipStream_t stream);

/*
 * gemm_fp8_scaled — C = (sA·A)(sB·B) for E4M3 operands, FP32 accumulation.
 * P2 §2.1 (FP8 inputs, FP32 accumulator), §3.2 (per-tensor scales applied
 * once to the accumulator at write-back; an FP8 output is divided by its own
 * output scale), §4.3 (the call takes A, B, M, N, K and the scales; output
 * FP32 or FP8, FP8 needing an output scale).
 *   A, B       device, uint8 E4M3 codes, A[M*K] and B[K*N] row-major
 *   sA, sB     device pointers to one float each (per-tensor scales)
 *   sOut       device pointer to one float; required iff out_dtype ==
 *              GEMM_OUT_E4M3 (else ignored, may be NULL)
 *   C          device, float / _Float16 / uint8 per out_dtype, [M*N]
 *   out_dtype  GEMM_OUT_F32, GEMM_OUT_F16 or GEMM_OUT_E4M3
 * Element value: y = acc·(sA·sB) with acc the FP32 sum of decoded products;
 * F32 writes y, F16 writes RNE(y), E4M3 / E5M2 write FP8(y / sOut); the
 * kernels form y / sOut as acc·(sA·sB/sOut), one FP32 factor, which may differ
 * from the two-step quotient by a few FP32 ulps (within one FP8 code step).
 * out_dtype GEMM_OUT_E5M2 is accepted as well (sOut required).
 */
int gemm_fp8_scaled(const uint8_t* A, const uint8_t* B, const float* sA, const float* sB,
                    const float* sOut, void* C, int out_dtype,
                    int64_t M, int64_t N, int64_t K, hipStream_t stream);

/*
 * gemm_fp8_fmt — gemm_fp8_scaled with a format per operand: A holds codes of
 * format fmt_a, B of fmt_b (GEMM_FMT_E4M3 or GEMM_FMT_E5M2; P2 §2.1 names both
 * FP8 formats, each with its own range). Same arguments, element value,
 * outputs (F32, F16, E4M3, E5M2) and errors as gemm_fp8_scaled; an unknown
 * format gives GEMM_ERR_DTYPE. Products of E4M3 and E5M2 codes accumulate in
 * FP32 on the FP8 matrix cores, whose format selectors take both formats.
 */
int gemm_fp8_fmt(const uint8_t* A, int fmt_a, const uint8_t* B, int fmt_b,
                 const float* sA, const float* sB, const float* sOut, void* C, int out_dtype,
                 int64_t M, int64_t N, int64_t K, hipStream_t stream);

/*
 * quantize_fp8 — q[i] = E4M3(fl32(x[i] / scale)).
 * P2 §4.3 (fp8 = clamp(round(x / scale), -448, 448)): the quotient is the
 * correctly rounded FP32 division; it is rounded to the nearest E4M3 value
 * (ties to the even code) and saturated at +-448; +-inf saturate, NaN gives
 * the code 0x7F; -0 and negative values that round to zero give 0x80.
 *   x      device, float[n]
 *   n      number of elements (0: no-op)
 *   scale  device pointer to one float (e.g. the one amax_f32 writes)
 *   q      device, uint8[n], written; must not overlap x
 */
int quantize_fp8(const float* x, int64_t n, const float* scale, uint8_t* q, hipStream_t stream);

/*
 * quantize_fp8_fmt — quantize_fp8 into FP8 format fmt: E4M3 as above, or E5M2
 * (P2 §4.3: the clamp bound is 57344 for E5M2): the FP32 quotient rounded to
 * the nearest E5M2 value (ties to the even code), saturated at +-57344, +-inf
 * saturating too, NaN giving 0x7F. Unknown fmt: GEMM_ERR_DTYPE. Arguments and
 * errors otherwise as quantize_fp8.
 */
int quantize_fp8_fmt(const float* x, int64_t n, const float* scale, uint8_t* q, int fmt, hipStream_t stream);

/*
 * amax_f32 — *amax = max_i |x[i]| (exact; NaN if any x[i] is NaN; 0 for
 * n = 0) and, when scale != NULL, *scale = fl32(*amax / 448), replaced by 1
 * when that is 0 (P2 §3.2: per-tensor scale = max|x| / 448, 448 being the
 * largest E4M3 value; P1 §3.3: the maximum is taken on the GPU on a stream).
 *   x      device, float[n]
 *   amax   device pointer to one float, written
 *   scale  device pointer to one float or NULL; written when non-NULL
 * amax serves as the running maximum while the call's kernels run: both
 * outputs are defined once that work has completed in stream order, and they
 * must not overlap x or each other (GEMM_ERR_ALIAS). Up to three launches;
 * no allocation.
 */
int amax_f32(const float* x, int64_t n, float* amax, float* scale, hipStream_t stream);

/*
 * amax_scale_f32 — amax_f32 with the scale rule chosen by the caller:
 *   pow2 == 0: *scale = fl32(*amax / fmax), replaced by 1 when that is 0,
 *              fmax = 448 (GEMM_FMT_E4M3) or 57344 (GEMM_FMT_E5M2) (P2 §3.2,
 *              §4.3);
 *   pow2 != 0: *scale = the smallest power of two s with *amax / s <= fmax
 *              (P2 §2.1: a power of two just above the calibrated maximum, so
 *              scaling is exponent arithmetic), not below 2^-149; amax 0 gives
 *              1, inf gives inf, NaN gives NaN.
 * Unknown fmt: GEMM_ERR_DTYPE. Arguments, aliasing rules and errors otherwise
 * as amax_f32 (amax_f32 is this call with GEMM_FMT_E4M3 and pow2 = 0).
 */
int amax_scale_f32(const float* x, int64_t n, float* amax, float* scale, int fmt, int pow2,
                   hipStream_t stream);

/* ------------------------------------------------ per-channel scaling */
/* P2 §2.1 and §3.2 name per-channel scaling as the finer alternative to one
 * scale per tensor. A scale applied to the accumulator at write-back (P2 §3.2)
 * must be constant along K, so the channels are the rows of A[M,K] and the
 * columns of B[K,N]. The channel calls take a row-major x[rows, cols] and an
 * axis: GEMM_AXIS_ROW gives one value per row (rows values; use it for A),
 * GEMM_AXIS_COL one per column (cols values; use it for B). */
#define GEMM_AXIS_ROW 0
#define GEMM_AXIS_COL 1

/*
 * gemm_fp8_channel — gemm_fp8_fmt with a scale per channel:
 *   C[i,j] = acc[i,j] · sA[i] · sB[j]   (F32, F16 outputs)
 *   C[i,j] = FP8(acc[i,j] · (1/sOut) · sA[i] · sB[j])   (E4M3 / E5M2 outputs)
 *   sA     device, float[M]: one scale per row of A
 *   sB     device, float[N]: one scale per column of B
 *   sOut   device pointer to one float (per-tensor output scale), required
 *          iff out_dtype is an FP8 output
 * Every other argument, output and error as gemm_fp8_fmt. The kernels read
 * sA[i] and sB[j] only for the elements they store, and form the element's
 * value as three FP32 products (a few FP32 ulps from the exact product).
 */
int gemm_fp8_channel(const uint8_t* A, int fmt_a, const uint8_t* B, int fmt_b,
                     const float* sA, const float* sB, const float* sOut, void* C, int out_dtype,
                     int64_t M, int64_t N, int64_t K, hipStream_t stream);

/*
 * amax_scale_channel_f32 — per channel c of x[rows, cols] (axis as above):
 *   amax[c]  = max |x| over the channel (exact; NaN if the channel holds a
 *              NaN; 0 for an empty channel)
 *   scale[c] = the rule of amax_scale_f32 (fmt, pow2) applied to amax[c];
 *              written when scale != NULL
 *   x       device, float[rows*cols] row-major (may be NULL when it is empty)
 *   amax    device, float[rows] (GEMM_AXIS_ROW) or float[cols] (GEMM_AXIS_COL)
 *   scale   device, the same length as amax, or NULL
 * With GEMM_AXIS_COL, amax serves as the running maximum while the call's
 * kernels run (three launches; one launch for GEMM_AXIS_ROW). Outputs must
 * not overlap x or each other (GEMM_ERR_ALIAS). Unknown fmt: GEMM_ERR_DTYPE;
 * an axis other than the two: GEMM_ERR_DIM. No allocation.
 */
int amax_scale_channel_f32(const float* x, int64_t rows, int64_t cols, int axis, float* amax,
                           float* scale, int fmt, int pow2, hipStream_t stream);

/*
 * quantize_fp8_channel — q[i,j] = FP8_fmt(fl32(x[i,j] / scale[c])) with c = i
 * (GEMM_AXIS_ROW) or c = j (GEMM_AXIS_COL); rounding, saturation and NaN as
 * quantize_fp8_fmt (P2 §4.3).
 *   x      device, float[rows*cols] row-major
 *   scale  device, float[rows] or float[cols] per the axis
 *   q      device, uint8[rows*cols], written; must not overlap x or scale
 * Errors as quantize_fp8_fmt, plus GEMM_ERR_DIM for an unknown axis.
 */
int quantize_fp8_channel(const float* x, int64_t rows, int64_t cols, int axis,
                         const float* scale, uint8_t* q, int fmt, hipStream_t stream);

/* ------------------------------------------------------------ split-K */
/* Decode and mid-M shapes (e.g. M <= 256 with N = K = 4096) have too few
 * output tiles to occupy 256 compute units while B streams from HBM. The
 * workspace entry points then cut K into ranges summed by separate
 * workgroups into FP32 slices of a caller-provided workspace, and a second
 * launch adds the slices in a fixed order and applies the epilogue once to
 * the full sum (P3 §6 names splitting K as the way to spread one GEMM over
 * more compute; P2 §3.2: scale, then convert, at write-back). */

/*
 * gemm_splitk_plan — host-only query: the configuration, the number of K
 * ranges (*splits; 1 = no split) and the workspace size in bytes
 * (*workspace_bytes = splits * M * N * 4, or 0) that gemm_fp8_splitk (kind 1)
 * or gemm_f16_splitk (kind 0) would use for this request. buf receives the
 * configuration name (NUL-terminated, truncated to buflen); buf, splits and
 * workspace_bytes may each be NULL. Returns GEMM_OK or a negative status for
 * invalid arguments; makes no HIP call. The plan depends only on the shape,
 * the kinds, formats and output type (and the LIBGEMM_CONFIG / LIBGEMM_SPLITS
 * overrides).
 */
int gemm_splitk_plan(int kind, int out_dtype, int64_t M, int64_t N, int64_t K,
                     int fmt_a, int fmt_b, char* buf, int buflen, int* splits,
                     int64_t* workspace_bytes);

/*
 * gemm_fp8_splitk — gemm_fp8_fmt (per-tensor scales) that may split K.
 *   workspace        device memory of workspace_bytes bytes, 16-byte aligned,
 *                    used as FP32 scratch; or NULL: no split (the plain call)
 *   workspace_bytes  at least what gemm_splitk_plan reports for the request
 * When the plan splits, the workspace must be large enough and 16-byte
 * aligned (else GEMM_ERR_WORKSPACE) and must not overlap A, B, C or the
 * scales (GEMM_ERR_ALIAS); its contents on entry do not matter and on return
 * are unspecified. Two launches on `stream`; calls that share a workspace
 * must not run concurrently. Element values, outputs and other errors as
 * gemm_fp8_fmt; the FP32 sum is formed in another order (per K range, then
 * across ranges in range order), so results are deterministic and within the
 * same bounds.
 */
int gemm_fp8_splitk(const uint8_t* A, int fmt_a, const uint8_t* B, int fmt_b,
                    const float* sA, const float* sB, const float* sOut, void* C, int out_dtype,
                    int64_t M, int64_t N, int64_t K, void* workspace, int64_t workspace_bytes,
                    hipStream_t stream);

/*
 * gemm_fp8_splitk_noalloc — gemm_fp8_splitk for callers that cannot allocate
 * device memory (code under HIP graph capture, serving loops, harnesses that
 * forbid hipMalloc): the FP32 partial sums go to a 16 MiB array that the
 * library holds on every GPU it runs on (the first call on a device looks up
 * that device's copy), so no workspace argument. A plan that needs more than
 * gemm_fp8_splitk_noalloc_max_bytes() bytes (splits * M * N * 4) returns
 * GEMM_ERR_WORKSPACE before any launch; a plan that does not split is the
 * plain call. The call allocates nothing. All calls on one GPU share the
 * array: calls that overlap in time on one GPU (other streams, other host
 * threads) race and must be serialised by the caller. Results, other errors
 * and determinism as gemm_fp8_splitk.
 */
int gemm_fp8_splitk_noalloc(const uint8_t* A, int fmt_a, const uint8_t* B, int fmt_b,
                            const float* sA, const float* sB, const float* sOut, void* C,
                            int out_dtype, int64_t M, int64_t N, int64_t K, hipStream_t stream);

/* gemm_fp8_splitk_noalloc_max_bytes — the size of that array in bytes. */
int64_t gemm_fp8_splitk_noalloc_max_bytes(void);

/* gemm_f16_splitk — gemm_f16 that may split K, with the workspace rules of
 * gemm_fp8_splitk (the M = 1 decode of P1 §4.1 is such a shape). */
int gemm_f16_splitk(const void* A, const void* B, void* C, int out_dtype,
                    int64_t M, int64_t N, int64_t K, void* workspace, int64_t workspace_bytes,
                    hipStream_t stream);

/* ------------------------------------------- FP16 dynamic-range guard */

/*
 * gemm_f16_guarded — C = A·B for FP32 inputs computed as an FP16 GEMM under
 * P1's dynamic-range guard (mixed-precision section): FP16 holds at most
 * ±65504, so max|A| and max|B| are taken on the GPU first, then
 *   s  = min(1, 65504 / (max|A| · max|B|))   (product and quotient in double,
 *        rounded once to FP32; 1 when A or B is all zero)
 *   A' = FP16(fl32(A · fl32(sqrt(s)))),  B' likewise   (RNE, IEEE overflow)
 *   C  = (A'·B', FP32 accumulation) · fl32(1/s)   (F32, or RNE to F16)
 * so every product of the scaled operands stays within the FP16 range. Both
 * operands stay finite when max|A| / max|B| (and its inverse) is at most
 * 65504; beyond that the larger one can still overflow to inf, as the
 * formula stands.
 *   A          device, float[M*K], row-major
 *   B          device, float[K*N], row-major
 *   C          device, float or _Float16 [M*N] per out_dtype (GEMM_OUT_F32 or
 *              GEMM_OUT_F16)
 *   scale      device pointer to one float receiving s, or NULL
 *   workspace  device memory, 16-byte aligned, of at least
 *              gemm_f16_guarded_workspace_size(M, N, K) bytes. On return it
 *              holds at offset 0 the floats max|A|, max|B|, s, sqrt(s), 1/s;
 *              at offset 256 the scaled FP16 A' (M*K halves, row-major); and
 *              at offset 256 + M*K*2 rounded up to a multiple of 256 the
 *              scaled FP16 B' (K*N halves).
 * Errors: GEMM_ERR_NULL (C or workspace NULL, or A/B NULL with K > 0),
 * GEMM_ERR_WORKSPACE (too small or misaligned), GEMM_ERR_ALIAS (C, the
 * workspace, scale, A and B must not overlap), and those of gemm_f16.
 * M = 0 or N = 0 is a no-op; K = 0 writes zeros (and s = 1). Eight launches
 * on `stream` (amax x2 with their clears, the scale, two conversions, the
 * GEMM); calls that share a workspace must not run concurrently.
 */
int gemm_f16_guarded(const float* A, const float* B, void* C, int out_dtype,
                     int64_t M, int64_t N, int64_t K, float* scale,
                     void* workspace, int64_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace gemm_f16_guarded needs (GEMM_ERR_DIM for a bad size). */
int64_t gemm_f16_guarded_workspace_size(int64_t M, int64_t N, int64_t K);

/* Human-readable name of a status code (a static string). */
const char* gemm_status_str(int status);

/*
 * gemm_select_config — host-only query of the shape-to-kernel selector
 * (P3 §3.1: tile sizes chosen from M, N and K; P2 §3.3: a smaller tile when
 * edge waste is high). Writes the name of the kernel configuration that
 * gemm_f16 (kind 0) or gemm_fp8_scaled (kind 1) would launch for this shape
 * into buf (NUL-terminated, truncated to buflen) and returns GEMM_OK, or a
 * negative status for invalid arguments. Makes no HIP call.
 */
int gemm_select_config(int kind, int out_dtype, int64_t M, int64_t N, int64_t K,
                       char* buf, int buflen);

/* gemm_select_config for gemm_fp8_fmt's operand formats (kind 1), or kind 0
 * with formats ignored; unknown formats give GEMM_ERR_DTYPE. */
int gemm_select_config_fmt(int kind, int out_dtype, int64_t M, int64_t N, int64_t K,
                           int fmt_a, int fmt_b, char* buf, int buflen);

/* ------------------------------------------------ K-major B (weight layout) */
/* P1 §3.2 ("Data Layout"): the weight matrix B need not be kept row-major;
 * it may be stored in a layout chosen for the kernel. The calls below take B
 * K-major, as Bt[N,K] row-major (element (k, n) of B at Bt[n*K + k]), which is
 * how a linear layer keeps its weight. Every B row is then a contiguous K
 * vector: the MFMA tile kernels stage B exactly like A (no LDS transpose
 * reads), and decode shapes (M <= 8) read each weight row once as a dot
 * product (P1 §2.1, §4.1: the [1,4096]x[4096,12288] projection reads each
 * weight once). The results are those of gemm_f16 / gemm_fp8_scaled on
 * B = transpose(Bt). */

/*
 * gemm_f16_bt — gemm_f16 with B given as Bt[N,K]:
 *   A          device, _Float16[M*K], row-major
 *   Bt         device, _Float16[N*K], row-major (B transposed)
 *   C, out_dtype, M, N, K, stream, errors: as gemm_f16.
 * M <= 8 runs the K-major decode kernel, larger M the MFMA tile kernel.
 */
int gemm_f16_bt(const void* A, const void* Bt, void* C, int out_dtype,
                int64_t M, int64_t N, int64_t K, hipStream_t stream);

/*
 * gemm_fp8_scaled_bt — gemm_fp8_scaled (E4M3 operands, per-tensor scales,
 * outputs F32, F16, E4M3 or E5M2) with B given as Bt[N,K] E4M3 codes,
 * row-major. Arguments, element value and errors as gemm_fp8_scaled.
 */
int gemm_fp8_scaled_bt(const uint8_t* A, const uint8_t* Bt, const float* sA, const float* sB,
                       const float* sOut, void* C, int out_dtype,
                       int64_t M, int64_t N, int64_t K, hipStream_t stream);

/*
 * quantize_fp8_transposed — quantize_fp8 of a row-major x[rows, cols] written
 * transposed: q[c*rows + r] = E4M3(fl32(x[r*cols + c] / scale)) (same
 * rounding, saturation and NaN rules as quantize_fp8, P2 §4.3). Quantizing a
 * row-major FP32 B[K,N] this way gives the Bt[N,K] codes gemm_fp8_scaled_bt
 * takes, in the same pass over B.
 *   x      device, float[rows*cols], row-major
 *   rows, cols  sizes (either 0: no-op; each at most 2^31 - 1)
 *   scale  device pointer to one float
 *   q      device, uint8[cols*rows], written; must not overlap x or scale
 */
int quantize_fp8_transposed(const float* x, int64_t rows, int64_t cols, const float* scale,
                            uint8_t* q, hipStream_t stream);

/*
 * gemm_fp8_fmt_bt — gemm_fp8_fmt (A in FP8 format fmt_a, B in fmt_b: E4M3 or
 * E5M2, P2 §2.1) with B given as Bt[N,K] codes, row-major. Arguments, element
 * value, outputs and errors as gemm_fp8_fmt.
 */
int gemm_fp8_fmt_bt(const uint8_t* A, int fmt_a, const uint8_t* Bt, int fmt_b,
                    const float* sA, const float* sB, const float* sOut, void* C, int out_dtype,
                    int64_t M, int64_t N, int64_t K, hipStream_t stream);

/*
 * quantize_fp8_transposed_fmt — quantize_fp8_transposed into FP8 format fmt
 * (E4M3 as quantize_fp8, E5M2 as quantize_fp8_fmt: saturate at +-57344, P2
 * §4.3). Unknown fmt: GEMM_ERR_DTYPE; otherwise as quantize_fp8_transposed.
 */
int quantize_fp8_transposed_fmt(const float* x, int64_t rows, int64_t cols, const float* scale,
                                uint8_t* q, int fmt, hipStream_t stream);

/*
 * pack_b_kmajor — the one-time re-layout of a weight into the K-major form the
 * _bt calls take (P1 §3.2: the weight is stored in a layout chosen for the
 * kernel, ahead of the GEMMs that read it): Bt[n*K + k] = B[k*N + n].
 *   B           device, row-major [K, N] elements of elem_bytes bytes (2: FP16,
 *               1: FP8 codes); read only
 *   K, N        sizes (either 0: no-op; each at most 2^31 - 1)
 *   elem_bytes  1 or 2 (else GEMM_ERR_DTYPE)
 *   Bt          device, [N, K] elements, written; must not overlap B
 * One launch on `stream`; bytes are moved unchanged.
 */
int pack_b_kmajor(const void* B, int64_t K, int64_t N, int elem_bytes, void* Bt, hipStream_t stream);

/* gemm_select_config for gemm_f16_bt (kind 0) and gemm_fp8_scaled_bt (kind 1). */
int gemm_select_config_bt(int kind, int out_dtype, int64_t M, int64_t N, int64_t K,
                          char* buf, int buflen);

/*
 * gemm_fp8_splitk_bt / gemm_f16_splitk_bt — gemm_fp8_scaled_bt / gemm_f16_bt
 * that may split K over a caller-provided workspace, exactly as
 * gemm_fp8_splitk / gemm_f16_splitk do for row-major B (P3 §6: K split to
 * spread one GEMM over more compute; the epilogue's scale and rounding are
 * applied once, to the full sum). Shapes up to M = 256 may split; decode
 * shapes (M <= 8) keep the K-major decode kernels and never split. Workspace
 * rules, errors and the determinism of the result as gemm_fp8_splitk; the
 * FP8 call takes E4M3 operands.
 */
int gemm_fp8_splitk_bt(const uint8_t* A, const uint8_t* Bt, const float* sA, const float* sB,
                       const float* sOut, void* C, int out_dtype, int64_t M, int64_t N, int64_t K,
                       void* workspace, int64_t workspace_bytes, hipStream_t stream);
int gemm_f16_splitk_bt(const void* A, const void* Bt, void* C, int out_dtype,
                       int64_t M, int64_t N, int64_t K, void* workspace, int64_t workspace_bytes,
                       hipStream_t stream);

/* gemm_splitk_plan for the two calls above (kind 0: FP16, 1: E4M3). */
int gemm_splitk_plan_bt(int kind, int out_dtype, int64_t M, int64_t N, int64_t K,
                        char* buf, int buflen, int* splits, int64_t* workspace_bytes);

/*
 * amax_quantize_fp8_pair — both operands of an FP8 GEMM in two launches:
 * amax[0] = max|A|, scale[0] = the scale of amax[0] for format fmt (pow2 = 0:
 * fl32(amax / fmax) with 0 -> 1, as amax_f32 / amax_scale_f32; pow2 != 0: the
 * power of two of amax_scale_f32), qa = FP8(fl32(A / scale[0])) as
 * quantize_fp8_fmt; the same for B into amax[1], scale[1], qb. Every value is
 * bit-identical to the separate calls. P2 §3.2 (per-tensor scale max/448 for
 * each operand), §4.3 (the quantize formula), §4.4 (launch overhead dominates
 * small work: batch it); P1 §3.3 (maxima on the GPU, on a stream).
 *   A, na      device, float[na]; na = 0 gives amax 0, scale 1, no codes
 *   B, nb      device, float[nb]; nb = 0: only A is processed, amax[1] and
 *              scale[1] are not written
 *   fmt, pow2  GEMM_FMT_E4M3 or GEMM_FMT_E5M2; scale rule as amax_scale_f32
 *   amax, scale  device, float[2] (float[1] when nb = 0), written
 *   qa, qb     device, uint8[na] and uint8[nb], written
 *   workspace  device scratch of at least
 *              amax_quantize_fp8_pair_workspace_size() bytes, 16-byte
 *              aligned, owned by the caller; its contents are overwritten
 * Errors: GEMM_ERR_DTYPE (fmt), GEMM_ERR_DIM (a count negative or of 2^62
 * bytes or more), GEMM_ERR_NULL, GEMM_ERR_WORKSPACE, GEMM_ERR_ALIAS (any two
 * written ranges, or a written range and an input, overlap). No allocation.
 */
int amax_quantize_fp8_pair(const float* A, int64_t na, const float* B, int64_t nb, int fmt, int pow2,
                           float* amax, float* scale, uint8_t* qa, uint8_t* qb, void* workspace,
                           int64_t workspace_bytes, hipStream_t stream);
/* Bytes of scratch amax_quantize_fp8_pair needs (a constant, 4096). */
int64_t amax_quantize_fp8_pair_workspace_size(void);

/*
 * amax_quantize_fp8_pair_bt — amax_quantize_fp8_pair for a GEMM whose B is
 * given row-major, with B's codes written K-major for the _bt GEMM calls:
 * qbt[n * K + k] = FP8(fl32(B[k * N + n] / scale[1])). amax, scale and qa are
 * those of amax_quantize_fp8_pair on (A, na, B, K * N), and qbt is its qb
 * transposed, bit for bit. P1 §3.2 (the weight held in the layout the kernel
 * reads), with P2 §3.2 / §4.3 / §4.4 and P1 §3.3 as for the call above.
 *   A, na      device, float[na]
 *   B, K, N    device, float[K * N], row-major [K, N]; K * N = 0: only A is
 *              processed, amax[1] and scale[1] are not written
 *   fmt, pow2, amax, scale, qa, workspace  as amax_quantize_fp8_pair
 *   qbt        device, uint8[N * K], row-major [N, K], written
 * Errors: as amax_quantize_fp8_pair (GEMM_ERR_DIM also for K or N negative or
 * above 2^31 - 1).
 * No allocation.
 */
int amax_quantize_fp8_pair_bt(const float* A, int64_t na, const float* B, int64_t K, int64_t N, int fmt,
                              int pow2, float* amax, float* scale, uint8_t* qa, uint8_t* qbt, void* workspace,
                              int64_t workspace_bytes, hipStream_t stream);

/*
 * gemm_fp8_exact / gemm_fp8_exact_bt — gemm_fp8_fmt / gemm_fp8_fmt_bt with
 * every product exact and every addition an FP32 addition (P2 §2.1: FP8
 * inputs with FP32 accumulation; §4.3: results are checked against an FP32
 * computation). The FP8 matrix cores used by the other calls add the 8
 * products of each aligned group of k after aligning them to the group's
 * largest exponent and dropping the bits more than 13 places below it; for
 * operands spanning a wide exponent range that can exceed an FP32
 * accumulation's error. These calls never use them: the codes are widened
 * exactly to FP16 as they are staged (every E4M3 and E5M2 value is an FP16
 * value) and summed on the FP16 matrix cores, which add FP16 products at FP32
 * precision; decode shapes (M <= 4 with row-major B, M <= 8 with K-major Bt)
 * run the FP32-FMA streaming kernels, which are exact in the same sense. The
 * FP16 matrix cores run at half the FP8 rate.
 *   A, fmt_a, B (or Bt[N*K]), fmt_b, sA, sB, sOut, C, out_dtype, M, N, K:
 *   as gemm_fp8_fmt; outputs F32, F16, E4M3 or E5M2; same errors. No
 *   allocation, no split of K.
 */
int gemm_fp8_exact(const uint8_t* A, int fmt_a, const uint8_t* B, int fmt_b,
                   const float* sA, const float* sB, const float* sOut, void* C, int out_dtype,
                   int64_t M, int64_t N, int64_t K, hipStream_t stream);
int gemm_fp8_exact_bt(const uint8_t* A, int fmt_a, const uint8_t* Bt, int fmt_b,
                      const float* sA, const float* sB, const float* sOut, void* C, int out_dtype,
                      int64_t M, int64_t N, int64_t K, hipStream_t stream);

/* The configuration gemm_fp8_exact (b_kmajor 0) or gemm_fp8_exact_bt
 * (b_kmajor 1) would launch; host only. Errors as gemm_select_config_fmt. */
int gemm_select_config_exact(int out_dtype, int64_t M, int64_t N, int64_t K, int fmt_a, int fmt_b,
                             int b_kmajor, char* buf, int buflen);

#ifdef __cplusplus
}
#endif

#endif /* LIBGEMM_H */
