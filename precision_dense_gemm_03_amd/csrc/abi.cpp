// C-ABI entry points of libgemm (declared in include/libgemm.h).
//
// Every entry point validates its arguments before any HIP call, so invalid
// requests return a status and enqueue nothing; then it checks (once per
// device) that the current device is gfx950, selects a kernel configuration
// from the shape and launches on the caller's stream without synchronising.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>
#include <cstring>

#include "kernels.h"
#include "libgemm.h"

using namespace libgemm;

namespace {

constexpr int64_t kMaxDim = 0x7FFFFFFF;
constexpr int kMaxDevices = 64;

bool dim_ok(int64_t d) { return d >= 0 && d <= kMaxDim; }

// Byte counts are formed only after this check: an operand of 2^62 bytes or
// more is a GEMM_ERR_DIM (no device holds one), so every later product of a
// dimension pair and an element size fits in int64.
constexpr unsigned __int128 kMaxBytes = (unsigned __int128)1 << 62;
bool bytes_ok(int64_t a, int64_t b, int64_t es) {
    if (a < 0 || b < 0) return false;
    return (unsigned __int128)a * (unsigned __int128)b * (unsigned __int128)es < kMaxBytes;
}
// A[M,K] with element size ea, B[K,N] with eb, C[M,N] with ec.
bool gemm_sizes_ok(int64_t M, int64_t N, int64_t K, int64_t ea, int64_t eb, int64_t ec) {
    return dim_ok(M) && dim_ok(N) && dim_ok(K) && bytes_ok(M, K, ea) && bytes_ok(K, N, eb) && bytes_ok(M, N, ec);
}

// Byte ranges [p, p+n) and [q, q+m) overlap (empty ranges never do).
bool overlaps(const void* p, int64_t n, const void* q, int64_t m) {
    if (!p || !q || n <= 0 || m <= 0) return false;
    const uintptr_t a = (uintptr_t)p, b = (uintptr_t)q;
    return a < b + (uintptr_t)m && b < a + (uintptr_t)n;
}

int64_t out_size(int out_dtype) { return out_dtype == GEMM_OUT_F32 ? 4 : (out_dtype == GEMM_OUT_F16 ? 2 : 1); }

// 0 unknown, 1 gfx950, 2 other architecture; filled once per device.
std::atomic<int> g_device_state[kMaxDevices];

int check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return GEMM_ERR_DEVICE;
    }
    int st = g_device_state[dev].load(std::memory_order_acquire);
    if (st == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
            (void)hipGetLastError();
            return GEMM_ERR_DEVICE;
        }
        st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
        g_device_state[dev].store(st, std::memory_order_release);
    }
    return st == 1 ? GEMM_OK : GEMM_ERR_DEVICE;
}

int status_of(hipError_t e) {
    if (e == hipSuccess) return GEMM_OK;
    (void)hipGetLastError();
    return GEMM_ERR_LAUNCH;
}

bool fp8_out(int out_dtype) { return out_dtype == GEMM_OUT_E4M3 || out_dtype == GEMM_OUT_E5M2; }

int run_gemm(int kind, const GemmArgs& a) {
    int st = check_device();
    if (st != GEMM_OK) return st;
    if (a.M == 0 || a.N == 0) return GEMM_OK;
    if (a.K == 0) return status_of(launch_fill_zero(a.C, a.M * a.N, a.out_dtype, a.stream));
    const GemmConfig* cfg = select_config(kind, a.out_dtype, a.M, a.N, a.K, a.fmt_a, a.fmt_b, a.b_kmajor);
    if (!cfg) return GEMM_ERR_UNSUPPORTED;
    return status_of(cfg->launch(a));
}

// The exact-accumulation FP8 mode: validated arguments, the exact selector.
int run_gemm_exact(const GemmArgs& a) {
    int st = check_device();
    if (st != GEMM_OK) return st;
    if (a.M == 0 || a.N == 0) return GEMM_OK;
    if (a.K == 0) return status_of(launch_fill_zero(a.C, a.M * a.N, a.out_dtype, a.stream));
    const GemmConfig* cfg = select_config_exact(a.out_dtype, a.M, a.N, a.K, a.fmt_a, a.fmt_b, a.b_kmajor);
    if (!cfg) return GEMM_ERR_UNSUPPORTED;
    return status_of(cfg->launch(a));
}

int64_t splitk_bytes(const SplitPlan& p, int64_t M, int64_t N) { return p.splits > 1 ? p.splits * M * N * 4 : 0; }

// Workspace entry points: after the caller's arguments were validated, the
// workspace is checked (host only), then the split launch and the reduce run,
// or the plain launch when the plan does not split or no workspace was given.
// `inputs` lists the byte ranges the workspace must not overlap.
int run_gemm_splitk(int kind, GemmArgs a, void* ws, int64_t ws_bytes, const void* const* in_ptr,
                    const int64_t* in_bytes, int n_in) {
    if (a.M == 0 || a.N == 0 || a.K == 0 || !ws) return run_gemm(kind, a);
    if (ws_bytes < 0) return GEMM_ERR_WORKSPACE;
    const SplitPlan p = plan_splitk(kind, a.out_dtype, a.M, a.N, a.K, a.fmt_a, a.fmt_b, a.b_kmajor);
    if (!p.cfg) return GEMM_ERR_UNSUPPORTED;
    const int64_t need = splitk_bytes(p, a.M, a.N);
    if (need == 0) return run_gemm(kind, a);
    if (ws_bytes < need || ((uintptr_t)ws & 15u) != 0) return GEMM_ERR_WORKSPACE;
    for (int i = 0; i < n_in; ++i)
        if (overlaps(ws, need, in_ptr[i], in_bytes[i])) return GEMM_ERR_ALIAS;
    const int st = check_device();
    if (st != GEMM_OK) return st;
    a.ws = reinterpret_cast<float*>(ws);
    a.splits = p.splits;
    a.k_chunk = p.k_chunk;
    const int s1 = status_of(p.cfg->launch(a));
    if (s1 != GEMM_OK) return s1;
    return status_of(launch_splitk_reduce(a));
}

}  // namespace

extern "C" {

// gemm_f16 and gemm_f16_bt: b_kmajor = 1 when B is given as Bt[N,K].
static int gemm_f16_common(const void* A, const void* B, void* C, int out_dtype, int64_t M, int64_t N, int64_t K,
                           hipStream_t stream, int b_kmajor) {
    if (out_dtype != GEMM_OUT_F32 && out_dtype != GEMM_OUT_F16) return GEMM_ERR_DTYPE;
    if (!gemm_sizes_ok(M, N, K, 2, 2, out_size(out_dtype))) return GEMM_ERR_DIM;
    if (M > 0 && N > 0) {
        if (!C) return GEMM_ERR_NULL;
        if (K > 0 && (!A || !B)) return GEMM_ERR_NULL;
        const int64_t cbytes = M * N * out_size(out_dtype);
        if (K > 0 && (overlaps(C, cbytes, A, M * K * 2) || overlaps(C, cbytes, B, K * N * 2))) return GEMM_ERR_ALIAS;
    }
    GemmArgs a{A, B, C, nullptr, nullptr, nullptr, out_dtype, M, N, K, stream};
    a.b_kmajor = b_kmajor;
    return run_gemm(KIND_F16, a);
}

int gemm_f16(const void* A, const void* B, void* C, int out_dtype, int64_t M, int64_t N, int64_t K,
             hipStream_t stream) {
    return gemm_f16_common(A, B, C, out_dtype, M, N, K, stream, 0);
}

int gemm_f16_bt(const void* A, const void* Bt, void* C, int out_dtype, int64_t M, int64_t N, int64_t K,
                hipStream_t stream) {
    return gemm_f16_common(A, Bt, C, out_dtype, M, N, K, stream, 1);
}

// Shared by gemm_fp8_scaled, gemm_fp8_fmt, gemm_fp8_channel and
// gemm_fp8_splitk: validation, then the launch. channel: sA holds M floats and
// sB N floats. ws: the split-K workspace (NULL: none).
static int gemm_fp8_common(const uint8_t* A, int fmt_a, const uint8_t* B, int fmt_b, const float* sA,
                           const float* sB, const float* sOut, void* C, int out_dtype, int64_t M, int64_t N,
                           int64_t K, hipStream_t stream, int channel = 0, void* ws = nullptr,
                           int64_t ws_bytes = 0, int b_kmajor = 0, int exact = 0) {
    if (out_dtype < GEMM_OUT_F32 || out_dtype > GEMM_OUT_E5M2) return GEMM_ERR_DTYPE;
    if ((fmt_a != GEMM_FMT_E4M3 && fmt_a != GEMM_FMT_E5M2) || (fmt_b != GEMM_FMT_E4M3 && fmt_b != GEMM_FMT_E5M2))
        return GEMM_ERR_DTYPE;
    if (!gemm_sizes_ok(M, N, K, 1, 1, out_size(out_dtype))) return GEMM_ERR_DIM;
    if (M > 0 && N > 0) {
        if (!C || !sA || !sB) return GEMM_ERR_NULL;
        if (fp8_out(out_dtype) && !sOut) return GEMM_ERR_SCALE;
        if (K > 0 && (!A || !B)) return GEMM_ERR_NULL;
        const int64_t cbytes = M * N * out_size(out_dtype);
        if (K > 0 && (overlaps(C, cbytes, A, M * K) || overlaps(C, cbytes, B, K * N))) return GEMM_ERR_ALIAS;
        const int64_t sa_bytes = channel ? 4 * M : 4, sb_bytes = channel ? 4 * N : 4;
        if (overlaps(C, cbytes, sA, sa_bytes) || overlaps(C, cbytes, sB, sb_bytes) ||
            (fp8_out(out_dtype) && overlaps(C, cbytes, sOut, 4)))
            return GEMM_ERR_ALIAS;
    }
    GemmArgs a{A, B, C, sA, sB, fp8_out(out_dtype) ? sOut : nullptr, out_dtype, M, N, K, stream, fmt_a, fmt_b,
               channel};
    a.b_kmajor = b_kmajor;
    if (exact) return run_gemm_exact(a);
    if (!ws) return run_gemm(KIND_FP8, a);
    const void* in_ptr[6] = {A, B, C, sA, sB, fp8_out(out_dtype) ? sOut : nullptr};
    const int64_t in_bytes[6] = {M * K, K * N, M * N * out_size(out_dtype), channel ? 4 * M : 4, channel ? 4 * N : 4,
                                 4};
    return run_gemm_splitk(KIND_FP8, a, ws, ws_bytes, in_ptr, in_bytes, 6);
}

int gemm_fp8_scaled(const uint8_t* A, const uint8_t* B, const float* sA, const float* sB, const float* sOut,
                    void* C, int out_dtype, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
    return gemm_fp8_common(A, GEMM_FMT_E4M3, B, GEMM_FMT_E4M3, sA, sB, sOut, C, out_dtype, M, N, K, stream);
}

int gemm_fp8_scaled_bt(const uint8_t* A, const uint8_t* Bt, const float* sA, const float* sB, const float* sOut,
                       void* C, int out_dtype, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
    return gemm_fp8_common(A, GEMM_FMT_E4M3, Bt, GEMM_FMT_E4M3, sA, sB, sOut, C, out_dtype, M, N, K, stream, 0,
                           nullptr, 0, 1);
}

int gemm_fp8_fmt_bt(const uint8_t* A, int fmt_a, const uint8_t* Bt, int fmt_b, const float* sA, const float* sB,
                    const float* sOut, void* C, int out_dtype, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
    return gemm_fp8_common(A, fmt_a, Bt, fmt_b, sA, sB, sOut, C, out_dtype, M, N, K, stream, 0, nullptr, 0, 1);
}

int gemm_fp8_fmt(const uint8_t* A, int fmt_a, const uint8_t* B, int fmt_b, const float* sA, const float* sB,
                 const float* sOut, void* C, int out_dtype, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
    return gemm_fp8_common(A, fmt_a, B, fmt_b, sA, sB, sOut, C, out_dtype, M, N, K, stream);
}

int gemm_fp8_exact(const uint8_t* A, int fmt_a, const uint8_t* B, int fmt_b, const float* sA, const float* sB,
                   const float* sOut, void* C, int out_dtype, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
    return gemm_fp8_common(A, fmt_a, B, fmt_b, sA, sB, sOut, C, out_dtype, M, N, K, stream, 0, nullptr, 0, 0, 1);
}

int gemm_fp8_exact_bt(const uint8_t* A, int fmt_a, const uint8_t* Bt, int fmt_b, const float* sA, const float* sB,
                      const float* sOut, void* C, int out_dtype, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
    return gemm_fp8_common(A, fmt_a, Bt, fmt_b, sA, sB, sOut, C, out_dtype, M, N, K, stream, 0, nullptr, 0, 1, 1);
}

int gemm_select_config_exact(int out_dtype, int64_t M, int64_t N, int64_t K, int fmt_a, int fmt_b, int b_kmajor,
                             char* buf, int buflen) {
    if (out_dtype < GEMM_OUT_F32 || out_dtype > GEMM_OUT_E5M2) return GEMM_ERR_DTYPE;
    if ((fmt_a != GEMM_FMT_E4M3 && fmt_a != GEMM_FMT_E5M2) || (fmt_b != GEMM_FMT_E4M3 && fmt_b != GEMM_FMT_E5M2))
        return GEMM_ERR_DTYPE;
    if (!gemm_sizes_ok(M, N, K, 1, 1, 4)) return GEMM_ERR_DIM;
    if (!buf || buflen <= 0) return GEMM_ERR_NULL;
    const GemmConfig* cfg = select_config_exact(out_dtype, M, N, K, fmt_a, fmt_b, b_kmajor ? 1 : 0);
    if (!cfg) return GEMM_ERR_UNSUPPORTED;
    std::snprintf(buf, (size_t)buflen, "%s", cfg->name);
    return GEMM_OK;
}

int gemm_fp8_splitk(const uint8_t* A, int fmt_a, const uint8_t* B, int fmt_b, const float* sA, const float* sB,
                    const float* sOut, void* C, int out_dtype, int64_t M, int64_t N, int64_t K, void* workspace,
                    int64_t workspace_bytes, hipStream_t stream) {
    return gemm_fp8_common(A, fmt_a, B, fmt_b, sA, sB, sOut, C, out_dtype, M, N, K, stream, 0, workspace,
                           workspace_bytes);
}

int gemm_fp8_splitk_bt(const uint8_t* A, const uint8_t* Bt, const float* sA, const float* sB, const float* sOut,
                       void* C, int out_dtype, int64_t M, int64_t N, int64_t K, void* workspace,
                       int64_t workspace_bytes, hipStream_t stream) {
    return gemm_fp8_common(A, GEMM_FMT_E4M3, Bt, GEMM_FMT_E4M3, sA, sB, sOut, C, out_dtype, M, N, K, stream, 0,
                           workspace, workspace_bytes, 1);
}

// gemm_f16_splitk and gemm_f16_splitk_bt.
static int gemm_f16_splitk_common(const void* A, const void* B, void* C, int out_dtype, int64_t M, int64_t N,
                                  int64_t K, void* workspace, int64_t workspace_bytes, hipStream_t stream,
                                  int b_kmajor) {
    if (out_dtype != GEMM_OUT_F32 && out_dtype != GEMM_OUT_F16) return GEMM_ERR_DTYPE;
    if (!gemm_sizes_ok(M, N, K, 2, 2, out_size(out_dtype))) return GEMM_ERR_DIM;
    if (M > 0 && N > 0) {
        if (!C) return GEMM_ERR_NULL;
        if (K > 0 && (!A || !B)) return GEMM_ERR_NULL;
        const int64_t cbytes = M * N * out_size(out_dtype);
        if (K > 0 && (overlaps(C, cbytes, A, M * K * 2) || overlaps(C, cbytes, B, K * N * 2))) return GEMM_ERR_ALIAS;
    }
    GemmArgs a{A, B, C, nullptr, nullptr, nullptr, out_dtype, M, N, K, stream};
    a.b_kmajor = b_kmajor;
    const void* in_ptr[3] = {A, B, C};
    const int64_t in_bytes[3] = {M * K * 2, K * N * 2, M * N * out_size(out_dtype)};
    return run_gemm_splitk(KIND_F16, a, workspace, workspace_bytes, in_ptr, in_bytes, 3);
}

int gemm_f16_splitk(const void* A, const void* B, void* C, int out_dtype, int64_t M, int64_t N, int64_t K,
                    void* workspace, int64_t workspace_bytes, hipStream_t stream) {
    return gemm_f16_splitk_common(A, B, C, out_dtype, M, N, K, workspace, workspace_bytes, stream, 0);
}

int gemm_f16_splitk_bt(const void* A, const void* Bt, void* C, int out_dtype, int64_t M, int64_t N, int64_t K,
                       void* workspace, int64_t workspace_bytes, hipStream_t stream) {
    return gemm_f16_splitk_common(A, Bt, C, out_dtype, M, N, K, workspace, workspace_bytes, stream, 1);
}

// Workspace of gemm_f16_guarded: 256 bytes of scalars (amax of A and B, s,
// sqrt(s), 1/s), then the scaled FP16 copies of A and of B, each starting on
// a 256-byte boundary.
static int64_t round256(int64_t b) { return (b + 255) / 256 * 256; }
static int64_t guard_ws_a16(int64_t, int64_t, int64_t) { return 256; }
static int64_t guard_ws_b16(int64_t M, int64_t, int64_t K) { return 256 + round256(M * K * 2); }

int64_t gemm_f16_guarded_workspace_size(int64_t M, int64_t N, int64_t K) {
    if (!gemm_sizes_ok(M, N, K, 4, 4, 4)) return GEMM_ERR_DIM;
    return guard_ws_b16(M, N, K) + round256(K * N * 2);
}

int gemm_f16_guarded(const float* A, const float* B, void* C, int out_dtype, int64_t M, int64_t N, int64_t K,
                     float* scale, void* workspace, int64_t workspace_bytes, hipStream_t stream) {
    if (out_dtype != GEMM_OUT_F32 && out_dtype != GEMM_OUT_F16) return GEMM_ERR_DTYPE;
    if (!gemm_sizes_ok(M, N, K, 4, 4, 4)) return GEMM_ERR_DIM;
    if (M == 0 || N == 0) return GEMM_OK;
    if (!C || !workspace) return GEMM_ERR_NULL;
    if (K > 0 && (!A || !B)) return GEMM_ERR_NULL;
    const int64_t need = gemm_f16_guarded_workspace_size(M, N, K);
    if (workspace_bytes < need || ((uintptr_t)workspace & 15u) != 0) return GEMM_ERR_WORKSPACE;
    const int64_t cbytes = M * N * out_size(out_dtype);
    const void* in_ptr[3] = {A, B, scale};
    const int64_t in_bytes[3] = {M * K * 4, K * N * 4, 4};
    for (int i = 0; i < 3; ++i)
        if (overlaps(C, cbytes, in_ptr[i], in_bytes[i]) || overlaps(workspace, need, in_ptr[i], in_bytes[i]))
            return GEMM_ERR_ALIAS;
    if (overlaps(workspace, need, C, cbytes) || overlaps(scale, 4, A, M * K * 4) || overlaps(scale, 4, B, K * N * 4))
        return GEMM_ERR_ALIAS;
    const int st = check_device();
    if (st != GEMM_OK) return st;
    uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
    float* amax_a = reinterpret_cast<float*>(ws);
    float* amax_b = amax_a + 1;
    float* scalars = amax_a + 2;   // s, sqrt(s), 1/s
    _Float16* a16 = reinterpret_cast<_Float16*>(ws + guard_ws_a16(M, N, K));
    _Float16* b16 = reinterpret_cast<_Float16*>(ws + guard_ws_b16(M, N, K));
    int s1 = status_of(launch_amax(A, M * K, amax_a, nullptr, GEMM_FMT_E4M3, 0, stream));
    if (s1 == GEMM_OK) s1 = status_of(launch_amax(B, K * N, amax_b, nullptr, GEMM_FMT_E4M3, 0, stream));
    if (s1 == GEMM_OK) s1 = status_of(launch_guard_scale(amax_a, amax_b, scalars, scale, stream));
    if (s1 == GEMM_OK) s1 = status_of(launch_guard_to_f16(A, M * K, scalars, a16, stream));
    if (s1 == GEMM_OK) s1 = status_of(launch_guard_to_f16(B, K * N, scalars, b16, stream));
    if (s1 != GEMM_OK) return s1;
    // The FP16 GEMM; its epilogue multiplies the FP32 sum by *sA = 1/s.
    GemmArgs a{a16, b16, C, scalars + 2, nullptr, nullptr, out_dtype, M, N, K, stream};
    return run_gemm(KIND_F16, a);
}

// gemm_splitk_plan and gemm_splitk_plan_bt.
static int splitk_plan_common(int kind, int out_dtype, int64_t M, int64_t N, int64_t K, int fmt_a, int fmt_b,
                              char* buf, int buflen, int* splits, int64_t* workspace_bytes, int b_kmajor) {
    if (kind != KIND_F16 && kind != KIND_FP8) return GEMM_ERR_DTYPE;
    if (out_dtype < GEMM_OUT_F32 || out_dtype > GEMM_OUT_E5M2 || (kind == KIND_F16 && fp8_out(out_dtype)))
        return GEMM_ERR_DTYPE;
    if ((fmt_a != GEMM_FMT_E4M3 && fmt_a != GEMM_FMT_E5M2) || (fmt_b != GEMM_FMT_E4M3 && fmt_b != GEMM_FMT_E5M2))
        return GEMM_ERR_DTYPE;
    if (!gemm_sizes_ok(M, N, K, 2, 2, 4)) return GEMM_ERR_DIM;
    const SplitPlan p = plan_splitk(kind, out_dtype, M, N, K, fmt_a, fmt_b, b_kmajor);
    if (!p.cfg) return GEMM_ERR_UNSUPPORTED;
    if (buf && buflen > 0) {
        std::strncpy(buf, p.cfg->name, (size_t)buflen - 1);
        buf[buflen - 1] = '\0';
    }
    if (splits) *splits = p.splits;
    if (workspace_bytes) *workspace_bytes = splitk_bytes(p, M, N);
    return GEMM_OK;
}

int gemm_splitk_plan(int kind, int out_dtype, int64_t M, int64_t N, int64_t K, int fmt_a, int fmt_b, char* buf,
                     int buflen, int* splits, int64_t* workspace_bytes) {
    return splitk_plan_common(kind, out_dtype, M, N, K, fmt_a, fmt_b, buf, buflen, splits, workspace_bytes, 0);
}

int gemm_splitk_plan_bt(int kind, int out_dtype, int64_t M, int64_t N, int64_t K, char* buf, int buflen, int* splits,
                        int64_t* workspace_bytes) {
    return splitk_plan_common(kind, out_dtype, M, N, K, GEMM_FMT_E4M3, GEMM_FMT_E4M3, buf, buflen, splits,
                              workspace_bytes, 1);
}

int gemm_fp8_channel(const uint8_t* A, int fmt_a, const uint8_t* B, int fmt_b, const float* sA, const float* sB,
                     const float* sOut, void* C, int out_dtype, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
    return gemm_fp8_common(A, fmt_a, B, fmt_b, sA, sB, sOut, C, out_dtype, M, N, K, stream, 1);
}

int amax_scale_channel_f32(const float* x, int64_t rows, int64_t cols, int axis, float* amax, float* scale, int fmt,
                           int pow2, hipStream_t stream) {
    if (fmt != GEMM_FMT_E4M3 && fmt != GEMM_FMT_E5M2) return GEMM_ERR_DTYPE;
    if (axis != GEMM_AXIS_ROW && axis != GEMM_AXIS_COL) return GEMM_ERR_DIM;
    if (!dim_ok(rows) || !dim_ok(cols) || !bytes_ok(rows, cols, 4)) return GEMM_ERR_DIM;
    const int64_t nch = axis == GEMM_AXIS_ROW ? rows : cols;
    if (nch == 0) return GEMM_OK;
    if (!amax) return GEMM_ERR_NULL;
    const int64_t xbytes = 4 * rows * cols;
    if (xbytes > 0 && !x) return GEMM_ERR_NULL;
    if (overlaps(amax, 4 * nch, x, xbytes) || overlaps(scale, 4 * nch, x, xbytes) ||
        overlaps(amax, 4 * nch, scale, 4 * nch))
        return GEMM_ERR_ALIAS;
    const int st = check_device();
    if (st != GEMM_OK) return st;
    return status_of(launch_amax_channel(x, rows, cols, axis, amax, scale, fmt, pow2 ? 1 : 0, stream));
}

int quantize_fp8_channel(const float* x, int64_t rows, int64_t cols, int axis, const float* scale, uint8_t* q,
                         int fmt, hipStream_t stream) {
    if (fmt != GEMM_FMT_E4M3 && fmt != GEMM_FMT_E5M2) return GEMM_ERR_DTYPE;
    if (axis != GEMM_AXIS_ROW && axis != GEMM_AXIS_COL) return GEMM_ERR_DIM;
    if (!dim_ok(rows) || !dim_ok(cols) || !bytes_ok(rows, cols, 4)) return GEMM_ERR_DIM;
    const int64_t n = rows * cols;
    if (n == 0) return GEMM_OK;
    if (!x || !scale || !q) return GEMM_ERR_NULL;
    const int64_t nch = axis == GEMM_AXIS_ROW ? rows : cols;
    if (overlaps(q, n, x, 4 * n) || overlaps(q, n, scale, 4 * nch)) return GEMM_ERR_ALIAS;
    const int st = check_device();
    if (st != GEMM_OK) return st;
    return status_of(launch_quantize_channel(x, rows, cols, axis, scale, q, fmt, stream));
}

int quantize_fp8_fmt(const float* x, int64_t n, const float* scale, uint8_t* q, int fmt, hipStream_t stream) {
    if (fmt != GEMM_FMT_E4M3 && fmt != GEMM_FMT_E5M2) return GEMM_ERR_DTYPE;
    if (!bytes_ok(n, 1, 4)) return GEMM_ERR_DIM;
    if (n == 0) return GEMM_OK;
    if (!x || !scale || !q) return GEMM_ERR_NULL;
    if (overlaps(q, n, x, 4 * n) || overlaps(q, n, scale, 4)) return GEMM_ERR_ALIAS;
    const int st = check_device();
    if (st != GEMM_OK) return st;
    return status_of(launch_quantize(x, n, scale, q, fmt, stream));
}

int quantize_fp8_transposed_fmt(const float* x, int64_t rows, int64_t cols, const float* scale, uint8_t* q,
                                int fmt, hipStream_t stream) {
    if (fmt != GEMM_FMT_E4M3 && fmt != GEMM_FMT_E5M2) return GEMM_ERR_DTYPE;
    if (!dim_ok(rows) || !dim_ok(cols) || !bytes_ok(rows, cols, 4)) return GEMM_ERR_DIM;
    const int64_t n = rows * cols;
    if (n == 0) return GEMM_OK;
    if (!x || !scale || !q) return GEMM_ERR_NULL;
    if (overlaps(q, n, x, 4 * n) || overlaps(q, n, scale, 4)) return GEMM_ERR_ALIAS;
    const int st = check_device();
    if (st != GEMM_OK) return st;
    return status_of(launch_quantize_transposed(x, rows, cols, scale, q, fmt, stream));
}

int quantize_fp8_transposed(const float* x, int64_t rows, int64_t cols, const float* scale, uint8_t* q,
                            hipStream_t stream) {
    return quantize_fp8_transposed_fmt(x, rows, cols, scale, q, GEMM_FMT_E4M3, stream);
}

int pack_b_kmajor(const void* B, int64_t K, int64_t N, int elem_bytes, void* Bt, hipStream_t stream) {
    if (elem_bytes != 1 && elem_bytes != 2) return GEMM_ERR_DTYPE;
    if (!dim_ok(K) || !dim_ok(N) || !bytes_ok(K, N, elem_bytes)) return GEMM_ERR_DIM;
    const int64_t bytes = K * N * elem_bytes;
    if (bytes == 0) return GEMM_OK;
    if (!B || !Bt) return GEMM_ERR_NULL;
    if (overlaps(Bt, bytes, B, bytes)) return GEMM_ERR_ALIAS;
    const int st = check_device();
    if (st != GEMM_OK) return st;
    return status_of(launch_transpose(B, K, N, elem_bytes, Bt, stream));
}

int quantize_fp8(const float* x, int64_t n, const float* scale, uint8_t* q, hipStream_t stream) {
    return quantize_fp8_fmt(x, n, scale, q, GEMM_FMT_E4M3, stream);
}

int amax_scale_f32(const float* x, int64_t n, float* amax, float* scale, int fmt, int pow2, hipStream_t stream) {
    if (fmt != GEMM_FMT_E4M3 && fmt != GEMM_FMT_E5M2) return GEMM_ERR_DTYPE;
    if (!bytes_ok(n, 1, 4)) return GEMM_ERR_DIM;
    if (!amax) return GEMM_ERR_NULL;
    if (n > 0 && !x) return GEMM_ERR_NULL;
    if (overlaps(amax, 4, x, 4 * n) || overlaps(scale, 4, x, 4 * n) || overlaps(amax, 4, scale, 4))
        return GEMM_ERR_ALIAS;
    const int st = check_device();
    if (st != GEMM_OK) return st;
    return status_of(launch_amax(x, n, amax, scale, fmt, pow2 ? 1 : 0, stream));
}

int64_t amax_quantize_fp8_pair_workspace_size(void) { return (int64_t)kPairSlots * 4; }

int amax_quantize_fp8_pair(const float* A, int64_t na, const float* B, int64_t nb, int fmt, int pow2, float* amax,
                           float* scale, uint8_t* qa, uint8_t* qb, void* workspace, int64_t workspace_bytes,
                           hipStream_t stream) {
    if (fmt != GEMM_FMT_E4M3 && fmt != GEMM_FMT_E5M2) return GEMM_ERR_DTYPE;
    if (!bytes_ok(na, 1, 4) || !bytes_ok(nb, 1, 4)) return GEMM_ERR_DIM;
    if (!amax || !scale || !workspace) return GEMM_ERR_NULL;
    if ((na > 0 && (!A || !qa)) || (nb > 0 && (!B || !qb))) return GEMM_ERR_NULL;
    const int64_t ws_need = amax_quantize_fp8_pair_workspace_size();
    if (workspace_bytes < ws_need || ((uintptr_t)workspace & 15u) != 0) return GEMM_ERR_WORKSPACE;
    const int64_t sb = nb > 0 ? 8 : 4;  // bytes of amax and of scale
    // every written range against every other range
    const void* w_ptr[5] = {amax, scale, workspace, qa, qb};
    const int64_t w_bytes[5] = {sb, sb, ws_need, na, nb};
    const void* r_ptr[2] = {A, B};
    const int64_t r_bytes[2] = {4 * na, 4 * nb};
    for (int i = 0; i < 5; ++i) {
        for (int j = 0; j < 2; ++j)
            if (overlaps(w_ptr[i], w_bytes[i], r_ptr[j], r_bytes[j])) return GEMM_ERR_ALIAS;
        for (int j = i + 1; j < 5; ++j)
            if (overlaps(w_ptr[i], w_bytes[i], w_ptr[j], w_bytes[j])) return GEMM_ERR_ALIAS;
    }
    const int st = check_device();
    if (st != GEMM_OK) return st;
    return status_of(launch_amax_quantize_pair(A, na, B, nb, fmt, pow2 ? 1 : 0, amax, scale, qa, qb,
                                               reinterpret_cast<uint32_t*>(workspace), stream));
}

int amax_quantize_fp8_pair_bt(const float* A, int64_t na, const float* B, int64_t K, int64_t N, int fmt, int pow2,
                              float* amax, float* scale, uint8_t* qa, uint8_t* qbt, void* workspace,
                              int64_t workspace_bytes, hipStream_t stream) {
    if (fmt != GEMM_FMT_E4M3 && fmt != GEMM_FMT_E5M2) return GEMM_ERR_DTYPE;
    if (!dim_ok(K) || !dim_ok(N) || !bytes_ok(na, 1, 4) || !bytes_ok(K, N, 4)) return GEMM_ERR_DIM;
    const int64_t nb = K * N;
    if (!amax || !scale || !workspace) return GEMM_ERR_NULL;
    if ((na > 0 && (!A || !qa)) || (nb > 0 && (!B || !qbt))) return GEMM_ERR_NULL;
    const int64_t ws_need = amax_quantize_fp8_pair_workspace_size();
    if (workspace_bytes < ws_need || ((uintptr_t)workspace & 15u) != 0) return GEMM_ERR_WORKSPACE;
    const int64_t sb = nb > 0 ? 8 : 4;  // bytes of amax and of scale
    const void* w_ptr[5] = {amax, scale, workspace, qa, qbt};
    const int64_t w_bytes[5] = {sb, sb, ws_need, na, nb};
    const void* r_ptr[2] = {A, B};
    const int64_t r_bytes[2] = {4 * na, 4 * nb};
    for (int i = 0; i < 5; ++i) {
        for (int j = 0; j < 2; ++j)
            if (overlaps(w_ptr[i], w_bytes[i], r_ptr[j], r_bytes[j])) return GEMM_ERR_ALIAS;
        for (int j = i + 1; j < 5; ++j)
            if (overlaps(w_ptr[i], w_bytes[i], w_ptr[j], w_bytes[j])) return GEMM_ERR_ALIAS;
    }
    const int st = check_device();
    if (st != GEMM_OK) return st;
    return status_of(launch_amax_quantize_pair_bt(A, na, B, K, N, fmt, pow2 ? 1 : 0, amax, scale, qa, qbt,
                                                  reinterpret_cast<uint32_t*>(workspace), stream));
}

int amax_f32(const float* x, int64_t n, float* amax, float* scale, hipStream_t stream) {
    return amax_scale_f32(x, n, amax, scale, GEMM_FMT_E4M3, 0, stream);
}

const char* gemm_status_str(int status) {
    switch (status) {
        case GEMM_OK: return "ok";
        case GEMM_ERR_NULL: return "a required pointer is NULL";
        case GEMM_ERR_DIM: return "a dimension is negative or above 2^31-1, or an operand spans 2^62 bytes or more";
        case GEMM_ERR_DTYPE: return "unsupported output dtype";
        case GEMM_ERR_SCALE: return "sOut is required for FP8 output";
        case GEMM_ERR_LAUNCH: return "kernel launch failed";
        case GEMM_ERR_UNSUPPORTED: return "no kernel for this request";
        case GEMM_ERR_DEVICE: return "no current HIP device, or it is not gfx950";
        case GEMM_ERR_ALIAS: return "output overlaps an input";
        case GEMM_ERR_WORKSPACE: return "workspace too small or not 16-byte aligned";
        default: return "unknown status";
    }
}

int gemm_select_config_fmt(int kind, int out_dtype, int64_t M, int64_t N, int64_t K, int fmt_a, int fmt_b,
                           char* buf, int buflen) {
    if (kind != KIND_F16 && kind != KIND_FP8) return GEMM_ERR_DTYPE;
    if (out_dtype < GEMM_OUT_F32 || out_dtype > GEMM_OUT_E5M2 || (kind == KIND_F16 && fp8_out(out_dtype)))
        return GEMM_ERR_DTYPE;
    if ((fmt_a != GEMM_FMT_E4M3 && fmt_a != GEMM_FMT_E5M2) || (fmt_b != GEMM_FMT_E4M3 && fmt_b != GEMM_FMT_E5M2))
        return GEMM_ERR_DTYPE;
    if (!gemm_sizes_ok(M, N, K, 2, 2, 4)) return GEMM_ERR_DIM;
    if (!buf || buflen <= 0) return GEMM_ERR_NULL;
    const GemmConfig* cfg = select_config(kind, out_dtype, M, N, K, fmt_a, fmt_b);
    if (!cfg) return GEMM_ERR_UNSUPPORTED;
    std::snprintf(buf, (size_t)buflen, "%s", cfg->name);
    return GEMM_OK;
}

int gemm_select_config_bt(int kind, int out_dtype, int64_t M, int64_t N, int64_t K, char* buf, int buflen) {
    if (kind != KIND_F16 && kind != KIND_FP8) return GEMM_ERR_DTYPE;
    if (out_dtype < GEMM_OUT_F32 || out_dtype > GEMM_OUT_E5M2 || (kind == KIND_F16 && fp8_out(out_dtype)))
        return GEMM_ERR_DTYPE;
    if (!gemm_sizes_ok(M, N, K, 2, 2, 4)) return GEMM_ERR_DIM;
    if (!buf || buflen <= 0) return GEMM_ERR_NULL;
    const GemmConfig* cfg = select_config(kind, out_dtype, M, N, K, GEMM_FMT_E4M3, GEMM_FMT_E4M3, 1);
    if (!cfg) return GEMM_ERR_UNSUPPORTED;
    std::snprintf(buf, (size_t)buflen, "%s", cfg->name);
    return GEMM_OK;
}

int gemm_select_config(int kind, int out_dtype, int64_t M, int64_t N, int64_t K, char* buf, int buflen) {
    return gemm_select_config_fmt(kind, out_dtype, M, N, K, GEMM_FMT_E4M3, GEMM_FMT_E4M3, buf, buflen);
}

}  // extern "C"
