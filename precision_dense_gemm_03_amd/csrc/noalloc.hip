// gemm_fp8_splitk_noalloc: gemm_fp8_splitk with its FP32 partial sums in a
// fixed device array of this library instead of a caller's workspace, for
// callers that cannot allocate device memory (code under HIP graph capture,
// serving loops, harnesses that forbid hipMalloc).
//
// `scratch` is a file-scope device array; every GPU the library runs on holds
// its own copy, at its own address, until the process ends. Host code never
// uses the array's name as a device address: the first call on a device, with
// that device current, asks the runtime for the copy's address
// (hipGetSymbolAddress) and keeps it per device; kernels receive that
// address. The split-K kernels write every element of the slices they later
// read, so nothing is cleared. Calls that overlap on one GPU share the array
// and race.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <mutex>

#include "libgemm.h"

namespace {

constexpr int64_t kScratchBytes = 16ll << 20;   // 16 MiB: splits * M * N * 4 bytes at most
constexpr int kMaxScratchDevices = 64;

__device__ __align__(256) uint8_t scratch[kScratchBytes];

std::atomic<void*> g_scratch_ptr[kMaxScratchDevices];
std::mutex g_scratch_mu;

// The current device's copy of `scratch`, or nullptr with *status set.
void* scratch_for_current_device(int* status) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) {
        (void)hipGetLastError();
        *status = GEMM_ERR_DEVICE;
        return nullptr;
    }
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p) return p;
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) {
        (void)hipGetLastError();
        *status = GEMM_ERR_DEVICE;
        return nullptr;
    }
    g_scratch_ptr[dev].store(q, std::memory_order_release);
    return q;
}

}  // namespace

extern "C" {

int64_t gemm_fp8_splitk_noalloc_max_bytes(void) { return kScratchBytes; }

int gemm_fp8_splitk_noalloc(const uint8_t* A, int fmt_a, const uint8_t* B, int fmt_b, const float* sA,
                            const float* sB, const float* sOut, void* C, int out_dtype, int64_t M, int64_t N,
                            int64_t K, hipStream_t stream) {
    int splits = 1;
    int64_t need = 0;
    const int st = gemm_splitk_plan(1, out_dtype, M, N, K, fmt_a, fmt_b, nullptr, 0, &splits, &need);
    if (st != GEMM_OK) return st;
    if (need > kScratchBytes) return GEMM_ERR_WORKSPACE;
    if (need == 0)  // the plan does not split: the plain call, no scratch
        return gemm_fp8_splitk(A, fmt_a, B, fmt_b, sA, sB, sOut, C, out_dtype, M, N, K, nullptr, 0, stream);
    int dst = GEMM_OK;
    void* ws = scratch_for_current_device(&dst);
    if (!ws) return dst;
    return gemm_fp8_splitk(A, fmt_a, B, fmt_b, sA, sB, sOut, C, out_dtype, M, N, K, ws, kScratchBytes, stream);
}

}  // extern "C"
