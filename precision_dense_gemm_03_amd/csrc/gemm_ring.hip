// Deep-ring MFMA tile GEMM for skinny shapes: the configuration table and the
// E4M3 x E4M3 and FP16 instantiations. The kernel, its data flow and its
// citations are in gemm_ring_impl.h.
#include "gemm_ring_impl.h"

namespace libgemm {
namespace ring {
// The other FP8 operand pairs: gemm_ring_mixed.hip.
#define LIBGEMM_RING_EXTERN(BM, BN, BT)                                          \
    extern template hipError_t launch_ring<1, BM, BN, 0, 1, BT>(const GemmArgs&); \
    extern template hipError_t launch_ring<1, BM, BN, 1, 0, BT>(const GemmArgs&); \
    extern template hipError_t launch_ring<1, BM, BN, 1, 1, BT>(const GemmArgs&);
LIBGEMM_RING_CONFIGS(LIBGEMM_RING_EXTERN)
#undef LIBGEMM_RING_EXTERN
}  // namespace ring

#define RING_FP8(BM, BN, BT, SUF)                                                                               \
    {"ring_fp8_" #BM "x" #BN "x128" SUF, KIND_FP8, 6, BM, BN, 128, ring::launch_ring_fp8_any<BM, BN, BT>, \
     kAllFp8Pairs, 0, BT}
#define RING_F16(BM, BN, BT, SUF) \
    {"ring_f16_" #BM "x" #BN "x64" SUF, KIND_F16, 6, BM, BN, 64, ring::launch_ring<2, BM, BN, 0, 0, BT>, 0, 0, BT}

// family 6; bm x bn = output tile, bk = K values per LDS stage
const GemmConfig* ring_configs(int* count) {
    static const GemmConfig table[] = {
        RING_FP8(16, 16, 0, ""),    RING_FP8(16, 32, 0, ""),    RING_FP8(16, 64, 0, ""),    RING_FP8(32, 32, 0, ""),
        RING_FP8(32, 64, 0, ""),    RING_FP8(64, 64, 0, ""),    RING_F16(16, 16, 0, ""),    RING_F16(16, 32, 0, ""),
        RING_F16(16, 64, 0, ""),    RING_F16(32, 32, 0, ""),    RING_F16(32, 64, 0, ""),    RING_F16(64, 64, 0, ""),
        RING_FP8(16, 16, 1, "_bt"), RING_FP8(16, 32, 1, "_bt"), RING_FP8(16, 64, 1, "_bt"), RING_FP8(32, 32, 1, "_bt"),
        RING_FP8(32, 64, 1, "_bt"), RING_FP8(64, 64, 1, "_bt"), RING_F16(16, 16, 1, "_bt"), RING_F16(16, 32, 1, "_bt"),
        RING_F16(16, 64, 1, "_bt"), RING_F16(32, 32, 1, "_bt"), RING_F16(32, 64, 1, "_bt"), RING_F16(64, 64, 1, "_bt"),
    };
    *count = (int)(sizeof(table) / sizeof(table[0]));
    return table;
}
#undef RING_FP8
#undef RING_F16

}  // namespace libgemm
