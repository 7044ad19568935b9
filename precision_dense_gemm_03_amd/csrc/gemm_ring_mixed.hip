// Deep-ring MFMA tile GEMM: the FP8 operand pairs other than E4M3 x E4M3
// (their own translation unit, so the build runs in parallel).
#include "gemm_ring_impl.h"

namespace libgemm {
namespace ring {
#define LIBGEMM_RING_INST(BM, BN, BT)                                      \
    template hipError_t launch_ring<1, BM, BN, 0, 1, BT>(const GemmArgs&); \
    template hipError_t launch_ring<1, BM, BN, 1, 0, BT>(const GemmArgs&); \
    template hipError_t launch_ring<1, BM, BN, 1, 1, BT>(const GemmArgs&);
LIBGEMM_RING_CONFIGS(LIBGEMM_RING_INST)
#undef LIBGEMM_RING_INST
}  // namespace ring
}  // namespace libgemm
