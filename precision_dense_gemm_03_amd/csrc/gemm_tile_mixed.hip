// The FP8 operand-format pairs other than E4M3 x E4M3 (E4M3 x E5M2, E5M2 x
// E4M3, E5M2 x E5M2) of the register-staged tile kernel, compiled apart from
// gemm_tile.hip so that the two translation units build in parallel.
#include "gemm_tile_impl.h"

namespace libgemm {
namespace tile {
#define LIBGEMM_TILE_INSTANTIATE(BM, BN, BK, WM, WN, BT)                             \
    template hipError_t launch_tile<1, BM, BN, BK, WM, WN, 0, 1, BT>(const GemmArgs&); \
    template hipError_t launch_tile<1, BM, BN, BK, WM, WN, 1, 0, BT>(const GemmArgs&); \
    template hipError_t launch_tile<1, BM, BN, BK, WM, WN, 1, 1, BT>(const GemmArgs&);
LIBGEMM_TILE_MIXED_CONFIGS(LIBGEMM_TILE_INSTANTIATE)
#undef LIBGEMM_TILE_INSTANTIATE
}  // namespace tile
}  // namespace libgemm
