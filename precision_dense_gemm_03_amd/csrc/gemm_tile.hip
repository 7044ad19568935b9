// MFMA tile GEMM for gfx950 (register-staged loads): the configuration table
// and the E4M3 x E4M3 and FP16 instantiations. The kernel itself, its data
// flow and its citations are in gemm_tile_impl.h.
#include "gemm_tile_impl.h"

namespace libgemm {
namespace tile {
// The other FP8 operand pairs are compiled in gemm_tile_mixed.hip.
#define LIBGEMM_TILE_EXTERN(BM, BN, BK, WM, WN, BT)                                         \
    extern template hipError_t launch_tile<1, BM, BN, BK, WM, WN, 0, 1, BT>(const GemmArgs&); \
    extern template hipError_t launch_tile<1, BM, BN, BK, WM, WN, 1, 0, BT>(const GemmArgs&); \
    extern template hipError_t launch_tile<1, BM, BN, BK, WM, WN, 1, 1, BT>(const GemmArgs&);
LIBGEMM_TILE_MIXED_CONFIGS(LIBGEMM_TILE_EXTERN)
#undef LIBGEMM_TILE_EXTERN
}  // namespace tile

// The table lives in a host function so that the kernels it names are
// instantiated for the device while the table itself stays host data.
const GemmConfig* tile_configs(int* count) {
    static const GemmConfig table[] = {
        {"tile_f16_64x64x64_w2x2", KIND_F16, 0, 64, 64, 64, tile::launch_tile<2, 64, 64, 64, 2, 2, 0, 0>, 0, 64},
        {"tile_f16_128x128x64_w2x2", KIND_F16, 0, 128, 128, 64, tile::launch_tile<2, 128, 128, 64, 2, 2, 0, 0>, 0, 64},
        {"tile_fp8_64x64x128_w2x2", KIND_FP8, 0, 64, 64, 128, tile::launch_tile_fp8_any<64, 64, 128, 2, 2>, kAllFp8Pairs, 128},
        {"tile_fp8_128x128x128_w2x2", KIND_FP8, 0, 128, 128, 128, tile::launch_tile_fp8_any<128, 128, 128, 2, 2>, kAllFp8Pairs, 128},
        {"tile_fp8_256x256x128_w2x4", KIND_FP8, 0, 256, 256, 128, tile::launch_tile_fp8_any<256, 256, 128, 2, 4>, kAllFp8Pairs, 128},
        {"tile_f16_256x256x64_w2x4", KIND_F16, 0, 256, 256, 64, tile::launch_tile<2, 256, 256, 64, 2, 4, 0, 0>, 0, 64},
        // K-major B (Bt[N,K]): B staged and read like A; every FP8 operand pair, and FP16.
        {"tile_f16_64x64x64_w2x2_bt", KIND_F16, 0, 64, 64, 64, tile::launch_tile<2, 64, 64, 64, 2, 2, 0, 0, true>, 0, 64, 1},
        {"tile_f16_128x128x64_w2x2_bt", KIND_F16, 0, 128, 128, 64, tile::launch_tile<2, 128, 128, 64, 2, 2, 0, 0, true>, 0, 64, 1},
        {"tile_f16_256x256x64_w2x4_bt", KIND_F16, 0, 256, 256, 64, tile::launch_tile<2, 256, 256, 64, 2, 4, 0, 0, true>, 0, 64, 1},
        {"tile_fp8_64x64x128_w2x2_bt", KIND_FP8, 0, 64, 64, 128, tile::launch_tile_fp8_any<64, 64, 128, 2, 2, true>, kAllFp8Pairs, 128, 1},
        {"tile_fp8_128x128x128_w2x2_bt", KIND_FP8, 0, 128, 128, 128, tile::launch_tile_fp8_any<128, 128, 128, 2, 2, true>, kAllFp8Pairs, 128, 1},
        {"tile_fp8_256x256x128_w2x4_bt", KIND_FP8, 0, 256, 256, 128, tile::launch_tile_fp8_any<256, 256, 128, 2, 4, true>, kAllFp8Pairs, 128, 1},
    };
    *count = (int)(sizeof(table) / sizeof(table[0]));
    return table;
}

// The exact-accumulation FP8 mode (family 5): FP8 codes widened to FP16 as
// they are staged, FP16 matrix cores, every FP8 operand pair (formats read at
// run time). Never chosen by the plain selector; select_config_exact does.
const GemmConfig* exact_configs(int* count) {
    static const GemmConfig table[] = {
        // 256x256: the ping-pong kernel with FP16 matrix cores (listed first,
        // so the selector's 256 rule takes it), then the register-staged kernels
        {"exact_pp_fp8_256x256x64", KIND_FP8, 5, 256, 256, 64, launch_pp_exact_rm, kAllFp8Pairs},
        {"exact_pp_fp8_256x256x64_bt", KIND_FP8, 5, 256, 256, 64, launch_pp_exact_bt, kAllFp8Pairs, 0, 1},
        {"exact_fp8_64x64x64_w2x2", KIND_FP8, 5, 64, 64, 64, tile::launch_tile_fp8_exact<64, 64, 64, 2, 2>, kAllFp8Pairs},
        {"exact_fp8_128x128x64_w2x2", KIND_FP8, 5, 128, 128, 64, tile::launch_tile_fp8_exact<128, 128, 64, 2, 2>, kAllFp8Pairs},
        {"exact_fp8_256x256x64_w2x4", KIND_FP8, 5, 256, 256, 64, tile::launch_tile_fp8_exact<256, 256, 64, 2, 4>, kAllFp8Pairs},
        {"exact_fp8_64x64x64_w2x2_bt", KIND_FP8, 5, 64, 64, 64, tile::launch_tile_fp8_exact<64, 64, 64, 2, 2, true>, kAllFp8Pairs, 0, 1},
        {"exact_fp8_128x128x64_w2x2_bt", KIND_FP8, 5, 128, 128, 64, tile::launch_tile_fp8_exact<128, 128, 64, 2, 2, true>, kAllFp8Pairs, 0, 1},
        {"exact_fp8_256x256x64_w2x4_bt", KIND_FP8, 5, 256, 256, 64, tile::launch_tile_fp8_exact<256, 256, 64, 2, 4, true>, kAllFp8Pairs, 0, 1},
    };
    *count = (int)(sizeof(table) / sizeof(table[0]));
    return table;
}

}  // namespace libgemm
