// Ping-pong MFMA tile GEMM for gfx950: the configuration table and the
// E4M3 x E4M3 and FP16 instantiations. The kernel itself, its data flow and
// its citations are in gemm_pp_impl.h.
#include "gemm_pp_impl.h"

namespace libgemm {
namespace pp {
// The other FP8 operand pairs: gemm_pp_mixed.hip.
#define LIBGEMM_PP_EXTERN(BT, BM)                                                \
    extern template hipError_t launch_pp<1, 0, 1, BT, false, BM>(const GemmArgs&); \
    extern template hipError_t launch_pp<1, 1, 0, BT, false, BM>(const GemmArgs&); \
    extern template hipError_t launch_pp<1, 1, 1, BT, false, BM>(const GemmArgs&);
LIBGEMM_PP_EXTERN(false, 256)
LIBGEMM_PP_EXTERN(true, 256)
LIBGEMM_PP_EXTERN(false, 192)
LIBGEMM_PP_EXTERN(true, 192)
#undef LIBGEMM_PP_EXTERN
}  // namespace pp

const GemmConfig* pp_configs(int* count) {
    static const GemmConfig table[] = {
        {"pp_fp8_256x256x64", KIND_FP8, 4, 256, 256, 64, pp::launch_pp_fp8_any<false>, kAllFp8Pairs},
        {"pp_f16_256x256x32", KIND_F16, 4, 256, 256, 32, pp::launch_pp<2, 0, 0, false>},
        {"pp_fp8_256x256x64_bt", KIND_FP8, 4, 256, 256, 64, pp::launch_pp_fp8_any<true>, kAllFp8Pairs, 0, 1},
        {"pp_f16_256x256x32_bt", KIND_F16, 4, 256, 256, 32, pp::launch_pp<2, 0, 0, true>, 0, 0, 1},
        // 192-row tiles: grids whose 256-row tiles leave CUs idle (selector)
        {"pp_fp8_192x256x64", KIND_FP8, 4, 192, 256, 64, pp::launch_pp_fp8_any<false, 192>, kAllFp8Pairs},
        {"pp_f16_192x256x32", KIND_F16, 4, 192, 256, 32, pp::launch_pp<2, 0, 0, false, false, 192>},
        {"pp_fp8_192x256x64_bt", KIND_FP8, 4, 192, 256, 64, pp::launch_pp_fp8_any<true, 192>, kAllFp8Pairs, 0, 1},
        {"pp_f16_192x256x32_bt", KIND_F16, 4, 192, 256, 32, pp::launch_pp<2, 0, 0, true, false, 192>, 0, 0, 1},
    };
    *count = (int)(sizeof(table) / sizeof(table[0]));
    return table;
}

}  // namespace libgemm
