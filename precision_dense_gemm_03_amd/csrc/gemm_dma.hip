// Direct-to-LDS MFMA tile GEMM for gfx950: the configuration table and the
// E4M3 x E4M3 and FP16 instantiations. The kernel itself, its data flow and its
// citations are in gemm_dma_impl.h.
#include "gemm_dma_impl.h"

namespace libgemm {
namespace dma {
// The other FP8 operand pairs of the 4-stage configuration: gemm_dma_mixed.hip.
extern template hipError_t launch_dma<1, 4, 0, 1>(const GemmArgs&);
extern template hipError_t launch_dma<1, 4, 1, 0>(const GemmArgs&);
extern template hipError_t launch_dma<1, 4, 1, 1>(const GemmArgs&);
}  // namespace dma

const GemmConfig* dma_configs(int* count) {
    static const GemmConfig table[] = {
        {"dma_fp8_256x256x64_s4", KIND_FP8, 2, 256, 256, 64, dma::launch_dma_fp8_any<4>, kAllFp8Pairs},
        {"dma_f16_256x256x32_s4", KIND_F16, 2, 256, 256, 32, dma::launch_dma<2, 4, 0, 0>},
        {"dma_fp8_256x256x64_s5", KIND_FP8, 2, 256, 256, 64, dma::launch_dma<1, 5, 0, 0>},
        {"dma_f16_256x256x32_s5", KIND_F16, 2, 256, 256, 32, dma::launch_dma<2, 5, 0, 0>},
        // K-major B (Bt[N,K]), E4M3 x E4M3 and FP16
        {"dma_fp8_256x256x64_s4_bt", KIND_FP8, 2, 256, 256, 64, dma::launch_dma<1, 4, 0, 0, true>, 0, 0, 1},
        {"dma_f16_256x256x32_s4_bt", KIND_F16, 2, 256, 256, 32, dma::launch_dma<2, 4, 0, 0, true>, 0, 0, 1},
    };
    *count = (int)(sizeof(table) / sizeof(table[0]));
    return table;
}

}  // namespace libgemm
