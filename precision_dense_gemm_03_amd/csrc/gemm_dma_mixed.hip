// The FP8 operand-format pairs other than E4M3 x E4M3 of the 4-stage
// direct-to-LDS kernel, compiled apart from gemm_dma.hip so that the two
// translation units build in parallel.
#include "gemm_dma_impl.h"

namespace libgemm {
namespace dma {
template hipError_t launch_dma<1, 4, 0, 1>(const GemmArgs&);
template hipError_t launch_dma<1, 4, 1, 0>(const GemmArgs&);
template hipError_t launch_dma<1, 4, 1, 1>(const GemmArgs&);
}  // namespace dma
}  // namespace libgemm
