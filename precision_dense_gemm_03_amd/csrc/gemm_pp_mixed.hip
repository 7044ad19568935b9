// Ping-pong MFMA tile GEMM: the FP8 operand pairs other than E4M3 x E4M3
// (compiled in their own translation unit so the build runs in parallel).
#include "gemm_pp_impl.h"

namespace libgemm {
namespace pp {
template hipError_t launch_pp<1, 0, 1, false>(const GemmArgs&);
template hipError_t launch_pp<1, 1, 0, false>(const GemmArgs&);
template hipError_t launch_pp<1, 1, 1, false>(const GemmArgs&);
template hipError_t launch_pp<1, 0, 1, true>(const GemmArgs&);
template hipError_t launch_pp<1, 1, 0, true>(const GemmArgs&);
template hipError_t launch_pp<1, 1, 1, true>(const GemmArgs&);
template hipError_t launch_pp<1, 0, 1, false, false, 192>(const GemmArgs&);
template hipError_t launch_pp<1, 1, 0, false, false, 192>(const GemmArgs&);
template hipError_t launch_pp<1, 1, 1, false, false, 192>(const GemmArgs&);
template hipError_t launch_pp<1, 0, 1, true, false, 192>(const GemmArgs&);
template hipError_t launch_pp<1, 1, 0, true, false, 192>(const GemmArgs&);
template hipError_t launch_pp<1, 1, 1, true, false, 192>(const GemmArgs&);
}  // namespace pp
}  // namespace libgemm
