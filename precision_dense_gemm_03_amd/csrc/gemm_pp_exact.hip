// Ping-pong MFMA tile GEMM in exact-accumulation mode (FP8 codes staged as in
// the FP8 kernel, widened to FP16 in registers, FP16 matrix cores): the
// launchers behind exact_configs()' 256x256 entries. The kernel and its
// citations are in gemm_pp_impl.h.
#include "gemm_pp_impl.h"

namespace libgemm {

hipError_t launch_pp_exact_rm(const GemmArgs& a) { return pp::launch_pp_fp8_exact<false>(a); }
hipError_t launch_pp_exact_bt(const GemmArgs& a) { return pp::launch_pp_fp8_exact<true>(a); }

}  // namespace libgemm
