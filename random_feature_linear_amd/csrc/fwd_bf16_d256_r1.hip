// Forward instantiation: element type bf16, head dimension 256, rank blocks 1.
#include "prf_kernels.cuh"

namespace dk {
dark_status fwd_bf16_d256_r1(const FwdArgs& a, const Plan& p, void* ws, void* s) {
  return launch_fwd_impl<bf16, 256, 1, 1>(a, p, ws, s);
}
dark_status exact_bf16_d256_r1(const FwdArgs& a, void* ws, void* s) {
  return launch_exact_impl<bf16, 256, 1>(a, ws, s);
}
}  // namespace dk
