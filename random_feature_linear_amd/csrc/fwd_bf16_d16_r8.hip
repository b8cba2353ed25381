// Forward instantiation: element type bf16, head dimension 16, rank blocks 8.
#include "prf_kernels.cuh"

namespace dk {
dark_status fwd_bf16_d16_r8(const FwdArgs& a, const Plan& p, void* ws, void* s) {
  return launch_fwd_impl<bf16, 16, 8, 2>(a, p, ws, s);
}
dark_status exact_bf16_d16_r8(const FwdArgs& a, void* ws, void* s) {
  return launch_exact_impl<bf16, 16, 8>(a, ws, s);
}
}  // namespace dk
