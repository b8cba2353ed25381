// Forward instantiation: element type float, head dimension 64, rank blocks 8.
#include "prf_kernels.cuh"

namespace dk {
dark_status fwd_f32_d64_r8(const FwdArgs& a, const Plan& p, void* ws, void* s) {
  return launch_fwd_impl<float, 64, 8, 2>(a, p, ws, s);
}
dark_status exact_f32_d64_r8(const FwdArgs& a, void* ws, void* s) {
  return launch_exact_impl<float, 64, 8>(a, ws, s);
}
}  // namespace dk
