// Forward instantiation: element type float, head dimension 32, rank blocks 16.
#include "prf_kernels.cuh"

namespace dk {
dark_status fwd_f32_d32_r16(const FwdArgs& a, const Plan& p, void* ws, void* s) {
  return launch_fwd_impl<float, 32, 16, 2>(a, p, ws, s);
}
dark_status exact_f32_d32_r16(const FwdArgs& a, void* ws, void* s) {
  return launch_exact_impl<float, 32, 16>(a, ws, s);
}
}  // namespace dk
