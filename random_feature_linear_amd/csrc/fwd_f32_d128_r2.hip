// Forward instantiation: element type float, head dimension 128, rank blocks 2.
#include "prf_kernels.cuh"

namespace dk {
dark_status fwd_f32_d128_r2(const FwdArgs& a, const Plan& p, void* ws, void* s) {
  return launch_fwd_impl<float, 128, 2, 1>(a, p, ws, s);
}
dark_status exact_f32_d128_r2(const FwdArgs& a, void* ws, void* s) {
  return launch_exact_impl<float, 128, 2>(a, ws, s);
}
}  // namespace dk
