// Instantiation unit: element type float, head dimension 16.
#include "prf_kernels.cuh"
#include "decode_kernels.cuh"

namespace dk {
dark_status fwd_f32_d16_r1(const FwdArgs& a, const Plan& p, void* ws, void* s) { return launch_fwd_impl<float, 16, 1, 64>(a, p, ws, s); }
dark_status fwd_f32_d16_r2(const FwdArgs& a, const Plan& p, void* ws, void* s) { return launch_fwd_impl<float, 16, 2, 64>(a, p, ws, s); }
dark_status fwd_f32_d16_r4(const FwdArgs& a, const Plan& p, void* ws, void* s) { return launch_fwd_impl<float, 16, 4, 64>(a, p, ws, s); }
dark_status fwd_f32_d16_r8(const FwdArgs& a, const Plan& p, void* ws, void* s) { return launch_fwd_impl<float, 16, 8, 64>(a, p, ws, s); }
dark_status fwd_f32_d16_r16(const FwdArgs& a, const Plan& p, void* ws, void* s) { return launch_fwd_impl<float, 16, 16, 64>(a, p, ws, s); }
dark_status dec_f32_d16(const dark_prf_desc& d, const void* q, const void* k, const void* v, const float* M,
                         const float* om, float* S, float* z, void* out, void* s) {
  return launch_decode_impl<float, 16>(d, q, k, v, M, om, S, z, out, s);
}
}  // namespace dk
