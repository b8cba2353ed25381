// Instantiation unit: element type bf16, head dimension 128.
#include "prf_kernels.cuh"
#include "decode_kernels.cuh"

namespace dk {
dark_status fwd_bf16_d128_r1(const FwdArgs& a, const Plan& p, void* ws, void* s) { return launch_fwd_impl<bf16, 128, 1, 32>(a, p, ws, s); }
dark_status fwd_bf16_d128_r2(const FwdArgs& a, const Plan& p, void* ws, void* s) { return launch_fwd_impl<bf16, 128, 2, 32>(a, p, ws, s); }
dark_status fwd_bf16_d128_r4(const FwdArgs& a, const Plan& p, void* ws, void* s) { return launch_fwd_impl<bf16, 128, 4, 32>(a, p, ws, s); }
dark_status fwd_bf16_d128_r8(const FwdArgs& a, const Plan& p, void* ws, void* s) { return launch_fwd_impl<bf16, 128, 8, 32>(a, p, ws, s); }
dark_status fwd_bf16_d128_r16(const FwdArgs& a, const Plan& p, void* ws, void* s) { return launch_fwd_impl<bf16, 128, 16, 32>(a, p, ws, s); }
dark_status dec_bf16_d128(const dark_prf_desc& d, const void* q, const void* k, const void* v, const float* M,
                         const float* om, float* S, float* z, void* out, void* s) {
  return launch_decode_impl<bf16, 128>(d, q, k, v, M, om, S, z, out, s);
}
}  // namespace dk
