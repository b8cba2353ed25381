// Decode instantiation: element type bf16, head dimension 32.
#include "prf_kernels.cuh"
#include "decode_kernels.cuh"

namespace dk {
dark_status dec_bf16_d32(const dark_prf_desc& d, const void* q, const void* k, const void* v, const float* M,
                         const float* om, float* S, float* z, void* out, const uint8_t* qm, int upd, void* s) {
  return launch_decode_impl<bf16, 32>(d, q, k, v, M, om, S, z, out, qm, upd, s);
}
}  // namespace dk
