// la_prefill_prf.hip -- instantiation and dispatch of the positive-random-feature bf16
// prefill kernels (see la_prefill_prf.hpp): chunk 64, d_k = d_v = 128, n_psi 128 or 256.
#include "la_prefill_prf.hpp"

namespace la {

bool prefill_prf_bf16_supported(int C, int d_k, int d_v, int n_psi) {
  return C == 64 && d_k == 128 && d_v == 128 && (n_psi == 128 || n_psi == 256);
}

hipError_t launch_prefill_prf_bf16(const PrefillParams& p, hipStream_t s, bool out) {
  if (p.C == 64 && p.d_k == 128 && p.n_psi == 256) return prf::launch_np<64, 128, 256>(p, s, out);
  if (p.C == 64 && p.d_k == 128 && p.n_psi == 128) return prf::launch_np<64, 128, 128>(p, s, out);
  return hipErrorInvalidValue;
}

}  // namespace la
