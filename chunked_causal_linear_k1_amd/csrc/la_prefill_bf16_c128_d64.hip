// Instantiations of the bf16 prefill kernels for chunk C = 128, head width D = 64.
#include "la_prefill_bf16.hpp"

namespace la {
hipError_t launch_prefill_bf16_c128_d64(const PrefillParams& p, hipStream_t s, bool out) {
  return pf::launch_cd<128, 64>(p, s, out);
}
}  // namespace la
