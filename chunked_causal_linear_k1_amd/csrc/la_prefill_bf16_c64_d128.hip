// Instantiations of the bf16 prefill kernels for chunk C = 64, head width D = 128.
#include "la_prefill_bf16.hpp"

namespace la {
hipError_t launch_prefill_bf16_c64_d128(const PrefillParams& p, hipStream_t s, bool out) {
  return pf::launch_cd<64, 128>(p, s, out);
}
}  // namespace la
