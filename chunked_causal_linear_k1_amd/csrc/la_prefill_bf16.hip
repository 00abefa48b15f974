// la_prefill_bf16.hip -- dispatch of the bf16 prefill kernels (la_prefill_bf16.hpp for the
// identity and elu+1 feature maps, la_prefill_prf.hip for positive random features) over the
// supported chunk sizes and head widths.
#include "la_prefill_bf16.hpp"

namespace la {

bool prefill_prf_bf16_supported(int C, int d_k, int d_v, int n_psi);
hipError_t launch_prefill_prf_bf16(const PrefillParams& p, hipStream_t s, bool out);

bool prefill_bf16_supported(int C, int d_k, int d_v, int n_psi, int psi) {
  if (is_prf(psi)) return prefill_prf_bf16_supported(C, d_k, d_v, n_psi);
  if (psi != LA_PSI_IDENTITY && psi != LA_PSI_ELU1) return false;
  if (d_k != d_v || n_psi != d_k) return false;
  return (d_k == 64 || d_k == 128) && (C == 64 || C == 128);
}

static hipError_t dispatch(const PrefillParams& p, hipStream_t s, bool out) {
  if (is_prf(p.psi)) return launch_prefill_prf_bf16(p, s, out);
  if (p.C == 64 && p.d_k == 64) return launch_prefill_bf16_c64_d64(p, s, out);
  if (p.C == 64 && p.d_k == 128) return launch_prefill_bf16_c64_d128(p, s, out);
  return hipErrorInvalidValue;  // C = 128 arrives here as 64-token steps
}

// Neither pass depends on how a segment's tokens are grouped into chunks: the segment
// summary is the decayed sum of psi(k_i) v_i^T over the segment's tokens, and each output is
// the same sum over the tokens before it however the prefix is split between the carried
// state and the chunk's own scores. So at C = 128 both passes walk the segment in 64-token
// steps (segment boundaries, multiples of seg_chunks * C tokens, are unchanged): the 64-token
// kernels need half the LDS, two workgroups share a CU and hide each other's latency. The
// results differ from a 128-token grouping only by rounding. (128k retention workload: output
// pass 2.21 ms in 64-token steps against 2.50 ms in 128-token chunks.)
static PrefillParams in_64_token_steps(const PrefillParams& p) {
  if (p.C != 128 || is_prf(p.psi)) return p;
  PrefillParams q = p;
  q.C = 64;
  q.n_chunks = 2 * p.n_chunks;  // kernels count each sequence's chunks from its own length
  q.seg_chunks = 2 * p.seg_chunks;
  return q;
}

hipError_t launch_prefill_bf16_summary(const PrefillParams& p, hipStream_t s) {
  return dispatch(in_64_token_steps(p), s, false);
}
hipError_t launch_prefill_bf16_output(const PrefillParams& p, hipStream_t s) {
  return dispatch(in_64_token_steps(p), s, true);
}

}  // namespace la
