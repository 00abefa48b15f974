// la_prefill_bf16.hip -- dispatch of the bf16 prefill kernels (la_prefill_bf16.hpp for the
// identity and elu+1 feature maps, la_prefill_prf.hip for positive random features) over the
// supported chunk sizes and head widths.
#include "la_prefill_bf16.hpp"

namespace la {

bool prefill_prf_bf16_supported(int C, int d_k, int d_v, int n_psi);
hipError_t launch_prefill_prf_bf16(const PrefillParams& p, hipStream_t s, bool out);

// Chunks of 32, 64 or 128 tokens: the kernels walk 64-token steps (see in_64_token_steps), so
// the planner keeps segment boundaries on multiples of 64 tokens (an even chunk count per
// segment at C = 32).
bool prefill_bf16_supported(int C, int d_k, int d_v, int n_psi, int psi) {
  if (C != 32 && C != 64 && C != 128) return false;
  if (is_prf(psi)) return prefill_prf_bf16_supported(64, d_k, d_v, n_psi);
  if (psi != LA_PSI_IDENTITY && psi != LA_PSI_ELU1) return false;
  if (d_k != d_v || n_psi != d_k) return false;
  return d_k == 64 || d_k == 128;
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
// state and the chunk's own scores. So both passes walk every segment in 64-token steps
// (segment boundaries, multiples of seg_chunks * C tokens and of 64, are unchanged): at C =
// 128 the 64-token kernels need half the LDS, two workgroups share a CU and hide each other's
// latency, and C = 32 needs no kernels of its own. The results differ from another grouping
// only by rounding. (128k retention workload: output pass 2.21 ms in 64-token steps against
// 2.50 ms in 128-token chunks.)
static PrefillParams in_64_token_steps(const PrefillParams& p) {
  if (p.C == 64) return p;
  PrefillParams q = p;
  q.C = 64;
  // kernels count each sequence's steps from its own length; C = 32 segments hold an even
  // number of chunks (the planner's rule)
  q.n_chunks = p.C == 128 ? 2 * p.n_chunks : (p.n_chunks + 1) / 2;
  q.seg_chunks = p.C == 128 ? 2 * p.seg_chunks : p.seg_chunks / 2;
  // an end that is not the sequence's last chunk is a segment or record boundary: even at C = 32
  q.sum_end = p.C == 128 ? 2 * p.sum_end : (p.sum_end + 1) / 2;
  return q;
}

// The eight-wave output kernels (d = 128 with elu+1 features or a denominator, and random
// features) fold up to kMaxFold records themselves: a few loads per lane and record, against a
// scan launch.
constexpr int kMaxFold = 8;
bool prefill_bf16_output_folds(const PrefillParams& p) {
  if (p.cu_seqlens || p.d_k != 128 || p.d_v != 128) return false;
  if (!is_prf(p.psi) && p.psi != LA_PSI_ELU1 && !p.normalize) return false;  // the shared-score kernel reads scanned prefixes
  if (p.rec_per_seg < 1 || p.seg_chunks % p.rec_per_seg != 0) return false;
  return (long long)(p.n_seg - 1) * p.rec_per_seg <= kMaxFold;
}

hipError_t launch_prefill_bf16_summary(const PrefillParams& p, hipStream_t s) {
  return dispatch(in_64_token_steps(p), s, false);
}
hipError_t launch_prefill_bf16_output(const PrefillParams& p, hipStream_t s) {
  return dispatch(in_64_token_steps(p), s, true);
}

}  // namespace la
