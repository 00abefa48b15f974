// la_kernels.hpp -- parameter blocks and launchers shared by the C-ABI layer and the
// HIP kernels. Internal to liblinattn.so.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "linattn.h"

namespace la {

// Everything the prefill kernels need, passed by value as the kernel argument.
//
// Work decomposition: each (batch, head) sequence of T tokens is cut into
// n_chunks = ceil(T / C) chunks, and consecutive chunks are grouped into n_seg
// segments of seg_chunks chunks (the last segment and the last chunk may be
// short). The workspace holds one summary (a, S, Z) per segment, scanned in place.
struct PrefillParams {
  const void* q;
  const void* k;
  const void* v;
  const void* prf_w;     // [H, n_psi, d_k] or null
  void* o;
  float* ws;             // [BH, n_seg, E] with E = n_psi*d_v + n_psi (segment summaries)
  int B, H, T;
  int d_k, d_v, n_psi, C;
  int psi;               // la_psi
  int normalize;
  float eps;
  int n_chunks, seg_chunks, n_seg;
  int has_decay;
  float log2g[LA_MAX_DECAY_HEADS];  // log2(gamma_h), 0 when gamma_h == 1
};

struct ScanParams {
  float* ws;             // [BH, n_seg, E], replaced by exclusive prefixes
  const float* init_S;   // [BH, n_psi, d_v] or null
  const float* init_Z;   // [BH, n_psi] or null
  float* final_S;        // [BH, n_psi, d_v] or null
  float* final_Z;        // [BH, n_psi] or null
  int BH, H, T;
  int n_psi, d_v;
  int n_seg, seg_len;    // segment length in tokens (the last one may be short)
  int has_decay;
  float log2g[LA_MAX_DECAY_HEADS];
};

struct DecodeParams {
  const void* q;
  const void* k;
  const void* v;
  const void* prf_w;
  float* S;
  float* Z;
  float* o;
  int N, H;
  int d_k, d_v, n_psi;
  int psi;
  int normalize;
  float eps;
  int in_f32;            // 1: q, k, v, prf_w are fp32; 0: bf16
  int has_decay;
  float gamma[LA_MAX_DECAY_HEADS];
};

// Launchers: return hipSuccess or the launch error. Shapes are validated by the caller.
bool prefill_bf16_supported(int C, int d_k, int d_v, int n_psi, int psi);
hipError_t launch_prefill_bf16_summary(const PrefillParams& p, hipStream_t s);
hipError_t launch_prefill_bf16_output(const PrefillParams& p, hipStream_t s);

bool prefill_f32_supported(int C, int d_k, int d_v, int n_psi, int psi);
hipError_t launch_prefill_f32_summary(const PrefillParams& p, hipStream_t s);
hipError_t launch_prefill_f32_output(const PrefillParams& p, hipStream_t s);

hipError_t launch_segment_scan(const ScanParams& p, hipStream_t s);

bool decode_supported(int d_k, int d_v, int n_psi, int psi);
hipError_t launch_decode_step(const DecodeParams& p, hipStream_t s);

}  // namespace la
