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
// short). The workspace holds summary records (a, S, Z), n_rec per sequence, scanned in
// place into exclusive prefixes; the output pass of segment s starts from record
// s * rec_per_seg. The summary pass may fold sub-segments (rec_per_seg records per
// segment) and may stop at chunk sum_end: records past it are empty, which is enough
// when no final state is asked for (the last segment's records feed only that state).
// One workgroup per (sequence, segment or record): blockIdx.x = b * H + h.
// With per-sequence lengths (cu_seqlens) T is the longest sequence: segments that
// start past a shorter sequence's end are empty (identity summaries, no outputs).
//
// Token tensors are seen as rows of d elements, one row per (token, head). Token t of
// sequence (b, h) is row row0(b, h) + t * tok_rows, where row0 = b * seq_rows + h * head_rows
// for fixed-length batches ([B,H,T,d]: tok_rows 1, head_rows T, seq_rows H*T; [B,T,H,d]:
// tok_rows H, head_rows 1, seq_rows T*H) and row0 = cu_seqlens[b] * H + h for packed
// sequences ([total, H, d]).
struct PrefillParams {
  const void* q;
  const void* k;
  const void* v;
  const void* prf_w;     // [H, n_psi, d_k] or null
  void* o;
  float* ws;             // [BH, n_seg, E] with E = n_psi*d_v + n_psi (segment summaries)
  const int* cu_seqlens; // [B + 1] first token of each packed sequence, or null
  const float* log_gate; // per-token, per-feature log forget gates (gated prefill), rows like k; or null
  int B, H, T;
  int total;             // tokens in the packed tensors (cu_seqlens only)
  int tok_rows;
  long long seq_rows, head_rows;
  int d_k, d_v, n_psi, C;
  int psi;               // la_psi
  int normalize;
  int out_bf16;          // o is bf16 (round to nearest even of the fp32 result)
  int in_f32;            // q, k, v are fp32 (gated path; the other paths dispatch on dtype)
  float eps;
  int n_chunks, seg_chunks, n_seg;
  int n_rec;             // summary records per sequence in ws (the record stride)
  int rec_per_seg;       // records per segment
  int sum_end;           // the summary pass folds chunks below this index only
  int fold_records;      // 1: no scan ran; the output pass folds the summary records before its
                         // segment itself (few records, no initial or final state)
  int sum_rounded;       // 1: no final state is asked for, so the bf16 summary pass may round
                         // elu+1 key features (denominator, no decay) to bf16 once, as the
                         // output pass does; 0: every inexact operand stays hi + lo
  int has_decay;
  float log2g[LA_MAX_DECAY_HEADS];  // log2(gamma_h), 0 when gamma_h == 1
};

struct ScanParams {
  float* ws;             // [BH, n_seg, E], replaced by exclusive prefixes
  const float* init_S;   // [BH, n_psi, d_v] or null
  const float* init_Z;   // [BH, n_psi] or null
  float* final_S;        // [BH, n_psi, d_v] or null
  float* final_Z;        // [BH, n_psi] or null
  const int* cu_seqlens; // [B + 1] or null (then every sequence has T tokens)
  int total;             // tokens in the packed tensors (cu_seqlens only)
  int BH, H, T;
  int n_psi, d_v;
  int n_seg, seg_len;    // segment length in tokens (the last one may be short)
  int gated;             // 1: per-row decays stored after each segment's S and Z (gated prefill)
  int reverse;           // 1: scan the segments from the last to the first (the adjoint state of
                         // the backward pass); the prefix of segment s then folds segments > s
  int has_decay;
  float log2g[LA_MAX_DECAY_HEADS];
  // Work the prefill's output pass does not need (0: none skipped): records at or past n_read
  // are not read (taken as empty; only a final state would need them), and only every
  // write_every-th prefix is written (the output pass reads the record at each segment start).
  int n_read;
  int write_every;
  int* rounds = nullptr;  // diagnostic record when set: the length of the scan's longest chain of
                          // dependent (+) steps (device int, raised by atomic max)
};

// Backward pass of the prefill: the forward problem plus the upstream gradient, the gradient
// outputs and three workspace regions.
struct BackwardParams {
  PrefillParams f;       // q, k, v, spans, chunking, decay (f.ws: the forward segment prefixes)
  const void* dout;      // dL/do, rows like o, dout_bf16 ? bf16 : fp32
  float* dq;             // fp32, rows like q
  float* dk;             // fp32, rows like k
  float* dv;             // fp32, rows like v
  float* rev;            // [BH, n_seg, E] segment summaries of the adjoint state, then their reverse prefixes
  float* tok;            // [rows, 2]: 1/den and dden per token row, rows as q's (normalize only)
  const uint16_t* wt;    // random features: the bank transposed per head, [H][d_k][n_psi] bf16
  int dout_bf16;
};

struct DecodeParams {
  const void* q;
  const void* k;
  const void* v;
  const void* prf_w;
  float* S;
  float* Z;
  void* o;               // [N, H, d_v]: fp32, or bf16 (the fp32 result rounded to nearest even) with out_bf16
  int out_bf16;
  int N, H;
  int d_k, d_v, n_psi;
  int psi;
  int normalize;
  float eps;
  int in_f32;            // 1: q, k, v, prf_w are fp32; 0: bf16
  int has_decay;
  float gamma[LA_MAX_DECAY_HEADS];
  const float* log_gate; // [N, H, n_psi] per-row log forget gates (gated step), or null
};

// Positive random features, with or without the query-row shift.
__host__ __device__ inline bool is_prf(int psi) { return psi == LA_PSI_PRF || psi == LA_PSI_PRF_QSHIFT; }

// Length of packed sequence b, clamped so that malformed offsets never address rows
// outside [0, total) and no sequence exceeds max_len; its first token is *start.
__device__ __forceinline__ int packed_len(const int* cu, int b, int total, int max_len, int* start) {
  const int s0 = min(max(cu[b], 0), total);
  const int s1 = min(max(cu[b + 1], s0), total);
  *start = s0;
  return min(s1 - s0, max_len);
}

// Where the sequence of (batch, head) bh lives: its length and its first token row.
// The workspace record that segment seg of sequence bh starts from (output pass), or
// record seg itself when rec_per_seg is 1 (summary pass).
__device__ __forceinline__ size_t rec_index(const PrefillParams& p, int bh, int seg) {
  return (size_t)bh * p.n_rec + (size_t)seg * p.rec_per_seg;
}

struct SeqSpan {
  int T;
  long long row0;
};
__device__ __forceinline__ SeqSpan seq_span(const PrefillParams& p, int bh) {
  const int b = bh / p.H, h = bh - b * p.H;
  SeqSpan s;
  if (p.cu_seqlens) {
    int start;
    s.T = packed_len(p.cu_seqlens, b, p.total, p.T, &start);
    s.row0 = (long long)start * p.H + h;
  } else {
    s.T = p.T;
    s.row0 = (long long)b * p.seq_rows + (long long)h * p.head_rows;
  }
  return s;
}

// Launchers: return hipSuccess or the launch error. Shapes are validated by the caller.
bool prefill_bf16_supported(int C, int d_k, int d_v, int n_psi, int psi);
// Whether the bf16 output kernel for these parameters can fold the summary records before its
// segment itself (then the scan between the passes is not launched).
bool prefill_bf16_output_folds(const PrefillParams& p);
hipError_t launch_prefill_bf16_summary(const PrefillParams& p, hipStream_t s);
hipError_t launch_prefill_bf16_output(const PrefillParams& p, hipStream_t s);

bool prefill_f32_supported(int C, int d_k, int d_v, int n_psi, int psi);
hipError_t launch_prefill_f32_summary(const PrefillParams& p, hipStream_t s);
hipError_t launch_prefill_f32_output(const PrefillParams& p, hipStream_t s);

hipError_t launch_segment_scan(const ScanParams& p, hipStream_t s);
// The scan over n_seg segments of a one-sequence problem with 4 x 4 states in ws (n_seg x 20
// floats, replaced by their exclusive prefixes), recording its (+) depth in *rounds (device int).
hipError_t scan_depth_probe(int n_seg, float* ws, int* rounds, hipStream_t s);

bool prefill_gated_supported(int C, int d_k, int d_v, int n_psi, int psi);
hipError_t launch_prefill_gated(const PrefillParams& p, hipStream_t s, bool out);

bool prefill_backward_supported(int C, int d_k, int d_v, int n_psi, int psi);
hipError_t launch_prefill_backward(const BackwardParams& p, hipStream_t s, bool key_sweep);

// The fp32 vector-ALU backward (la_backward_gen.hip) for the shapes the matrix-core kernels do
// not take: fp32 inputs (f.in_f32 set; dout fp32), bf16 inputs at d = 64. Same two sweeps over
// the same segment records.
bool prefill_backward_gen_supported(int C, int d_k, int d_v, int n_psi, int psi, bool in_f32);
hipError_t launch_prefill_backward_gen(const BackwardParams& p, hipStream_t s, bool state_sweep);

// Random features (la_backward_prf.hip): one 64-token step per workgroup; the forward summary
// pass of la_prefill_prf.hpp gives one record per step.
bool prefill_backward_prf_supported(int C, int d_k, int d_v, int n_psi);
hipError_t launch_prefill_backward_prf(const BackwardParams& p, hipStream_t s, bool key_sweep);
hipError_t launch_bank_transpose(const void* w, uint16_t* wt, int H, int n_psi, hipStream_t s);
hipError_t launch_prefill_prf_bf16(const PrefillParams& p, hipStream_t s, bool out);

// lin_attn_prefill on a caller-sized workspace whose segment plan is fitted to it (la_api.cpp):
// the host-only checks, then the call itself.
la_status prefill_capped_check(const la_prefill_desc* d, size_t ws_cap);
la_status prefill_capped(const la_prefill_desc* d, const void* q, const void* k, const void* v, const float* gamma,
                         const void* prf_w, const float* init_S, const float* init_Z, void* o, float* final_S,
                         float* final_Z, void* workspace, size_t ws_cap, hipStream_t stream);

bool decode_supported(int d_k, int d_v, int n_psi, int psi);
hipError_t launch_decode_step(const DecodeParams& p, hipStream_t s);

}  // namespace la
