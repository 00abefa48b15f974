// la_api.cpp -- the extern "C" boundary of liblinattn.so (declared in include/linattn.h).
//
// Host side only: validates every argument before anything is enqueued, plans the
// segment decomposition, carves the caller's workspace, and launches
//   prefill: segment summaries -> segment scan -> output walk   (three launches)
//   decode : one launch
// on the caller's stream. No allocation, no synchronisation, no device switch.
#include <math.h>
#include <string.h>

#include <algorithm>

#include "la_kernels.hpp"

namespace {

using la::PrefillParams;
using la::ScanParams;

// Prefill decomposition (segments of consecutive chunks, one workgroup each):
constexpr int kTargetWorkgroups = 2048;  // enough to fill 256 CUs several times over
constexpr int kMinWorkgroups = 256;      // at least one per CU where the sequences allow it
constexpr int kMinSegTokens = 2048;      // per-segment state traffic (n_psi*d_v floats written,
                                         // scanned, read back) small next to the token traffic
constexpr int kMinSubTokens = 1024;      // the same bound for the summary pass's sub-segments
constexpr int kMaxRecPerSeg = 4;

bool aligned16(const void* p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

la_status check_gamma(const float* gamma, int H) {
  if (!gamma) return LA_OK;
  if (H > LA_MAX_DECAY_HEADS) return LA_ERR_UNSUPPORTED;
  for (int h = 0; h < H; ++h) {
    const float g = gamma[h];
    if (!(g > 0.f && g <= 1.f)) return LA_ERR_VALUE;  // also rejects NaN
  }
  return LA_OK;
}

// log2(gamma) evaluated in double from the fp32 value, stored as float (0 for gamma == 1).
int fill_log2g(const float* gamma, int H, float* out) {
  int any = 0;
  for (int h = 0; h < LA_MAX_DECAY_HEADS; ++h) out[h] = 0.f;
  if (!gamma) return 0;
  for (int h = 0; h < H; ++h) {
    out[h] = gamma[h] == 1.f ? 0.f : (float)log2((double)gamma[h]);
    any |= gamma[h] != 1.f;
  }
  return any;
}

la_status validate_prefill_desc(const la_prefill_desc* d, bool gated = false) {
  if (!d) return LA_ERR_NULL;
  if (d->B < 1 || d->H < 1 || d->T < 1 || d->d_k < 1 || d->d_v < 1 || d->n_psi < 1 || d->chunk < 1)
    return LA_ERR_SHAPE;
  if (d->psi < LA_PSI_IDENTITY || d->psi > LA_PSI_PRF_QSHIFT) return LA_ERR_VALUE;
  if (d->normalize != 0 && d->normalize != 1) return LA_ERR_VALUE;
  if (!(d->eps >= 0.f) || !isfinite(d->eps)) return LA_ERR_VALUE;
  if (d->in_dtype != LA_BF16 && d->in_dtype != LA_F32) return LA_ERR_VALUE;
  if (d->out_dtype != LA_BF16 && d->out_dtype != LA_F32) return LA_ERR_VALUE;
  if (d->layout != LA_LAYOUT_BHTD && d->layout != LA_LAYOUT_BTHD) return LA_ERR_VALUE;
  if (!la::is_prf(d->psi) && d->n_psi != d->d_k) return LA_ERR_SHAPE;
  // the query-row shift cancels only against a denominator; without one each output would be
  // scaled by the query's exp(-max log-feature), a different function from plain PRF's
  if (d->psi == LA_PSI_PRF_QSHIFT && !d->normalize) return LA_ERR_UNSUPPORTED;
  if (d->d_v % 4 != 0 || d->n_psi % 4 != 0) return LA_ERR_UNSUPPORTED;  // 16-byte state rows
  // element counts must fit comfortably in 64-bit offsets; sequences go on the grid's x
  // extent (segments and element blocks on y, each capped at 65535 by the planner)
  const double tokens = (double)d->B * d->H * d->T;
  if (tokens * std::max(d->d_k, d->d_v) > 9.0e15) return LA_ERR_SHAPE;
  if ((long long)d->B * d->H > 2147483647LL) return LA_ERR_SHAPE;
  // one chunk of one head spans (C - 1) * H + 1 rows in the interleaved layout: its byte
  // extent must fit a buffer resource's 32-bit range
  if (d->layout == LA_LAYOUT_BTHD && (double)d->chunk * d->H * std::max(d->d_k, d->d_v) * 4 >= 2147483648.0)
    return LA_ERR_UNSUPPORTED;
  if (d->out_dtype == LA_BF16 && d->in_dtype != LA_BF16) return LA_ERR_UNSUPPORTED;
  if (gated) return la::prefill_gated_supported(d->chunk, d->d_k, d->d_v, d->n_psi, d->psi) ? LA_OK
                                                                                           : LA_ERR_UNSUPPORTED;
  const bool ok = d->in_dtype == LA_BF16
                      ? la::prefill_bf16_supported(d->chunk, d->d_k, d->d_v, d->n_psi, d->psi)
                      : la::prefill_f32_supported(d->chunk, d->d_k, d->d_v, d->n_psi, d->psi);
  return ok ? LA_OK : LA_ERR_UNSUPPORTED;
}

struct Plan {
  int chunk;  // the chunk the kernels walk (the caller's, or kF32LatencyChunk, see make_plan)
  int n_chunks, seg_chunks, n_seg;
  int rec_per_seg, n_rec;  // summary records per segment and per sequence (at most)
  size_t ws_bytes;
};

// total_tokens < 0: a fixed-length batch (every sequence T tokens), cut into the same number
// of segments per sequence. total_tokens >= 0: a packed batch whose lengths only the device
// knows (T is the longest); segments then have a fixed token count sized from the batch's
// total, so the non-empty workgroups number about kTargetWorkgroups and carry similar work
// whatever the length mix (segments past a shorter sequence's end are empty and exit at once).
//
// sub (fixed-length bf16 forward only, gated or not): when the segments leave the summary
// pass short of workgroups, it folds rec_per_seg sub-segments per segment (whole steps of
// the kernels: 64 tokens, or the gated path's 32-token chunks; at least kMinSubTokens each),
// so that the pass takes a fraction of a segment's time; the scan then runs over the
// sub-segment records and each segment reads the record at its start.
//
// ws_cap (fixed-length batches, nonzero only for lin_attn_prefill_noalloc): when the records
// exceed it, the plan takes fewer, longer segments, one record each, at most as many per
// sequence as fit; if not even one record per sequence fits, ws_bytes stays above the cap.
//
// latency_chunk (the prefill and its backward, fixed-length batches): fp32 inputs whose chunks cannot
// fill the GPU walk chunks of kF32LatencyChunk tokens instead of the caller's, for more and
// shorter workgroups. The result does not depend on the grouping of tokens into chunks (the
// same function; only the rounding differs).
constexpr int kF32LatencyChunk = 16;
Plan make_plan(const la_prefill_desc* d, long long total_tokens = -1, bool gated = false, bool sub = false,
               size_t ws_cap = 0, bool latency_chunk = false) {
  Plan pl;
  const long long BH = (long long)d->B * d->H;
  int C = d->chunk;
  if (latency_chunk && total_tokens < 0 && !gated && d->in_dtype == LA_F32 && C > kF32LatencyChunk &&
      BH * ((d->T + C - 1) / C) < kTargetWorkgroups)
    C = kF32LatencyChunk;
  pl.chunk = C;
  pl.n_chunks = (int)((d->T + (long long)C - 1) / C);
  if (total_tokens < 0) {
    long long want = (kTargetWorkgroups + BH - 1) / BH;  // segments per sequence
    want = std::min<long long>(want, std::max(1LL, (long long)d->T / kMinSegTokens));
    if (want * BH < kMinWorkgroups) want = (kMinWorkgroups + BH - 1) / BH;
    want = std::max(1LL, std::min<long long>(want, pl.n_chunks));
    pl.seg_chunks = (int)((pl.n_chunks + want - 1) / want);
  } else {
    const long long work = total_tokens * d->H;  // token-heads in the batch
    const long long seg_tokens = std::max<long long>(kMinSegTokens, (work + kTargetWorkgroups - 1) / kTargetWorkgroups);
    pl.seg_chunks = (int)std::min<long long>(pl.n_chunks, (seg_tokens + C - 1) / C);
  }
  pl.n_seg = (pl.n_chunks + pl.seg_chunks - 1) / pl.seg_chunks;
  if (pl.n_seg > 65535) {  // the grid's y extent
    pl.seg_chunks = (pl.n_chunks + 65534) / 65535;
    pl.n_seg = (pl.n_chunks + pl.seg_chunks - 1) / pl.seg_chunks;
  }
  // the bf16 kernels walk 64-token steps: with 32-token chunks a segment holds an even number
  if (!gated && d->in_dtype == LA_BF16 && C == 32 && (pl.seg_chunks & 1)) {
    pl.seg_chunks += 1;
    pl.n_seg = (pl.n_chunks + pl.seg_chunks - 1) / pl.seg_chunks;
  }
  pl.rec_per_seg = 1;
  if (sub && total_tokens < 0 && d->in_dtype == LA_BF16) {
    const int step = !gated && C == 32 ? 2 : 1;  // chunks per kernel step
    // workgroups that fold tokens when the last segment (only the final state needs it) is skipped
    const long long folded = BH * std::max(1, pl.n_seg - 1);
    while (pl.rec_per_seg < kMaxRecPerSeg) {
      const int k2 = 2 * pl.rec_per_seg;
      if (pl.seg_chunks % (k2 * step) != 0) break;
      if ((long long)(pl.seg_chunks / k2) * C < kMinSubTokens) break;
      if (folded * k2 > kTargetWorkgroups || (long long)pl.n_seg * k2 > 65535) break;
      pl.rec_per_seg = k2;
    }
  }
  pl.n_rec = pl.n_seg * pl.rec_per_seg;
  // one record per segment or sub-segment: S, Z (and, gated, the segment's per-row decay)
  const size_t E = (size_t)d->n_psi * d->d_v + (gated ? 2 : 1) * (size_t)d->n_psi;
  pl.ws_bytes = (size_t)BH * pl.n_rec * E * sizeof(float);
  if (ws_cap && total_tokens < 0 && pl.ws_bytes > ws_cap) {
    const long long max_rec = (long long)(ws_cap / ((size_t)BH * E * sizeof(float)));
    if (max_rec >= 1) {
      pl.rec_per_seg = 1;
      pl.seg_chunks = (int)((pl.n_chunks + max_rec - 1) / max_rec);
      if (!gated && d->in_dtype == LA_BF16 && C == 32 && (pl.seg_chunks & 1)) pl.seg_chunks += 1;
      pl.n_seg = (pl.n_chunks + pl.seg_chunks - 1) / pl.seg_chunks;
      pl.n_rec = pl.n_seg;
      pl.ws_bytes = (size_t)BH * pl.n_rec * E * sizeof(float);
    }
  }
  return pl;
}

}  // namespace

extern "C" {

const char* lin_attn_status_string(la_status s) {
  switch (s) {
    case LA_OK: return "ok";
    case LA_ERR_NULL: return "a required pointer is NULL";
    case LA_ERR_SHAPE: return "a size is out of range or inconsistent";
    case LA_ERR_UNSUPPORTED: return "combination not supported by this build";
    case LA_ERR_WORKSPACE: return "workspace missing or too small";
    case LA_ERR_ALIGN: return "device pointer not 16-byte aligned";
    case LA_ERR_VALUE: return "invalid value (eps, gamma or enum)";
    case LA_ERR_HIP: return "HIP runtime error at launch";
  }
  return "unknown status";
}

const char* lin_attn_version(void) { return "0.4.0"; }

la_status lin_attn_prefill_workspace_size(const la_prefill_desc* d, size_t* bytes) {
  if (!bytes) return LA_ERR_NULL;
  const la_status st = validate_prefill_desc(d);
  if (st != LA_OK) return st;
  *bytes = make_plan(d, -1, false, true, 0, true).ws_bytes;
  return LA_OK;
}

la_status lin_attn_prefill_gated_workspace_size(const la_prefill_desc* d, size_t* bytes) {
  if (!bytes) return LA_ERR_NULL;
  const la_status st = validate_prefill_desc(d, true);
  if (st != LA_OK) return st;
  *bytes = make_plan(d, -1, true, true).ws_bytes;
  return LA_OK;
}

// The backward pass: the forward segment prefixes, the adjoint segment records (same size) and,
// with a denominator, two floats per token (1/den and dden).
// varlen: the packed form. Random features have a backward for fixed-length batches only: it
// keeps one record per 64-token step and sequence, which for a packed batch would scale with the
// longest sequence times the batch.
la_status validate_backward_desc(const la_prefill_desc* d, bool varlen = false) {
  const la_status st = validate_prefill_desc(d);
  if (st != LA_OK) return st;
  if (d->in_dtype == LA_F32)  // the fp32 vector-ALU sweeps, segment records as for bf16 inputs
    return la::prefill_backward_gen_supported(d->chunk, d->d_k, d->d_v, d->n_psi, d->psi, true) ? LA_OK
                                                                                               : LA_ERR_UNSUPPORTED;
  if (la::is_prf(d->psi)) {
    // one workgroup per 64-token step on the grid's y extent
    if ((d->T + 63) / 64 > 65535) return LA_ERR_UNSUPPORTED;
    return !varlen && la::prefill_backward_prf_supported(d->chunk, d->d_k, d->d_v, d->n_psi) ? LA_OK
                                                                                             : LA_ERR_UNSUPPORTED;
  }
  if (la::prefill_backward_supported(d->chunk, d->d_k, d->d_v, d->n_psi, d->psi)) return LA_OK;
  return la::prefill_backward_gen_supported(d->chunk, d->d_k, d->d_v, d->n_psi, d->psi, false) ? LA_OK
                                                                                              : LA_ERR_UNSUPPORTED;
}

// Random features with bf16 inputs: one record per 64-token step (la_backward_prf.hip). With fp32
// inputs they take the vector-ALU sweeps over segment records like every other feature map.
constexpr int kPrfBwdStep = 64;
bool prf_steps(const la_prefill_desc* d) { return la::is_prf(d->psi) && d->in_dtype == LA_BF16; }
Plan prf_backward_plan(const la_prefill_desc* d) {
  Plan pl;
  pl.n_chunks = (d->T + kPrfBwdStep - 1) / kPrfBwdStep;
  pl.seg_chunks = 1;
  pl.n_seg = pl.n_rec = pl.n_chunks;
  pl.rec_per_seg = 1;
  const size_t E = (size_t)d->n_psi * d->d_v + d->n_psi;
  pl.ws_bytes = (size_t)d->B * d->H * pl.n_rec * E * sizeof(float);
  return pl;
}

// total_tokens < 0: a fixed-length batch; otherwise a packed batch of that many tokens. Two
// record regions (forward prefixes, adjoint states), 1/den and dden per token row with a
// denominator, and for random features the transposed bank.
size_t backward_ws_bytes(const la_prefill_desc* d, long long total_tokens = -1) {
  const long long rows = total_tokens < 0 ? (long long)d->B * d->T * d->H : total_tokens * d->H;
  const size_t tok = d->normalize ? (size_t)rows * 2 * sizeof(float) : 0;
  if (prf_steps(d)) {
    const size_t bank = ((size_t)d->H * d->n_psi * d->d_k * 2 + 15) & ~(size_t)15;
    return 2 * prf_backward_plan(d).ws_bytes + tok + bank;
  }
  return 2 * make_plan(d, total_tokens, false, false, 0, true).ws_bytes + tok;
}

la_status lin_attn_prefill_backward_workspace_size(const la_prefill_desc* d, size_t* bytes) {
  if (!bytes) return LA_ERR_NULL;
  const la_status st = validate_backward_desc(d);
  if (st != LA_OK) return st;
  *bytes = backward_ws_bytes(d);
  return LA_OK;
}

la_status lin_attn_prefill_backward_varlen_workspace_size(const la_prefill_desc* d, int32_t total_tokens,
                                                          size_t* bytes) {
  if (!bytes) return LA_ERR_NULL;
  const la_status st = validate_backward_desc(d, true);
  if (st != LA_OK) return st;
  if (total_tokens < 0) return LA_ERR_SHAPE;
  *bytes = backward_ws_bytes(d, total_tokens);
  return LA_OK;
}

la_status lin_attn_prefill_varlen_workspace_size(const la_prefill_desc* d, int32_t total_tokens, size_t* bytes) {
  if (!bytes) return LA_ERR_NULL;
  const la_status st = validate_prefill_desc(d);
  if (st != LA_OK) return st;
  if (total_tokens < 0) return LA_ERR_SHAPE;
  *bytes = make_plan(d, total_tokens).ws_bytes;
  return LA_OK;
}

}  // extern "C"

namespace {

// Both prefill entry points: fixed-length batches (cu_seqlens == nullptr) and packed
// variable-length batches.
la_status prefill_impl(const la_prefill_desc* d, const int32_t* cu_seqlens, int32_t total_tokens, const void* q,
                       const void* k, const void* v, const float* gamma, const void* prf_w, const float* init_S,
                       const float* init_Z, void* o, float* final_S, float* final_Z, void* workspace,
                       size_t workspace_bytes, hipStream_t stream, hipEvent_t* events,
                       const float* log_gate = nullptr, size_t ws_cap = 0) {
  const bool gated = log_gate != nullptr;
  la_status st = validate_prefill_desc(d, gated);
  if (st != LA_OK) return st;
  if (cu_seqlens) {
    if (d->layout != LA_LAYOUT_BTHD) return LA_ERR_VALUE;
    if (total_tokens < 0) return LA_ERR_SHAPE;
    if ((reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) != 0) return LA_ERR_ALIGN;
  }
  if (!q || !k || !v || !o) return LA_ERR_NULL;
  if (la::is_prf(d->psi) && !prf_w) return LA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(prf_w) ||
      !aligned16(init_S) || !aligned16(init_Z) || !aligned16(final_S) || !aligned16(final_Z) ||
      !aligned16(workspace))
    return LA_ERR_ALIGN;
  st = check_gamma(gamma, d->H);
  if (st != LA_OK) return st;
  if (gated && !aligned16(log_gate)) return LA_ERR_ALIGN;
  const bool sub = !cu_seqlens;
  const Plan pl = make_plan(d, cu_seqlens ? (long long)total_tokens : -1LL, gated, sub, ws_cap, true);
  if (pl.ws_bytes > 0 && (!workspace || workspace_bytes < pl.ws_bytes)) return LA_ERR_WORKSPACE;

  PrefillParams p;
  memset(&p, 0, sizeof p);
  p.q = q; p.k = k; p.v = v; p.prf_w = prf_w; p.o = o;
  p.ws = (float*)workspace;
  p.cu_seqlens = cu_seqlens;
  p.log_gate = log_gate;
  p.in_f32 = d->in_dtype == LA_F32;
  p.total = cu_seqlens ? total_tokens : 0;
  p.B = d->B; p.H = d->H; p.T = d->T;
  if (d->layout == LA_LAYOUT_BTHD) {
    p.tok_rows = d->H; p.head_rows = 1; p.seq_rows = (long long)d->T * d->H;
  } else {
    p.tok_rows = 1; p.head_rows = d->T; p.seq_rows = (long long)d->H * d->T;
  }
  p.d_k = d->d_k; p.d_v = d->d_v; p.n_psi = d->n_psi; p.C = pl.chunk;
  p.psi = d->psi; p.normalize = d->normalize; p.eps = d->eps;
  p.out_bf16 = d->out_dtype == LA_BF16;
  p.n_chunks = pl.n_chunks; p.seg_chunks = pl.seg_chunks; p.n_seg = pl.n_seg;
  p.n_rec = pl.n_rec; p.rec_per_seg = pl.rec_per_seg; p.sum_end = pl.n_chunks;
  p.has_decay = fill_log2g(gamma, d->H, p.log2g);
  // The last segment's records feed only the final state: without one, the summary pass stops
  // at the last segment's start, whose single empty record the scan turns into its prefix.
  const bool want_final = final_S || (d->normalize && final_Z);
  if (sub && d->in_dtype == LA_BF16 && !want_final) {  // the bf16 kernels (gated too) honour sum_end and n_rec
    p.n_rec = pl.rec_per_seg * (pl.n_seg - 1) + 1;
    p.sum_end = (pl.n_seg - 1) * pl.seg_chunks;
  }
  p.sum_rounded = !want_final && !gated;  // the records reach only outputs
  // few records before each segment, no initial or final state: the output pass folds them
  p.fold_records = d->in_dtype == LA_BF16 && !gated && !want_final && !init_S && !(d->normalize && init_Z) &&
                   la::prefill_bf16_output_folds(p);
  // the summary pass: one workgroup per record
  PrefillParams ps = p;
  ps.seg_chunks = pl.seg_chunks / pl.rec_per_seg;
  ps.n_seg = p.n_rec;
  ps.rec_per_seg = 1;

  ScanParams sp;
  memset(&sp, 0, sizeof sp);
  sp.ws = p.ws;
  sp.init_S = init_S; sp.final_S = final_S;
  // without normalisation the normaliser is not maintained: init_Z / final_Z are ignored
  sp.init_Z = d->normalize ? init_Z : nullptr;
  sp.final_Z = d->normalize ? final_Z : nullptr;
  sp.cu_seqlens = cu_seqlens; sp.total = p.total;
  sp.gated = gated;
  sp.BH = d->B * d->H; sp.H = d->H; sp.T = d->T;
  sp.n_psi = d->n_psi; sp.d_v = d->d_v;
  sp.n_seg = ps.n_seg; sp.seg_len = ps.seg_chunks * pl.chunk;
  sp.has_decay = p.has_decay;
  memcpy(sp.log2g, p.log2g, sizeof sp.log2g);
  sp.write_every = pl.rec_per_seg;       // the output pass reads the record at each segment start
  if (!want_final) sp.n_read = p.n_rec - 1;  // the last record feeds only the final state

  auto mark = [&](int i) -> hipError_t {
    return (events && events[i]) ? hipEventRecord(events[i], stream) : hipSuccess;
  };
  const bool bf = d->in_dtype == LA_BF16;
  hipError_t e = mark(0);
  if (e == hipSuccess)
    e = gated ? la::launch_prefill_gated(ps, stream, false)
              : bf ? la::launch_prefill_bf16_summary(ps, stream) : la::launch_prefill_f32_summary(ps, stream);
  if (e == hipSuccess) e = mark(1);
  if (e == hipSuccess && !p.fold_records) e = la::launch_segment_scan(sp, stream);
  if (e == hipSuccess) e = mark(2);
  if (e == hipSuccess)
    e = gated ? la::launch_prefill_gated(p, stream, true)
              : bf ? la::launch_prefill_bf16_output(p, stream) : la::launch_prefill_f32_output(p, stream);
  if (e == hipSuccess) e = mark(3);
  return e == hipSuccess ? LA_OK : LA_ERR_HIP;
}

}  // namespace

namespace la {

// The checks lin_attn_prefill makes on the host that do not touch pointers, plus the segment
// plan under a workspace cap: LA_ERR_WORKSPACE when not even one record per sequence fits.
la_status prefill_capped_check(const la_prefill_desc* d, size_t ws_cap) {
  const la_status st = validate_prefill_desc(d);
  if (st != LA_OK) return st;
  return make_plan(d, -1, false, true, ws_cap, true).ws_bytes > ws_cap ? LA_ERR_WORKSPACE : LA_OK;
}

// lin_attn_prefill with a workspace of ws_cap bytes and the plan fitted to it.
la_status prefill_capped(const la_prefill_desc* d, const void* q, const void* k, const void* v, const float* gamma,
                         const void* prf_w, const float* init_S, const float* init_Z, void* o, float* final_S,
                         float* final_Z, void* workspace, size_t ws_cap, hipStream_t stream) {
  return prefill_impl(d, nullptr, 0, q, k, v, gamma, prf_w, init_S, init_Z, o, final_S, final_Z, workspace, ws_cap,
                      stream, nullptr, nullptr, ws_cap);
}

}  // namespace la

extern "C" {

la_status lin_attn_prefill_profiled(const la_prefill_desc* d, const void* q, const void* k, const void* v,
                                    const float* gamma, const void* prf_w, const float* init_S,
                                    const float* init_Z, void* o, float* final_S, float* final_Z, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream, hipEvent_t* events) {
  return prefill_impl(d, nullptr, 0, q, k, v, gamma, prf_w, init_S, init_Z, o, final_S, final_Z, workspace,
                      workspace_bytes, stream, events);
}

la_status lin_attn_prefill_varlen(const la_prefill_desc* d, const int32_t* cu_seqlens, int32_t total_tokens,
                                  const void* q, const void* k, const void* v, const float* gamma,
                                  const void* prf_w, const float* init_S, const float* init_Z, void* o,
                                  float* final_S, float* final_Z, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream) {
  if (!cu_seqlens) return LA_ERR_NULL;
  return prefill_impl(d, cu_seqlens, total_tokens, q, k, v, gamma, prf_w, init_S, init_Z, o, final_S, final_Z,
                      workspace, workspace_bytes, stream, nullptr);
}

la_status lin_attn_prefill(const la_prefill_desc* d, const void* q, const void* k, const void* v,
                           const float* gamma, const void* prf_w, const float* init_S, const float* init_Z,
                           void* o, float* final_S, float* final_Z, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  return lin_attn_prefill_profiled(d, q, k, v, gamma, prf_w, init_S, init_Z, o, final_S, final_Z, workspace,
                                   workspace_bytes, stream, nullptr);
}

}  // extern "C"

namespace {

la_status decode_impl(const la_decode_desc* d, const void* q, const void* k, const void* v, const float* gamma,
                      const float* log_gate, const void* prf_w, float* S, float* Z, void* o, hipStream_t stream) {
  if (!d) return LA_ERR_NULL;
  if (d->N < 1 || d->H < 1 || d->d_k < 1 || d->d_v < 1 || d->n_psi < 1) return LA_ERR_SHAPE;
  if (d->psi < LA_PSI_IDENTITY || d->psi > LA_PSI_PRF_QSHIFT) return LA_ERR_VALUE;
  if (d->normalize != 0 && d->normalize != 1) return LA_ERR_VALUE;
  if (!(d->eps >= 0.f) || !isfinite(d->eps)) return LA_ERR_VALUE;
  if (d->in_dtype != LA_BF16 && d->in_dtype != LA_F32) return LA_ERR_VALUE;
  if (d->out_dtype != LA_BF16 && d->out_dtype != LA_F32) return LA_ERR_VALUE;
  if (!la::is_prf(d->psi) && d->n_psi != d->d_k) return LA_ERR_SHAPE;
  if (d->psi == LA_PSI_PRF_QSHIFT && !d->normalize) return LA_ERR_UNSUPPORTED;  // as in prefill
  if ((long long)d->N * d->H > 2147483647LL) return LA_ERR_SHAPE;
  if (d->out_dtype == LA_BF16 && d->in_dtype != LA_BF16) return LA_ERR_UNSUPPORTED;  // as in prefill
  if (!la::decode_supported(d->d_k, d->d_v, d->n_psi, d->psi)) return LA_ERR_UNSUPPORTED;
  if (!q || !k || !v || !S || !o) return LA_ERR_NULL;
  if (d->normalize && !Z) return LA_ERR_NULL;
  if (la::is_prf(d->psi) && !prf_w) return LA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(S) || !aligned16(Z) || !aligned16(o) ||
      !aligned16(prf_w) || !aligned16(log_gate))
    return LA_ERR_ALIGN;
  la_status st = check_gamma(gamma, d->H);
  if (st != LA_OK) return st;

  la::DecodeParams p;
  memset(&p, 0, sizeof p);
  p.q = q; p.k = k; p.v = v; p.prf_w = prf_w; p.S = S; p.Z = Z; p.o = o;
  p.out_bf16 = d->out_dtype == LA_BF16;
  p.N = d->N; p.H = d->H; p.d_k = d->d_k; p.d_v = d->d_v; p.n_psi = d->n_psi;
  p.psi = d->psi; p.normalize = d->normalize; p.eps = d->eps;
  p.in_f32 = d->in_dtype == LA_F32;
  p.log_gate = log_gate;
  if (gamma) {
    for (int h = 0; h < d->H; ++h) {
      p.gamma[h] = gamma[h];
      p.has_decay |= gamma[h] != 1.f;
    }
  }
  return la::launch_decode_step(p, stream) == hipSuccess ? LA_OK : LA_ERR_HIP;
}

}  // namespace

extern "C" {

la_status lin_attn_decode_step(const la_decode_desc* d, const void* q, const void* k, const void* v,
                               const float* gamma, const void* prf_w, float* S, float* Z, void* o,
                               hipStream_t stream) {
  return decode_impl(d, q, k, v, gamma, nullptr, prf_w, S, Z, o, stream);
}

la_status lin_attn_decode_step_gated(const la_decode_desc* d, const void* q, const void* k, const void* v,
                                     const float* log_gate, const void* prf_w, float* S, float* Z, void* o,
                                     hipStream_t stream) {
  if (!log_gate) return LA_ERR_NULL;
  return decode_impl(d, q, k, v, nullptr, log_gate, prf_w, S, Z, o, stream);
}

}  // extern "C"

namespace {

// Both backward entry points: fixed-length batches (cu_seqlens == nullptr) and packed
// variable-length batches.
la_status backward_impl(const la_prefill_desc* d, const int32_t* cu_seqlens, int32_t total_tokens, const void* q,
                        const void* k, const void* v, const float* gamma, const void* prf_w, const float* init_S,
                        const float* init_Z, const void* dout, float* dq, float* dk, float* dv, float* dinit_S,
                        float* dinit_Z, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  la_status st = validate_backward_desc(d, cu_seqlens != nullptr);
  if (st != LA_OK) return st;
  const bool prf = prf_steps(d);
  if (la::is_prf(d->psi) && !prf_w) return LA_ERR_NULL;
  if (!aligned16(prf_w)) return LA_ERR_ALIGN;
  if (cu_seqlens) {
    if (d->layout != LA_LAYOUT_BTHD) return LA_ERR_VALUE;
    if (total_tokens < 0) return LA_ERR_SHAPE;
    if ((reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) != 0) return LA_ERR_ALIGN;
  }
  if (!q || !k || !v || !dout || !dq || !dk || !dv) return LA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dout) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv) || !aligned16(init_S) || !aligned16(init_Z) || !aligned16(dinit_S) ||
      !aligned16(dinit_Z) || !aligned16(workspace))
    return LA_ERR_ALIGN;
  st = check_gamma(gamma, d->H);
  if (st != LA_OK) return st;
  const long long tt = cu_seqlens ? (long long)total_tokens : -1LL;
  const Plan pl = prf ? prf_backward_plan(d) : make_plan(d, tt, false, false, 0, true);
  const size_t need = backward_ws_bytes(d, tt);
  if (!workspace || workspace_bytes < need) return LA_ERR_WORKSPACE;

  la::BackwardParams bp;
  memset(&bp, 0, sizeof bp);
  PrefillParams& p = bp.f;
  p.q = q; p.k = k; p.v = v;
  p.ws = (float*)workspace;
  p.cu_seqlens = cu_seqlens;
  p.total = cu_seqlens ? total_tokens : 0;
  p.B = d->B; p.H = d->H; p.T = d->T;
  if (d->layout == LA_LAYOUT_BTHD) {
    p.tok_rows = d->H; p.head_rows = 1; p.seq_rows = (long long)d->T * d->H;
  } else {
    p.tok_rows = 1; p.head_rows = d->T; p.seq_rows = (long long)d->H * d->T;
  }
  p.d_k = d->d_k; p.d_v = d->d_v; p.n_psi = d->n_psi;
  // random features walk one 64-token step per segment (the same function for every chunk size)
  p.C = prf ? kPrfBwdStep : pl.chunk;
  p.prf_w = prf_w;
  p.psi = d->psi; p.normalize = d->normalize; p.eps = d->eps;
  p.n_chunks = pl.n_chunks; p.seg_chunks = pl.seg_chunks; p.n_seg = pl.n_seg;
  p.n_rec = pl.n_seg; p.rec_per_seg = 1; p.sum_end = pl.n_chunks;
  p.has_decay = fill_log2g(gamma, d->H, p.log2g);
  bp.dout = dout;
  bp.dq = dq; bp.dk = dk; bp.dv = dv;
  bp.rev = (float*)((char*)workspace + pl.ws_bytes);
  const size_t tok_bytes = d->normalize ? (size_t)(cu_seqlens ? (long long)total_tokens * d->H
                                                              : (long long)d->B * d->T * d->H) * 2 * sizeof(float)
                                        : 0;
  bp.tok = d->normalize ? (float*)((char*)workspace + 2 * pl.ws_bytes) : nullptr;
  bp.wt = prf ? (const uint16_t*)((char*)workspace + 2 * pl.ws_bytes + tok_bytes) : nullptr;
  bp.dout_bf16 = d->out_dtype == LA_BF16;

  ScanParams sp;
  memset(&sp, 0, sizeof sp);
  sp.ws = p.ws;
  sp.init_S = init_S;
  sp.init_Z = d->normalize ? init_Z : nullptr;
  sp.cu_seqlens = cu_seqlens; sp.total = p.total;
  sp.BH = d->B * d->H; sp.H = d->H; sp.T = d->T;
  sp.n_psi = d->n_psi; sp.d_v = d->d_v;
  sp.n_seg = pl.n_seg; sp.seg_len = pl.seg_chunks * p.C;
  sp.has_decay = p.has_decay;
  memcpy(sp.log2g, p.log2g, sizeof sp.log2g);
  ScanParams rp = sp;  // the adjoint state: no initial element; its total is the initial state's gradient
  rp.ws = bp.rev;
  rp.init_S = nullptr; rp.init_Z = nullptr;
  rp.final_S = dinit_S;
  rp.final_Z = d->normalize ? dinit_Z : nullptr;
  rp.reverse = 1;

  if (prf) {
    uint16_t* wt = const_cast<uint16_t*>(bp.wt);
    hipError_t e = la::launch_bank_transpose(prf_w, wt, d->H, d->n_psi, stream);  // the bank, [d][p] per head
    if (e == hipSuccess) e = la::launch_prefill_prf_bf16(p, stream, false);       // per-step forward summaries
    if (e == hipSuccess) e = la::launch_segment_scan(sp, stream);                 // the state before each step
    if (e == hipSuccess) e = la::launch_prefill_backward_prf(bp, stream, false);  // dq, per-step adjoint records
    if (e == hipSuccess) e = la::launch_segment_scan(rp, stream);                 // the adjoint state after each step
    if (e == hipSuccess) e = la::launch_prefill_backward_prf(bp, stream, true);   // dk, dv
    return e == hipSuccess ? LA_OK : LA_ERR_HIP;
  }
  if (d->in_dtype == LA_F32 || !la::prefill_backward_supported(d->chunk, d->d_k, d->d_v, d->n_psi, d->psi)) {
    // fp32 inputs, or bf16 at d = 64: the vector-ALU sweeps over the same records
    p.in_f32 = d->in_dtype == LA_F32;
    hipError_t e = p.in_f32 ? la::launch_prefill_f32_summary(p, stream) : la::launch_prefill_bf16_summary(p, stream);
    if (e == hipSuccess) e = la::launch_segment_scan(sp, stream);
    if (e == hipSuccess) e = la::launch_prefill_backward_gen(bp, stream, false);  // query sweep
    if (e == hipSuccess) e = la::launch_segment_scan(rp, stream);
    if (e == hipSuccess) e = la::launch_prefill_backward_gen(bp, stream, true);   // state sweep
    return e == hipSuccess ? LA_OK : LA_ERR_HIP;
  }
  hipError_t e = la::launch_prefill_bf16_summary(p, stream);            // forward segment summaries
  if (e == hipSuccess) e = la::launch_segment_scan(sp, stream);          // forward prefixes
  if (e == hipSuccess) e = la::launch_prefill_backward(bp, stream, false);  // query sweep: dq, adjoint summaries
  if (e == hipSuccess) e = la::launch_segment_scan(rp, stream);          // adjoint state after each segment
  if (e == hipSuccess) e = la::launch_prefill_backward(bp, stream, true);   // state sweep: dk, dv
  return e == hipSuccess ? LA_OK : LA_ERR_HIP;
}

}  // namespace

extern "C" {

la_status lin_attn_prefill_backward(const la_prefill_desc* d, const void* q, const void* k, const void* v,
                                    const float* gamma, const void* prf_w, const float* init_S, const float* init_Z,
                                    const void* dout, float* dq, float* dk, float* dv, float* dinit_S,
                                    float* dinit_Z, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return backward_impl(d, nullptr, 0, q, k, v, gamma, prf_w, init_S, init_Z, dout, dq, dk, dv, dinit_S, dinit_Z,
                       workspace, workspace_bytes, stream);
}

la_status lin_attn_prefill_backward_varlen(const la_prefill_desc* d, const int32_t* cu_seqlens, int32_t total_tokens,
                                           const void* q, const void* k, const void* v, const float* gamma,
                                           const void* prf_w, const float* init_S, const float* init_Z,
                                           const void* dout, float* dq, float* dk, float* dv, float* dinit_S,
                                           float* dinit_Z, void* workspace, size_t workspace_bytes,
                                           hipStream_t stream) {
  if (!cu_seqlens) return LA_ERR_NULL;
  return backward_impl(d, cu_seqlens, total_tokens, q, k, v, gamma, prf_w, init_S, init_Z, dout, dq, dk, dv, dinit_S,
                       dinit_Z, workspace, workspace_bytes, stream);
}

la_status lin_attn_prefill_gated(const la_prefill_desc* d, const void* q, const void* k, const void* v,
                                 const float* log_gate, const float* init_S, const float* init_Z, void* o,
                                 float* final_S, float* final_Z, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
  if (!log_gate) return LA_ERR_NULL;
  return prefill_impl(d, nullptr, 0, q, k, v, nullptr, nullptr, init_S, init_Z, o, final_S, final_Z, workspace,
                      workspace_bytes, stream, nullptr, log_gate);
}

la_status lin_attn_scan_depth(int32_t n_seg, float* ws, int32_t* rounds, hipStream_t stream) {
  if (!ws || !rounds) return LA_ERR_NULL;
  if (n_seg < 1 || n_seg > 65535) return LA_ERR_SHAPE;
  if (!aligned16(ws)) return LA_ERR_ALIGN;
  return la::scan_depth_probe(n_seg, ws, rounds, stream) == hipSuccess ? LA_OK : LA_ERR_HIP;
}

}  // extern "C"
