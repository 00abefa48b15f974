// la_gla.hip -- chunkwise causal linear attention with data-dependent forget gates.
//
// "Linear Attention and Retentive Networks", Data-Dependent Gating Mechanism: the state
// update S_t = G_t . S_{t-1} + k_t^T v_t with G_t = alpha_t 1^T, one gate per state row
// (key feature) and token, alpha_t = exp(log_gate_t) taken from the caller. The chunk
// algebra is that of the decayed form ("Log-Depth Chunked Linear-Attention Scan",
// Implementation notes; the same page's chunkwise representation C) with the scalar
// powers gamma^(j-i) replaced by per-feature gate products. With G_j[p] the cumulative
// log gate inside a chunk of L real tokens (token j inclusive) and G = G_{L-1}:
//   A_ji   = sum_p psi(q_j)_p psi(k_i)_p exp(G_j[p] - G_i[p])          (i <= j)
//   num_j  = sum_p psi(q_j)_p exp(G_j[p]) S_prev[p, :] + sum_i A_ji v_i
//   den_j  = sum_p psi(q_j)_p exp(G_j[p]) Z_prev[p]    + sum_i A_ji + eps
//   S_next = diag(exp(G)) S_prev + sum_i diag(exp(G - G_i)) psi(k_i) v_i^T    (Z likewise)
// Every exponent here is a sum of log gates over tokens between a writer and a reader, so
// it is <= 0 whatever the gates: nothing overflows. Segments combine as
// (a1, X1) (+) (a2, X2) = (a1 a2, diag(a2) X1 + X2) with vector a (the scan, la_scan.hip).
//
// Two implementations, both with chunks of 32 tokens:
//  - bf16 inputs: the state terms on MFMA (outputs psi(q_j) e^{G_j} S_prev and the update
//    psi(k_i) e^{G - G_i} v_i^T, both factors carried as bf16 hi + lo), the intra-chunk
//    scores A on the vector ALUs as running products of the gates (for a fixed key i the
//    factor exp(G_j - G_i) is the product of the gates of tokens i+1..j, so it is built by
//    one multiply per token with every factor <= 1: no exponential per pair, no overflow).
//  - fp32 inputs: fp32 on the vector ALUs throughout (the fp32 tolerance leaves no room for
//    two-term bf16 products); each thread keeps an 8 x 8 block of the state in registers
//    (rows 8 pb.., columns 8 eb..; the pb lanes of a column block are adjacent, so the sums
//    over state rows reduce across 16 (or 8) consecutive lanes).
#include "la_device.hpp"
#include "la_kernels.hpp"

namespace la {
namespace {

constexpr int GC = 32;  // chunk

template <int NP, int DV>
struct GlaGeo {
  static constexpr int PB = NP / 8, EB = DV / 8, NT = PB * EB;  // thread grid: row blocks x column blocks
  // LDS (floats)
  static constexpr int Q = 0;                // psi(q) [GC][NP]
  static constexpr int K = Q + GC * NP;      // psi(k) [GC][NP]
  static constexpr int V = K + GC * NP;      // v [GC][DV]
  static constexpr int G = V + GC * DV;      // log gates, then their cumulative sums [GC][NP]
  static constexpr int QH = G + GC * NP;     // psi(q_j) exp(G_j) [GC][NP]
  static constexpr int KH = QH + GC * NP;    // psi(k_i) exp(G - G_i) [GC][NP]
  static constexpr int A = KH + GC * NP;     // scores [GC][GC]
  static constexpr int DEN = A + GC * GC;    // [GC]
  static constexpr int Z = DEN + GC;         // normaliser [NP]
  static constexpr int AT = Z + NP;          // exp(G) [NP]
  static constexpr int FLOATS = AT + NP;
  static_assert(PB == 8 || PB == 16, "row blocks reduce within 8 or 16 lanes");
  static_assert(NT % 64 == 0 || NT == 64, "whole waves");
};

__device__ __forceinline__ float in_elem(const void* base, size_t i, bool f32) {
  return f32 ? ((const float*)base)[i] : bf16_bits_to_f32(((const uint16_t*)base)[i]);
}

// One chunk tile of `width` columns from rows [0, valid) of a token-row tensor (rows `rs`
// elements apart) into LDS fp32; rows past `valid` are zero. psi = identity or elu+1.
__device__ __forceinline__ void load_tile(float* dst, const void* src, size_t row0, size_t rs, int width, int valid,
                                          bool f32, bool elu, int nt) {
  for (int idx = threadIdx.x; idx < GC * width; idx += nt) {
    const int r = idx / width, c = idx - r * width;
    float x = 0.f;
    if (r < valid) {
      x = in_elem(src, row0 + (size_t)r * rs + c, f32);
      if (elu) x = elu1(x);
    }
    dst[idx] = x;
  }
}

__device__ __forceinline__ void load_gates(float* dst, const float* lg, size_t row0, size_t rs, int width, int valid,
                                           int nt) {
  for (int idx = threadIdx.x; idx < GC * width; idx += nt) {
    const int r = idx / width, c = idx - r * width;
    dst[idx] = r < valid ? lg[row0 + (size_t)r * rs + c] : 0.f;  // padded tokens: gate 1
  }
}

// Cumulative log gates per feature (in place) and exp(G) of the chunk; returns G for
// thread p < NP (else 0).
template <int NP>
__device__ __forceinline__ float gate_cumsum(float* sm, int g_off, int at_off) {
  float c = 0.f;
  if (threadIdx.x < NP) {
    const int p = threadIdx.x;
#pragma unroll
    for (int r = 0; r < GC; ++r) {
      c += sm[g_off + r * NP + p];
      sm[g_off + r * NP + p] = c;
    }
    sm[at_off + p] = expf(c);
  }
  return c;
}

// S block += sum_i KH[i][rows] v[i][cols]; S block *= exp(G) first. Z likewise (threads p < NP).
template <int NP, int DV>
__device__ __forceinline__ void state_update(float (&S)[8][8], const float* sm, int pb, int eb, bool norm) {
  using G = GlaGeo<NP, DV>;
  float at[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) at[r] = sm[G::AT + 8 * pb + r];
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int c = 0; c < 8; ++c) S[r][c] *= at[r];
  for (int i = 0; i < GC; ++i) {
    const f32x4 k0 = *(const f32x4*)(sm + G::KH + i * NP + 8 * pb), k1 = *(const f32x4*)(sm + G::KH + i * NP + 8 * pb + 4);
    const f32x4 v0 = *(const f32x4*)(sm + G::V + i * DV + 8 * eb), v1 = *(const f32x4*)(sm + G::V + i * DV + 8 * eb + 4);
    const float kr[8] = {k0[0], k0[1], k0[2], k0[3], k1[0], k1[1], k1[2], k1[3]};
    const float vc[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
      for (int c = 0; c < 8; ++c) S[r][c] += kr[r] * vc[c];
  }
  (void)norm;
}

template <int NP, int DV>
__device__ __forceinline__ void z_update(float* sm) {
  using G = GlaGeo<NP, DV>;
  if (threadIdx.x < NP) {
    const int p = threadIdx.x;
    float z = sm[G::AT + p] * sm[G::Z + p];
    for (int i = 0; i < GC; ++i) z += sm[G::KH + i * NP + p];
    sm[G::Z + p] = z;
  }
}

template <int NP, int DV>
__device__ __forceinline__ void build_kh(float* sm, int nt) {
  using G = GlaGeo<NP, DV>;
  for (int idx = threadIdx.x; idx < GC * NP; idx += nt) {
    const int p = idx % NP;
    sm[G::KH + idx] = sm[G::K + idx] * expf(sm[G::G + (GC - 1) * NP + p] - sm[G::G + idx]);
  }
}

// Segment summaries: fold the segment's chunks into (S, Z) and the segment's per-row decay
// exp(sum of its log gates). Workspace record [S (NP*DV)][Z (NP)][decay (NP)].
template <int NP, int DV>
__global__ __launch_bounds__((GlaGeo<NP, DV>::NT)) void k_summary_gla(PrefillParams p) {
  using G = GlaGeo<NP, DV>;
  extern __shared__ __align__(16) float sm[];
  const int bh = blockIdx.x, seg = blockIdx.y, tid = threadIdx.x;
  const int pb = tid % G::PB, eb = tid / G::PB;
  const bool f32 = p.in_f32 != 0, elu = p.psi == LA_PSI_ELU1, norm = p.normalize != 0;
  const SeqSpan sq = seq_span(p, bh);
  const int T = sq.T, n_chunks = (T + GC - 1) / GC;
  const size_t rk = (size_t)p.tok_rows * NP, rv = (size_t)p.tok_rows * DV;
  const int c0 = seg * p.seg_chunks, c1 = min(c0 + p.seg_chunks, n_chunks);
  float S[8][8];
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int c = 0; c < 8; ++c) S[r][c] = 0.f;
  if (tid < NP) sm[G::Z + tid] = 0.f;
  float segtot = 0.f;  // thread p: the segment's summed log gate of row p
  for (int c = c0; c < c1; ++c) {
    const int L = min(GC, T - c * GC);
    __syncthreads();
    const size_t t0 = (size_t)c * GC;
    load_tile(sm + G::K, p.k, (sq.row0 + t0 * p.tok_rows) * NP, rk, NP, L, f32, elu, G::NT);
    load_tile(sm + G::V, p.v, (sq.row0 + t0 * p.tok_rows) * DV, rv, DV, L, f32, false, G::NT);
    load_gates(sm + G::G, p.log_gate, (sq.row0 + t0 * p.tok_rows) * NP, rk, NP, L, G::NT);
    __syncthreads();
    segtot += gate_cumsum<NP>(sm, G::G, G::AT);
    __syncthreads();
    build_kh<NP, DV>(sm, G::NT);
    __syncthreads();
    state_update<NP, DV>(S, sm, pb, eb, norm);
    if (norm) z_update<NP, DV>(sm);
  }
  __syncthreads();
  const size_t REC = (size_t)NP * DV + 2 * NP;
  float* out = p.ws + ((size_t)bh * p.n_seg + seg) * REC;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    float* row = out + (size_t)(8 * pb + r) * DV + 8 * eb;
    *(f32x4*)row = f32x4{S[r][0], S[r][1], S[r][2], S[r][3]};
    *(f32x4*)(row + 4) = f32x4{S[r][4], S[r][5], S[r][6], S[r][7]};
  }
  if (tid < NP) {
    out[(size_t)NP * DV + tid] = norm ? sm[G::Z + tid] : 0.f;
    out[(size_t)NP * DV + NP + tid] = expf(segtot);
  }
}

// Sum over the PB row-block lanes (adjacent lanes) of a column block.
template <int PB>
__device__ __forceinline__ float rowblock_sum(float x) {
#pragma unroll
  for (int off = 1; off < PB; off <<= 1) x += __shfl_xor(x, off);
  return x;
}

template <int NP, int DV, bool OBF>
__global__ __launch_bounds__((GlaGeo<NP, DV>::NT)) void k_output_gla(PrefillParams p) {
  using G = GlaGeo<NP, DV>;
  extern __shared__ __align__(16) float sm[];
  const int bh = blockIdx.x, seg = blockIdx.y, tid = threadIdx.x;
  const int pb = tid % G::PB, eb = tid / G::PB;
  const bool f32 = p.in_f32 != 0, elu = p.psi == LA_PSI_ELU1, norm = p.normalize != 0;
  const SeqSpan sq = seq_span(p, bh);
  const int T = sq.T, n_chunks = (T + GC - 1) / GC;
  const size_t rk = (size_t)p.tok_rows * NP, rv = (size_t)p.tok_rows * DV;
  const int c0 = seg * p.seg_chunks, c1 = min(c0 + p.seg_chunks, n_chunks);
  if (c0 >= c1) return;
  // the segment's exclusive prefix (written by the scan)
  const size_t REC = (size_t)NP * DV + 2 * NP;
  const float* pre = p.ws + ((size_t)bh * p.n_seg + seg) * REC;
  float S[8][8];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const float* row = pre + (size_t)(8 * pb + r) * DV + 8 * eb;
    const f32x4 a = *(const f32x4*)row, b = *(const f32x4*)(row + 4);
    S[r][0] = a[0]; S[r][1] = a[1]; S[r][2] = a[2]; S[r][3] = a[3];
    S[r][4] = b[0]; S[r][5] = b[1]; S[r][6] = b[2]; S[r][7] = b[3];
  }
  if (tid < NP) sm[G::Z + tid] = norm ? pre[(size_t)NP * DV + tid] : 0.f;
  constexpr int OES = OBF ? 2 : 4;
  unsigned char* ob = (unsigned char*)p.o + sq.row0 * DV * OES;
  for (int c = c0; c < c1; ++c) {
    const int L = min(GC, T - c * GC);
    __syncthreads();
    const size_t t0 = (size_t)c * GC;
    load_tile(sm + G::Q, p.q, (sq.row0 + t0 * p.tok_rows) * NP, rk, NP, L, f32, elu, G::NT);
    load_tile(sm + G::K, p.k, (sq.row0 + t0 * p.tok_rows) * NP, rk, NP, L, f32, elu, G::NT);
    load_tile(sm + G::V, p.v, (sq.row0 + t0 * p.tok_rows) * DV, rv, DV, L, f32, false, G::NT);
    load_gates(sm + G::G, p.log_gate, (sq.row0 + t0 * p.tok_rows) * NP, rk, NP, L, G::NT);
    __syncthreads();
    gate_cumsum<NP>(sm, G::G, G::AT);
    __syncthreads();
    // psi(q_j) exp(G_j), psi(k_i) exp(G - G_i), and the scores
    for (int idx = tid; idx < GC * NP; idx += G::NT) sm[G::QH + idx] = sm[G::Q + idx] * expf(sm[G::G + idx]);
    build_kh<NP, DV>(sm, G::NT);
    for (int idx = tid; idx < GC * GC; idx += G::NT) {
      const int j = idx / GC, i = idx - j * GC;
      float a = 0.f;
      if (i <= j) {
        const float* qj = sm + G::Q + j * NP;
        const float* ki = sm + G::K + i * NP;
        const float* gj = sm + G::G + j * NP;
        const float* gi = sm + G::G + i * NP;
        for (int f = 0; f < NP; ++f) a += qj[f] * ki[f] * expf(gj[f] - gi[f]);
      }
      sm[G::A + idx] = a;
    }
    __syncthreads();
    if (norm && tid < GC) {
      const int j = tid;
      float d = 0.f;
      for (int f = 0; f < NP; ++f) d += sm[G::QH + j * NP + f] * sm[G::Z + f];
      for (int i = 0; i <= j; ++i) d += sm[G::A + j * GC + i];
      sm[G::DEN + j] = d + p.eps;
    }
    __syncthreads();
    // outputs: inter part reduced over the row blocks; the lane pb == j % PB finishes token j
    for (int j = 0; j < GC; ++j) {
      float part[8];
      {
        float qh[8];
        const f32x4 a = *(const f32x4*)(sm + G::QH + j * NP + 8 * pb), b = *(const f32x4*)(sm + G::QH + j * NP + 8 * pb + 4);
        qh[0] = a[0]; qh[1] = a[1]; qh[2] = a[2]; qh[3] = a[3]; qh[4] = b[0]; qh[5] = b[1]; qh[6] = b[2]; qh[7] = b[3];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float s = 0.f;
#pragma unroll
          for (int r = 0; r < 8; ++r) s += qh[r] * S[r][e];
          part[e] = rowblock_sum<G::PB>(s);
        }
      }
      if (pb == j % G::PB && j < L) {
        for (int i = 0; i <= j; ++i) {
          const float a = sm[G::A + j * GC + i];
          const f32x4 v0 = *(const f32x4*)(sm + G::V + i * DV + 8 * eb), v1 = *(const f32x4*)(sm + G::V + i * DV + 8 * eb + 4);
          part[0] += a * v0[0]; part[1] += a * v0[1]; part[2] += a * v0[2]; part[3] += a * v0[3];
          part[4] += a * v1[0]; part[5] += a * v1[1]; part[6] += a * v1[2]; part[7] += a * v1[3];
        }
        const float inv = norm ? 1.f / sm[G::DEN + j] : 1.f;
        unsigned char* orow = ob + (size_t)(t0 + j) * rv * OES + (size_t)(8 * eb) * OES;
        if (OBF) {
          uint16_t h[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) h[e] = __builtin_bit_cast(uint16_t, (__bf16)(part[e] * inv));
          *(uint4*)orow = __builtin_bit_cast(uint4, h);
        } else {
          *(f32x4*)orow = f32x4{part[0] * inv, part[1] * inv, part[2] * inv, part[3] * inv};
          *(f32x4*)(orow + 16) = f32x4{part[4] * inv, part[5] * inv, part[6] * inv, part[7] * inv};
        }
      }
    }
    __syncthreads();  // Z is read by the denominators above before it is updated
    state_update<NP, DV>(S, sm, pb, eb, norm);
    if (norm) z_update<NP, DV>(sm);
  }
}

// ======================= bf16 inputs: state terms on MFMA ===============================

// LDS image of the MFMA kernels (D = n_psi = d_k = d_v). bf16 tiles have pitch D + 8.
template <int D>
struct MGeo {
  static constexpr int NT = 2 * D, NW = D / 32, P = D + 8, AP = GC + 8;
  // fp32 regions (float offsets)
  static constexpr int PQ = 0;              // psi(q) [GC][D]
  static constexpr int PK = PQ + GC * D;    // psi(k) [GC][D]
  static constexpr int AL = PK + GC * D;    // log gates, then the gates exp(log_gate) [GC][D]
  static constexpr int APART = AL + GC * D; // score partials [NW][GC][GC]
  static constexpr int AEND = APART + NW * GC * GC;  // exp(G) [D]
  static constexpr int ZV = AEND + D;       // Z_prev [D]
  static constexpr int DEN = ZV + D;        // [GC]
  static constexpr int FEND = DEN + GC;
  // bf16 regions (element offsets from the end of the fp32 image)
  static constexpr int H0 = 2 * FEND;
  static constexpr int QH = H0, QL = QH + GC * P, KH = QL + GC * P, KL = KH + GC * P, V = KL + GC * P;
  static constexpr int SAH = V + GC * P, SAL = SAH + GC * AP;  // A hi / lo [GC][AP]
  // the off-diagonal half block of the scores: q~ (rows GC/2.., zero above) and k~ (rows
  // ..GC/2, zero below), referenced to the last token of the first half
  static constexpr int XQH = SAL + GC * AP, XQL = XQH + GC * P, XKH = XQL + GC * P, XKL = XKH + GC * P;
  static constexpr int HEND = XKL + GC * P;
  static constexpr int BYTES = HEND * 2;
  static_assert(FEND % 4 == 0 && (GC * P) % 8 == 0 && (GC * AP) % 8 == 0, "16-byte aligned regions");
};

// The summary pass's LDS image: psi(k), the gates, the chunk's end decays and the k^ and v
// tiles, without the output pass's query, score and off-diagonal regions (59 KiB at d = 128,
// so two summary workgroups share a CU). Offsets as in MGeo.
template <int D>
struct MSumGeo {
  static constexpr int NT = 2 * D, NW = D / 32, P = D + 8;
  static constexpr int PK = 0, AL = PK + GC * D, AEND = AL + GC * D, FEND = AEND + D;
  static constexpr int H0 = 2 * FEND;
  static constexpr int KH = H0, KL = KH + GC * P, V = KL + GC * P;
  static constexpr int HEND = V + GC * P;
  static constexpr int BYTES = HEND * 2;
  static_assert(FEND % 4 == 0 && (GC * P) % 8 == 0, "16-byte aligned regions");
};

// Global tile of GC token rows x D bf16 (16-byte pieces) / fp32 log gates.
template <int D>
struct MLoad {
  static constexpr int NT = 2 * D;
  static constexpr int PB = GC * D / 8 / NT;   // bf16 pieces per thread per tensor (2)
  static constexpr int PF = GC * D / 4 / NT;   // fp32 pieces per thread (4)
  uint4 q[PB], k[PB], v[PB];
  uint4 g[PF];
};
template <int D>
__device__ __forceinline__ void mload(MLoad<D>& T, const PrefillParams& p, long long r0, int L) {
  constexpr int NT = 2 * D, RP = D / 8, RPF = D / 4;  // pieces per row
  const uint32_t rsb = (uint32_t)p.tok_rows * D * 2, rsf = (uint32_t)p.tok_rows * D * 4;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc((const uint16_t*)p.q + r0 * D, rows_extent(L, rsb, D * 2));
  const __amdgpu_buffer_rsrc_t rk = make_rsrc((const uint16_t*)p.k + r0 * D, rows_extent(L, rsb, D * 2));
  const __amdgpu_buffer_rsrc_t rv = make_rsrc((const uint16_t*)p.v + r0 * D, rows_extent(L, rsb, D * 2));
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(p.log_gate + r0 * D, rows_extent(L, rsf, D * 4));
#pragma unroll
  for (int i = 0; i < MLoad<D>::PB; ++i) {
    const int pc = threadIdx.x + i * NT, row = pc / RP, col = (pc % RP) * 8;
    const uint32_t off = (uint32_t)row * rsb + (uint32_t)col * 2;
    T.q[i] = buf_load16(rq, off);
    T.k[i] = buf_load16(rk, off);
    T.v[i] = buf_load16(rv, off);
  }
#pragma unroll
  for (int i = 0; i < MLoad<D>::PF; ++i) {
    const int pc = threadIdx.x + i * NT, row = pc / RPF, col = (pc % RPF) * 4;
    T.g[i] = buf_load16(rg, (uint32_t)row * rsf + (uint32_t)col * 4);
  }
}

// Commit: psi(q), psi(k) as fp32 (rows >= L zero), v, and the log gates (summary) or the
// gates exp(log_gate) (output pass, Q); padded rows have gate 1.
template <int D, bool Q, typename G = MGeo<D>>
__device__ __forceinline__ void mcommit(const MLoad<D>& T, float* sf, __bf16* sh, int L, bool elu) {
  constexpr int NT = 2 * D, RP = D / 8, RPF = D / 4;
#pragma unroll
  for (int i = 0; i < MLoad<D>::PB; ++i) {
    const int pc = threadIdx.x + i * NT, row = pc / RP, col = (pc % RP) * 8;
    const bf16x8 kx = __builtin_bit_cast(bf16x8, T.k[i]);
    f32x4 k0, k1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a = from_bf16(kx[j]), b = from_bf16(kx[4 + j]);
      k0[j] = row < L ? (elu ? elu1(a) : a) : 0.f;
      k1[j] = row < L ? (elu ? elu1(b) : b) : 0.f;
    }
    *(f32x4*)(sf + G::PK + row * D + col) = k0;
    *(f32x4*)(sf + G::PK + row * D + col + 4) = k1;
    if constexpr (Q) {
      const bf16x8 qx = __builtin_bit_cast(bf16x8, T.q[i]);
      f32x4 q0, q1;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float a = from_bf16(qx[j]), b = from_bf16(qx[4 + j]);
        q0[j] = row < L ? (elu ? elu1(a) : a) : 0.f;
        q1[j] = row < L ? (elu ? elu1(b) : b) : 0.f;
      }
      *(f32x4*)(sf + G::PQ + row * D + col) = q0;
      *(f32x4*)(sf + G::PQ + row * D + col + 4) = q1;
    }
    *(uint4*)(sh + G::V + row * G::P + col) = T.v[i];
  }
#pragma unroll
  for (int i = 0; i < MLoad<D>::PF; ++i) {
    const int pc = threadIdx.x + i * NT, row = pc / RPF, col = (pc % RPF) * 4;
    const f32x4 g = __builtin_bit_cast(f32x4, T.g[i]);
    f32x4 x = row < L ? g : f32x4{0.f, 0.f, 0.f, 0.f};  // padded tokens: log gate 0, gate 1
    if constexpr (Q) x = f32x4{__expf(x[0]), __expf(x[1]), __expf(x[2]), __expf(x[3])};
    *(f32x4*)(sf + G::AL + row * D + col) = x;
  }
}

// Per feature p (threads p < D): G_j = cumulative log gate, k^_i = psi(k_i) e^{G_end - G_i}
// (hi + lo), and with Q also q^_j = psi(q_j) e^{G_j} (hi + lo) and the gates exp(log_gate)
// in place of the log gates. Returns G_end (this feature's summed log gate over the chunk)
// and adds sum_i k^_i to *ksum.
template <int D, bool Q, typename G = MGeo<D>>
__device__ __forceinline__ float feature_pass(float* sf, __bf16* sh, float* ksum) {
  const int p = threadIdx.x;
  float g[GC];
  float c = 0.f;
#pragma unroll
  for (int j = 0; j < GC; ++j) {
    const float lg = sf[G::AL + j * D + p];
    c += lg;
    g[j] = c;
    if constexpr (Q) {
      sf[G::AL + j * D + p] = __expf(lg);
      const bf16_pair pr = split_bf16(sf[G::PQ + j * D + p] * __expf(c));
      sh[G::QH + j * G::P + p] = pr.hi;
      sh[G::QL + j * G::P + p] = pr.lo;
    }
  }
  float ks = 0.f;
#pragma unroll
  for (int i = 0; i < GC; ++i) {
    const float kh = sf[G::PK + i * D + p] * __expf(c - g[i]);
    ks += kh;
    const bf16_pair pr = split_bf16(kh);
    sh[G::KH + i * G::P + p] = pr.hi;
    sh[G::KL + i * G::P + p] = pr.lo;
  }
  *ksum = ks;
  return c;
}

// State update of wave w's columns: S[p][e] = e^{G_end[p]} S[p][e] + sum_i k^_i[p] v_i[e].
template <int D, typename G = MGeo<D>>
__device__ __forceinline__ void mstate(f32x16 (&S)[D / 32], const float* sf, const __bf16* sh, int w, int lane) {
#pragma unroll
  for (int pt = 0; pt < D / 32; ++pt) {
#pragma unroll
    for (int r = 0; r < 16; ++r) S[pt][r] *= sf[G::AEND + 32 * pt + dtile_row(r, lane)];
#pragma unroll
    for (int i0 = 0; i0 < GC; i0 += 16) {
      const bf16x8 v = ld_rows8(sh + G::V, G::P, i0, 32 * w, lane);    // B[k=i][n=e] = v_i[e]
      S[pt] = mfma32(ld_rows8(sh + G::KH, G::P, i0, 32 * pt, lane), v, S[pt]);  // A[m=p][k=i] = k^_i[p]
      S[pt] = mfma32(ld_rows8(sh + G::KL, G::P, i0, 32 * pt, lane), v, S[pt]);
    }
  }
}

template <int D>
__global__ __launch_bounds__(2 * D) void k_summary_gla_m(PrefillParams p) {
  using G = MSumGeo<D>;
  extern __shared__ __align__(16) unsigned char smem[];
  float* sf = (float*)smem;
  __bf16* sh = (__bf16*)smem;
  const int bh = blockIdx.x, seg = blockIdx.y, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const bool elu = p.psi == LA_PSI_ELU1, norm = p.normalize != 0;
  const SeqSpan sq = seq_span(p, bh);
  const int T = sq.T, n_chunks = (T + GC - 1) / GC;
  const int c0 = seg * p.seg_chunks, c1 = min(min(c0 + p.seg_chunks, n_chunks), p.sum_end);
  f32x16 S[D / 32];
#pragma unroll
  for (int pt = 0; pt < D / 32; ++pt)
#pragma unroll
    for (int r = 0; r < 16; ++r) S[pt][r] = 0.f;
  float z = 0.f, segtot = 0.f;  // thread p < D: Z[p] and the segment's summed log gate
  MLoad<D> T0;
  if (c0 < c1) mload<D>(T0, p, sq.row0 + (long long)c0 * GC * p.tok_rows, min(GC, T - c0 * GC));
  for (int c = c0; c < c1; ++c) {
    const int L = min(GC, T - c * GC);
    lds_barrier();
    mcommit<D, false, G>(T0, sf, sh, L, elu);
    if (c + 1 < c1) mload<D>(T0, p, sq.row0 + (long long)(c + 1) * GC * p.tok_rows, min(GC, T - (c + 1) * GC));
    lds_barrier();
    if (tid < D) {
      float ks;
      const float ge = feature_pass<D, false, G>(sf, sh, &ks);
      const float ae = __expf(ge);
      sf[G::AEND + tid] = ae;
      z = ae * z + ks;
      segtot += ge;
    }
    lds_barrier();
    mstate<D, G>(S, sf, sh, w, lane);
  }
  const size_t REC = (size_t)D * D + 2 * D;
  float* out = p.ws + rec_index(p, bh, seg) * REC;
#pragma unroll
  for (int pt = 0; pt < D / 32; ++pt)
#pragma unroll
    for (int r = 0; r < 16; ++r) out[(size_t)(32 * pt + dtile_row(r, lane)) * D + 32 * w + (lane & 31)] = S[pt][r];
  if (tid < D) {
    out[(size_t)D * D + tid] = norm ? z : 0.f;
    out[(size_t)D * D + D + tid] = __expf(segtot);
  }
}

template <int D, bool OBF>
__global__ __launch_bounds__(2 * D) void k_output_gla_m(PrefillParams p) {
  using G = MGeo<D>;
  constexpr int NT = 2 * D, NW = D / 32, TPT = NT / GC;  // threads per token in the reductions
  extern __shared__ __align__(16) unsigned char smem[];
  float* sf = (float*)smem;
  __bf16* sh = (__bf16*)smem;
  const int bh = blockIdx.x, seg = blockIdx.y, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const bool elu = p.psi == LA_PSI_ELU1, norm = p.normalize != 0;
  const SeqSpan sq = seq_span(p, bh);
  const int T = sq.T, n_chunks = (T + GC - 1) / GC;
  const int c0 = seg * p.seg_chunks, c1 = min(c0 + p.seg_chunks, n_chunks);
  if (c0 >= c1) return;
  const size_t REC = (size_t)D * D + 2 * D;
  const float* pre = p.ws + rec_index(p, bh, seg) * REC;
  f32x16 S[D / 32];  // S[p][e]: rows p in tile pt, column e = 32 w + lane % 32
#pragma unroll
  for (int pt = 0; pt < D / 32; ++pt)
#pragma unroll
    for (int r = 0; r < 16; ++r) S[pt][r] = pre[(size_t)(32 * pt + dtile_row(r, lane)) * D + 32 * w + (lane & 31)];
  float z = (norm && tid >= D) ? pre[(size_t)D * D + tid - D] : 0.f;  // Z_prev[p] of thread D + p
  constexpr int OES = OBF ? 2 : 4;
  constexpr int HC = GC / 2;
  const uint32_t rso = (uint32_t)p.tok_rows * D * OES;
  // rows 0..HC-1 of q~ and HC.. of k~ stay zero: the MFMA over the full tile then yields the
  // off-diagonal half block only
  for (int x = tid; x < HC * G::P; x += NT) {
    sh[G::XQH + x] = to_bf16(0.f);
    sh[G::XQL + x] = to_bf16(0.f);
    sh[G::XKH + HC * G::P + x] = to_bf16(0.f);
    sh[G::XKL + HC * G::P + x] = to_bf16(0.f);
  }
  MLoad<D> T0;
  mload<D>(T0, p, sq.row0 + (long long)c0 * GC * p.tok_rows, min(GC, T - c0 * GC));
  for (int c = c0; c < c1; ++c) {
    const int L = min(GC, T - c * GC);
    const long long r0 = sq.row0 + (long long)c * GC * p.tok_rows;
    lds_barrier();
    mcommit<D, true>(T0, sf, sh, L, elu);
    if (tid >= D) sf[G::ZV + tid - D] = z;
    if (c + 1 < c1) mload<D>(T0, p, sq.row0 + (long long)(c + 1) * GC * p.tok_rows, min(GC, T - (c + 1) * GC));
    lds_barrier();
    // q^_j = psi(q_j) prod_{s<=j} alpha_s (threads p < D) and k^_i = psi(k_i) prod_{s>i} alpha_s
    // (threads D + p): running products of the gates, every factor <= 1
    // (the chunk's gates and features of this thread's feature are read into registers first,
    // so the chains wait on no LDS read)
    float ks = 0.f;
    if (tid < D) {
      const int pf = tid;
      float av[GC], qv[GC];
#pragma unroll
      for (int j = 0; j < GC; ++j) {
        av[j] = sf[G::AL + j * D + pf];
        qv[j] = sf[G::PQ + j * D + pf];
      }
      float eg = 1.f, ex = 1.f;  // prod_{s<=j} alpha_s, and prod_{HC<=s<=j} alpha_s
#pragma unroll
      for (int j = 0; j < GC; ++j) {
        const float a = av[j], q = qv[j];
        eg *= a;
        const bf16_pair pr = split_bf16(q * eg);
        sh[G::QH + j * G::P + pf] = pr.hi;
        sh[G::QL + j * G::P + pf] = pr.lo;
        if (j >= HC) {
          ex *= a;
          const bf16_pair px = split_bf16(q * ex);
          sh[G::XQH + j * G::P + pf] = px.hi;
          sh[G::XQL + j * G::P + pf] = px.lo;
        }
      }
      sf[G::AEND + pf] = eg;
    } else {
      const int pf = tid - D;
      float av[GC], kv[GC];
#pragma unroll
      for (int i = 0; i < GC; ++i) {
        av[i] = sf[G::AL + i * D + pf];
        kv[i] = sf[G::PK + i * D + pf];
      }
      float f = 1.f, fx = 1.f;  // prod_{s>i} alpha_s, and prod_{i<s<HC} alpha_s
#pragma unroll
      for (int i = GC - 1; i >= 0; --i) {
        const float k = kv[i], a = av[i];
        const float kh = k * f;
        ks += kh;
        const bf16_pair pr = split_bf16(kh);
        sh[G::KH + i * G::P + pf] = pr.hi;
        sh[G::KL + i * G::P + pf] = pr.lo;
        f *= a;
        if (i < HC) {
          const bf16_pair px = split_bf16(k * fx);
          sh[G::XKH + i * G::P + pf] = px.hi;
          sh[G::XKL + i * G::P + pf] = px.lo;
          fx *= a;
        }
      }
    }
    lds_barrier();

    // scores A_ji = sum_p psi(q_j)[p] psi(k_i)[p] prod_{s=i+1..j} alpha_s[p]
    //  - i, j in the same half: thread (i, slice of 16 features) walks j upwards through its
    //    half, multiplying its running key features by each token's gates (every factor <= 1)
    //  - j in the second half, i in the first: sum_p q~_j[p] k~_i[p] with both factors
    //    referenced to token HC - 1 (so both <= 1), one MFMA tile per wave over its features
    {
      const int i = tid & 31, f0 = (tid >> 5) * 16, jb = i & HC;
      float kk[16];
#pragma unroll
      for (int f = 0; f < 16; f += 4) *(f32x4*)(kk + f) = *(const f32x4*)(sf + G::PK + i * D + f0 + f);
#pragma unroll
      for (int j0 = 0; j0 < HC; j0 += 4) {
        float part[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int j = jb + j0 + jj;
          // branch-free (a select after the product), so the gate reads need not wait on a branch
          const bool on = j > i;
#pragma unroll
          for (int f = 0; f < 16; f += 4) {
            const f32x4 a = *(const f32x4*)(sf + G::AL + j * D + f0 + f);
#pragma unroll
            for (int u = 0; u < 4; ++u) kk[f + u] = on ? kk[f + u] * a[u] : kk[f + u];
          }
          float acc[4];
#pragma unroll
          for (int f = 0; f < 16; f += 4) {
            const f32x4 qv = *(const f32x4*)(sf + G::PQ + j * D + f0 + f);
            acc[f / 4] = qv[0] * kk[f] + qv[1] * kk[f + 1] + qv[2] * kk[f + 2] + qv[3] * kk[f + 3];
          }
          part[jj] = j >= i ? (acc[0] + acc[1]) + (acc[2] + acc[3]) : 0.f;
        }
        // lanes l and l + 32 hold the same key i: combine, then one partial per wave to LDS
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) part[jj] += __shfl_xor(part[jj], 32);
        if (lane < 32) {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) sf[G::APART + (w * GC + jb + j0 + jj) * GC + i] = part[jj];
        }
      }
      f32x16 x;
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = 0.f;
#pragma unroll
      for (int k0 = 0; k0 < 32; k0 += 16) {
        const bf16x8 qh = ld_cols8(sh + G::XQH, G::P, 0, 32 * w + k0, lane);  // A[m=j][k=p] = q~_j[p]
        const bf16x8 ql = ld_cols8(sh + G::XQL, G::P, 0, 32 * w + k0, lane);
        const bf16x8 kh = ld_cols8(sh + G::XKH, G::P, 0, 32 * w + k0, lane);  // B[k=p][n=i] = k~_i[p]
        const bf16x8 kl = ld_cols8(sh + G::XKL, G::P, 0, 32 * w + k0, lane);
        x = mfma32(qh, kh, x);
        x = mfma32(qh, kl, x);
        x = mfma32(ql, kh, x);
      }
      if (i < HC) {  // rows j >= HC: registers 8..15
#pragma unroll
        for (int r = 8; r < 16; ++r) sf[G::APART + (w * GC + dtile_row(r, lane)) * GC + i] = x[r];
      }
    }
    lds_barrier();
    // A as hi + lo; den_j = q^_j . Z_prev + sum_i A_ji + eps (TPT threads per token)
    {
      const int j = tid / TPT, r = tid % TPT;
      constexpr int IW = GC / TPT, FW = D / TPT;
      float rs = 0.f;
#pragma unroll
      for (int ii = 0; ii < IW; ++ii) {
        const int i = r * IW + ii;
        float a = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) a += sf[G::APART + (ww * GC + j) * GC + i];
        a = i <= j ? a : 0.f;  // the first half's rows against the second half's keys are never written
        rs += a;
        const bf16_pair pr = split_bf16(a);
        sh[G::SAH + j * G::AP + i] = pr.hi;
        sh[G::SAL + j * G::AP + i] = pr.lo;
      }
      if (norm) {
        float zs = 0.f;
        for (int f = r * FW; f < r * FW + FW; ++f)
          zs += (from_bf16(sh[G::QH + j * G::P + f]) + from_bf16(sh[G::QL + j * G::P + f])) * sf[G::ZV + f];
        rs += zs;
#pragma unroll
        for (int o = 1; o < TPT; o <<= 1) rs += __shfl_xor(rs, o);
        if (r == 0) sf[G::DEN + j] = rs + p.eps;
      }
    }
    if (norm && tid >= D) z = sf[G::AEND + tid - D] * z + ks;  // Z_prev read above; written at the next commit
    lds_barrier();

    // outputs, transposed: num^T[e][j] = sum_p S[p][e] q^_j[p] + sum_i v_i[e] A_ji (M = e, N = j)
    {
      f32x16 acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
      for (int pt = 0; pt < D / 32; ++pt) {
        bf16x8 shi[2], slo[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          float x[8];
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) x[jj] = S[pt][8 * q + jj];
          split8_trunc(x, shi[q], slo[q]);
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const bf16x8 qh = ld_cols8_perm(sh + G::QH, G::P, 0, 32 * pt, q, lane);  // B[k=p][n=j] = q^_j[p]
          const bf16x8 ql = ld_cols8_perm(sh + G::QL, G::P, 0, 32 * pt, q, lane);
          acc = mfma32(shi[q], qh, acc);  // A[m=e][k=p] = S[p][e] (the D-tile, transposed)
          acc = mfma32(shi[q], ql, acc);
          acc = mfma32(slo[q], qh, acc);
        }
      }
#pragma unroll
      for (int i0 = 0; i0 < GC; i0 += 16) {
        const bf16x8 va = ld_rows8(sh + G::V, G::P, i0, 32 * w, lane);  // A[m=e][k=i] = v_i[e]
        acc = mfma32(va, ld_cols8(sh + G::SAH, G::AP, 0, i0, lane), acc);  // B[k=i][n=j] = A_ji
        acc = mfma32(va, ld_cols8(sh + G::SAL, G::AP, 0, i0, lane), acc);
      }
      const int j = lane & 31;
      const float inv = norm ? 1.f / sf[G::DEN + j] : 1.f;
      const __amdgpu_buffer_rsrc_t ro = make_rsrc((unsigned char*)p.o + r0 * D * OES, rows_extent(L, rso, D * OES));
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int e = 32 * w + dtile_row(4 * g, lane);  // four consecutive columns
        store_out4<OBF>(ro, (uint32_t)j * (rso / OES) + e, acc[4 * g] * inv, acc[4 * g + 1] * inv,
                        acc[4 * g + 2] * inv, acc[4 * g + 3] * inv);
      }
    }
    mstate<D>(S, sf, sh, w, lane);
  }
}

template <int D>
hipError_t launch_m(const PrefillParams& p, hipStream_t s, bool out) {
  using G = MGeo<D>;
  const void* kern = !out ? (const void*)k_summary_gla_m<D>
                     : p.out_bf16 ? (const void*)k_output_gla_m<D, true> : (const void*)k_output_gla_m<D, false>;
  const int lds = out ? G::BYTES : MSumGeo<D>::BYTES;
  hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  dim3 grid(p.B * p.H, p.n_seg);
  void* args[] = {(void*)&p};
  e = hipLaunchKernel(kern, grid, dim3(G::NT), args, lds, s);
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

template <int NP, int DV>
hipError_t launch_nd(const PrefillParams& p, hipStream_t s, bool out) {
  using G = GlaGeo<NP, DV>;
  const void* kern = !out ? (const void*)k_summary_gla<NP, DV>
                     : p.out_bf16 ? (const void*)k_output_gla<NP, DV, true> : (const void*)k_output_gla<NP, DV, false>;
  const int lds = 4 * G::FLOATS;
  hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  dim3 grid(p.B * p.H, p.n_seg);  // sequences on x: every XCD gets all segments of its sequences
  void* args[] = {(void*)&p};
  e = hipLaunchKernel(kern, grid, dim3(G::NT), args, lds, s);
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace

bool prefill_gated_supported(int C, int d_k, int d_v, int n_psi, int psi) {
  if (psi != LA_PSI_IDENTITY && psi != LA_PSI_ELU1) return false;
  if (n_psi != d_k || d_k != d_v) return false;
  return C == GC && (d_k == 64 || d_k == 128);
}

hipError_t launch_prefill_gated(const PrefillParams& p, hipStream_t s, bool out) {
  if (!p.in_f32) {
    if (p.d_k == 64) return launch_m<64>(p, s, out);
    if (p.d_k == 128) return launch_m<128>(p, s, out);
    return hipErrorInvalidValue;
  }
  if (p.d_k == 64) return launch_nd<64, 64>(p, s, out);
  if (p.d_k == 128) return launch_nd<128, 128>(p, s, out);
  return hipErrorInvalidValue;
}

}  // namespace la
