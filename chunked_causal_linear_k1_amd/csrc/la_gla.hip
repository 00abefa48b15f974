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
// This path runs in fp32 on the vector ALUs: the gate factors make every operand inexact
// in bf16. Chunks of 16 tokens; each thread keeps an 8 x 8 block of the state in
// registers (rows 8 pb.., columns 8 eb..; the pb lanes of a column block are adjacent,
// so the sums over state rows reduce across 16 (or 8) consecutive lanes).
#include "la_device.hpp"
#include "la_kernels.hpp"

namespace la {
namespace {

constexpr int GC = 16;  // chunk

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
  if (p.d_k == 64) return launch_nd<64, 64>(p, s, out);
  if (p.d_k == 128) return launch_nd<128, 128>(p, s, out);
  return hipErrorInvalidValue;
}

}  // namespace la
