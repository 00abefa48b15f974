// la_backward_gen.hip -- backward pass of the prefill on the vector ALUs in fp32, for the shapes
// the matrix-core backward kernels do not take: fp32 inputs (identity, elu+1 and positive random
// features, with or without the query-row shift) and bf16 inputs at d = 64 (identity, elu+1).
//
// Same two sweeps as la_backward.hip ("Linearized 2-Simplicial Attention", 4.2 Custom Triton
// kernel, Backward, and appendix B.2, backward query sweep and backward state sweep), with the
// token recurrence's adjoint written per step of CB tokens (j, i, u: positions in the step,
// S_prev / Z_prev: the forward state before it, g = psi(q), f = psi(k), theta_j = gamma^(j+1),
// xi_j = gamma^(L-1-j)):
//   query sweep, forward over a segment from its forward prefix:
//     den_j  = theta_j g_j . Z_prev + sum_{i<=j} A_ji + eps,  A_ji = gamma^(j-i) g_j . f_i
//     num_j  = theta_j g_j^T S_prev + sum_{i<=j} A_ji v_i
//     dnum_j = dout_j / den_j,  dden_j = -(dout_j . num_j) / den_j^2   (no denominator: dout_j, 0)
//     dg_j   = theta_j (S_prev dnum_j + Z_prev dden_j) + sum_{i<=j} gamma^(j-i) (v_i . dnum_j + dden_j) f_i
//     dq_j   = the feature map's vector-Jacobian product at q_j applied to dg_j
//   and the segment's adjoint record sum_t gamma^(t - start + 1) g_t dnum_t^T (and g_t dden_t);
//   state sweep, backward over a segment from the adjoint state after it (R, RZ: the reverse
//   segment scan of those records), per step:
//     df_j = xi_j (R v_j + RZ) + sum_{u>=j} gamma^(u-j) (dnum_u . v_j + dden_u) g_u
//     dv_j = xi_j R^T f_j + sum_{u>=j} gamma^(u-j) (g_u . f_j) dnum_u
//     dk_j = the feature map's vector-Jacobian product at k_j applied to df_j
//     R    = gamma^L R + sum_u theta_u g_u dnum_u^T,  RZ likewise with dden_u.
// The feature maps' products: identity dx = dpsi; elu+1 dx = dpsi * (x > 0 ? 1 : e^x); random
// features ("Linearized 2-Simplicial Attention", 3.2) dx = sum_p a_p w_p - (sum_p a_p) x with
// a_p = dpsi_p psi_p, where under the query-row shift the last term takes the bank row that attains
// the shift (keys never take it).
//
// One workgroup of 256 threads per (sequence, segment); the state (or adjoint state) and one step's
// tiles live in LDS, the query sweep's adjoint record in registers (4 x 4 blocks per thread).
#include "la_device.hpp"
#include "la_kernels.hpp"

namespace la {
namespace {

constexpr int kT = 256;  // threads per workgroup
constexpr int CB = 16;   // tokens per step (segments are multiples of 16 tokens)
using F4 = f32x4;

struct GenLayout {
  int S, Z, FQ, FK, RQ, RK, V, DN, A, B, DG, DEN, DD, TH, XI, WT, AMX, total;  // float offsets
};

__host__ __device__ inline GenLayout gen_layout(int d_k, int d_v, int n_psi) {
  GenLayout L;
  int off = 0;
  L.S = off; off += n_psi * d_v;  // S_prev (query sweep) or R (state sweep)
  L.Z = off; off += n_psi;        // Z_prev or RZ
  L.FQ = off; off += CB * n_psi;  // psi(q) of the step's rows
  L.FK = off; off += CB * n_psi;  // psi(k)
  L.RQ = off; off += CB * d_k;    // raw q
  L.RK = off; off += CB * d_k;    // raw k
  L.V = off; off += CB * d_v;
  L.DN = off; off += CB * d_v;    // dout, then dnum
  L.A = off; off += CB * CB;      // A (query sweep) or its transpose (state sweep)
  L.B = off; off += CB * CB;      // the v . dnum + dden weights, likewise
  L.DG = off; off += CB * n_psi;  // dpsi of the query (query sweep) or of the key (state sweep)
  L.DEN = off; off += CB;         // 1 / den
  L.DD = off; off += CB;          // dden
  L.TH = off; off += CB;          // gamma^(j+1)
  L.XI = off; off += CB;          // gamma^(L-1-j), 0 past L
  L.WT = off; off += CB;          // gamma^(t - segment start + 1), 0 past L (adjoint record)
  L.AMX = off; off += CB;         // query-row shift: the bank row attaining each row's maximum
  L.total = off;
  return L;
}

size_t gen_lds_bytes(int d_k, int d_v, int n_psi) { return sizeof(float) * (size_t)gen_layout(d_k, d_v, n_psi).total; }

__device__ __forceinline__ F4 ld4s(const float* p) { return *(const F4*)p; }

// Four consecutive elements of a global row as fp32 (16-byte fp32 or 8-byte bf16 loads).
__device__ __forceinline__ F4 load4(const float* p) { return *(const F4*)p; }
__device__ __forceinline__ F4 load4(const uint16_t* p) {
  const uint2 u = *(const uint2*)p;
  return F4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
            __uint_as_float(u.y & 0xffff0000u)};
}
__device__ __forceinline__ float load1(const float* p) { return *p; }
__device__ __forceinline__ float load1(const uint16_t* p) { return __uint_as_float((uint32_t)*p << 16); }

// Rows [0, valid) of x (row length d, rows rs elements apart) into out[CB][d]; rows past valid 0.
template <typename TI>
__device__ void load_rows(const TI* __restrict__ x, long long rs, float* out, int valid, int d) {
  const int d4 = d / 4;
  for (int q = threadIdx.x; q < CB * d4; q += kT) {
    const int r = q / d4, c = (q - r * d4) * 4;
    ((F4*)out)[q] = r < valid ? load4(x + (long long)r * rs + c) : F4{0.f, 0.f, 0.f, 0.f};
  }
}

// psi of the raw rows [0, valid) (LDS, CB x d_k) into out (CB x n_psi), rows past valid 0. With the
// query-row shift each row's log-features drop by their maximum and amx[r] takes the index of the
// first bank row attaining it. Ends with a barrier.
template <typename TW>
__device__ void features(const float* raw, float* out, int valid, int d_k, int n_psi, int psi,
                         const TW* __restrict__ w, float* amx) {
  for (int idx = threadIdx.x; idx < CB * n_psi; idx += kT) {
    const int r = idx / n_psi, f = idx - r * n_psi;
    float val = 0.f;
    if (r < valid) {
      const float* xr = raw + r * d_k;
      if (psi == LA_PSI_IDENTITY) {
        val = xr[f];
      } else if (psi == LA_PSI_ELU1) {
        val = xr[f] > 0.f ? xr[f] + 1.f : expf(xr[f]);
      } else {
        float dot = 0.f, sq = 0.f;
        const TW* wr = w + (size_t)f * d_k;
        for (int j = 0; j < d_k; j += 4) {
          const F4 a = load4(wr + j), x = ld4s(xr + j);
          dot += (a[0] * x[0] + a[1] * x[1]) + (a[2] * x[2] + a[3] * x[3]);
          sq += (x[0] * x[0] + x[1] * x[1]) + (x[2] * x[2] + x[3] * x[3]);
        }
        val = dot - 0.5f * sq;  // the log-feature, exponentiated below
      }
    }
    out[idx] = val;
  }
  __syncthreads();
  if (is_prf(psi)) {
    if (psi == LA_PSI_PRF_QSHIFT) {
      for (int r = threadIdx.x; r < valid; r += kT) {
        float mx = out[r * n_psi];
        int arg = 0;
        for (int f = 1; f < n_psi; ++f)
          if (out[r * n_psi + f] > mx) {
            mx = out[r * n_psi + f];
            arg = f;
          }
        for (int f = 0; f < n_psi; ++f) out[r * n_psi + f] -= mx;
        amx[r] = (float)arg;
      }
      __syncthreads();
    }
    const float sc = rsqrtf((float)n_psi);
    for (int idx = threadIdx.x; idx < CB * n_psi; idx += kT)
      if (idx / n_psi < valid) out[idx] = expf(out[idx]) * sc;
    __syncthreads();
  }
}

// dx (global row, d_k floats) of the feature map at the raw row x for the upstream gradient dpsi
// (row j of DG); the threads of one 16-lane group share the row, lane g takes columns 4g, 4g + 64..
// a: dpsi_p psi_p, formed in place in DG by the caller for random features.
template <typename TW>
__device__ void feature_vjp_row(int psi, const float* x, const float* dpsi, const float* psirow, float amx,
                                int d_k, int n_psi, const TW* __restrict__ w, float* __restrict__ dx, int g) {
  if (psi == LA_PSI_IDENTITY) {
    for (int c = 4 * g; c < d_k; c += 64) *(F4*)(dx + c) = ld4s(dpsi + c);
  } else if (psi == LA_PSI_ELU1) {
    for (int c = 4 * g; c < d_k; c += 64) {
      const F4 xv = ld4s(x + c), gv = ld4s(dpsi + c);
      F4 r;
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = gv[e] * (xv[e] > 0.f ? 1.f : expf(xv[e]));
      *(F4*)(dx + c) = r;
    }
  } else {
    float csum = 0.f;
    for (int pp = 0; pp < n_psi; ++pp) csum += dpsi[pp] * psirow[pp];
    const TW* wstar = w + (size_t)(int)amx * d_k;
    for (int c = 4 * g; c < d_k; c += 64) {
      F4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int pp = 0; pp < n_psi; ++pp) acc += (dpsi[pp] * psirow[pp]) * load4(w + (size_t)pp * d_k + c);
      const F4 sub = psi == LA_PSI_PRF_QSHIFT ? load4(wstar + c) : ld4s(x + c);
      *(F4*)(dx + c) = acc - csum * sub;
    }
  }
}

// acc[r][c] += sum_k wk[k] X[k ldx + m0 + r] Y[k ldy + n0 + c] over k < K   (X^T diag(w) Y)
__device__ __forceinline__ void mm_atb(float (&acc)[4][4], const float* X, int ldx, const float* Y, int ldy,
                                       const float* wk, int m0, int n0, int K) {
  for (int k = 0; k < K; ++k) {
    const F4 x = ld4s(X + k * ldx + m0) * wk[k];
    const F4 y = ld4s(Y + k * ldy + n0);
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[r][c] += x[r] * y[c];
  }
}

// X <- a X + sum_k wk[k] P[k]^T Q[k] (n_psi x d_v, 4 x 4 blocks) and Xz <- a Xz + sum_k wk[k] P[k]
// (zw: per-row weight of P's rows in Xz). Ends with a barrier.
__device__ void rank_update(float* X, float* Xz, const float* P, const float* Q, const float* wk, const float* zw,
                            float a, int n_psi, int d_v) {
  const int nb = d_v / 4, blocks = (n_psi / 4) * nb;
  for (int b = threadIdx.x; b < blocks; b += kT) {
    const int m0 = (b / nb) * 4, n0 = (b % nb) * 4;
    float acc[4][4] = {};
    mm_atb(acc, P, n_psi, Q, d_v, wk, m0, n0, CB);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      F4* sp = (F4*)(X + (m0 + r) * d_v + n0);
      *sp = *sp * a + F4{acc[r][0], acc[r][1], acc[r][2], acc[r][3]};
    }
  }
  for (int pp = threadIdx.x; pp < n_psi; pp += kT) {
    float acc = 0.f;
    for (int k = 0; k < CB; ++k) acc += zw[k] * P[k * n_psi + pp];
    Xz[pp] = a * Xz[pp] + acc;
  }
  __syncthreads();
}

// Row bases of one sequence: token t of a tensor with rows of d elements is element (row0 + t tok_rows) d.
struct Rows {
  long long row0;
  long long step;  // tok_rows
};

template <typename TI, typename TO>
__global__ __launch_bounds__(kT) void k_bwd_gen_query(BackwardParams bp) {
  const PrefillParams& p = bp.f;
  extern __shared__ __align__(16) float sm[];
  const GenLayout Ly = gen_layout(p.d_k, p.d_v, p.n_psi);
  const int n = p.n_psi, dv = p.d_v, dk = p.d_k, tid = threadIdx.x;
  const int bh = blockIdx.x, seg = blockIdx.y, head = bh % p.H;
  const float lg = p.has_decay ? p.log2g[head] : 0.f;
  const TI* w = is_prf(p.psi) ? (const TI*)p.prf_w + (size_t)head * n * dk : nullptr;
  const int kpsi = p.psi == LA_PSI_PRF_QSHIFT ? LA_PSI_PRF : p.psi;  // keys take no query shift
  const size_t E = (size_t)n * dv + n;
  const SeqSpan sq = seq_span(p, bh);
  const int seg_tok = p.seg_chunks * p.C;
  const int s0 = seg * seg_tok, s1 = min(s0 + seg_tok, sq.T);
  float* rec = bp.rev + rec_index(p, bh, seg) * E;

  const int nbv = dv / 4, nblk = (n / 4) * nbv;  // adjoint record blocks, at most 4 per thread
  float adj[4][4][4] = {};
  float adjz = 0.f;

  if (s0 < s1) {
    const float* pre = p.ws + rec_index(p, bh, seg) * E;
    for (int q = tid; q < (int)(E / 4); q += kT) ((F4*)(sm + Ly.S))[q] = ld4s(pre + 4 * q);  // S then Z
    const long long rk = (long long)p.tok_rows * dk, rv = (long long)p.tok_rows * dv;
    const TI* qb = (const TI*)p.q + sq.row0 * dk;
    const TI* kb = (const TI*)p.k + sq.row0 * dk;
    const TI* vb = (const TI*)p.v + sq.row0 * dv;
    const TO* ob = (const TO*)bp.dout + sq.row0 * dv;
    const int j = tid / CB, gi = tid % CB;  // a (row, lane-of-16) pair per thread
    for (int t0 = s0; t0 < s1; t0 += CB) {
      const int L = min(CB, s1 - t0);
      __syncthreads();
      load_rows(qb + t0 * rk, rk, sm + Ly.RQ, L, dk);
      load_rows(kb + t0 * rk, rk, sm + Ly.RK, L, dk);
      load_rows(vb + t0 * rv, rv, sm + Ly.V, L, dv);
      load_rows(ob + t0 * rv, rv, sm + Ly.DN, L, dv);
      if (tid < CB) {
        sm[Ly.TH + tid] = gpow(lg, (float)(tid + 1));
        sm[Ly.XI + tid] = tid < L ? gpow(lg, (float)(L - 1 - tid)) : 0.f;
        sm[Ly.WT + tid] = tid < L ? gpow(lg, (float)(t0 + tid - s0 + 1)) : 0.f;
        sm[Ly.AMX + tid] = 0.f;
      }
      __syncthreads();
      features(sm + Ly.RQ, sm + Ly.FQ, L, dk, n, p.psi, w, sm + Ly.AMX);
      features(sm + Ly.RK, sm + Ly.FK, L, dk, n, kpsi, w, sm + Ly.AMX);  // no shift: amx untouched
      // A[j][i] = gamma^(j-i) g_j . f_i and B[j][i] = gamma^(j-i) v_i . dout_j (dnum scaling below)
      {
        float a = 0.f, b = 0.f;
        if (gi <= j && j < L) {
          for (int f = 0; f < n; f += 4) {
            const F4 x = ld4s(sm + Ly.FQ + j * n + f), y = ld4s(sm + Ly.FK + gi * n + f);
            a += (x[0] * y[0] + x[1] * y[1]) + (x[2] * y[2] + x[3] * y[3]);
          }
          for (int e = 0; e < dv; e += 4) {
            const F4 x = ld4s(sm + Ly.V + gi * dv + e), y = ld4s(sm + Ly.DN + j * dv + e);
            b += (x[0] * y[0] + x[1] * y[1]) + (x[2] * y[2] + x[3] * y[3]);
          }
          const float dec = gpow(lg, (float)(j - gi));
          a *= dec;
          b *= dec;
        }
        sm[Ly.A + tid] = a;
        sm[Ly.B + tid] = b;
      }
      __syncthreads();
      // den_j, dout_j . num_j -> 1/den_j, dden_j; then dnum_j = dout_j / den_j (row j, 16 lanes)
      if (p.normalize) {
        float part = 0.f;
        for (int c = 4 * gi; c < dv; c += 64) {
          F4 num = {0.f, 0.f, 0.f, 0.f};
          for (int pp = 0; pp < n; ++pp) num += sm[Ly.FQ + j * n + pp] * ld4s(sm + Ly.S + pp * dv + c);
          num *= sm[Ly.TH + j];
          for (int i = 0; i <= j; ++i) num += sm[Ly.A + j * CB + i] * ld4s(sm + Ly.V + i * dv + c);
          const F4 d = ld4s(sm + Ly.DN + j * dv + c);
          part += (num[0] * d[0] + num[1] * d[1]) + (num[2] * d[2] + num[3] * d[3]);
        }
        float qz = 0.f, rs = 0.f;
        for (int pp = gi; pp < n; pp += CB) qz += sm[Ly.FQ + j * n + pp] * sm[Ly.Z + pp];
        if (gi <= j) rs = sm[Ly.A + j * CB + gi];
#pragma unroll
        for (int off = 1; off < CB; off <<= 1) {
          part += __shfl_xor(part, off);
          qz += __shfl_xor(qz, off);
          rs += __shfl_xor(rs, off);
        }
        const float den = sm[Ly.TH + j] * qz + rs + p.eps;
        const float inv = 1.f / den;
        __syncthreads();  // every row's num is formed before dout turns into dnum
        if (gi == 0) {
          sm[Ly.DEN + j] = j < L ? inv : 0.f;
          sm[Ly.DD + j] = j < L ? -part * inv * inv : 0.f;
        }
        for (int c = 4 * gi; c < dv; c += 64) *(F4*)(sm + Ly.DN + j * dv + c) = ld4s(sm + Ly.DN + j * dv + c) * inv;
        __syncthreads();
        // B[j][i] was formed with dout_j: scale to dnum_j and add dden_j gamma^(j-i)
        if (gi <= j && j < L) {
          const float dd = sm[Ly.DD + j];
          sm[Ly.B + tid] = sm[Ly.B + tid] * sm[Ly.DEN + j] + dd * gpow(lg, (float)(j - gi));
        }
      } else if (gi == 0) {
        sm[Ly.DEN + j] = 1.f;
        sm[Ly.DD + j] = 0.f;
      }
      __syncthreads();
      // dg_j = theta_j (S_prev dnum_j + Z_prev dden_j) + sum_i B_ji f_i
      for (int pp = gi; pp < n; pp += CB) {
        float acc = 0.f;
        for (int e = 0; e < dv; e += 4) {
          const F4 x = ld4s(sm + Ly.S + pp * dv + e), y = ld4s(sm + Ly.DN + j * dv + e);
          acc += (x[0] * y[0] + x[1] * y[1]) + (x[2] * y[2] + x[3] * y[3]);
        }
        acc = sm[Ly.TH + j] * (acc + sm[Ly.Z + pp] * sm[Ly.DD + j]);
        for (int i = 0; i <= j; ++i) acc += sm[Ly.B + j * CB + i] * sm[Ly.FK + i * n + pp];
        sm[Ly.DG + j * n + pp] = j < L ? acc : 0.f;
      }
      __syncthreads();
      if (j < L) {
        feature_vjp_row(p.psi, sm + Ly.RQ + j * dk, sm + Ly.DG + j * n, sm + Ly.FQ + j * n, sm[Ly.AMX + j], dk, n,
                        w, bp.dq + (sq.row0 + (long long)(t0 + j) * p.tok_rows) * dk, gi);
        if (p.normalize && gi == 0) {
          float* tk = bp.tok + (sq.row0 + (long long)(t0 + j) * p.tok_rows) * 2;
          tk[0] = sm[Ly.DEN + j];
          tk[1] = sm[Ly.DD + j];
        }
      }
      // the segment's adjoint record: sum_t gamma^(t - start + 1) g_t dnum_t^T, and g_t dden_t
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int b = tid + kT * s;
        if (b < nblk) mm_atb(adj[s], sm + Ly.FQ, n, sm + Ly.DN, dv, sm + Ly.WT, (b / nbv) * 4, (b % nbv) * 4, CB);
      }
      if (tid < n)
        for (int k = 0; k < CB; ++k) adjz += sm[Ly.WT + k] * sm[Ly.DD + k] * sm[Ly.FQ + k * n + tid];
      if (t0 + CB < s1) {  // S_prev, Z_prev <- the state after this step
        __syncthreads();
        rank_update(sm + Ly.S, sm + Ly.Z, sm + Ly.FK, sm + Ly.V, sm + Ly.XI, sm + Ly.XI, gpow(lg, (float)L), n, dv);
      }
    }
  }
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int b = tid + kT * s;
    if (b < nblk) {
      const int m0 = (b / nbv) * 4, n0 = (b % nbv) * 4;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        *(F4*)(rec + (m0 + r) * dv + n0) = F4{adj[s][r][0], adj[s][r][1], adj[s][r][2], adj[s][r][3]};
    }
  }
  for (int pp = tid; pp < n; pp += kT) rec[(size_t)n * dv + pp] = pp == tid ? adjz : 0.f;
}

template <typename TI, typename TO>
__global__ __launch_bounds__(kT) void k_bwd_gen_state(BackwardParams bp) {
  const PrefillParams& p = bp.f;
  extern __shared__ __align__(16) float sm[];
  const GenLayout Ly = gen_layout(p.d_k, p.d_v, p.n_psi);
  const int n = p.n_psi, dv = p.d_v, dk = p.d_k, tid = threadIdx.x;
  const int bh = blockIdx.x, seg = blockIdx.y, head = bh % p.H;
  const float lg = p.has_decay ? p.log2g[head] : 0.f;
  const TI* w = is_prf(p.psi) ? (const TI*)p.prf_w + (size_t)head * n * dk : nullptr;
  const int kpsi = p.psi == LA_PSI_PRF_QSHIFT ? LA_PSI_PRF : p.psi;
  const size_t E = (size_t)n * dv + n;
  const SeqSpan sq = seq_span(p, bh);
  const int seg_tok = p.seg_chunks * p.C;
  const int s0 = seg * seg_tok, s1 = min(s0 + seg_tok, sq.T);
  if (s0 >= s1) return;
  const float* after = bp.rev + rec_index(p, bh, seg) * E;  // the adjoint state after the segment
  for (int q = tid; q < (int)(E / 4); q += kT) ((F4*)(sm + Ly.S))[q] = ld4s(after + 4 * q);  // R then RZ
  const long long rk = (long long)p.tok_rows * dk, rv = (long long)p.tok_rows * dv;
  const TI* qb = (const TI*)p.q + sq.row0 * dk;
  const TI* kb = (const TI*)p.k + sq.row0 * dk;
  const TI* vb = (const TI*)p.v + sq.row0 * dv;
  const TO* ob = (const TO*)bp.dout + sq.row0 * dv;
  const int j = tid / CB, gu = tid % CB;
  const int nsteps = (s1 - s0 + CB - 1) / CB;
  for (int st = nsteps - 1; st >= 0; --st) {
    const int t0 = s0 + st * CB, L = min(CB, s1 - t0);
    __syncthreads();
    load_rows(qb + t0 * rk, rk, sm + Ly.RQ, L, dk);
    load_rows(kb + t0 * rk, rk, sm + Ly.RK, L, dk);
    load_rows(vb + t0 * rv, rv, sm + Ly.V, L, dv);
    load_rows(ob + t0 * rv, rv, sm + Ly.DN, L, dv);
    if (tid < CB) {
      sm[Ly.TH + tid] = tid < L ? gpow(lg, (float)(tid + 1)) : 0.f;
      sm[Ly.XI + tid] = tid < L ? gpow(lg, (float)(L - 1 - tid)) : 0.f;
      float inv = 1.f, dd = 0.f;
      if (p.normalize && tid < L) {
        const float* tk = bp.tok + (sq.row0 + (long long)(t0 + tid) * p.tok_rows) * 2;
        inv = tk[0];
        dd = tk[1];
      }
      sm[Ly.DEN + tid] = inv;
      sm[Ly.DD + tid] = tid < L ? dd : 0.f;
      sm[Ly.AMX + tid] = 0.f;
    }
    __syncthreads();
    if (p.normalize)
      for (int c = 4 * gu; c < dv; c += 64) *(F4*)(sm + Ly.DN + j * dv + c) = ld4s(sm + Ly.DN + j * dv + c) * sm[Ly.DEN + j];
    features(sm + Ly.RQ, sm + Ly.FQ, L, dk, n, p.psi, w, sm + Ly.AMX);
    features(sm + Ly.RK, sm + Ly.FK, L, dk, n, kpsi, w, sm + Ly.AMX);
    // At[j][u] = gamma^(u-j) g_u . f_j and Bt[j][u] = gamma^(u-j) (dnum_u . v_j + dden_u), j <= u < L
    {
      float a = 0.f, b = 0.f;
      if (j <= gu && gu < L) {
        for (int f = 0; f < n; f += 4) {
          const F4 x = ld4s(sm + Ly.FQ + gu * n + f), y = ld4s(sm + Ly.FK + j * n + f);
          a += (x[0] * y[0] + x[1] * y[1]) + (x[2] * y[2] + x[3] * y[3]);
        }
        for (int e = 0; e < dv; e += 4) {
          const F4 x = ld4s(sm + Ly.DN + gu * dv + e), y = ld4s(sm + Ly.V + j * dv + e);
          b += (x[0] * y[0] + x[1] * y[1]) + (x[2] * y[2] + x[3] * y[3]);
        }
        const float dec = gpow(lg, (float)(gu - j));
        a *= dec;
        b = (b + sm[Ly.DD + gu]) * dec;
      }
      sm[Ly.A + tid] = a;
      sm[Ly.B + tid] = b;
    }
    __syncthreads();
    if (j < L) {
      const float xi = sm[Ly.XI + j];
      // df_j = xi_j (R v_j + RZ) + sum_u Bt_ju g_u
      for (int pp = gu; pp < n; pp += CB) {
        float acc = 0.f;
        for (int e = 0; e < dv; e += 4) {
          const F4 x = ld4s(sm + Ly.S + pp * dv + e), y = ld4s(sm + Ly.V + j * dv + e);
          acc += (x[0] * y[0] + x[1] * y[1]) + (x[2] * y[2] + x[3] * y[3]);
        }
        acc = xi * (acc + sm[Ly.Z + pp]);
        for (int u = j; u < L; ++u) acc += sm[Ly.B + j * CB + u] * sm[Ly.FQ + u * n + pp];
        sm[Ly.DG + j * n + pp] = acc;
      }
      // dv_j = xi_j R^T f_j + sum_u At_ju dnum_u
      float* dvr = bp.dv + (sq.row0 + (long long)(t0 + j) * p.tok_rows) * dv;
      for (int c = 4 * gu; c < dv; c += 64) {
        F4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int pp = 0; pp < n; ++pp) acc += sm[Ly.FK + j * n + pp] * ld4s(sm + Ly.S + pp * dv + c);
        acc *= xi;
        for (int u = j; u < L; ++u) acc += sm[Ly.A + j * CB + u] * ld4s(sm + Ly.DN + u * dv + c);
        *(F4*)(dvr + c) = acc;
      }
    }
    __syncthreads();
    if (j < L)
      feature_vjp_row(kpsi, sm + Ly.RK + j * dk, sm + Ly.DG + j * n, sm + Ly.FK + j * n, 0.f, dk, n, w,
                      bp.dk + (sq.row0 + (long long)(t0 + j) * p.tok_rows) * dk, gu);
    if (st > 0) {  // R, RZ <- the adjoint state before this step
      __syncthreads();
      // RZ weights: theta_u dden_u, formed in XI (no longer needed) by the first 16 threads
      if (tid < CB) sm[Ly.XI + tid] = sm[Ly.TH + tid] * sm[Ly.DD + tid];
      __syncthreads();
      rank_update(sm + Ly.S, sm + Ly.Z, sm + Ly.FQ, sm + Ly.DN, sm + Ly.TH, sm + Ly.XI, gpow(lg, (float)L), n, dv);
    }
  }
}

template <typename TI, typename TO>
hipError_t launch_gen(const BackwardParams& bp, hipStream_t s, bool state_sweep) {
  const PrefillParams& p = bp.f;
  const void* kern = state_sweep ? (const void*)k_bwd_gen_state<TI, TO> : (const void*)k_bwd_gen_query<TI, TO>;
  const size_t lds = gen_lds_bytes(p.d_k, p.d_v, p.n_psi);
  hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  dim3 grid(p.B * p.H, p.n_seg);
  void* args[] = {(void*)&bp};
  e = hipLaunchKernel(kern, grid, dim3(kT), args, lds, s);
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace

bool prefill_backward_gen_supported(int C, int d_k, int d_v, int n_psi, int psi, bool in_f32) {
  if (d_k % 4 != 0 || d_v % 4 != 0 || n_psi % 4 != 0) return false;
  if ((size_t)n_psi * d_v > 4u * 4 * 4 * kT) return false;  // the query sweep's record: 4 blocks per thread
  if (gen_lds_bytes(d_k, d_v, n_psi) > 160 * 1024) return false;
  if (in_f32) return prefill_f32_supported(C, d_k, d_v, n_psi, psi) && C % CB == 0;  // its forward summary pass
  // bf16: the shapes of the bf16 forward that the matrix-core backward does not take
  if (psi != LA_PSI_IDENTITY && psi != LA_PSI_ELU1) return false;
  return prefill_bf16_supported(C, d_k, d_v, n_psi, psi) && !prefill_backward_supported(C, d_k, d_v, n_psi, psi);
}

hipError_t launch_prefill_backward_gen(const BackwardParams& p, hipStream_t s, bool state_sweep) {
  const bool f32 = p.f.in_f32 != 0;
  if (f32) return p.dout_bf16 ? hipErrorInvalidValue : launch_gen<float, float>(p, s, state_sweep);
  return p.dout_bf16 ? launch_gen<uint16_t, uint16_t>(p, s, state_sweep) : launch_gen<uint16_t, float>(p, s, state_sweep);
}

}  // namespace la
