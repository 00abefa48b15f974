// la_prefill_f32.hip -- chunkwise causal linear attention for fp32 inputs.
//
// fp32 inputs come with an fp32-level accuracy contract, which bf16 MFMA operands
// cannot meet, so this path runs every contraction as fp32 FMAs on the vector ALUs
// with LDS-staged chunk tiles. It follows the same decomposition as the bf16 path
// (segment summaries -> scan -> output walk over each segment's chunks) and the same
// chunk algebra ("Log-Depth Chunked Linear-Attention Scan", Implementation notes;
// "Linear Attention and Retentive Networks", chunkwise representation C):
//   A_ji  = psi(q_j).psi(k_i) gamma^(j-i), i <= j
//   num_j = gamma^(j+1) psi(q_j) S_prev + sum_i A_ji v_i,   den_j likewise with Z
//   S     = gamma^L S + sum_i gamma^(L-1-i) psi(k_i) v_i^T
// It is sized for small problems (all of one chunk plus the state in LDS).
#include "la_device.hpp"
#include "la_kernels.hpp"

namespace la {
namespace {

constexpr int kThreads = 256;

struct F32Layout {
  int S, Z, FQ, FK, RQ, RK, V, A, DEN, THETA, XI, total;  // float offsets
  int PF;  // feature row pitch: n_psi + 4, so that rows 4 apart fall in different LDS banks
};

__host__ __device__ inline F32Layout f32_layout(int C, int d_k, int d_v, int n_psi) {
  F32Layout L;
  int off = 0;
  L.S = off; off += n_psi * d_v;
  L.Z = off; off += n_psi;
  L.PF = n_psi + 4;
  L.FQ = off; off += C * L.PF;
  L.FK = off; off += C * L.PF;
  L.RQ = off; off += C * d_k;    // raw q and k rows, loaded together with v (PRF needs them
  L.RK = off; off += C * d_k;    // beside the features)
  L.V = off; off += C * d_v;
  L.A = off; off += C * C;
  L.DEN = off; off += C;
  L.THETA = off; off += C;
  L.XI = off; off += C;
  L.total = off;
  return L;
}

// psi of the raw chunk rows [0, valid) (LDS, row length d_k, loaded and made visible by the
// caller) into out[C][pf] (row pitch pf >= n_psi); rows >= valid -> 0.
__device__ void features_f32(const float* raw, float* out, int pf, int C, int valid, int d_k, int n_psi, int psi,
                             const float* __restrict__ w) {
  for (int idx = threadIdx.x; idx < C * n_psi; idx += kThreads) {
    const int r = idx / n_psi, f = idx % n_psi;
    float val = 0.f;
    if (r < valid) {
      const float* xr = raw + r * d_k;
      if (psi == LA_PSI_IDENTITY) {
        val = xr[f];
      } else if (psi == LA_PSI_ELU1) {
        val = xr[f] > 0.f ? xr[f] + 1.f : expf(xr[f]);
      } else {
        float dot = 0.f, sq = 0.f;
        const float* wr = w + (size_t)f * d_k;
        for (int j = 0; j < d_k; ++j) {
          dot += wr[j] * xr[j];
          sq += xr[j] * xr[j];
        }
        val = dot - 0.5f * sq;  // log-feature; exponentiated below
      }
    }
    out[(idx / n_psi) * pf + idx % n_psi] = val;
  }
  __syncthreads();
  if (is_prf(psi)) {
    // PRF_QSHIFT: subtract each row's largest log-feature (rows past `valid` stay zero)
    if (psi == LA_PSI_PRF_QSHIFT) {
      for (int r = threadIdx.x; r < valid; r += kThreads) {
        float mx = out[r * pf];
        for (int f = 1; f < n_psi; ++f) mx = fmaxf(mx, out[r * pf + f]);
        for (int f = 0; f < n_psi; ++f) out[r * pf + f] -= mx;
      }
      __syncthreads();
    }
    for (int idx = threadIdx.x; idx < C * n_psi; idx += kThreads) {
      const int r = idx / n_psi, o = r * pf + idx % n_psi;
      if (r < valid) out[o] = expf(out[o]) * rsqrtf((float)n_psi);
    }
    __syncthreads();
  }
}

// Rows [0, valid) of x (row length d, a multiple of 4; rows rs elements apart) into out[C][d],
// rows past `valid` zero: 16-byte loads, several in flight per thread.
__device__ void load_rows_f32(const float* __restrict__ x, size_t rs, float* out, int C, int valid, int d) {
  const int n4 = C * d / 4, d4 = d / 4;
#pragma unroll 4
  for (int q = threadIdx.x; q < n4; q += kThreads) {
    const int r = q / d4, c = (q - r * d4) * 4;
    ((f32x4*)out)[q] = r < valid ? *(const f32x4*)(x + (size_t)r * rs + c) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

// n floats (a multiple of 4) from global to LDS or back, 16 bytes at a time
__device__ __forceinline__ void copy4(float* dst, const float* __restrict__ src, int n) {
#pragma unroll 4
  for (int q = threadIdx.x; q < n / 4; q += kThreads) ((f32x4*)dst)[q] = ((const f32x4*)src)[q];
}

// 4 x 4 output blocks of fp32 products over LDS operands, one block per thread per pass;
// every operand read is 16 bytes (the tile sizes, offsets and leading dimensions are
// multiples of 4 floats), so each pair of reads feeds 16 or 64 FMAs.
using F4 = f32x4;
__device__ __forceinline__ F4 ld4s(const float* p) { return *(const F4*)p; }

// acc[r][c] += sum_k X[(m0 + r) ldx + k] Y[(n0 + c) ldy + k]            (X Y^T)
__device__ __forceinline__ void mm_abt(float (&acc)[4][4], const float* X, int ldx, const float* Y, int ldy, int m0,
                                       int n0, int K) {
  for (int k = 0; k < K; k += 4) {
    F4 x[4], y[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = ld4s(X + (m0 + r) * ldx + k);
#pragma unroll
    for (int c = 0; c < 4; ++c) y[c] = ld4s(Y + (n0 + c) * ldy + k);
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) acc[r][c] += x[r][kk] * y[c][kk];
  }
}

// acc[r][c] += sum_k X[(m0 + r) ldx + k] Y[k ldy + n0 + c]               (X Y)
__device__ __forceinline__ void mm_ab(float (&acc)[4][4], const float* X, int ldx, const float* Y, int ldy, int m0,
                                      int n0, int K) {
  for (int k = 0; k < K; k += 4) {
    F4 x[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = ld4s(X + (m0 + r) * ldx + k);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const F4 y = ld4s(Y + (k + kk) * ldy + n0);
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[r][c] += x[r][kk] * y[c];
    }
  }
}

// acc[r][c] += sum_k w[k] X[k ldx + m0 + r] Y[k ldy + n0 + c]            (X^T diag(w) Y)
__device__ __forceinline__ void mm_atb(float (&acc)[4][4], const float* X, int ldx, const float* Y, int ldy,
                                       const float* w, int m0, int n0, int K) {
  for (int k = 0; k < K; ++k) {
    const F4 x = ld4s(X + k * ldx + m0) * w[k];
    const F4 y = ld4s(Y + k * ldy + n0);
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[r][c] += x[r] * y[c];
  }
}

// S <- a S + sum_i xi_i fK_i v_i^T ; Z likewise. Needs FK, V in LDS; writes XI.
__device__ void state_update_f32(float* sm, const F32Layout& Ly, int C, int L, int d_v, int n_psi, float lg) {
  for (int i = threadIdx.x; i < C; i += kThreads) sm[Ly.XI + i] = i < L ? gpow(lg, (float)(L - 1 - i)) : 0.f;
  __syncthreads();
  const float a = gpow(lg, (float)L);
  const int nb = d_v / 4, blocks = (n_psi / 4) * nb;
  const int K = (L + 3) & ~3;  // rows past L are zero in FK and XI
  for (int b = threadIdx.x; b < blocks; b += kThreads) {
    const int m0 = (b / nb) * 4, n0 = (b % nb) * 4;
    float acc[4][4] = {};
    mm_atb(acc, sm + Ly.FK, Ly.PF, sm + Ly.V, d_v, sm + Ly.XI, m0, n0, K);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      F4* sp = (F4*)(sm + Ly.S + (m0 + r) * d_v + n0);
      *sp = *sp * a + F4{acc[r][0], acc[r][1], acc[r][2], acc[r][3]};
    }
  }
  for (int pp = threadIdx.x; pp < n_psi; pp += kThreads) {
    float acc = 0.f;
    for (int i = 0; i < L; ++i) acc += sm[Ly.XI + i] * sm[Ly.FK + i * Ly.PF + pp];
    sm[Ly.Z + pp] = a * sm[Ly.Z + pp] + acc;
  }
  __syncthreads();
}

__global__ __launch_bounds__(kThreads) void k_summary_f32(PrefillParams p) {
  extern __shared__ __align__(16) float sm[];
  const F32Layout Ly = f32_layout(p.C, p.d_k, p.d_v, p.n_psi);
  const int bh = blockIdx.x, seg = blockIdx.y, head = bh % p.H;
  const float lg = p.has_decay ? p.log2g[head] : 0.f;
  const float* w = is_prf(p.psi) ? (const float*)p.prf_w + (size_t)head * p.n_psi * p.d_k : nullptr;
  const int kpsi = p.psi == LA_PSI_PRF_QSHIFT ? LA_PSI_PRF : p.psi;  // keys take no query shift
  for (int idx = threadIdx.x; idx < p.n_psi * p.d_v + p.n_psi; idx += kThreads) sm[Ly.S + idx] = 0.f;  // S then Z
  const SeqSpan sq = seq_span(p, bh);
  const int T = sq.T, n_chunks = (T + p.C - 1) / p.C;
  const size_t rk = (size_t)p.tok_rows * p.d_k, rv = (size_t)p.tok_rows * p.d_v;  // elements between token rows
  const float* kb = (const float*)p.k + sq.row0 * p.d_k;
  const float* vb = (const float*)p.v + sq.row0 * p.d_v;
  const int c0 = seg * p.seg_chunks, c1 = min(c0 + p.seg_chunks, n_chunks);
  for (int c = c0; c < c1; ++c) {
    const int t0 = c * p.C, L = min(p.C, T - t0);
    __syncthreads();
    load_rows_f32(vb + (size_t)t0 * rv, rv, sm + Ly.V, p.C, L, p.d_v);
    load_rows_f32(kb + (size_t)t0 * rk, rk, sm + Ly.RK, p.C, L, p.d_k);
    __syncthreads();
    features_f32(sm + Ly.RK, sm + Ly.FK, Ly.PF, p.C, L, p.d_k, p.n_psi, kpsi, w);
    state_update_f32(sm, Ly, p.C, L, p.d_v, p.n_psi, lg);
  }
  __syncthreads();
  const size_t E = (size_t)p.n_psi * p.d_v + p.n_psi;
  copy4(p.ws + ((size_t)bh * p.n_seg + seg) * E, sm + Ly.S, (int)E);
}

__global__ __launch_bounds__(kThreads) void k_output_f32(PrefillParams p) {
  extern __shared__ __align__(16) float sm[];
  const F32Layout Ly = f32_layout(p.C, p.d_k, p.d_v, p.n_psi);
  const int bh = blockIdx.x, seg = blockIdx.y, head = bh % p.H;
  const float lg = p.has_decay ? p.log2g[head] : 0.f;
  const int C = p.C, n_psi = p.n_psi, d_v = p.d_v;
  const float* w = is_prf(p.psi) ? (const float*)p.prf_w + (size_t)head * n_psi * p.d_k : nullptr;
  const int kpsi = p.psi == LA_PSI_PRF_QSHIFT ? LA_PSI_PRF : p.psi;  // keys take no query shift
  const size_t E = (size_t)n_psi * d_v + n_psi;
  const float* pre = p.ws + ((size_t)bh * p.n_seg + seg) * E;
  copy4(sm + Ly.S, pre, (int)E);  // S then Z
  for (int j = threadIdx.x; j < C; j += kThreads) sm[Ly.THETA + j] = gpow(lg, (float)(j + 1));
  const SeqSpan sq = seq_span(p, bh);
  const int T = sq.T, n_chunks = (T + C - 1) / C;
  const size_t rk = (size_t)p.tok_rows * p.d_k, rv = (size_t)p.tok_rows * d_v;  // elements between token rows
  const float* qb = (const float*)p.q + sq.row0 * p.d_k;
  const float* kb = (const float*)p.k + sq.row0 * p.d_k;
  const float* vb = (const float*)p.v + sq.row0 * d_v;
  float* ob = (float*)p.o + sq.row0 * d_v;
  const int c0 = seg * p.seg_chunks, c1 = min(c0 + p.seg_chunks, n_chunks);
  for (int c = c0; c < c1; ++c) {
    const int t0 = c * C, L = min(C, T - t0);
    __syncthreads();
    // v, q and k rows in one round of loads, then both feature maps
    load_rows_f32(vb + (size_t)t0 * rv, rv, sm + Ly.V, C, L, d_v);
    load_rows_f32(qb + (size_t)t0 * rk, rk, sm + Ly.RQ, C, L, p.d_k);
    load_rows_f32(kb + (size_t)t0 * rk, rk, sm + Ly.RK, C, L, p.d_k);
    __syncthreads();
    features_f32(sm + Ly.RQ, sm + Ly.FQ, Ly.PF, C, L, p.d_k, n_psi, p.psi, w);
    features_f32(sm + Ly.RK, sm + Ly.FK, Ly.PF, C, L, p.d_k, n_psi, kpsi, w);
    // scores A[j][i] = psi(q_j).psi(k_i) gamma^(j-i), i <= j < L, in 4 x 4 blocks on or below
    // the diagonal (blocks above it are zero)
    {
      const int nb = C / 4;
      for (int b = threadIdx.x; b < nb * nb; b += kThreads) {
        const int m0 = (b / nb) * 4, n0 = (b % nb) * 4;
        float acc[4][4] = {};
        if (n0 <= m0 && m0 < L) mm_abt(acc, sm + Ly.FQ, Ly.PF, sm + Ly.FK, Ly.PF, m0, n0, n_psi);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float o4[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int j = m0 + r, i = n0 + c;
            o4[c] = (i <= j && j < L) ? acc[r][c] * gpow(lg, (float)(j - i)) : 0.f;
          }
          *(F4*)(sm + Ly.A + (m0 + r) * C + n0) = F4{o4[0], o4[1], o4[2], o4[3]};
        }
      }
    }
    __syncthreads();
    if (p.normalize) {
      for (int j = threadIdx.x; j < C; j += kThreads) {
        F4 qz = {0.f, 0.f, 0.f, 0.f}, r = {0.f, 0.f, 0.f, 0.f};
        for (int f = 0; f < n_psi; f += 4) qz += ld4s(sm + Ly.FQ + j * Ly.PF + f) * ld4s(sm + Ly.Z + f);
        for (int i = 0; i <= j; i += 4) r += ld4s(sm + Ly.A + j * C + i);  // zero above the diagonal
        sm[Ly.DEN + j] = sm[Ly.THETA + j] * ((qz[0] + qz[1]) + (qz[2] + qz[3])) + ((r[0] + r[1]) + (r[2] + r[3])) + p.eps;
      }
      __syncthreads();
    }
    // outputs: theta_j psi(q_j) S_prev + sum_{i <= j} A_ji v_i, over the denominator
    {
      const int nb = d_v / 4;
      for (int b = threadIdx.x; b < (C / 4) * nb; b += kThreads) {
        const int m0 = (b / nb) * 4, n0 = (b % nb) * 4;
        if (m0 >= L) continue;
        float inter[4][4] = {}, intra[4][4] = {};
        mm_ab(inter, sm + Ly.FQ, Ly.PF, sm + Ly.S, d_v, m0, n0, n_psi);
        mm_ab(intra, sm + Ly.A, C, sm + Ly.V, d_v, m0, n0, m0 + 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = m0 + r;
          if (j >= L) break;
          const float th = sm[Ly.THETA + j];
          F4 o4;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const float num = th * inter[r][c] + intra[r][c];
            o4[c] = p.normalize ? num / sm[Ly.DEN + j] : num;
          }
          *(F4*)(ob + (size_t)(t0 + j) * rv + n0) = o4;
        }
      }
    }
    __syncthreads();
    if (c + 1 < c1) state_update_f32(sm, Ly, C, L, d_v, n_psi, lg);  // the segment's last state is not needed
  }
}

}  // namespace

static size_t f32_lds_bytes(int C, int d_k, int d_v, int n_psi) {
  return sizeof(float) * (size_t)f32_layout(C, d_k, d_v, n_psi).total;
}

bool prefill_f32_supported(int C, int d_k, int d_v, int n_psi, int psi) {
  if (psi < LA_PSI_IDENTITY || psi > LA_PSI_PRF_QSHIFT) return false;
  if (!is_prf(psi) && n_psi != d_k) return false;
  if (d_k > 128 || d_v > 128 || n_psi > 256) return false;
  if (d_k % 4 != 0) return false;  // 16-byte row loads
  if (C != 16 && C != 32 && C != 64) return false;
  return f32_lds_bytes(C, d_k, d_v, n_psi) <= 160 * 1024;
}

static hipError_t launch_f32(const void* kern, const PrefillParams& p, hipStream_t s) {
  const size_t lds = f32_lds_bytes(p.C, p.d_k, p.d_v, p.n_psi);
  hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  // x = (batch, head), y = segment: workgroups are dealt to the 8 XCDs round-robin by linear id
  // x + y * B * H, so every XCD gets a share of the sequences with all their segments. With the
  // segment on x, segment s would always land on the same XCDs: for variable-length batches the
  // heavy first segments would pile onto a few of them.
  dim3 grid(p.B * p.H, p.n_seg);
  void* args[] = {(void*)&p};
  e = hipLaunchKernel(kern, grid, dim3(kThreads), args, lds, s);
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

hipError_t launch_prefill_f32_summary(const PrefillParams& p, hipStream_t s) {
  return launch_f32((const void*)k_summary_f32, p, s);
}
hipError_t launch_prefill_f32_output(const PrefillParams& p, hipStream_t s) {
  return launch_f32((const void*)k_output_f32, p, s);
}

}  // namespace la
