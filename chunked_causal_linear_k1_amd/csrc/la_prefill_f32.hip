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
  int S, Z, FQ, FK, RAW, V, A, DEN, THETA, XI, total;  // float offsets
};

__host__ __device__ inline F32Layout f32_layout(int C, int d_k, int d_v, int n_psi) {
  F32Layout L;
  int off = 0;
  L.S = off; off += n_psi * d_v;
  L.Z = off; off += n_psi;
  L.FQ = off; off += C * n_psi;
  L.FK = off; off += C * n_psi;
  L.RAW = off; off += C * d_k;   // raw rows (PRF needs them beside the features)
  L.V = off; off += C * d_v;
  L.A = off; off += C * C;
  L.DEN = off; off += C;
  L.THETA = off; off += C;
  L.XI = off; off += C;
  L.total = off;
  return L;
}

// psi of the chunk rows [0, valid) of x (fp32, row length d_k, rows rs elements apart) into
// out[C][n_psi]; rows >= valid -> 0.
__device__ void features_f32(const float* __restrict__ x, size_t rs, float* raw, float* out, int C, int valid,
                             int d_k, int n_psi, int psi, const float* __restrict__ w) {
  for (int idx = threadIdx.x; idx < C * d_k; idx += kThreads) {
    const int r = idx / d_k;
    raw[idx] = r < valid ? x[(size_t)r * rs + (idx - r * d_k)] : 0.f;
  }
  __syncthreads();
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
    out[idx] = val;
  }
  __syncthreads();
  if (is_prf(psi)) {
    // PRF_QSHIFT: subtract each row's largest log-feature (rows past `valid` stay zero)
    if (psi == LA_PSI_PRF_QSHIFT) {
      for (int r = threadIdx.x; r < valid; r += kThreads) {
        float mx = out[r * n_psi];
        for (int f = 1; f < n_psi; ++f) mx = fmaxf(mx, out[r * n_psi + f]);
        for (int f = 0; f < n_psi; ++f) out[r * n_psi + f] -= mx;
      }
      __syncthreads();
    }
    for (int idx = threadIdx.x; idx < C * n_psi; idx += kThreads)
      if (idx / n_psi < valid) out[idx] = expf(out[idx]) * rsqrtf((float)n_psi);
    __syncthreads();
  }
}

__device__ void load_rows_f32(const float* __restrict__ x, size_t rs, float* out, int C, int valid, int d) {
  for (int idx = threadIdx.x; idx < C * d; idx += kThreads) {
    const int r = idx / d;
    out[idx] = r < valid ? x[(size_t)r * rs + (idx - r * d)] : 0.f;
  }
}

// S <- a S + sum_i xi_i fK_i v_i^T ; Z likewise. Needs FK, V, XI in LDS.
__device__ void state_update_f32(float* sm, const F32Layout& Ly, int C, int L, int d_v, int n_psi, float lg) {
  for (int i = threadIdx.x; i < C; i += kThreads) sm[Ly.XI + i] = i < L ? gpow(lg, (float)(L - 1 - i)) : 0.f;
  __syncthreads();
  const float a = gpow(lg, (float)L);
  for (int idx = threadIdx.x; idx < n_psi * d_v; idx += kThreads) {
    const int pp = idx / d_v, e = idx % d_v;
    float acc = 0.f;
    for (int i = 0; i < L; ++i) acc += sm[Ly.XI + i] * sm[Ly.FK + i * n_psi + pp] * sm[Ly.V + i * d_v + e];
    sm[Ly.S + idx] = a * sm[Ly.S + idx] + acc;
  }
  for (int pp = threadIdx.x; pp < n_psi; pp += kThreads) {
    float acc = 0.f;
    for (int i = 0; i < L; ++i) acc += sm[Ly.XI + i] * sm[Ly.FK + i * n_psi + pp];
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
    features_f32(kb + (size_t)t0 * rk, rk, sm + Ly.RAW, sm + Ly.FK, p.C, L, p.d_k, p.n_psi, kpsi, w);
    state_update_f32(sm, Ly, p.C, L, p.d_v, p.n_psi, lg);
  }
  __syncthreads();
  const size_t E = (size_t)p.n_psi * p.d_v + p.n_psi;
  float* out = p.ws + ((size_t)bh * p.n_seg + seg) * E;
  for (int idx = threadIdx.x; idx < (int)E; idx += kThreads) out[idx] = sm[Ly.S + idx];
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
  for (int idx = threadIdx.x; idx < (int)E; idx += kThreads) sm[Ly.S + idx] = pre[idx];  // S then Z
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
    load_rows_f32(vb + (size_t)t0 * rv, rv, sm + Ly.V, C, L, d_v);
    features_f32(qb + (size_t)t0 * rk, rk, sm + Ly.RAW, sm + Ly.FQ, C, L, p.d_k, n_psi, p.psi, w);
    features_f32(kb + (size_t)t0 * rk, rk, sm + Ly.RAW, sm + Ly.FK, C, L, p.d_k, n_psi, kpsi, w);
    // scores
    for (int idx = threadIdx.x; idx < C * C; idx += kThreads) {
      const int j = idx / C, i = idx % C;
      float a = 0.f;
      if (i <= j && j < L) {
        for (int f = 0; f < n_psi; ++f) a += sm[Ly.FQ + j * n_psi + f] * sm[Ly.FK + i * n_psi + f];
        a *= gpow(lg, (float)(j - i));
      }
      sm[Ly.A + idx] = a;
    }
    __syncthreads();
    if (p.normalize) {
      for (int j = threadIdx.x; j < C; j += kThreads) {
        float qz = 0.f, r = 0.f;
        for (int f = 0; f < n_psi; ++f) qz += sm[Ly.FQ + j * n_psi + f] * sm[Ly.Z + f];
        for (int i = 0; i <= j; ++i) r += sm[Ly.A + j * C + i];
        sm[Ly.DEN + j] = sm[Ly.THETA + j] * qz + r + p.eps;
      }
      __syncthreads();
    }
    for (int idx = threadIdx.x; idx < C * d_v; idx += kThreads) {
      const int j = idx / d_v, e = idx % d_v;
      if (j >= L) continue;
      float inter = 0.f, intra = 0.f;
      for (int f = 0; f < n_psi; ++f) inter += sm[Ly.FQ + j * n_psi + f] * sm[Ly.S + f * d_v + e];
      for (int i = 0; i <= j; ++i) intra += sm[Ly.A + j * C + i] * sm[Ly.V + i * d_v + e];
      float num = sm[Ly.THETA + j] * inter + intra;
      if (p.normalize) num = num / sm[Ly.DEN + j];
      ob[(size_t)(t0 + j) * rv + e] = num;
    }
    __syncthreads();
    state_update_f32(sm, Ly, C, L, d_v, n_psi, lg);
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
