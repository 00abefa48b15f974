// la_decode.hip -- one recurrent decode step for N streams x H heads, state in place.
//
// "Linear Attention and Retentive Networks", The Recurrent Dual and Retentive
// Networks representation B: the whole history lives in a fixed-size state, so a
// step is a rank-1 update plus a vector-matrix product, independent of how many
// tokens came before:
//   S <- gamma S + psi(k) v^T,  Z <- gamma Z + psi(k),  o = psi(q)^T S / (psi(q).Z + eps)
// (update first, then read: the new token attends to itself). With per-row forget gates
// ("Linear Attention and Retentive Networks", Data-Dependent Gating Mechanism) gamma is
// replaced, row by row, by alpha[p] = exp(log_gate[p]).
//
// The step is a pure stream over the fp32 state (n_psi*d_v*4 bytes read and written
// per head). One workgroup per (stream, head): psi(k), psi(q) go to LDS, then every
// thread owns a 4-column slice of the value axis and a strided set of state rows,
// reads and writes its rows with 16-byte accesses (a wave covers whole contiguous
// rows), and accumulates its share of psi(q)^T S in registers; the row-group
// partials are summed in a fixed order through LDS.
#include "la_device.hpp"
#include "la_kernels.hpp"

namespace la {
namespace {

constexpr int kDecThreads = 256;
constexpr int kMaxFeat = 256;
constexpr int kMaxDv = 128;

__device__ __forceinline__ float load_in(const void* p, size_t i, bool f32) {
  return f32 ? ((const float*)p)[i] : bf16_bits_to_f32(((const uint16_t*)p)[i]);
}

__global__ __launch_bounds__(kDecThreads) void k_decode(DecodeParams p) {
  __shared__ float sf[kMaxFeat], sg[kMaxFeat], sx[2 * 128], sv[kMaxDv];
  __shared__ float sred[kDecThreads];
  __shared__ float snum[kDecThreads / 16][kMaxDv];  // [row group][d_v]; d_v >= 64 -> <= 16 groups
  __shared__ float sden;
  const int b = blockIdx.x, head = b % p.H, tid = threadIdx.x;
  const int d_k = p.d_k, d_v = p.d_v, n_psi = p.n_psi;
  const bool f32 = p.in_f32 != 0;
  const float gam = p.has_decay ? p.gamma[head] : 1.f;

  // raw q, k and v
  for (int i = tid; i < d_k; i += kDecThreads) {
    sx[i] = load_in(p.k, (size_t)b * d_k + i, f32);
    sx[128 + i] = load_in(p.q, (size_t)b * d_k + i, f32);
  }
  for (int i = tid; i < d_v; i += kDecThreads) sv[i] = load_in(p.v, (size_t)b * d_v + i, f32);
  __syncthreads();
  // features: f = psi(k), g = psi(q)
  for (int idx = tid; idx < 2 * n_psi; idx += kDecThreads) {
    const int which = idx / n_psi, f = idx % n_psi;
    const float* x = sx + 128 * which;
    float val;
    if (p.psi == LA_PSI_IDENTITY) {
      val = x[f];
    } else if (p.psi == LA_PSI_ELU1) {
      val = x[f] > 0.f ? x[f] + 1.f : expf(x[f]);
    } else {
      float dot = 0.f, sq = 0.f;
      for (int j = 0; j < d_k; ++j) {
        const float wj = load_in(p.prf_w, ((size_t)head * n_psi + f) * d_k + j, f32);
        dot += wj * x[j];
        sq += x[j] * x[j];
      }
      const float l = dot - 0.5f * sq;
      // with the query-row shift the query's log-features are exponentiated below
      val = (which == 1 && p.psi == LA_PSI_PRF_QSHIFT) ? l : expf(l) * rsqrtf((float)n_psi);
    }
    (which == 0 ? sf : sg)[f] = val;
  }
  __syncthreads();
  if (p.psi == LA_PSI_PRF_QSHIFT) {  // psi(q)_p = exp(l_p - max_r l_r) / sqrt(m)
    float mx = -__builtin_huge_valf();
    for (int f = tid; f < n_psi; f += kDecThreads) mx = fmaxf(mx, sg[f]);
    sred[tid] = mx;
    __syncthreads();
    for (int s = kDecThreads / 2; s > 0; s >>= 1) {
      if (tid < s) sred[tid] = fmaxf(sred[tid], sred[tid + s]);
      __syncthreads();
    }
    const float shift = sred[0];
    __syncthreads();  // every thread has the shift before sred is reused
    for (int f = tid; f < n_psi; f += kDecThreads) sg[f] = expf(sg[f] - shift) * rsqrtf((float)n_psi);
    __syncthreads();
  }

  // normaliser: Z <- gamma Z + f, den = g . Z + eps
  if (p.normalize) {
    float part = 0.f;
    for (int f = tid; f < n_psi; f += kDecThreads) {
      float* zp = p.Z + (size_t)b * n_psi + f;
      const float gz = p.log_gate ? expf(p.log_gate[(size_t)b * n_psi + f]) : gam;
      const float z = gz * *zp + sf[f];
      *zp = z;
      part += sg[f] * z;
    }
    sred[tid] = part;
    __syncthreads();
    for (int s = kDecThreads / 2; s > 0; s >>= 1) {
      if (tid < s) sred[tid] += sred[tid + s];
      __syncthreads();
    }
    if (tid == 0) sden = sred[0] + p.eps;
  }

  // state rows: thread -> (4-column group cg, row group rg)
  const int CG = d_v / 4, RG = kDecThreads / CG;
  const int cg = tid % CG, rg = tid / CG;
  float* Sb = p.S + (size_t)b * n_psi * d_v;
  const f32x4 v4 = {sv[4 * cg], sv[4 * cg + 1], sv[4 * cg + 2], sv[4 * cg + 3]};
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int row = rg; row < n_psi; row += RG) {
    f32x4* sp = (f32x4*)(Sb + (size_t)row * d_v + 4 * cg);
    f32x4 s = *sp;
    const float fk = sf[row], gq = sg[row];
    const float gr = p.log_gate ? expf(p.log_gate[(size_t)b * n_psi + row]) : gam;  // this row's forget gate
    s = gr * s + fk * v4;
    *sp = s;
    acc += gq * s;
  }
  for (int j = 0; j < 4; ++j) snum[rg][4 * cg + j] = acc[j];
  __syncthreads();
  for (int e = tid; e < d_v; e += kDecThreads) {
    float num = 0.f;
    for (int r = 0; r < RG; ++r) num += snum[r][e];
    p.o[(size_t)b * d_v + e] = p.normalize ? num / sden : num;
  }
}

}  // namespace

bool decode_supported(int d_k, int d_v, int n_psi, int psi) {
  if (d_k != 64 && d_k != 128) return false;
  if (d_v != 64 && d_v != 128) return false;
  if (is_prf(psi)) return n_psi == 64 || n_psi == 128 || n_psi == 256;
  return (psi == LA_PSI_IDENTITY || psi == LA_PSI_ELU1) && n_psi == d_k;
}

hipError_t launch_decode_step(const DecodeParams& p, hipStream_t s) {
  hipLaunchKernelGGL(k_decode, dim3(p.N * p.H), dim3(kDecThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace la
