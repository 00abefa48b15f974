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
// per head). One workgroup per (stream, head). In the general kernel (random features,
// whose feature map is a GEMV with the bank) psi(k), psi(q) go to LDS, then every
// thread owns a 4-column slice of the value axis and a strided set of state rows,
// reads and writes its rows with 16-byte accesses (a wave covers whole contiguous
// rows), and accumulates its share of psi(q)^T S in registers; the row-group
// partials are summed in a fixed order through LDS.
#include "la_device.hpp"
#include "la_kernels.hpp"

namespace la {
namespace {

// One output element: fp32, or the fp32 result rounded to bf16 (nearest even).
__device__ __forceinline__ void store_o(const DecodeParams& p, size_t idx, float x) {
  if (p.out_bf16)
    ((__bf16*)p.o)[idx] = to_bf16(x);
  else
    ((float*)p.o)[idx] = x;
}


constexpr int kDecThreads = 256;   // general kernel
constexpr int kElemThreads = 512;  // streaming kernel (elementwise features)
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
    store_o(p, (size_t)b * d_v + e, p.normalize ? num / sden : num);
  }
}

// The step for identity or elu+1 features with d_k == d_v == n_psi == D (64 or 128): the
// feature maps are elementwise, so the prologue is one global load per feature and one LDS
// hand-off, and the stream over the state dominates. Thread t owns the 4-column group
// cg = t % (D/4) and the rows rg + RG*i (rg = t / (D/4)); a wave covers 64 / (D/4) whole
// consecutive rows per 16-byte access. All of a thread's state rows are loaded before the
// prologue, so the whole state slice is in flight while the features are formed; the
// prologue's barrier waits for LDS only. The state is read once and written once per step,
// with nothing to reuse it before the next step, so both accesses are non-temporal (they do
// not displace other data in the caches): with 512 threads per (stream, head) this ran at
// 21.3k steps/s on 32 x 64 heads of d = 128 with the state rotating over four copies, against
// 17.6k with ordinary accesses and 256 threads. Row-group partials of psi(q)^T S meet by lane
// shuffles within a wave and through LDS across the waves, in a fixed order.
template <int D, bool ELU, bool NORM, bool F32IN, bool GATED>
__global__ __launch_bounds__(kElemThreads) void k_decode_elem(DecodeParams p) {
  constexpr int CG = D / 4, RG = kElemThreads / CG, RPT = D / RG, NWV = kElemThreads / 64;
  static_assert(2 * D <= kElemThreads && RPT * RG == D, "decode tiling");
  __shared__ float sF[2 * D];   // psi(k) [0, D), psi(q) [D, 2D)
  __shared__ float sA[D];       // per-row decay (gated: exp(log_gate))
  __shared__ float sNum[NWV][D];
  __shared__ float sDen[NWV];
  const int b = blockIdx.x, head = b % p.H, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int cg = tid % CG, rg = tid / CG;
  float* Sb = p.S + (size_t)b * D * D;

  // the state slice first: RPT independent 16-byte loads per thread
  f32x4 s[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i)
    s[i] = __builtin_nontemporal_load((const f32x4*)(Sb + (size_t)(rg + RG * i) * D + 4 * cg));
  float z = 0.f;
  if (NORM && tid < D) z = p.Z[(size_t)b * D + tid];
  f32x4 v4;
  if (F32IN) {
    v4 = *(const f32x4*)((const float*)p.v + (size_t)b * D + 4 * cg);
  } else {
    const uint2 raw = *(const uint2*)((const uint16_t*)p.v + (size_t)b * D + 4 * cg);
    v4 = f32x4{__uint_as_float(raw.x << 16), __uint_as_float(raw.x & 0xffff0000u), __uint_as_float(raw.y << 16),
               __uint_as_float(raw.y & 0xffff0000u)};
  }
  // features: threads [0, D) take psi(k), [D, 2D) psi(q)
  if (tid < 2 * D) {
    const int f = tid % D;
    const void* x = tid < D ? p.k : p.q;
    const float xv = F32IN ? ((const float*)x)[(size_t)b * D + f] : bf16_bits_to_f32(((const uint16_t*)x)[(size_t)b * D + f]);
    sF[tid] = ELU ? (xv > 0.f ? xv + 1.f : expf(xv)) : xv;
  }
  const float gam = p.has_decay ? p.gamma[head] : 1.f;
  if (tid < D) sA[tid] = GATED ? expf(p.log_gate[(size_t)b * D + tid]) : gam;
  lds_barrier();

  // normaliser: Z <- a Z + psi(k), den = psi(q) . Z + eps (waves holding the first D threads)
  if (NORM && tid < D) {
    z = sA[tid] * z + sF[tid];
    p.Z[(size_t)b * D + tid] = z;
    float part = sF[D + tid] * z;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off);
    if (lane == 0) sDen[w] = part;
  }
  // state rows: S <- a S + psi(k) v^T, then psi(q)^T S
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int row = rg + RG * i;
    const f32x4 x = sA[row] * s[i] + sF[row] * v4;
    __builtin_nontemporal_store(x, (f32x4*)(Sb + (size_t)row * D + 4 * cg));
    acc += sF[D + row] * x;
  }
  // row groups within the wave (lanes CG apart), then across the waves
#pragma unroll
  for (int off = CG; off < 64; off <<= 1)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] += __shfl_xor(acc[j], off);
  if (lane < CG) *(f32x4*)&sNum[w][4 * cg] = acc;
  lds_barrier();
  if (tid < D) {
    float num = 0.f;
#pragma unroll
    for (int ww = 0; ww < NWV; ++ww) num += sNum[ww][tid];
    if (NORM) {
      float den = p.eps;
#pragma unroll
      for (int ww = 0; ww < (D + 63) / 64; ++ww) den += sDen[ww];
      num /= den;
    }
    store_o(p, (size_t)b * D + tid, num);
  }
}

template <int D, bool ELU, bool NORM>
hipError_t launch_elem(const DecodeParams& p, hipStream_t s) {
  const dim3 g(p.N * p.H), t(kElemThreads);
  if (p.in_f32) {
    if (p.log_gate) hipLaunchKernelGGL((k_decode_elem<D, ELU, NORM, true, true>), g, t, 0, s, p);
    else hipLaunchKernelGGL((k_decode_elem<D, ELU, NORM, true, false>), g, t, 0, s, p);
  } else {
    if (p.log_gate) hipLaunchKernelGGL((k_decode_elem<D, ELU, NORM, false, true>), g, t, 0, s, p);
    else hipLaunchKernelGGL((k_decode_elem<D, ELU, NORM, false, false>), g, t, 0, s, p);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_elem_d(const DecodeParams& p, hipStream_t s) {
  const bool elu = p.psi == LA_PSI_ELU1;
  if (elu) return p.normalize ? launch_elem<D, true, true>(p, s) : launch_elem<D, true, false>(p, s);
  return p.normalize ? launch_elem<D, false, true>(p, s) : launch_elem<D, false, false>(p, s);
}

}  // namespace

bool decode_supported(int d_k, int d_v, int n_psi, int psi) {
  if (d_k != 64 && d_k != 128) return false;
  if (d_v != 64 && d_v != 128) return false;
  if (is_prf(psi)) return n_psi == 64 || n_psi == 128 || n_psi == 256;
  return (psi == LA_PSI_IDENTITY || psi == LA_PSI_ELU1) && n_psi == d_k;
}

hipError_t launch_decode_step(const DecodeParams& p, hipStream_t s) {
  // elementwise features at equal widths take the streaming kernel; random features (a
  // feature GEMV per token) the general one
  if (!is_prf(p.psi) && p.d_k == p.d_v && p.n_psi == p.d_k) {
    if (p.d_k == 128) return launch_elem_d<128>(p, s);
    if (p.d_k == 64) return launch_elem_d<64>(p, s);
  }
  hipLaunchKernelGGL(k_decode, dim3(p.N * p.H), dim3(kDecThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace la
