// la_prefill_bf16.hip -- chunkwise causal linear attention, bf16 inputs, fp32 state,
// MFMA 32x32x16 bf16 -> fp32 on gfx950.
//
// Method ("Log-Depth Chunked Linear-Attention Scan", Implementation notes; decayed
// form: "Linear Attention and Retentive Networks", chunkwise recurrent
// representation C). For chunk c with L real tokens, 0-based local indices i, j:
//   A_ji    = (psi(q_j) . psi(k_i)) gamma^(j-i)  for i <= j, else 0
//   num_j   = gamma^(j+1) psi(q_j) S_prev + sum_i A_ji v_i
//   den_j   = gamma^(j+1) psi(q_j) . Z_prev + sum_i A_ji
//   S_next  = gamma^L S_prev + sum_i gamma^(L-1-i) psi(k_i) v_i^T   (Z likewise)
// Padded positions (past T) are zeroed after the feature map, so they add nothing.
//
// Two kernels share the chunk loop:
//   k_summary: one workgroup per (sequence, segment of chunks); folds its chunks'
//              summaries into one segment summary (Kernel 1's summaries, reduced
//              over the segment) and writes it to the workspace.
//   k_output : one workgroup per (sequence, segment); starts from the segment's
//              exclusive prefix (written there by the scan), walks its chunks,
//              emits o for every real token (Kernels 1 and 3 fused) and carries the
//              state from chunk to chunk on chip.
//
// Workgroup = D/32 waves; wave w owns value columns [32w, 32w+32) of the state
// S (all n_psi rows, fp32 in registers) and of every output tile. All LDS tiles are
// row-major; operands whose k runs over tokens are read with the gfx950 transpose
// read, and the score tile A is fed from the MFMA accumulators straight back into
// the next MFMA (no LDS round trip).
//
// Precision: q, k, v are exact bf16 operands. Derived operands that are not
// exact in bf16 are carried as two-term bf16 expansions (hi + lo): the state S
// when it multiplies psi(Q), the score tile A, and K~_i = gamma^(L-1-i) psi(k_i)
// in the state update (rebuilt in fp32 from the raw keys), so the carried state is
// accurate to about 2^-16. In the score tile psi(q) and psi(k) of elu+1 are
// rounded to bf16 once; numerator and denominator use the same rounded scores.
#include "la_device.hpp"
#include "la_kernels.hpp"

namespace la {
namespace {

template <int C, int D>
struct Geo {
  static constexpr int NW = D / 32;         // waves per workgroup
  static constexpr int NT = 64 * NW;        // threads per workgroup
  static constexpr int P = D + 32;          // LDS pitch (elements) of K, V and K~ lo
  static constexpr int PQ = D + 8;          // LDS pitch of Q
  static constexpr int PPR = D / 8;         // 16-byte pieces per token row
  static constexpr int TILE = C * P * 2;    // bytes per tile region
  static constexpr int OFF_Q = 0;           // Q (steps on scores); K~ lo during the state update
  static constexpr int OFF_K = TILE;        // psi(K); K~ hi in place during the state update
  static constexpr int OFF_V = 2 * TILE;
  static constexpr int OFF_F = 3 * TILE;    // fp32 scratch
  static constexpr int F_Z = 0;             // Z [D]
  static constexpr int F_ZRED = D;          // per-wave Z partials [NW][D]
  static constexpr int F_QZ = D + NW * D;   // psi(q_j) . Z_prev [C]
  static constexpr int F_DEN = F_QZ + C;    // denominators [C]
  static constexpr int F_THETA = F_DEN + C; // gamma^(j+1) [C]
  static constexpr int LDS_BYTES = OFF_F + 4 * (F_THETA + C);
  static_assert(NT % PPR == 0, "thread count must cover whole rows");
  static_assert(NT == 2 * D, "launch bounds assume 2*D threads");
};

// Global (bf16 rows of D elements) -> LDS tile, applying psi. Rows >= valid are not
// read; they are zero, and stay zero after psi when zero_pad (the key side).
template <int C, int D>
__device__ __forceinline__ void stage_tile(const uint16_t* __restrict__ g, __bf16* s, int pitch, int valid,
                                           bool elu, bool zero_pad) {
  using G = Geo<C, D>;
  for (int pc = threadIdx.x; pc < C * G::PPR; pc += G::NT) {
    const int row = pc / G::PPR, c8 = (pc % G::PPR) * 8;
    uint4 raw = make_uint4(0u, 0u, 0u, 0u);
    if (row < valid) raw = *(const uint4*)(g + (size_t)row * D + c8);
    if (elu) {
      bf16x8 x = __builtin_bit_cast(bf16x8, raw);
      bf16x8 y;
#pragma unroll
      for (int j = 0; j < 8; ++j) y[j] = to_bf16(elu1(from_bf16(x[j])));
      if (zero_pad && row >= valid) y = bf16x8{};
      raw = __builtin_bit_cast(uint4, y);
    }
    *(uint4*)(s + row * pitch + c8) = raw;
  }
}

// The chunk's contribution to the state: S <- gamma^L S + K~^T V, Z <- gamma^L Z + K~^T 1,
// K~_i = gamma^(L-1-i) psi(k_i). psi(K) and V are in LDS; S tiles are this wave's.
template <int C, int D>
__device__ __forceinline__ void state_update(unsigned char* smem, f32x16 (&S)[D / 32], const uint16_t* __restrict__ kg,
                                             int L, float lg, bool decay, bool elu, bool norm) {
  using G = Geo<C, D>;
  __bf16* sKlo = (__bf16*)(smem + G::OFF_Q);
  __bf16* sK = (__bf16*)(smem + G::OFF_K);
  const __bf16* sV = (const __bf16*)(smem + G::OFF_V);
  float* sF = (float*)(smem + G::OFF_F);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;

  // K~_i = Xi_i psi(k_i) is exact in bf16 only for identity psi without decay. Otherwise it
  // is rebuilt in fp32 from the raw keys (just staged, so the re-read hits L2) and kept
  // as hi (in place of psi(K)) + lo (in the Q region). Z partials use the same fp32 values.
  const bool split = decay || elu;
  float zp[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) zp[j] = 0.f;
  if (split) {
    for (int pc = tid; pc < C * G::PPR; pc += G::NT) {
      const int row = pc / G::PPR, c8 = (pc % G::PPR) * 8;
      uint4 raw = make_uint4(0u, 0u, 0u, 0u);
      if (row < L) raw = *(const uint4*)(kg + (size_t)row * D + c8);
      const bf16x8 x = __builtin_bit_cast(bf16x8, raw);
      const float xi = row < L ? gpow(lg, (float)(L - 1 - row)) : 0.f;
      bf16x8 hi, lo;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float xf = from_bf16(x[j]);
        const float f = (elu ? elu1(xf) : xf) * xi;
        zp[j] += f;
        const bf16_pair sp = split_bf16(f);
        hi[j] = sp.hi;
        lo[j] = sp.lo;
      }
      *(bf16x8*)(sK + row * G::P + c8) = hi;
      *(bf16x8*)(sKlo + row * G::P + c8) = lo;
    }
  } else if (norm) {
    for (int pc = tid; pc < C * G::PPR; pc += G::NT) {
      const int row = pc / G::PPR, c8 = (pc % G::PPR) * 8;
      const bf16x8 x = *(const bf16x8*)(sK + row * G::P + c8);
#pragma unroll
      for (int j = 0; j < 8; ++j) zp[j] += from_bf16(x[j]);
    }
  }
  const float a = decay ? gpow(lg, (float)L) : 1.f;
  if (norm) {
    // lanes with equal (lane % PPR) own the same 8 columns
#pragma unroll
    for (int j = 0; j < 8; ++j)
      for (int off = G::PPR; off < 64; off <<= 1) zp[j] += __shfl_xor(zp[j], off);
    if (lane < G::PPR) {
#pragma unroll
      for (int j = 0; j < 8; ++j) sF[G::F_ZRED + w * D + lane * 8 + j] = zp[j];
    }
  }
  __syncthreads();
  if (norm && tid < D) {
    float z = 0.f;
#pragma unroll
    for (int ww = 0; ww < G::NW; ++ww) z += sF[G::F_ZRED + ww * D + tid];
    sF[G::F_Z + tid] = a * sF[G::F_Z + tid] + z;
  }
  // S <- a S + K~^T V  (M = state row p, N = value column e, k = token i)
  const int Ew = 32 * w;
  if (decay) {
#pragma unroll
    for (int pt = 0; pt < D / 32; ++pt) S[pt] *= a;
  }
#pragma unroll 2
  for (int ik = 0; ik < C / 16; ++ik) {
    const bf16x8 vb = ld_rows8(sV, G::P, ik * 16, Ew, lane);
#pragma unroll
    for (int pt = 0; pt < D / 32; ++pt) {
      const bf16x8 kh = ld_rows8(sK, G::P, ik * 16, pt * 32, lane);
      S[pt] = mfma32(kh, vb, S[pt]);
      if (split) {
        const bf16x8 kl = ld_rows8(sKlo, G::P, ik * 16, pt * 32, lane);
        S[pt] = mfma32(kl, vb, S[pt]);
      }
    }
  }
}

template <int C, int D>
__global__ __launch_bounds__(2 * D) void k_summary(PrefillParams p) {
  using G = Geo<C, D>;
  extern __shared__ __align__(16) unsigned char smem[];
  const int seg = blockIdx.x, bh = blockIdx.y, head = bh % p.H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const bool decay = p.has_decay && p.log2g[head] != 0.f;
  const float lg = decay ? p.log2g[head] : 0.f;
  const bool norm = p.normalize != 0, elu = p.psi == LA_PSI_ELU1;
  float* sF = (float*)(smem + G::OFF_F);
  if (tid < D) sF[G::F_Z + tid] = 0.f;
  f32x16 S[D / 32];
#pragma unroll
  for (int pt = 0; pt < D / 32; ++pt) S[pt] = f32x16{};

  const uint16_t* kb = (const uint16_t*)p.k + (size_t)bh * p.T * D;
  const uint16_t* vb = (const uint16_t*)p.v + (size_t)bh * p.T * D;
  const int c0 = seg * p.seg_chunks, c1 = min(c0 + p.seg_chunks, p.n_chunks);
  for (int c = c0; c < c1; ++c) {
    const int t0 = c * C, L = min(C, p.T - t0);
    __syncthreads();
    stage_tile<C, D>(kb + (size_t)t0 * D, (__bf16*)(smem + G::OFF_K), G::P, L, elu, true);
    stage_tile<C, D>(vb + (size_t)t0 * D, (__bf16*)(smem + G::OFF_V), G::P, L, false, false);
    __syncthreads();
    state_update<C, D>(smem, S, kb + (size_t)t0 * D, L, lg, decay, elu, norm);
  }
  __syncthreads();
  // segment summary -> workspace [bh][seg][E], E = D*D + D
  const size_t E = (size_t)D * D + D;
  float* out = p.ws + ((size_t)bh * p.n_seg + seg) * E;
  const int Ew = 32 * w, n = lane & 31;
#pragma unroll
  for (int pt = 0; pt < D / 32; ++pt)
#pragma unroll
    for (int r = 0; r < 16; ++r) out[(size_t)(pt * 32 + dtile_row(r, lane)) * D + Ew + n] = S[pt][r];
  if (tid < D) out[(size_t)D * D + tid] = sF[G::F_Z + tid];
}

template <int C, int D>
__global__ __launch_bounds__(2 * D) void k_output(PrefillParams p) {
  using G = Geo<C, D>;
  extern __shared__ __align__(16) unsigned char smem[];
  const int seg = blockIdx.x, bh = blockIdx.y, head = bh % p.H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, n = lane & 31;
  const int Ew = 32 * w;
  const bool decay = p.has_decay && p.log2g[head] != 0.f;
  const float lg = decay ? p.log2g[head] : 0.f;
  const bool norm = p.normalize != 0, elu = p.psi == LA_PSI_ELU1;
  __bf16* sQ = (__bf16*)(smem + G::OFF_Q);
  const __bf16* sK = (const __bf16*)(smem + G::OFF_K);
  const __bf16* sV = (const __bf16*)(smem + G::OFF_V);
  float* sF = (float*)(smem + G::OFF_F);

  // exclusive prefix state of this segment (written by the scan)
  const size_t E = (size_t)D * D + D;
  const float* pre = p.ws + ((size_t)bh * p.n_seg + seg) * E;
  f32x16 S[D / 32];
#pragma unroll
  for (int pt = 0; pt < D / 32; ++pt)
#pragma unroll
    for (int r = 0; r < 16; ++r) S[pt][r] = pre[(size_t)(pt * 32 + dtile_row(r, lane)) * D + Ew + n];
  if (tid < D) sF[G::F_Z + tid] = norm ? pre[(size_t)D * D + tid] : 0.f;
  for (int j = tid; j < C; j += G::NT) sF[G::F_THETA + j] = gpow(lg, (float)(j + 1));

  // per-lane decay factors for off-diagonal score tiles: gamma^(j-i) = cj * ri[r] * gamma^(32 m)
  float cj = 1.f, ri[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) ri[r] = 1.f;
  if (decay) {
    cj = gpow(lg, (float)n);
#pragma unroll
    for (int r = 0; r < 16; ++r) ri[r] = gpow(lg, (float)(32 - dtile_row(r, lane)));
  }

  const uint16_t* qb = (const uint16_t*)p.q + (size_t)bh * p.T * D;
  const uint16_t* kb = (const uint16_t*)p.k + (size_t)bh * p.T * D;
  const uint16_t* vb = (const uint16_t*)p.v + (size_t)bh * p.T * D;
  float* ob = (float*)p.o + (size_t)bh * p.T * D;
  const int c0 = seg * p.seg_chunks, c1 = min(c0 + p.seg_chunks, p.n_chunks);
  constexpr int NJ = C / 32;

  for (int c = c0; c < c1; ++c) {
    const int t0 = c * C, L = min(C, p.T - t0);
    __syncthreads();
    stage_tile<C, D>(qb + (size_t)t0 * D, sQ, G::PQ, L, elu, false);
    stage_tile<C, D>(kb + (size_t)t0 * D, (__bf16*)(smem + G::OFF_K), G::P, L, elu, true);
    stage_tile<C, D>(vb + (size_t)t0 * D, (__bf16*)(smem + G::OFF_V), G::P, L, false, false);
    __syncthreads();

    if (norm) {  // psi(q_j) . Z_prev
      constexpr int TPR = G::NT / C >= 1 ? G::NT / C : 1;
      for (int base = 0; base < C * TPR; base += G::NT) {
        const int idx = base + tid, j = idx / TPR, part = idx % TPR;
        float acc = 0.f;
        if (j < C) {
          const __bf16* qr = sQ + j * G::PQ;
          for (int e = part * (D / TPR); e < (part + 1) * (D / TPR); ++e) acc += from_bf16(qr[e]) * sF[G::F_Z + e];
        }
        for (int off = 1; off < TPR; off <<= 1) acc += __shfl_xor(acc, off);
        if (j < C && part == 0) sF[G::F_QZ + j] = acc;
      }
      __syncthreads();
    }

    // num_j = gamma^(j+1) psi(q_j) S_prev   (M = j, N = e, k = state row p)
    f32x16 num[NJ];
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt) num[jt] = f32x16{};
#pragma unroll
    for (int pt = 0; pt < D / 32; ++pt) {
      bf16x8 bh8[2], bl8[2];
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const bf16_pair sp = split_bf16(S[pt][8 * q + j]);
          bh8[q][j] = sp.hi;
          bl8[q][j] = sp.lo;
        }
#pragma unroll
      for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const bf16x8 qa = ld_cols8_perm(sQ, G::PQ, jt * 32, pt * 32, q, lane);
          num[jt] = mfma32(qa, bh8[q], num[jt]);
          num[jt] = mfma32(qa, bl8[q], num[jt]);
        }
    }
    if (decay) {
#pragma unroll
      for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
        for (int r = 0; r < 16; ++r) num[jt][r] *= sF[G::F_THETA + jt * 32 + dtile_row(r, lane)];
    }

    // scores A^T (M = i, N = j, k = feature p), masked and decayed, then num += A V
    float rsum[NJ];
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt) rsum[jt] = 0.f;
#pragma unroll
    for (int it = 0; it < NJ; ++it) {
      bf16x8 ka[D / 16];
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) ka[kk] = ld_cols8(sK, G::P, it * 32, kk * 16, lane);
#pragma unroll
      for (int jt = it; jt < NJ; ++jt) {
        f32x16 acc = f32x16{};
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) acc = mfma32(ka[kk], ld_cols8(sQ, G::PQ, jt * 32, kk * 16, lane), acc);
        if (it == jt) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int ir = dtile_row(r, lane);
            acc[r] = ir <= n ? acc[r] * gpow(lg, (float)(n - ir)) : 0.f;
          }
        } else if (decay) {
          const float tf = cj * gpow(lg, (float)(32 * (jt - it - 1)));
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[r] *= tf * ri[r];
        }
        if (norm) {
#pragma unroll
          for (int r = 0; r < 16; ++r) rsum[jt] += acc[r];
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          bf16x8 ah, al;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const bf16_pair sp = split_bf16(acc[8 * q + j]);
            ah[j] = sp.hi;
            al[j] = sp.lo;
          }
          const bf16x8 vv = ld_rows8_perm(sV, G::P, it * 32, q, Ew, lane);
          num[jt] = mfma32(ah, vv, num[jt]);
          num[jt] = mfma32(al, vv, num[jt]);
        }
      }
    }

    if (norm) {
#pragma unroll
      for (int jt = 0; jt < NJ; ++jt) {
        const float rj = rsum[jt] + __shfl_xor(rsum[jt], 32);
        const int j = jt * 32 + n;
        if (w == 0 && lane < 32) sF[G::F_DEN + j] = sF[G::F_THETA + j] * sF[G::F_QZ + j] + rj + p.eps;
      }
    }
    __syncthreads();
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = jt * 32 + dtile_row(r, lane);
        if (j < L) {
          float val = num[jt][r];
          if (norm) val = val / sF[G::F_DEN + j];
          ob[(size_t)(t0 + j) * D + Ew + n] = val;
        }
      }
    state_update<C, D>(smem, S, kb + (size_t)t0 * D, L, lg, decay, elu, norm);
  }
}

template <int C, int D>
hipError_t launch_summary_t(const PrefillParams& p, hipStream_t s) {
  using G = Geo<C, D>;
  auto kern = k_summary<C, D>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, G::LDS_BYTES);
  if (e != hipSuccess) return e;
  dim3 grid(p.n_seg, p.B * p.H);
  hipLaunchKernelGGL(kern, grid, dim3(G::NT), G::LDS_BYTES, s, p);
  return hipGetLastError();
}

template <int C, int D>
hipError_t launch_output_t(const PrefillParams& p, hipStream_t s) {
  using G = Geo<C, D>;
  auto kern = k_output<C, D>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, G::LDS_BYTES);
  if (e != hipSuccess) return e;
  dim3 grid(p.n_seg, p.B * p.H);
  hipLaunchKernelGGL(kern, grid, dim3(G::NT), G::LDS_BYTES, s, p);
  return hipGetLastError();
}

}  // namespace

bool prefill_bf16_supported(int C, int d_k, int d_v, int n_psi, int psi) {
  if (psi != LA_PSI_IDENTITY && psi != LA_PSI_ELU1) return false;
  if (d_k != d_v || n_psi != d_k) return false;
  return (d_k == 64 || d_k == 128) && (C == 64 || C == 128);
}

#define LA_DISPATCH_CD(FN, p, s)                                   \
  do {                                                             \
    if (p.C == 64 && p.d_k == 64) return FN<64, 64>(p, s);         \
    if (p.C == 64 && p.d_k == 128) return FN<64, 128>(p, s);       \
    if (p.C == 128 && p.d_k == 64) return FN<128, 64>(p, s);       \
    if (p.C == 128 && p.d_k == 128) return FN<128, 128>(p, s);     \
    return hipErrorInvalidValue;                                   \
  } while (0)

hipError_t launch_prefill_bf16_summary(const PrefillParams& p, hipStream_t s) { LA_DISPATCH_CD(launch_summary_t, p, s); }
hipError_t launch_prefill_bf16_output(const PrefillParams& p, hipStream_t s) { LA_DISPATCH_CD(launch_output_t, p, s); }

}  // namespace la
