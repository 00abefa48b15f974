// la_prefill_bf16.hpp -- chunkwise causal linear attention, bf16 inputs, fp32 state,
// MFMA 32x32x16 bf16 -> fp32 on gfx950. Kernel templates; instantiated per (C, D) in
// la_prefill_bf16_c*.hip.
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
// Two kernels share the chunk machinery:
//   k_summary: one workgroup per (sequence, segment of chunks); folds its chunks'
//              summaries into one segment summary (Kernel 1's summaries, reduced
//              over the segment) and writes it to the workspace.
//   k_output : one workgroup per (sequence, segment); starts from the segment's
//              exclusive prefix (written there by the scan), walks its chunks,
//              emits o for every real token (Kernels 1 and 3 fused) and carries the
//              state from chunk to chunk on chip.
//
// Workgroup = D/32 waves; wave w owns value columns [32w, 32w+32) of the state
// S (all n_psi rows, fp32 in registers) and of every output tile. Each wave
// computes every score tile itself, so the score tile goes from the MFMA
// accumulators straight back into the next MFMA as an operand (no LDS round trip).
// All LDS tiles are row-major; operands whose k runs over tokens use the gfx950
// transpose read (ds_read_b64_tr_b16).
//
// Scheduling: decay, normalisation and the feature map are template parameters and
// the tile loops are fully unrolled, so each chunk's matrix work is straight-line
// code the compiler can interleave (LDS reads issued ahead of the MFMAs that use
// them, independent score tiles overlapping). The raw q, k, v of chunk c+1 are
// loaded into registers (bounded buffer loads: rows past T read as zero) while
// chunk c is computed and written to LDS at the top of the next iteration.
//
// Precision: q, k, v are exact bf16 operands. Derived operands that are not
// exact in bf16 are carried as two-term bf16 expansions (hi + lo): the state S
// when it multiplies psi(Q), the score tile A, and K~_i = gamma^(L-1-i) psi(k_i)
// in the state update, so the carried state is accurate to about 2^-16. In the
// score tile psi(q) and psi(k) of elu+1 are rounded to bf16 once; numerator and
// denominator use the same rounded scores.
#pragma once
#include "la_device.hpp"
#include "la_kernels.hpp"

namespace la {
namespace pf {

template <int C, int D, bool WITH_Q>
struct Geo {
  static constexpr int NW = D / 32;          // waves per workgroup
  static constexpr int NT = 64 * NW;         // threads per workgroup
  static constexpr int PQ = D + 8;           // LDS pitch (elements) of Q: row reads only
  static constexpr int PK = D + 16;          // pitch of K, K lo, V: row and transpose reads
  static constexpr int PPR = D / 8;          // 16-byte pieces per token row
  static constexpr int NPC = C * PPR / NT;   // pieces per thread per tile
  static constexpr int Q_BYTES = WITH_Q ? C * PQ * 2 : 0;
  static constexpr int K_BYTES = C * PK * 2;
  static constexpr int OFF_Q = 0;
  static constexpr int OFF_K = Q_BYTES;      // psi(K) (hi part); K~ hi during the state update
  static constexpr int OFF_KLO = OFF_K + K_BYTES;
  static constexpr int OFF_V = OFF_KLO + K_BYTES;
  static constexpr int OFF_F = OFF_V + K_BYTES;  // fp32 scratch
  static constexpr int F_Z = 0;              // Z [D]
  static constexpr int F_ZRED = D;           // per-wave Z partials [NW][D]
  static constexpr int F_THETA = D + NW * D; // gamma^(j+1) [C]
  static constexpr int LDS_BYTES = OFF_F + 4 * (F_THETA + C);
  static_assert(NT == 2 * D, "launch bounds assume 2*D threads");
  static_assert((C * PPR) % NT == 0 && NT % PPR == 0, "pieces must tile the threads");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

// Raw 16-byte pieces of one C x D chunk tile, held in registers between the load and
// the LDS write. Piece i of thread t covers row (t + i*NT) / PPR, columns 8*((t + i*NT) % PPR).
template <int C, int D>
struct Pieces {
  uint4 r[Geo<C, D, true>::NPC];
};

template <int C, int D>
__device__ __forceinline__ int piece_cols(int i) {
  using G = Geo<C, D, true>;
  return ((threadIdx.x + i * G::NT) % G::PPR) * 8;
}
template <int C, int D>
__device__ __forceinline__ int piece_row(int i) {
  using G = Geo<C, D, true>;
  return (threadIdx.x + i * G::NT) / G::PPR;
}

// Rows >= valid read as zeros (bounded buffer resource, no branches).
template <int C, int D>
__device__ __forceinline__ void load_pieces(Pieces<C, D>& P, const uint16_t* __restrict__ g, int valid) {
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(g, (uint32_t)valid * D * 2);
#pragma unroll
  for (int i = 0; i < Geo<C, D, true>::NPC; ++i)
    P.r[i] = buf_load16(rs, (uint32_t)(piece_row<C, D>(i) * D + piece_cols<C, D>(i)) * 2);
}

// Q: psi applied, rounded once to bf16.
template <int C, int D, bool ELU>
__device__ __forceinline__ void commit_q(const Pieces<C, D>& P, __bf16* sQ, int pitch) {
#pragma unroll
  for (int i = 0; i < Geo<C, D, true>::NPC; ++i) {
    uint4 raw = P.r[i];
    if (ELU) {
      const bf16x8 x = __builtin_bit_cast(bf16x8, raw);
      bf16x8 y;
#pragma unroll
      for (int j = 0; j < 8; ++j) y[j] = to_bf16(elu1(from_bf16(x[j])));
      raw = __builtin_bit_cast(uint4, y);
    }
    *(uint4*)(sQ + piece_row<C, D>(i) * pitch + piece_cols<C, D>(i)) = raw;
  }
}

// K: f = psi(k) in fp32 (zero past the sequence end), times Xi_i = gamma^(L-1-i) when
// FOLD. Writes hi = bf16(f) and, if LO, lo = bf16(f - hi). Adds this thread's
// contribution to the chunk's normaliser summary: zp += Xi_i psi(k_i).
template <int C, int D, bool ELU, bool DECAY, bool FOLD, bool LO>
__device__ __forceinline__ void commit_k(const Pieces<C, D>& P, __bf16* sK, __bf16* sKlo, int pitch, int L,
                                         float lg, float (&zp)[8]) {
#pragma unroll
  for (int i = 0; i < Geo<C, D, true>::NPC; ++i) {
    const int row = piece_row<C, D>(i), c8 = piece_cols<C, D>(i);
    const float live = row < L ? 1.f : 0.f;
    const float xi = DECAY ? live * exp2f((float)(L - 1 - row) * lg) : live;
    const float xs = FOLD ? xi : live;
    const bf16x8 x = __builtin_bit_cast(bf16x8, P.r[i]);
    bf16x8 hi, lo;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float xf = from_bf16(x[j]);
      const float f = (ELU ? elu1(xf) : xf) * xs;
      zp[j] += FOLD ? f : f * xi;
      const bf16_pair sp = split_bf16(f);
      hi[j] = sp.hi;
      lo[j] = sp.lo;
    }
    *(bf16x8*)(sK + row * pitch + c8) = hi;
    if (LO) *(bf16x8*)(sKlo + row * pitch + c8) = lo;
  }
}

template <int C, int D>
__device__ __forceinline__ void commit_v(const Pieces<C, D>& P, __bf16* sV, int pitch) {
#pragma unroll
  for (int i = 0; i < Geo<C, D, true>::NPC; ++i)
    *(uint4*)(sV + piece_row<C, D>(i) * pitch + piece_cols<C, D>(i)) = P.r[i];
}

// Reduce the per-thread normaliser partials (8 columns each) to one vector per wave in LDS.
template <int D>
__device__ __forceinline__ void reduce_zp(float (&zp)[8], float* sZred) {
  constexpr int PPR = D / 8;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int off = PPR; off < 64; off <<= 1) zp[j] += __shfl_xor(zp[j], off);
  if (lane < PPR) {
#pragma unroll
    for (int j = 0; j < 8; ++j) sZred[w * D + lane * 8 + j] = zp[j];
  }
}

// S[pt] += K~^T V over the chunk (M = state row p, N = value column e, k = token i).
template <int C, int D, bool SPLIT>
__device__ __forceinline__ void state_mfma(f32x16 (&S)[D / 32], const __bf16* sK, const __bf16* sKlo,
                                           const __bf16* sV, int Ew, int lane) {
  constexpr int PK = Geo<C, D, true>::PK;
#pragma unroll 2
  for (int ik = 0; ik < C / 16; ++ik) {
    const bf16x8 vb = ld_rows8(sV, PK, ik * 16, Ew, lane);
#pragma unroll
    for (int pt = 0; pt < D / 32; ++pt) {
      S[pt] = mfma32(ld_rows8(sK, PK, ik * 16, pt * 32, lane), vb, S[pt]);
      if (SPLIT) S[pt] = mfma32(ld_rows8(sKlo, PK, ik * 16, pt * 32, lane), vb, S[pt]);
    }
  }
}

// One score tile A^T[i-tile it][j-tile jt] (M = i, N = j, k = feature) with the causal
// mask (DIAG) and decay D_ji = gamma^(j-i); adds its row sums to rsum and A V to num.
// qk holds the j-tile's Q operands (k = feature); lane column j = 32 jt + n, register
// row i = 32 it + dtile_row(r).
template <int C, int D, bool DECAY, bool NORM, bool DIAG>
__device__ __forceinline__ void score_tile(int it, int jt, const bf16x8 (&qk)[D / 16], const __bf16* sK,
                                           const __bf16* sV, f32x16& num, float& rsum, float lg, int Ew,
                                           int lane) {
  constexpr int PK = Geo<C, D, true>::PK;
  const int n = lane & 31;
  f32x16 acc = f32x16{};
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) acc = mfma32(ld_cols8(sK, PK, it * 32, kk * 16, lane), qk[kk], acc);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int ir = dtile_row(r, lane);
    if (DIAG) {
      acc[r] = ir <= n ? (DECAY ? acc[r] * exp2f((float)(n - ir) * lg) : acc[r]) : 0.f;
    } else if (DECAY) {
      acc[r] *= exp2f((float)(32 * (jt - it) + n - ir) * lg);
    }
    if (NORM) rsum += acc[r];
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
    const bf16x8 vv = ld_rows8_perm(sV, PK, it * 32, q, Ew, lane);
    num = mfma32(ah, vv, num);
    num = mfma32(al, vv, num);
  }
}

template <int C, int D, bool DECAY, bool NORM, bool ELU>
__global__ __launch_bounds__(2 * D) void k_summary(PrefillParams p) {
  using G = Geo<C, D, false>;
  constexpr bool SPLIT = DECAY || ELU;  // K~ inexact in bf16: keep a lo part
  extern __shared__ __align__(16) unsigned char smem[];
  const int seg = blockIdx.x, bh = blockIdx.y, head = bh % p.H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const float lg = DECAY ? p.log2g[head] : 0.f;
  __bf16* sK = (__bf16*)(smem + G::OFF_K);
  __bf16* sKlo = (__bf16*)(smem + G::OFF_KLO);
  __bf16* sV = (__bf16*)(smem + G::OFF_V);
  float* sF = (float*)(smem + G::OFF_F);
  const int Ew = 32 * w;

  f32x16 S[D / 32];
#pragma unroll
  for (int pt = 0; pt < D / 32; ++pt) S[pt] = f32x16{};
  float zrun[8];  // this thread's share of the segment's Z (its 8 columns, its rows)
#pragma unroll
  for (int j = 0; j < 8; ++j) zrun[j] = 0.f;

  const uint16_t* kb = (const uint16_t*)p.k + (size_t)bh * p.T * D;
  const uint16_t* vb = (const uint16_t*)p.v + (size_t)bh * p.T * D;
  const int c0 = seg * p.seg_chunks, c1 = min(c0 + p.seg_chunks, p.n_chunks);
  Pieces<C, D> pk, pv;
  load_pieces<C, D>(pk, kb + (size_t)c0 * C * D, min(C, p.T - c0 * C));
  load_pieces<C, D>(pv, vb + (size_t)c0 * C * D, min(C, p.T - c0 * C));
  for (int c = c0; c < c1; ++c) {
    const int L = min(C, p.T - c * C);
    const float a = DECAY ? exp2f((float)L * lg) : 1.f;
    __syncthreads();  // the previous chunk is done with LDS
    float zp[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) zp[j] = 0.f;
    commit_k<C, D, ELU, DECAY, true, SPLIT>(pk, sK, sKlo, G::PK, L, lg, zp);
    commit_v<C, D>(pv, sV, G::PK);
#pragma unroll
    for (int j = 0; j < 8; ++j) zrun[j] = a * zrun[j] + zp[j];
    if (c + 1 < c1) {  // next chunk's loads overlap this chunk's matrix work
      const int Ln = min(C, p.T - (c + 1) * C);
      load_pieces<C, D>(pk, kb + (size_t)(c + 1) * C * D, Ln);
      load_pieces<C, D>(pv, vb + (size_t)(c + 1) * C * D, Ln);
    }
    __syncthreads();
    if (DECAY) {
#pragma unroll
      for (int pt = 0; pt < D / 32; ++pt) S[pt] *= a;
    }
    state_mfma<C, D, SPLIT>(S, sK, sKlo, sV, Ew, lane);
  }
  // segment summary -> workspace [bh][seg][E], E = D*D + D
  const size_t E = (size_t)D * D + D;
  float* out = p.ws + ((size_t)bh * p.n_seg + seg) * E;
  const int n = lane & 31;
#pragma unroll
  for (int pt = 0; pt < D / 32; ++pt)
#pragma unroll
    for (int r = 0; r < 16; ++r) out[(size_t)(pt * 32 + dtile_row(r, lane)) * D + Ew + n] = S[pt][r];
  if (NORM) {
    __syncthreads();
    reduce_zp<D>(zrun, sF + G::F_ZRED);
    __syncthreads();
    if (tid < D) {
      float z = 0.f;
#pragma unroll
      for (int ww = 0; ww < G::NW; ++ww) z += sF[G::F_ZRED + ww * D + tid];
      out[(size_t)D * D + tid] = z;
    }
  } else if (tid < D) {
    out[(size_t)D * D + tid] = 0.f;
  }
}

template <int C, int D, bool DECAY, bool NORM, bool ELU>
__global__ __launch_bounds__(2 * D) void k_output(PrefillParams p) {
  using G = Geo<C, D, true>;
  constexpr bool SPLIT = DECAY || ELU;
  constexpr int NJ = C / 32;
  extern __shared__ __align__(16) unsigned char smem[];
  const int seg = blockIdx.x, bh = blockIdx.y, head = bh % p.H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, n = lane & 31, hh = lane >> 5;
  const int Ew = 32 * w;
  const float lg = DECAY ? p.log2g[head] : 0.f;
  __bf16* sQ = (__bf16*)(smem + G::OFF_Q);
  __bf16* sK = (__bf16*)(smem + G::OFF_K);
  __bf16* sKlo = (__bf16*)(smem + G::OFF_KLO);
  __bf16* sV = (__bf16*)(smem + G::OFF_V);
  float* sF = (float*)(smem + G::OFF_F);

  // exclusive prefix state of this segment (written by the scan)
  const size_t E = (size_t)D * D + D;
  const float* pre = p.ws + ((size_t)bh * p.n_seg + seg) * E;
  f32x16 S[D / 32];
#pragma unroll
  for (int pt = 0; pt < D / 32; ++pt)
#pragma unroll
    for (int r = 0; r < 16; ++r) S[pt][r] = pre[(size_t)(pt * 32 + dtile_row(r, lane)) * D + Ew + n];
  if (tid < D) sF[G::F_Z + tid] = NORM ? pre[(size_t)D * D + tid] : 0.f;
  for (int j = tid; j < C; j += G::NT) sF[G::F_THETA + j] = DECAY ? exp2f((float)(j + 1) * lg) : 1.f;

  const uint16_t* qb = (const uint16_t*)p.q + (size_t)bh * p.T * D;
  const uint16_t* kb = (const uint16_t*)p.k + (size_t)bh * p.T * D;
  const uint16_t* vb = (const uint16_t*)p.v + (size_t)bh * p.T * D;
  float* ob = (float*)p.o + (size_t)bh * p.T * D;
  const int c0 = seg * p.seg_chunks, c1 = min(c0 + p.seg_chunks, p.n_chunks);

  Pieces<C, D> pq, pk, pv;
  {
    const int L0 = min(C, p.T - c0 * C);
    load_pieces<C, D>(pq, qb + (size_t)c0 * C * D, L0);
    load_pieces<C, D>(pk, kb + (size_t)c0 * C * D, L0);
    load_pieces<C, D>(pv, vb + (size_t)c0 * C * D, L0);
  }
  for (int c = c0; c < c1; ++c) {
    const int t0 = c * C, L = min(C, p.T - t0);
    const float a = DECAY ? exp2f((float)L * lg) : 1.f;
    __syncthreads();  // the previous chunk is done with LDS (and Z is updated)
    float zp[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) zp[j] = 0.f;
    commit_q<C, D, ELU>(pq, sQ, G::PQ);
    commit_k<C, D, ELU, DECAY, false, ELU>(pk, sK, sKlo, G::PK, L, lg, zp);
    commit_v<C, D>(pv, sV, G::PK);
    const bool more = c + 1 < c1;
    const int Ln = more ? min(C, p.T - (c + 1) * C) : 0;
    // next chunk's keys and values stream in during this chunk's matrix work (rows past
    // Ln, including every row when there is no next chunk, read as zeros)
    load_pieces<C, D>(pk, kb + (size_t)(c + 1) * C * D, Ln);
    load_pieces<C, D>(pv, vb + (size_t)(c + 1) * C * D, Ln);
    __syncthreads();
    // stores of this chunk's outputs: rows past L are dropped by the buffer bound
    const __amdgpu_buffer_rsrc_t ors = make_rsrc(ob + (size_t)t0 * D, (uint32_t)L * D * 4);

#pragma unroll 1
    for (int jt = 0; jt < NJ; ++jt) {
      // num = gamma^(j+1) psi(q_j) S_prev   (M = j, N = e, k = state row p); S enters as
      // the B operand straight from its accumulator layout (D-tile feedback order), hi + lo
      f32x16 num = f32x16{};
#pragma unroll
      for (int pt = 0; pt < D / 32; ++pt)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          bf16x8 sh, sl;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const bf16_pair sp = split_bf16(S[pt][8 * q + j]);
            sh[j] = sp.hi;
            sl[j] = sp.lo;
          }
          const bf16x8 qa = ld_cols8_perm(sQ, G::PQ, jt * 32, pt * 32, q, lane);
          num = mfma32(qa, sh, num);
          num = mfma32(qa, sl, num);
        }
      if (DECAY) {
#pragma unroll
        for (int r = 0; r < 16; ++r) num[r] *= sF[G::F_THETA + jt * 32 + dtile_row(r, lane)];
      }
      // psi(q_j) . Z_prev for j = jt*32 + n (the two lane halves split the features)
      float qz = 0.f;
      if (NORM) {
        const __bf16* qr = sQ + (jt * 32 + n) * G::PQ + hh * (D / 2);
        const f32x4* zr = (const f32x4*)(sF + G::F_Z + hh * (D / 2));
#pragma unroll
        for (int e8 = 0; e8 < D / 2; e8 += 8) {
          const bf16x8 qv = *(const bf16x8*)(qr + e8);
          const f32x4 z0 = zr[e8 / 4], z1 = zr[e8 / 4 + 1];
#pragma unroll
          for (int j = 0; j < 4; ++j) qz += from_bf16(qv[j]) * z0[j] + from_bf16(qv[4 + j]) * z1[j];
        }
        qz += __shfl_xor(qz, 32);
      }
      // this row tile's Q operands for the score tiles (k = feature), loaded once
      bf16x8 qk[D / 16];
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) qk[kk] = ld_cols8(sQ, G::PQ, jt * 32, kk * 16, lane);
      // scores A^T (M = i, N = j, k = feature), masked and decayed; then num += A V.
      // Off-diagonal tiles (it < jt) first, in a loop whose body is one basic block; the
      // diagonal tile (causal mask) last.
      float rsum = 0.f;
#pragma unroll 1
      for (int it = 0; it < jt; ++it) score_tile<C, D, DECAY, NORM, false>(it, jt, qk, sK, sV, num, rsum, lg, Ew, lane);
      score_tile<C, D, DECAY, NORM, true>(jt, jt, qk, sK, sV, num, rsum, lg, Ew, lane);
      // o_j = num_j / den_j; den_j is formed in lane j%32 and fetched by the lanes holding row j
      float den = 1.f;
      if (NORM) den = sF[G::F_THETA + jt * 32 + n] * qz + (rsum + __shfl_xor(rsum, 32)) + p.eps;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = jt * 32 + dtile_row(r, lane);
        const float val = NORM ? num[r] / __shfl(den, dtile_row(r, lane)) : num[r];
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(val), ors, (uint32_t)(j * D + Ew + n) * 4, 0, 0);
      }
    }

    // next chunk's queries: issued once this chunk's queries are no longer read
    load_pieces<C, D>(pq, qb + (size_t)(c + 1) * C * D, Ln);
    // state update: K~ = Xi psi(K) as hi + lo, S <- gamma^L S + K~^T V, Z <- gamma^L Z + K~^T 1
    if (NORM) reduce_zp<D>(zp, sF + G::F_ZRED);
    if (DECAY) {
      __syncthreads();  // every wave is done reading psi(K) for scores
#pragma unroll
      for (int i = 0; i < G::NPC; ++i) {
        const int row = piece_row<C, D>(i), c8 = piece_cols<C, D>(i);
        const float xi = row < L ? exp2f((float)(L - 1 - row) * lg) : 0.f;
        const bf16x8 h8 = *(const bf16x8*)(sK + row * G::PK + c8);
        bf16x8 l8 = bf16x8{};
        if (ELU) l8 = *(const bf16x8*)(sKlo + row * G::PK + c8);
        bf16x8 hi, lo;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const bf16_pair sp = split_bf16((from_bf16(h8[j]) + from_bf16(l8[j])) * xi);
          hi[j] = sp.hi;
          lo[j] = sp.lo;
        }
        *(bf16x8*)(sK + row * G::PK + c8) = hi;
        *(bf16x8*)(sKlo + row * G::PK + c8) = lo;
      }
    }
    __syncthreads();
    if (NORM && tid < D) {
      float z = 0.f;
#pragma unroll
      for (int ww = 0; ww < G::NW; ++ww) z += sF[G::F_ZRED + ww * D + tid];
      sF[G::F_Z + tid] = a * sF[G::F_Z + tid] + z;
    }
    if (DECAY) {
#pragma unroll
      for (int pt = 0; pt < D / 32; ++pt) S[pt] *= a;
    }
    state_mfma<C, D, SPLIT>(S, sK, sKlo, sV, Ew, lane);
  }
}

template <int C, int D, bool DECAY, bool NORM, bool ELU>
hipError_t launch_flags(const PrefillParams& p, hipStream_t s, bool out) {
  const void* kern = out ? (const void*)k_output<C, D, DECAY, NORM, ELU> : (const void*)k_summary<C, D, DECAY, NORM, ELU>;
  const int lds = out ? Geo<C, D, true>::LDS_BYTES : Geo<C, D, false>::LDS_BYTES;
  hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  dim3 grid(p.n_seg, p.B * p.H);
  void* args[] = {(void*)&p};
  e = hipLaunchKernel(kern, grid, dim3(2 * D), args, lds, s);
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

// Runtime flags -> template instantiation.
template <int C, int D>
hipError_t launch_cd(const PrefillParams& p, hipStream_t s, bool out) {
  const bool decay = p.has_decay != 0, norm = p.normalize != 0, elu = p.psi == LA_PSI_ELU1;
  if (decay) {
    if (norm) return elu ? launch_flags<C, D, true, true, true>(p, s, out) : launch_flags<C, D, true, true, false>(p, s, out);
    return elu ? launch_flags<C, D, true, false, true>(p, s, out) : launch_flags<C, D, true, false, false>(p, s, out);
  }
  if (norm) return elu ? launch_flags<C, D, false, true, true>(p, s, out) : launch_flags<C, D, false, true, false>(p, s, out);
  return elu ? launch_flags<C, D, false, false, true>(p, s, out) : launch_flags<C, D, false, false, false>(p, s, out);
}

}  // namespace pf

// Per-(C, D) entry points, each defined in its own translation unit.
hipError_t launch_prefill_bf16_c64_d64(const PrefillParams& p, hipStream_t s, bool out);
hipError_t launch_prefill_bf16_c64_d128(const PrefillParams& p, hipStream_t s, bool out);
hipError_t launch_prefill_bf16_c128_d64(const PrefillParams& p, hipStream_t s, bool out);
hipError_t launch_prefill_bf16_c128_d128(const PrefillParams& p, hipStream_t s, bool out);

}  // namespace la
