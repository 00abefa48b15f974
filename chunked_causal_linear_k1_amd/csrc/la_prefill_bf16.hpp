// la_prefill_bf16.hpp -- chunkwise causal linear attention, bf16 inputs, fp32 state,
// MFMA 32x32x16 bf16 -> fp32 on gfx950. Kernel templates; instantiated per head width D
// in la_prefill_bf16_c64_d*.hip.
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
// Two passes share the chunk machinery:
//   k_summary: one workgroup per (sequence, segment of chunks); folds its chunks'
//              summaries into one segment summary (Kernel 1's summaries, reduced
//              over the segment) and writes it to the workspace.
//   output   : one workgroup per (sequence, segment); starts from the segment's
//              exclusive prefix (written there by the scan), walks its chunks,
//              emits o for every real token (Kernels 1 and 3 fused) and carries the
//              state from chunk to chunk on chip. Two kernels: k_output_sh (D/32
//              waves, score tiles shared through LDS) and k_output_w8 (two waves per
//              SIMD within one workgroup, d = 128).
// Both are instantiated at C = 64: a 128-token chunk is walked in two 64-token steps
// (la_prefill_bf16.hip), since neither pass depends on how a segment's tokens are grouped.
//
// Wave w owns value columns [32w, 32w+32) of the state S (all n_psi rows, fp32 in
// registers) and of every output tile. All LDS tiles are row-major; operands whose k
// runs over tokens use the gfx950 transpose read (ds_read_b64_tr_b16).
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
// denominator use the same rounded scores. With elu+1 features, a denominator and no decay,
// the output pass also rounds S (in psi(Q) S) and psi(k) (in the state update) to bf16 once
// (see k_output_w8); the summary pass keeps them hi + lo.
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

// Token rows are rsb bytes apart (D * 2 when a head's tokens are contiguous). Rows >= valid
// read as zeros (bounded buffer resource, no branches).
template <int C, int D>
__device__ __forceinline__ void load_pieces(Pieces<C, D>& P, const uint16_t* __restrict__ g, int valid,
                                            uint32_t rsb) {
  using G = Geo<C, D, true>;
  static_assert(G::NT % G::PPR == 0, "piece i of a thread is i * NT / PPR rows below piece 0");
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(g, rows_extent(valid, rsb, D * 2));
  const uint32_t v0 = (uint32_t)piece_row<C, D>(0) * rsb + (uint32_t)piece_cols<C, D>(0) * 2;
#pragma unroll
  for (int i = 0; i < G::NPC; ++i) P.r[i] = buf_load16(rs, v0, (uint32_t)(i * (G::NT / G::PPR)) * rsb);
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
    const float xi = row < L ? (DECAY ? exp2_hw((float)(L - 1 - row) * lg) : 1.f) : 0.f;
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

// S[pt] += K^T (Xi V) over the chunk: keys exact (no lo part), the values of this wave's
// columns scaled by Xi (table sXi, per token) and split into hi + lo in registers. Element j
// of the V operand at step ik is token 16 ik + 8 h + j (h = lane / 32).
template <int C, int D>
__device__ __forceinline__ void state_mfma_vdec(f32x16 (&S)[D / 32], const __bf16* sK, const __bf16* sV,
                                                const float* sXi, int Ew, int lane) {
  constexpr int PK = Geo<C, D, true>::PK;
  const float* xr = sXi + 8 * (lane >> 5);
#pragma unroll 2
  for (int ik = 0; ik < C / 16; ++ik) {
    const bf16x8 vb = ld_rows8(sV, PK, ik * 16, Ew, lane);
    const f32x4 x0 = *(const f32x4*)(xr + ik * 16), x1 = *(const f32x4*)(xr + ik * 16 + 4);
    float vx[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      vx[j] = from_bf16(vb[j]) * x0[j];
      vx[4 + j] = from_bf16(vb[4 + j]) * x1[j];
    }
    bf16x8 vh, vl;
    split8_trunc(vx, vh, vl);
#pragma unroll
    for (int pt = 0; pt < D / 32; ++pt) {
      const bf16x8 ka = ld_rows8(sK, PK, ik * 16, pt * 32, lane);
      S[pt] = mfma32(ka, vh, S[pt]);
      S[pt] = mfma32(ka, vl, S[pt]);
    }
  }
}

// Summary-pass LDS image. With identity keys and decay the decay goes on the values (see
// k_summary), so there is no K lo tile and V moves up: about 40 KiB at C = 64, d = 128, so
// three workgroups share a CU instead of two.
template <int C, int D, bool VDEC>
struct SumGeo {
  using B = Geo<C, D, false>;
  static constexpr int NW = B::NW, PK = B::PK;
  static constexpr int OFF_K = B::OFF_K, OFF_KLO = B::OFF_KLO;
  static constexpr int OFF_V = VDEC ? B::OFF_KLO : B::OFF_V;
  static constexpr int OFF_F = OFF_V + B::K_BYTES;
  static constexpr int F_ZRED = B::F_ZRED;  // per-wave Z partials [NW][D]
  static constexpr int F_XI = B::F_THETA;   // Xi_i = gamma^(L-1-i), 0 past L [C]
  static constexpr int LDS_BYTES = OFF_F + 4 * (F_XI + C);
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

template <int C, int D, bool DECAY, bool NORM, bool ELU, bool ONE = false>
__global__ __launch_bounds__(2 * D) void k_summary(PrefillParams p) {
  // Identity keys are exact in bf16: the decay goes on the values, S += K^T (Xi V), with Xi V
  // split hi + lo in registers. elu+1 keys keep K~ = Xi psi(K) as hi + lo, except with ONE
  // (elu+1, a denominator, no decay, no final state asked for): psi(K) rounded to bf16 once
  // (nearest even), the policy of the output pass, since these records reach only outputs,
  // which average the rounding over the features; Z still sums the unrounded features.
  static_assert(!ONE || (ELU && NORM && !DECAY), "single rounding: elu+1 keys with a denominator, no decay");
  constexpr bool VDEC = DECAY && !ELU;
  constexpr bool SPLIT = (DECAY || ELU) && !VDEC && !ONE;  // K~ inexact in bf16: keep a lo part
  using G = SumGeo<C, D, VDEC>;
  extern __shared__ __align__(16) unsigned char smem[];
  const int bh = blockIdx.x, seg = blockIdx.y, head = bh % p.H;
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

  const SeqSpan sq = seq_span(p, bh);
  const int T = sq.T, n_chunks = (T + C - 1) / C;
  const uint32_t rse = (uint32_t)p.tok_rows * D, rsb = rse * 2;  // elements / bytes between token rows
  const uint16_t* kb = (const uint16_t*)p.k + sq.row0 * D;
  const uint16_t* vb = (const uint16_t*)p.v + sq.row0 * D;
  const int c0 = seg * p.seg_chunks, c1 = min(min(c0 + p.seg_chunks, n_chunks), p.sum_end);
  const int L0 = c0 < c1 ? min(C, T - c0 * C) : 0;
  Pieces<C, D> pk, pv;
  load_pieces<C, D>(pk, kb + (size_t)c0 * C * rse, L0, rsb);
  load_pieces<C, D>(pv, vb + (size_t)c0 * C * rse, L0, rsb);
  for (int c = c0; c < c1; ++c) {
    const int L = min(C, T - c * C);
    const float a = DECAY ? exp2_hw((float)L * lg) : 1.f;
    lds_barrier();  // the previous chunk is done with LDS
    float zp[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) zp[j] = 0.f;
    commit_k<C, D, ELU, DECAY, !VDEC, SPLIT>(pk, sK, sKlo, G::PK, L, lg, zp);
    commit_v<C, D>(pv, sV, G::PK);
    if (VDEC) {
      for (int j = tid; j < C; j += 2 * D) sF[G::F_XI + j] = j < L ? exp2_hw((float)(L - 1 - j) * lg) : 0.f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) zrun[j] = a * zrun[j] + zp[j];
    if (c + 1 < c1) {  // next chunk's loads overlap this chunk's matrix work
      const int Ln = min(C, T - (c + 1) * C);
      load_pieces<C, D>(pk, kb + (size_t)(c + 1) * C * rse, Ln, rsb);
      load_pieces<C, D>(pv, vb + (size_t)(c + 1) * C * rse, Ln, rsb);
    }
    lds_barrier();
    if (DECAY) {
#pragma unroll
      for (int pt = 0; pt < D / 32; ++pt) S[pt] *= a;
    }
    if (VDEC)
      state_mfma_vdec<C, D>(S, sK, sV, sF + G::F_XI, Ew, lane);
    else
      state_mfma<C, D, SPLIT>(S, sK, sKlo, sV, Ew, lane);
  }
  // segment summary -> workspace [bh][seg][E], E = D*D + D
  const size_t E = (size_t)D * D + D;
  float* out = p.ws + rec_index(p, bh, seg) * E;
  const int n = lane & 31;
#pragma unroll
  for (int pt = 0; pt < D / 32; ++pt)
#pragma unroll
    for (int r = 0; r < 16; ++r) out[(size_t)(pt * 32 + dtile_row(r, lane)) * D + Ew + n] = S[pt][r];
  if (NORM) {
    lds_barrier();
    reduce_zp<D>(zrun, sF + G::F_ZRED);
    lds_barrier();
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

// Output kernel with the score tiles computed once per workgroup.
//
// Each wave produces a share of the C/32 x (C/32 + 1)/2 score tiles A^T (masked, decayed,
// split into bf16 hi + lo) and writes them to LDS; after a barrier every wave reads the
// tiles it needs as MFMA operands for its value columns. Compared with every wave
// computing every tile, this removes 3/4 of the score MFMAs and of the score epilogue
// (mask, decay, split). For identity psi the score tiles share LDS with the K~ lo tile,
// which is only needed afterwards, in the state update.
template <int C, int D, bool ELU>
struct ShGeo {
  static constexpr int NW = D / 32;
  static constexpr int NJ = C / 32;
  static constexpr int NTILE = NJ * (NJ + 1) / 2;
  static constexpr int PQ = D + 8;          // Q: row reads
  static constexpr int PK = D;              // K (and K lo): XOR-swizzled, see swz_off
  static constexpr int PV = D;              // V: XOR-swizzled like K (transpose reads)
  static constexpr int PA = 40;             // score tiles: 32 x 32, row pitch 40
  static constexpr int A_TILE = 2 * 32 * PA * 2;  // hi + lo, bytes
  static constexpr int Q_BYTES = C * PQ * 2;
  static constexpr int K_BYTES = C * PK * 2;
  static constexpr int V_BYTES = C * PV * 2;
  static constexpr int A_BYTES = NTILE * A_TILE;
  // K lo directly after K, so one register addresses both (offsets stay below 64 KiB)
  static constexpr int OFF_Q = 0;
  static constexpr int OFF_K = Q_BYTES;
  static constexpr int OFF_KLO = OFF_K + K_BYTES;  // psi(k) lo (elu+1) or K~ lo (decay)
  static constexpr int OFF_A = ELU ? OFF_KLO + K_BYTES : OFF_KLO;  // aliases K lo for identity psi
  static constexpr int OFF_V = ELU ? OFF_A + A_BYTES : OFF_KLO + (A_BYTES > K_BYTES ? A_BYTES : K_BYTES);
  static constexpr int OFF_F = OFF_V + V_BYTES;
  static constexpr int F_Z = 0;               // Z [D]
  static constexpr int F_ZRED = D;            // per-wave Z partials [NW][D]
  static constexpr int F_THETA = D + NW * D;  // gamma^(j+1) [C]
  static constexpr int F_R = F_THETA + C;     // per-tile score row sums [NTILE][32]
  static constexpr int F_XI = F_R + NTILE * 32;  // Xi_i = gamma^(L-1-i), 0 past L [C] (decay on V)
  static constexpr int LDS_BYTES = OFF_F + 4 * (F_XI + C);
  static constexpr bool FITS = LDS_BYTES <= 160 * 1024;
  // waves per SIMD: two when two workgroups' LDS images fit in the CU (registers are then
  // capped at 256 per wave), so a second wave computes while the first one's global loads and
  // stores wait to issue; else one
  static constexpr int OCC = 2 * LDS_BYTES <= 160 * 1024 ? 2 : 1;
};

// The shared-score kernel's LDS image for (ELU, NORM, DECAY): elu+1 keys keep a K lo tile
// except under the single-rounding policy (elu+1 with a denominator and no decay, see
// k_output_w8), which takes the identity layout (score tiles where K lo would be).
template <int C, int D, bool DECAY, bool NORM, bool ELU>
using ShGeoF = ShGeo<C, D, ELU && (DECAY || !NORM)>;

// tile t <-> (it, jt) with it <= jt, t = jt (jt + 1) / 2 + it; branch-free (up to 16 row tiles)
__device__ __forceinline__ int tile_jt(int t) {
  int jt = 0;
#pragma unroll
  for (int k = 1; k < 16; ++k) jt += t >= k * (k + 1) / 2;
  return jt;
}

// S[pt] += K~^T V over the chunk, K~ = hi (+ lo) in LDS with pitch PK, V with pitch PV.
template <int C, int D, bool SPLIT, int PK, int PV>
__device__ __forceinline__ void state_mfma_p(f32x16 (&S)[D / 32], const __bf16* sK, const __bf16* sKlo,
                                             const __bf16* sV, int Ew, int lane) {
#pragma unroll 2
  for (int ik = 0; ik < C / 16; ++ik) {
    const bf16x8 vb = ld_rows8(sV, PV, ik * 16, Ew, lane);
#pragma unroll
    for (int pt = 0; pt < D / 32; ++pt) {
      S[pt] = mfma32(ld_rows8(sK, PK, ik * 16, pt * 32, lane), vb, S[pt]);
      if (SPLIT) S[pt] = mfma32(ld_rows8(sKlo, PK, ik * 16, pt * 32, lane), vb, S[pt]);
    }
  }
}

// Output kernel addressing. The LDS image (up to 160 KiB) is larger than the 64 KiB reach
// of a DS instruction's immediate offset, so each region is addressed from per-lane
// byte bases pinned in registers (see pin) plus compile-time immediates below 64 KiB.
// K and K lo are XOR-swizzled (swz_off); since swz<D>(r0 + x) == swz<D>(x) whenever r0
// is a multiple of 16 and x < 32, a swizzled read of any row block is one of a few
// per-lane bases plus the row block's constant offset.
template <int C, int D, bool DECAY, bool NORM, bool ELU, bool OBF>
__global__ __launch_bounds__(2 * D)
__attribute__((amdgpu_waves_per_eu(ShGeoF<C, D, DECAY, NORM, ELU>::OCC, ShGeoF<C, D, DECAY, NORM, ELU>::OCC)))
void k_output_sh(PrefillParams p) {
  using G = ShGeoF<C, D, DECAY, NORM, ELU>;
  using PG = Geo<C, D, true>;  // piece geometry of the global -> LDS copies
  static_assert(G::FITS, "LDS budget");
  static_assert(PG::NT / PG::PPR == 16, "piece i of a thread covers row 16 i + tid / PPR");
  // elu+1 with a denominator and no decay: S (in psi(Q) S) and psi(K) (scores, state update,
  // Z) are rounded to bf16 once, as in k_output_w8; the score tiles stay hi + lo
  constexpr bool PLAIN = ELU && NORM && !DECAY;
  constexpr bool SPLIT = (DECAY || ELU) && !PLAIN;
  // Identity keys are exact in bf16, so the decay of the state update goes on the values:
  // S += K^T (Xi V), with Xi V split into hi + lo in registers from the transpose reads of V.
  // K stays as committed: no K~ pass, no barrier around it. (elu+1 keys are already two-term,
  // and decayed values would make that four MFMAs per step, so elu+1 keeps K~ = Xi psi(K).)
  constexpr bool VDEC = DECAY && !ELU;
  constexpr int NJ = G::NJ, NW = G::NW, NPC = PG::NPC;
  constexpr int TPW = (G::NTILE + NW - 1) / NW;  // score tiles per wave (the last round partial)
  constexpr int PQ = G::PQ, PV = G::PV, PA = G::PA;
  constexpr int KLO = G::K_BYTES;    // K lo, relative to K
  constexpr int ALO = 32 * PA * 2;   // a score tile's lo half, relative to its hi half
  extern __shared__ __align__(16) unsigned char smem[];
  const int bh = blockIdx.x, seg = blockIdx.y, head = bh % p.H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, n = lane & 31, hh = lane >> 5;
  const int L16 = lane & 15, g = lane >> 4;
  const int Ew = 32 * w;
  const float lg = DECAY ? p.log2g[head] : 0.f;

  // per-lane LDS bases (bytes); pieces of this thread: row prow + 16 i, columns pcol..+7
  const int prow = tid / PG::PPR, pcol = (tid % PG::PPR) * 8;
  const int trow = 8 * (g >> 1) + (L16 >> 2), tcol = 16 * (g & 1) + 4 * (L16 & 3);  // transpose reads
  unsigned char* const qP = smem + pin(G::OFF_Q + (prow * PQ + pcol) * 2);
  const unsigned char* const qC = smem + pin(G::OFF_Q + (n * PQ + 4 * hh) * 2);  // psi(Q) S operand
  const unsigned char* const qS = smem + pin(G::OFF_Q + (n * PQ + 8 * hh) * 2);  // score operand
  const unsigned char* const qZ = smem + pin(G::OFF_Q + (n * PQ + hh * (D / 2)) * 2);  // psi(q) . Z
  unsigned char* const kP = smem + pin(G::OFF_K + swz_off<D>(prow, pcol) * 2);
  const unsigned char* kR[D / 16];     // score operand: row n, features 16 kk + 8 hh
  const unsigned char* kT[D / 32][2];  // state-update operand: rows trow (+4), columns 32 pt + tcol
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) kR[kk] = smem + pin(G::OFF_K + swz_off<D>(n, 16 * kk + 8 * hh) * 2);
#pragma unroll
  for (int pt = 0; pt < D / 32; ++pt) {
    kT[pt][0] = smem + pin(G::OFF_K + swz_off<D>(trow, 32 * pt + tcol) * 2);
    kT[pt][1] = smem + pin(G::OFF_K + swz_off<D>(trow + 4, 32 * pt + tcol) * 2);
  }
  unsigned char* const vP = smem + pin(G::OFF_V + swz_off<D>(prow, pcol) * 2);
  const unsigned char* const vT0 = smem + pin(G::OFF_V + swz_off<D>(trow, Ew + tcol) * 2);
  const unsigned char* const vT1 = smem + pin(G::OFF_V + swz_off<D>(trow + 4, Ew + tcol) * 2);
  unsigned char* const aW = smem + pin(G::OFF_A + (n * PA + 4 * hh) * 2);
  const unsigned char* const aR = smem + pin(G::OFF_A + (n * PA + 8 * hh) * 2);
  float* const sF = (float*)(smem + pin(G::OFF_F));
  float* const fN = (float*)(smem + pin(G::OFF_F + 4 * n));  // per-token entries of this lane's column

  // exclusive prefix state of this segment (written by the scan)
  const size_t E = (size_t)D * D + D;
  const float* pre = p.ws + rec_index(p, bh, seg) * E;
  f32x16 S[D / 32];
#pragma unroll
  for (int pt = 0; pt < D / 32; ++pt)
#pragma unroll
    for (int r = 0; r < 16; ++r) S[pt][r] = pre[(size_t)(pt * 32 + dtile_row(r, lane)) * D + Ew + n];
  if (tid < D) sF[G::F_Z + tid] = NORM ? pre[(size_t)D * D + tid] : 0.f;
  for (int j = tid; j < C; j += 2 * D) sF[G::F_THETA + j] = DECAY ? exp2_hw((float)(j + 1) * lg) : 1.f;

  // this lane's score-tile factors (column j%32 = n and register rows fixed):
  // diagonal tile gamma^(n - i_r) masked to i_r <= n; off-diagonal base gamma^(n + 32 - i_r)
  float fdiag[16], foff[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int ir = dtile_row(r, lane);
    fdiag[r] = ir <= n ? (DECAY ? exp2_hw((float)(n - ir) * lg) : 1.f) : 0.f;
    foff[r] = DECAY ? exp2_hw((float)(n + 32 - ir) * lg) : 1.f;
  }

  const SeqSpan sq = seq_span(p, bh);
  const int T = sq.T, n_chunks = (T + C - 1) / C;
  const uint32_t rse = (uint32_t)p.tok_rows * D, rsb = rse * 2;  // elements / bytes between token rows
  constexpr int OES = OBF ? 2 : 4;  // output element bytes
  const uint16_t* qb = (const uint16_t*)p.q + sq.row0 * D;
  const uint16_t* kb = (const uint16_t*)p.k + sq.row0 * D;
  const uint16_t* vb = (const uint16_t*)p.v + sq.row0 * D;
  unsigned char* ob = (unsigned char*)p.o + sq.row0 * D * OES;
  const int c0 = seg * p.seg_chunks, c1 = min(c0 + p.seg_chunks, n_chunks);
  if (c0 >= c1) return;  // segment past the end of a shorter sequence: nothing to write

  Pieces<C, D> pq, pk, pv;
  {
    const int L0 = min(C, T - c0 * C);
    load_pieces<C, D>(pq, qb + (size_t)c0 * C * rse, L0, rsb);
    load_pieces<C, D>(pk, kb + (size_t)c0 * C * rse, L0, rsb);
    load_pieces<C, D>(pv, vb + (size_t)c0 * C * rse, L0, rsb);
    vm_drain();  // entering the loop with nothing in flight, see the prefetch below
  }
  for (int c = c0; c < c1; ++c) {
    const int t0 = c * C, L = min(C, T - t0);
    const float a = DECAY ? exp2_hw((float)L * lg) : 1.f;
    lds_barrier();  // the previous chunk is done with LDS (and Z is updated)

    // ---- commit this chunk's tiles: psi(Q) rounded to bf16; K swizzled (psi(k) as hi + lo
    // for elu+1; raw keys for identity, rows past T zero from the bounded load); V raw
    float zp[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) zp[j] = 0.f;
#pragma unroll
    for (int i = 0; i < NPC; ++i) {
      uint4 raw = pq.r[i];
      if (ELU) {
        const bf16x8 x = __builtin_bit_cast(bf16x8, raw);
        bf16x8 y;
#pragma unroll
        for (int j = 0; j < 8; ++j) y[j] = to_bf16(elu1(from_bf16(x[j])));
        raw = __builtin_bit_cast(uint4, y);
      }
      *(uint4*)(qP + i * 16 * PQ * 2) = raw;
    }
#pragma unroll
    for (int i = 0; i < NPC; ++i) {
      const int off = i * 16 * D * 2;
      if (!ELU && !NORM) {
        *(uint4*)(kP + off) = pk.r[i];
        continue;
      }
      const int row = prow + 16 * i;
      const float live = row < L ? 1.f : 0.f;
      const float xi = row < L ? (DECAY ? exp2_hw((float)(L - 1 - row) * lg) : 1.f) : 0.f;
      const bf16x8 x = __builtin_bit_cast(bf16x8, pk.r[i]);
      float f[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) f[j] = ELU ? elu1(from_bf16(x[j])) * live : from_bf16(x[j]);
      if (PLAIN) {  // Z from the same rounded features as the state
        bf16x8 y;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          y[j] = to_bf16(f[j]);
          zp[j] += from_bf16(y[j]);
        }
        *(bf16x8*)(kP + off) = y;
        continue;
      }
      if (NORM) {
#pragma unroll
        for (int j = 0; j < 8; ++j) zp[j] += f[j] * xi;
      }
      if (ELU) {
        bf16x8 hi, lo;
        split8_rne(f, hi, lo);  // hi alone is the score operand
        *(bf16x8*)(kP + off) = hi;
        *(bf16x8*)(kP + off + KLO) = lo;
      } else {
        *(uint4*)(kP + off) = pk.r[i];
      }
    }
#pragma unroll
    for (int i = 0; i < NPC; ++i) *(uint4*)(vP + i * 16 * D * 2) = pv.r[i];
    if (VDEC) {  // Xi of this chunk (the previous chunk's state update is done: barrier above)
      for (int j = tid; j < C; j += 2 * D) sF[G::F_XI + j] = j < L ? exp2_hw((float)(L - 1 - j) * lg) : 0.f;
    }
    const bool more = c + 1 < c1;
    const int Ln = more ? min(C, T - (c + 1) * C) : 0;
    lds_barrier();
    // next chunk's tiles stream in during this chunk's matrix work (rows past Ln read as
    // zero). They are issued among the score MFMAs (one load after each, see below), so the
    // wave keeps the MFMA pipe fed while the vector memory unit accepts them, and before
    // this chunk's output stores: the vmcnt wait at the next commit then covers only these
    // loads, not the stores.
    load_pieces<C, D>(pq, qb + (size_t)(c + 1) * C * rse, Ln, rsb);
    load_pieces<C, D>(pk, kb + (size_t)(c + 1) * C * rse, Ln, rsb);
    load_pieces<C, D>(pv, vb + (size_t)(c + 1) * C * rse, Ln, rsb);

    // ---- score tiles A^T (M = i, N = j, k = feature), masked, decayed, split into hi + lo
    // and shared through LDS: wave w computes tiles w, w + NW, ... Software-pipelined: the
    // MFMA chain of the next tile is interleaved with the epilogue (mask, decay, split, LDS
    // writes) of the current one, so the VALU work fills the chain's latency.
    auto score_chain = [&](int t) {
      const int jt = tile_jt(t), it = t - jt * (jt + 1) / 2;
      bf16x8 ka[D / 16], qv[D / 16];
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        ka[kk] = *(const bf16x8*)(kR[kk] + it * 32 * D * 2);
        qv[kk] = *(const bf16x8*)(qS + (jt * 32 * PQ + kk * 16) * 2);
      }
      f32x16 acc = f32x16{};
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) acc = mfma32(ka[kk], qv[kk], acc);
      return acc;
    };
    auto score_epilogue = [&](int t, const f32x16& acc) {
      const int jt = tile_jt(t), it = t - jt * (jt + 1) / 2;
      const bool diag = it == jt;
      const float tf = (DECAY && !diag) ? exp2_hw((float)(32 * (jt - it - 1)) * lg) : 1.f;
      float av[16];
      float rs = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        av[r] = acc[r] * ((diag ? fdiag[r] : foff[r]) * tf);
        if (NORM) rs += av[r];
      }
      if (NORM) {
        rs += __shfl_xor(rs, 32);
        if (hh == 0) fN[G::F_R + t * 32] = rs;
      }
      // A[j = n][i = 8 q4 + 4 hh + 0..3] as 8-byte runs: registers 8q..8q+3 are columns
      // 16q + 4hh + 0..3, registers 8q+4..8q+7 columns 16q + 8 + 4hh + 0..3
      unsigned char* at = aW + t * G::A_TILE;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        bf16x8 h8, l8;
        split8_trunc(av + 8 * q, h8, l8);
        const u32x4 hv = __builtin_bit_cast(u32x4, h8), lv = __builtin_bit_cast(u32x4, l8);
        *(uint2*)(at + 32 * q) = make_uint2(hv[0], hv[1]);
        *(uint2*)(at + 32 * q + 16) = make_uint2(hv[2], hv[3]);
        *(uint2*)(at + 32 * q + ALO) = make_uint2(lv[0], lv[1]);
        *(uint2*)(at + 32 * q + 16 + ALO) = make_uint2(lv[2], lv[3]);
      }
    };
    // Every wave runs TPW tiles, so the phase is straight-line code the schedule can
    // interleave: a wave with fewer tiles (or none, when there are fewer tiles than waves)
    // recomputes the last tile and writes the same bytes to the same place as the wave that
    // owns it (it would wait at the barrier anyway).
    {
      // next-chunk loads per score MFMA (3 NPC loads over TPW tiles of D / 16 MFMAs)
      constexpr int LPM = (3 * NPC + TPW * (D / 16) - 1) / (TPW * (D / 16));
      int tp = min(w, G::NTILE - 1);
      f32x16 prev = score_chain(tp);
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * (D / 16), 0);  // the first tile's operands
#pragma unroll
      for (int i = 0; i < D / 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x020, LPM, 0);  // next-chunk loads
      }
#pragma unroll
      for (int u = 1; u < TPW; ++u) {
        const int t = min(w + u * NW, G::NTILE - 1);
        const f32x16 cur = score_chain(t);
        score_epilogue(tp, prev);
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * (D / 16), 0);  // the next tile's operands
#pragma unroll
        for (int i = 0; i < D / 16; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // one MFMA of the next tile
          __builtin_amdgcn_sched_group_barrier(0x020, LPM, 0);  // next-chunk loads
          __builtin_amdgcn_sched_group_barrier(0x002, 14, 0);   // epilogue VALU of this one
        }
        __builtin_amdgcn_sched_group_barrier(0x200, 8, 0);     // its LDS writes
        prev = cur;
        tp = t;
      }
      score_epilogue(tp, prev);
    }
    lds_barrier();

    // ---- outputs for this wave's value columns, computed transposed: numT[e][j] (M = value
    // column e, N = token j), so each lane ends up with 4 consecutive columns of one token
    // row (16-byte stores) and the per-token factors are lane scalars.
    const __amdgpu_buffer_rsrc_t ors = make_rsrc(ob + (size_t)t0 * rse * OES, rows_extent(L, rse * OES, D * OES));
    // All NJ row tiles accumulate together (NJ independent MFMA chains), in steps whose LDS
    // operands are read one step ahead (double-buffered registers; the schedule barriers keep
    // the next step's reads above this step's MFMAs). S steps (one per state-row tile pt):
    // numT[jt] += S_prev^T psi(Q)^T over the tile's 32 state rows (k in the D-tile feedback
    // order), with only that tile of S held as hi + lo. A V steps (one per 16-token half q of
    // token tile it): numT[jt] += V^T A^T for every jt >= it, so each V operand is read once.
    // For each row tile the MFMAs happen in the order one tile at a time would do them.
    constexpr int NPT = D / 32;
    f32x16 num[NJ];
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt) num[jt] = f32x16{};
    bf16x8 qo[2][NJ][2];  // S step operands: psi(Q) rows of every row tile, this state-row tile
    bf16x8 vo[2];         // A V step operands: V of the half token tile ...
    bf16x8 ao[2][NJ][2];  // ... and the score tiles (hi, lo) of every row tile jt >= it
    auto load_s = [&](int pt, int buf) {
#pragma unroll
      for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const unsigned char* qa = qC + (jt * 32 * PQ + pt * 32 + 16 * q) * 2;
          qo[buf][jt][q] = cat8(*(const bf16x4*)qa, *(const bf16x4*)(qa + 16));
        }
    };
    auto load_av = [&](int st, int buf) {  // step st: token tile st / 2, half st % 2
      const int it = st >> 1, q = st & 1, r0 = it * 32 + 16 * q;
      vo[buf] = cat8(lds_read_tr4((const __bf16*)(vT0 + r0 * D * 2)), lds_read_tr4((const __bf16*)(vT1 + r0 * D * 2)));
#pragma unroll
      for (int jt = it; jt < NJ; ++jt) {
        const unsigned char* at = aR + (jt * (jt + 1) / 2 + it) * G::A_TILE + 32 * q;
        ao[buf][jt][0] = *(const bf16x8*)at;
        ao[buf][jt][1] = *(const bf16x8*)(at + ALO);
      }
    };
    // DS read instructions of each step's operands (one read2 per psi(Q) pair; two transpose
    // reads and two reads per row tile for an A V step)
    constexpr int RD_S = 2 * NJ;
    auto rd_av = [](int st) constexpr { return 2 + 2 * (NJ - (st >> 1)); };
    load_s(0, 0);
    static_for<0, NPT>([&](auto ipt) {
      constexpr int pt = decltype(ipt)::value;
      if constexpr (pt + 1 < NPT) load_s(pt + 1, (pt + 1) & 1);
      else load_av(0, 0);
      bf16x8 sh[2], sl[2];  // this state-row tile of S_prev as hi + lo (or rounded once), from its accumulator
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = S[pt][8 * q + j];
        if (PLAIN) {
#pragma unroll
          for (int j = 0; j < 8; ++j) sh[q][j] = to_bf16(x[j]);
        } else {
          split8_trunc(x, sh[q], sl[q]);
        }
      }
#pragma unroll
      for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          num[jt] = mfma32(sh[q], qo[pt & 1][jt][q], num[jt]);
          if (!PLAIN) num[jt] = mfma32(sl[q], qo[pt & 1][jt][q], num[jt]);
        }
      __builtin_amdgcn_sched_group_barrier(0x100, pt + 1 < NPT ? RD_S : rd_av(0), 0);  // next step's reads
      __builtin_amdgcn_sched_group_barrier(0x008, (PLAIN ? 2 : 4) * NJ, 0);              // this step's MFMAs
    });
    if (DECAY) {
#pragma unroll
      for (int jt = 0; jt < NJ; ++jt) num[jt] *= fN[G::F_THETA + jt * 32];  // gamma^(j+1), j = this lane's token
    }
    static_for<0, 2 * NJ>([&](auto ist) {
      constexpr int st = decltype(ist)::value, it = st >> 1, b = st & 1;
      if constexpr (st + 1 < 2 * NJ) load_av(st + 1, b ^ 1);
#pragma unroll
      for (int jt = it; jt < NJ; ++jt) {
        num[jt] = mfma32(vo[b], ao[b][jt][0], num[jt]);
        num[jt] = mfma32(vo[b], ao[b][jt][1], num[jt]);
      }
      if constexpr (st + 1 < 2 * NJ) {
        __builtin_amdgcn_sched_group_barrier(0x100, rd_av(st + 1), 0);  // next step's reads
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * (NJ - it), 0);  // this step's MFMAs
      }
    });
    // unrolled so the store count per chunk is static: the wait for the prefetched tiles
    // at the next commit then leaves this chunk's output stores in flight
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt) {
      float inv = 1.f;
      if (NORM) {
        // psi(q_j) . Z_prev (the lane halves split the features) and the score row sums
        float qz = 0.f;
        const unsigned char* qr = qZ + jt * 32 * PQ * 2;
        const f32x4* zr = (const f32x4*)(sF + G::F_Z + hh * (D / 2));
#pragma unroll
        for (int e8 = 0; e8 < D / 2; e8 += 8) {
          const bf16x8 qv = *(const bf16x8*)(qr + e8 * 2);
          const f32x4 z0 = zr[e8 / 4], z1 = zr[e8 / 4 + 1];
#pragma unroll
          for (int j = 0; j < 4; ++j) qz += from_bf16(qv[j]) * z0[j] + from_bf16(qv[4 + j]) * z1[j];
        }
        qz += __shfl_xor(qz, 32);
        float r = 0.f;
#pragma unroll
        for (int it = 0; it <= jt; ++it) r += fN[G::F_R + (jt * (jt + 1) / 2 + it) * 32];
        inv = 1.f / (fN[G::F_THETA + jt * 32] * qz + r + p.eps);
      }
      // registers 4 q4 .. 4 q4 + 3 hold columns Ew + 8 q4 + 4 hh + 0..3 of token row j
      const uint32_t row_el = (uint32_t)(jt * 32 + n) * rse + Ew + 4 * hh;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        store_out4<OBF>(ors, row_el + 8 * q4, num[jt][4 * q4] * inv, num[jt][4 * q4 + 1] * inv,
                        num[jt][4 * q4 + 2] * inv, num[jt][4 * q4 + 3] * inv);
    }

    // ---- state update: S <- gamma^L S + K~^T V with K~ = Xi psi(K) as hi + lo (elu+1), or
    // S <- gamma^L S + K^T (Xi V) (identity); Z <- gamma^L Z + sum_i Xi_i psi(k_i)
    if (NORM) reduce_zp<D>(zp, sF + G::F_ZRED);
    if (DECAY && !VDEC) {
      lds_barrier();  // every wave is done with the score tiles (K lo aliases them) and K
#pragma unroll
      for (int i = 0; i < NPC; ++i) {
        const int row = prow + 16 * i, off = i * 16 * D * 2;
        const float xi = row < L ? exp2_hw((float)(L - 1 - row) * lg) : 0.f;
        const bf16x8 h8 = *(const bf16x8*)(kP + off);
        float x[8];
        if (ELU) {
          const bf16x8 l8 = *(const bf16x8*)(kP + off + KLO);
#pragma unroll
          for (int j = 0; j < 8; ++j) x[j] = (from_bf16(h8[j]) + from_bf16(l8[j])) * xi;
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) x[j] = from_bf16(h8[j]) * xi;
        }
        bf16x8 hi, lo;
        split8_trunc(x, hi, lo);
        *(bf16x8*)(kP + off) = hi;
        *(bf16x8*)(kP + off + KLO) = lo;
      }
    }
    // the Z partials (and a rewritten K~) must be complete; K, V and Xi were published before
    // the score tiles, and nothing else changes LDS until the next chunk's commit
    if (NORM || (DECAY && !VDEC)) lds_barrier();
    if (NORM && tid < D) {
      float z = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) z += sF[G::F_ZRED + ww * D + tid];
      sF[G::F_Z + tid] = a * sF[G::F_Z + tid] + z;
    }
    if (DECAY) {
#pragma unroll
      for (int pt = 0; pt < D / 32; ++pt) S[pt] *= a;
    }
    // S[pt] += K~^T V, or K^T (Xi V) (M = state row, N = value column, k = token),
    // software-pipelined: the operands of token step ik + 1 are read while the MFMAs of
    // step ik run. Element j of this lane's V operand at step ik is token 16 ik + 8 hh + j.
    {
      constexpr int NK = C / 16;
      constexpr int KP = (SPLIT && !VDEC) ? 2 : 1;  // key operand parts per state-row tile
      constexpr int NM = KP * (D / 32);
      bf16x8 ops[2][1 + NM];  // [buffer][V, then K (K~ hi and lo) per state-row tile]
      f32x4 xis[2][2];        // VDEC: Xi of this lane's 8 tokens of the step
      const float* const xiR = sF + G::F_XI + 8 * hh;
      auto load_ops = [&](bf16x8 (&o)[1 + NM], f32x4 (&x)[2], int ik) {
        const int r0 = ik * 16, ko = r0 * D * 2;
        o[0] = cat8(lds_read_tr4((const __bf16*)(vT0 + r0 * D * 2)), lds_read_tr4((const __bf16*)(vT1 + r0 * D * 2)));
#pragma unroll
        for (int pt = 0; pt < D / 32; ++pt) {
          o[1 + KP * pt] =
              cat8(lds_read_tr4((const __bf16*)(kT[pt][0] + ko)), lds_read_tr4((const __bf16*)(kT[pt][1] + ko)));
          if (KP == 2)
            o[2 + 2 * pt] = cat8(lds_read_tr4((const __bf16*)(kT[pt][0] + ko + KLO)),
                                 lds_read_tr4((const __bf16*)(kT[pt][1] + ko + KLO)));
        }
        if (VDEC) {
          x[0] = *(const f32x4*)(xiR + r0);
          x[1] = *(const f32x4*)(xiR + r0 + 4);
        }
      };
      load_ops(ops[0], xis[0], 0);
#pragma unroll
      for (int ik = 0; ik < NK; ++ik) {
        if (ik + 1 < NK) load_ops(ops[(ik + 1) & 1], xis[(ik + 1) & 1], ik + 1);
        const bf16x8(&o)[1 + NM] = ops[ik & 1];
        if (VDEC) {
          const f32x4(&x)[2] = xis[ik & 1];
          float vx[8];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            vx[j] = from_bf16(o[0][j]) * x[0][j];
            vx[4 + j] = from_bf16(o[0][4 + j]) * x[1][j];
          }
          bf16x8 vh, vl;
          split8_trunc(vx, vh, vl);
#pragma unroll
          for (int pt = 0; pt < D / 32; ++pt) {
            S[pt] = mfma32(o[1 + pt], vh, S[pt]);
            S[pt] = mfma32(o[1 + pt], vl, S[pt]);
          }
        } else {
#pragma unroll
          for (int pt = 0; pt < D / 32; ++pt) {
            S[pt] = mfma32(o[1 + KP * pt], o[0], S[pt]);
            if (KP == 2) S[pt] = mfma32(o[2 + 2 * pt], o[0], S[pt]);
          }
        }
        if (ik + 1 < NK) {  // keep the next step's reads ahead of this step's MFMAs
          __builtin_amdgcn_sched_group_barrier(0x100, 2 * (1 + NM) + (VDEC ? 2 : 0), 0);  // LDS reads
          __builtin_amdgcn_sched_group_barrier(0x008, VDEC ? 2 * (D / 32) : NM, 0);       // MFMA
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// Output kernel with two waves per SIMD (8 waves per workgroup, d = 128, chunk 64).
//
// The LDS image with elu+1 keys (or a denominator) keeps the CU to one workgroup, so
// occupancy comes from within it. Wave w = (cb, fh), cb = w % 4, fh = w / 4, owns value
// columns [32 cb, 32 cb + 32) and state rows [64 fh, 64 fh + 64): half the state per wave
// pair, so neither the hi + lo split of S nor the state update is done twice. Each half
// computes the inter-chunk part over its state rows for both token tiles; half h then
// finishes token tile h (adds the intra-chunk term V^T A^T and takes the other half's
// partial through LDS), so every wave stores the same rows. psi(q) . Z_prev is formed per
// token while psi(Q) is committed (DPP sums over the 16 threads of a row); Z's per-chunk
// column sums come from MFMAs of an all-ones operand inside the state update.
template <int C, int D, bool ELU>
struct W8Geo {
  using B = ShGeo<C, D, ELU>;
  static constexpr int NWV = 8, NT = 64 * NWV;
  static constexpr int NJ = B::NJ, NTILE = B::NTILE;
  static constexpr int NPH = D / 64;            // state-row tiles per wave (half of D / 32)
  static constexpr int PQ = B::PQ, PV = B::PV, PA = B::PA, A_TILE = B::A_TILE, K_BYTES = B::K_BYTES;
  static constexpr int OFF_Q = B::OFF_Q, OFF_K = B::OFF_K, OFF_A = B::OFF_A, OFF_V = B::OFF_V, OFF_F = B::OFF_F;
  static constexpr int F_Z = 0;                 // Z [D]
  static constexpr int F_THETA = D;             // gamma^(j+1) [C]
  static constexpr int F_R = F_THETA + C;       // per-tile score row sums [NTILE][32]
  static constexpr int F_QZ = F_R + NTILE * 32; // psi(q_j) . Z_prev [C]
  static constexpr int OFF_X = OFF_F + 4 * (F_QZ + C);      // partial outputs [4][NJ][16 / 4][64][4] floats
  static constexpr int LDS_BYTES = OFF_X + 4 * 4 * NJ * 16 * 64;
  static constexpr int PPR = D / 8;             // 16-byte pieces per token row
  static constexpr int RSTEP = NT / PPR;        // rows between a thread's pieces
  static constexpr int NPC = C * PPR / NT;      // pieces per thread per tile
  static_assert(OFF_X % 16 == 0, "16-byte exchange slots");
  // Laid out for C = 64, d = 128 (two token tiles, one per feature half).
  static constexpr bool FITS = B::FITS && LDS_BYTES <= 160 * 1024 && D == 128 && C == 64;
};

template <int NPC>
struct PiecesN {
  uint4 r[NPC];
};

// Rows >= valid read as zeros (bounded buffer resource, no branches); piece i of the thread
// at row prow + RSTEP i, columns pcol .. pcol + 7; token rows rsb bytes apart.
template <int D, int NPC, int RSTEP>
__device__ __forceinline__ void load_pieces_n(PiecesN<NPC>& P, const uint16_t* __restrict__ g, int valid, int prow,
                                              int pcol, uint32_t rsb) {
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(g, rows_extent(valid, rsb, D * 2));
  const uint32_t v0 = (uint32_t)prow * rsb + (uint32_t)pcol * 2;
#pragma unroll
  for (int i = 0; i < NPC; ++i) P.r[i] = buf_load16(rs, v0, (uint32_t)(i * RSTEP) * rsb);
}

template <int C, int D, bool DECAY, bool NORM, bool ELU, bool OBF>
__global__ __launch_bounds__(512) void k_output_w8(PrefillParams p) {
  using G = W8Geo<C, D, ELU>;
  static_assert(G::FITS, "8-wave layout");
  static_assert(G::RSTEP % 16 == 0, "piece rows advance in multiples of 16 (swizzle period)");
  static_assert(G::NJ == 2 && G::PPR == 16, "two token tiles, one DPP row per token row");
  constexpr bool SPLIT = DECAY || ELU;
  // elu+1 features with a denominator and no decay: the state and psi(k) enter the outputs
  // rounded to bf16 once (the features are positive and the outputs are ratios of sums over all
  // of them, so single roundings average out: see the precision readings); the score tiles stay
  // hi + lo. Elsewhere, and in the summary pass that gives the final state, every inexact
  // operand is hi + lo.
  constexpr bool PLAIN = ELU && NORM && !DECAY;
  constexpr int NJ = G::NJ, NPC = G::NPC, RSTEP = G::RSTEP, NPH = G::NPH;
  constexpr int PQ = G::PQ, PA = G::PA;
  constexpr int KLO = G::K_BYTES;
  constexpr int ALO = 32 * PA * 2;
  extern __shared__ __align__(16) unsigned char smem[];
  const int bh = blockIdx.x, seg = blockIdx.y, head = bh % p.H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, n = lane & 31, hh = lane >> 5;
  const int cb = w & 3, fh = w >> 2;
  const int L16 = lane & 15, g = lane >> 4;
  const int Ew = 32 * cb;
  const float lg = DECAY ? p.log2g[head] : 0.f;
  // this wave's state-row tiles: j-th = NPH fh + (j + rot) % NPH; the first one's column sums
  // give Z (waves cb < NPH of each half cover the half)
  const int rot = cb % NPH;
  const bool zw = __builtin_amdgcn_readfirstlane(cb) < NPH;

  const int prow = tid / G::PPR, pcol = (tid % G::PPR) * 8;
  const int trow = 8 * (g >> 1) + (L16 >> 2), tcol = 16 * (g & 1) + 4 * (L16 & 3);
  unsigned char* const qP = smem + pin(G::OFF_Q + (prow * PQ + pcol) * 2);
  const unsigned char* const qC = smem + pin(G::OFF_Q + (n * PQ + 4 * hh) * 2);
  const unsigned char* const qS = smem + pin(G::OFF_Q + (n * PQ + 8 * hh) * 2);
  unsigned char* const kP = smem + pin(G::OFF_K + swz_off<D>(prow, pcol) * 2);
  const unsigned char* kR[D / 16];
  const unsigned char* kT[NPH][2];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) kR[kk] = smem + pin(G::OFF_K + swz_off<D>(n, 16 * kk + 8 * hh) * 2);
#pragma unroll
  for (int j = 0; j < NPH; ++j) {
    const int pt = NPH * fh + (j + rot) % NPH;
    kT[j][0] = smem + pin(G::OFF_K + swz_off<D>(trow, 32 * pt + tcol) * 2);
    kT[j][1] = smem + pin(G::OFF_K + swz_off<D>(trow + 4, 32 * pt + tcol) * 2);
  }
  unsigned char* const vP = smem + pin(G::OFF_V + swz_off<D>(prow, pcol) * 2);
  const unsigned char* const vT0 = smem + pin(G::OFF_V + swz_off<D>(trow, Ew + tcol) * 2);
  const unsigned char* const vT1 = smem + pin(G::OFF_V + swz_off<D>(trow + 4, Ew + tcol) * 2);
  unsigned char* const aW = smem + pin(G::OFF_A + (n * PA + 4 * hh) * 2);
  const unsigned char* const aR = smem + pin(G::OFF_A + (n * PA + 8 * hh) * 2);
  float* const xch = (float*)(smem + pin(G::OFF_X)) + 4 * lane;  // [cb][jt][r / 4][lane][r % 4]
  float* const sF = (float*)(smem + pin(G::OFF_F));
  float* const fN = (float*)(smem + pin(G::OFF_F + 4 * n));

  const size_t E = (size_t)D * D + D;
  f32x16 S[NPH];
  if (p.fold_records) {
    // no scan ran: the state before this segment is the fold of the summary records before it,
    // X_0 (+) X_1 (+) ... in order (each record's decay gamma^len applied to what came before;
    // every one of them is a whole sub-segment), two records' loads in flight at a time
    const float* rec = p.ws + (size_t)bh * p.n_rec * E;
    const int nr = seg * p.rec_per_seg;
    const float a = DECAY ? exp2_hw((float)((p.seg_chunks / p.rec_per_seg) * C) * lg) : 1.f;
    float z = 0.f;
#pragma unroll
    for (int j = 0; j < NPH; ++j) S[j] = f32x16{};
    for (int r0 = 0; r0 < nr; r0 += 2) {
      const bool two = r0 + 1 < nr;
      const float* x0 = rec + (size_t)r0 * E;
      const float* x1 = rec + (size_t)(two ? r0 + 1 : r0) * E;
      f32x16 y0[NPH], y1[NPH];
#pragma unroll
      for (int j = 0; j < NPH; ++j) {
        const int pt = NPH * fh + (j + rot) % NPH;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const size_t o = (size_t)(pt * 32 + dtile_row(r, lane)) * D + Ew + n;
          y0[j][r] = x0[o];
          y1[j][r] = x1[o];
        }
      }
      const float z0 = (NORM && tid < D) ? x0[(size_t)D * D + tid] : 0.f;
      const float z1 = (NORM && tid < D) ? x1[(size_t)D * D + tid] : 0.f;
#pragma unroll
      for (int j = 0; j < NPH; ++j) {
        if (DECAY) S[j] *= a;
        S[j] += y0[j];
        if (two) {
          if (DECAY) S[j] *= a;
          S[j] += y1[j];
        }
      }
      z = a * z + z0;
      if (two) z = a * z + z1;
    }
    if (tid < D) sF[G::F_Z + tid] = NORM ? z : 0.f;
  } else {
    const float* pre = p.ws + rec_index(p, bh, seg) * E;
#pragma unroll
    for (int j = 0; j < NPH; ++j) {
      const int pt = NPH * fh + (j + rot) % NPH;
#pragma unroll
      for (int r = 0; r < 16; ++r) S[j][r] = pre[(size_t)(pt * 32 + dtile_row(r, lane)) * D + Ew + n];
    }
    if (tid < D) sF[G::F_Z + tid] = NORM ? pre[(size_t)D * D + tid] : 0.f;
  }
  for (int j = tid; j < C; j += G::NT) sF[G::F_THETA + j] = DECAY ? exp2_hw((float)(j + 1) * lg) : 1.f;

  const SeqSpan sq = seq_span(p, bh);
  const int T = sq.T, n_chunks = (T + C - 1) / C;
  const uint32_t rse = (uint32_t)p.tok_rows * D, rsb = rse * 2;  // elements / bytes between token rows
  constexpr int OES = OBF ? 2 : 4;  // output element bytes
  const uint16_t* qb = (const uint16_t*)p.q + sq.row0 * D;
  const uint16_t* kb = (const uint16_t*)p.k + sq.row0 * D;
  const uint16_t* vb = (const uint16_t*)p.v + sq.row0 * D;
  unsigned char* ob = (unsigned char*)p.o + sq.row0 * D * OES;
  const int c0 = seg * p.seg_chunks, c1 = min(c0 + p.seg_chunks, n_chunks);
  if (c0 >= c1) return;  // segment past the end of a shorter sequence: nothing to write

  PiecesN<NPC> pq, pk, pv;
  {
    const int L0 = min(C, T - c0 * C);
    load_pieces_n<D, NPC, RSTEP>(pq, qb + (size_t)c0 * C * rse, L0, prow, pcol, rsb);
    load_pieces_n<D, NPC, RSTEP>(pk, kb + (size_t)c0 * C * rse, L0, prow, pcol, rsb);
    load_pieces_n<D, NPC, RSTEP>(pv, vb + (size_t)c0 * C * rse, L0, prow, pcol, rsb);
    vm_drain();
  }
  for (int c = c0; c < c1; ++c) {
    const int t0 = c * C, L = min(C, T - t0);
    const float a = DECAY ? exp2_hw((float)L * lg) : 1.f;
    lds_barrier();  // the previous chunk is done with LDS (and Z is updated)

    // ---- commit (see k_output_sh); with a denominator, psi(q_j) . Z_prev per token row from
    // the rounded features (the 16 threads of a row are one DPP row)
    f32x4 zq[2];
    if (NORM) {
      zq[0] = *(const f32x4*)(sF + G::F_Z + pcol);
      zq[1] = *(const f32x4*)(sF + G::F_Z + pcol + 4);
    }
#pragma unroll
    for (int i = 0; i < NPC; ++i) {
      uint4 raw = pq.r[i];
      if (ELU) {
        const bf16x8 x = __builtin_bit_cast(bf16x8, raw);
        bf16x8 y;
#pragma unroll
        for (int j = 0; j < 8; ++j) y[j] = to_bf16(elu1(from_bf16(x[j])));
        raw = __builtin_bit_cast(uint4, y);
      }
      *(uint4*)(qP + i * RSTEP * PQ * 2) = raw;
      if (NORM) {
        const bf16x8 y = __builtin_bit_cast(bf16x8, raw);
        float qz = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) qz += from_bf16(y[j]) * zq[0][j] + from_bf16(y[4 + j]) * zq[1][j];
        qz = row16_sum(qz);
        if (tid % G::PPR == 0) sF[G::F_QZ + prow + RSTEP * i] = qz;
      }
    }
#pragma unroll
    for (int i = 0; i < NPC; ++i) {
      const int off = i * RSTEP * D * 2;
      if (!ELU) {
        *(uint4*)(kP + off) = pk.r[i];
        continue;
      }
      const int row = prow + RSTEP * i;
      const float live = row < L ? 1.f : 0.f;
      const bf16x8 x = __builtin_bit_cast(bf16x8, pk.r[i]);
      float f[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) f[j] = elu1(from_bf16(x[j])) * live;
      if (PLAIN) {
        bf16x8 y;
#pragma unroll
        for (int j = 0; j < 8; ++j) y[j] = to_bf16(f[j]);
        *(bf16x8*)(kP + off) = y;
        continue;
      }
      bf16x8 hi, lo;
      split8_rne(f, hi, lo);  // hi alone is the score operand
      *(bf16x8*)(kP + off) = hi;
      *(bf16x8*)(kP + off + KLO) = lo;
    }
#pragma unroll
    for (int i = 0; i < NPC; ++i) *(uint4*)(vP + i * RSTEP * D * 2) = pv.r[i];
    const bool more = c + 1 < c1;
    const int Ln = more ? min(C, T - (c + 1) * C) : 0;
    load_pieces_n<D, NPC, RSTEP>(pq, qb + (size_t)(c + 1) * C * rse, Ln, prow, pcol, rsb);
    load_pieces_n<D, NPC, RSTEP>(pk, kb + (size_t)(c + 1) * C * rse, Ln, prow, pcol, rsb);
    load_pieces_n<D, NPC, RSTEP>(pv, vb + (size_t)(c + 1) * C * rse, Ln, prow, pcol, rsb);
    lds_barrier();

    // ---- score tiles (shared): wave t < NTILE computes tile t; decay factors per tile
    if (w < G::NTILE) {
      const int t = w, jt = tile_jt(t), it = t - jt * (jt + 1) / 2;
      bf16x8 ka[D / 16], qv[D / 16];
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        ka[kk] = *(const bf16x8*)(kR[kk] + it * 32 * D * 2);
        qv[kk] = *(const bf16x8*)(qS + (jt * 32 * PQ + kk * 16) * 2);
      }
      f32x16 acc = f32x16{};
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) acc = mfma32(ka[kk], qv[kk], acc);
      const bool diag = it == jt;
      float av[16];
      float rs = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ir = dtile_row(r, lane);
        float f;
        if constexpr (DECAY) f = (diag && ir > n) ? 0.f : exp2_hw((float)(32 * (jt - it) + n - ir) * lg);
        else f = (diag && ir > n) ? 0.f : 1.f;
        av[r] = acc[r] * f;
        if (NORM) rs += av[r];
      }
      if (NORM) {
        rs += __shfl_xor(rs, 32);
        if (hh == 0) fN[G::F_R + t * 32] = rs;
      }
      unsigned char* at = aW + t * G::A_TILE;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        bf16x8 h8, l8;
        split8_trunc(av + 8 * q, h8, l8);
        const u32x4 hv = __builtin_bit_cast(u32x4, h8), lv = __builtin_bit_cast(u32x4, l8);
        *(uint2*)(at + 32 * q) = make_uint2(hv[0], hv[1]);
        *(uint2*)(at + 32 * q + 16) = make_uint2(hv[2], hv[3]);
        *(uint2*)(at + 32 * q + ALO) = make_uint2(lv[0], lv[1]);
        *(uint2*)(at + 32 * q + 16 + ALO) = make_uint2(lv[2], lv[3]);
      }
    }
    lds_barrier();

    // ---- outputs, transposed as in k_output_sh: numT[e][j] (M = value column, N = token).
    // The inter-chunk part over this wave's state rows for both token tiles (S split into
    // hi + lo one tile at a time), theta-weighted; then the intra-chunk term V^T A^T for
    // token tile fh, the tile this half finishes.
    // num[0] accumulates token tile fh (the one this half finishes), num[1] the other half's
    // tile (handed over through LDS): the accumulators are named by role, so no per-register
    // select between the tiles is needed afterwards
    f32x16 num[NJ];
#pragma unroll
    for (int u = 0; u < NJ; ++u) num[u] = f32x16{};
    const int jtu[2] = {fh, 1 - fh};
#pragma unroll
    for (int j = 0; j < NPH; ++j) {
      bf16x8 sh[2], sl[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        float x[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) x[jj] = S[j][8 * q + jj];
        if (PLAIN) {
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) sh[q][jj] = to_bf16(x[jj]);
        } else {
          split8_trunc(x, sh[q], sl[q]);
        }
      }
      const int fcol = (NPH * fh + (j + rot) % NPH) * 32;
#pragma unroll
      for (int u = 0; u < NJ; ++u)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const unsigned char* qa = qC + (jtu[u] * 32 * PQ + fcol + 16 * q) * 2;
          const bf16x8 qo = cat8(*(const bf16x4*)qa, *(const bf16x4*)(qa + 16));
          num[u] = mfma32(sh[q], qo, num[u]);
          if (!PLAIN) num[u] = mfma32(sl[q], qo, num[u]);
        }
    }
    if (DECAY) {
#pragma unroll
      for (int u = 0; u < NJ; ++u) num[u] *= fN[G::F_THETA + jtu[u] * 32];
    }
    f32x16 mine = num[0], give = num[1];
    {
      // the intra-chunk terms, in equal shares: each half adds the diagonal score tile of its
      // own token tile, and one 16-key half (k-half fh) of the off-diagonal tile (queries of
      // token tile 1, keys of token tile 0), half 0 into the partial it hands over
      auto av_step = [&](f32x16& acc, int t, int it, int q) {
        const unsigned char* at = aR + t * G::A_TILE;
        const int r0 = it * 32 + 16 * q;
        const bf16x8 vv = cat8(lds_read_tr4((const __bf16*)(vT0 + r0 * D * 2)),
                               lds_read_tr4((const __bf16*)(vT1 + r0 * D * 2)));
        acc = mfma32(vv, *(const bf16x8*)(at + 32 * q), acc);
        acc = mfma32(vv, *(const bf16x8*)(at + 32 * q + ALO), acc);
      };
      static_assert(NJ == 2, "tiles (0, 0) = 0, (1, 0) = 1, (1, 1) = 2");
      if (__builtin_amdgcn_readfirstlane(fh)) {
        av_step(mine, 2, 1, 0);
        av_step(mine, 2, 1, 1);
        av_step(mine, 1, 0, 1);
      } else {
        av_step(mine, 0, 0, 0);
        av_step(mine, 0, 0, 1);
        av_step(give, 1, 0, 0);
      }
      f32x4* const xo = (f32x4*)(xch + (cb * NJ + (1 - fh)) * 16 * 64);
#pragma unroll
      for (int q = 0; q < 4; ++q) xo[q * 64] = f32x4{give[4 * q], give[4 * q + 1], give[4 * q + 2], give[4 * q + 3]};
    }
    lds_barrier();  // partials published; every wave is done with the score tiles and with K

    // K~ = Xi psi(K) with decay: rescale the hi + lo tile in place (identity keys: K lo
    // aliases the score tiles, dead now)
    if (DECAY) {
#pragma unroll
      for (int i = 0; i < NPC; ++i) {
        const int row = prow + RSTEP * i, off = i * RSTEP * D * 2;
        const float xi = row < L ? exp2_hw((float)(L - 1 - row) * lg) : 0.f;
        const bf16x8 h8 = *(const bf16x8*)(kP + off);
        float x[8];
        if (ELU) {
          const bf16x8 l8 = *(const bf16x8*)(kP + off + KLO);
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) x[jj] = (from_bf16(h8[jj]) + from_bf16(l8[jj])) * xi;
        } else {
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) x[jj] = from_bf16(h8[jj]) * xi;
        }
        bf16x8 hi, lo;
        split8_trunc(x, hi, lo);
        *(bf16x8*)(kP + off) = hi;
        *(bf16x8*)(kP + off + KLO) = lo;
      }
    }
    {
      const int jt = fh;
      const f32x4* const xi4 = (const f32x4*)(xch + (cb * NJ + jt) * 16 * 64);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 o4 = xi4[q * 64];
#pragma unroll
        for (int e = 0; e < 4; ++e) mine[4 * q + e] += o4[e];
      }
      float inv = 1.f;
      if (NORM) {
        float r = fN[G::F_R + (jt * (jt + 1) / 2) * 32];
        if (jt) r += fN[G::F_R + 2 * 32];
        inv = 1.f / (fN[G::F_THETA + jt * 32] * fN[G::F_QZ + jt * 32] + r + p.eps);
      }
      const __amdgpu_buffer_rsrc_t ors = make_rsrc(ob + (size_t)t0 * rse * OES, rows_extent(L, rse * OES, D * OES));
      const uint32_t row_el = (uint32_t)(jt * 32 + n) * rse + Ew + 4 * hh;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        store_out4<OBF>(ors, row_el + 8 * q4, mine[4 * q4] * inv, mine[4 * q4 + 1] * inv, mine[4 * q4 + 2] * inv,
                        mine[4 * q4 + 3] * inv);
    }
    if (DECAY) lds_barrier();  // K~ complete

    // ---- state update: S <- gamma^L S + K~^T V over this wave's state rows, and Z's column
    // sums 1 K~ of its first tile (waves cb < NPH), read again only in the next chunk
    if (DECAY) {
#pragma unroll
      for (int j = 0; j < NPH; ++j) S[j] *= a;
    }
    {
      constexpr int NK = C / 16, KP = (SPLIT && !PLAIN) ? 2 : 1, NM = KP * NPH;
      const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
      f32x16 zc = f32x16{};
      bf16x8 ops[2][1 + NM];
      auto load_ops = [&](bf16x8 (&o)[1 + NM], int ik) {
        const int r0 = ik * 16, ko = r0 * D * 2;
        o[0] = cat8(lds_read_tr4((const __bf16*)(vT0 + r0 * D * 2)), lds_read_tr4((const __bf16*)(vT1 + r0 * D * 2)));
#pragma unroll
        for (int j = 0; j < NPH; ++j) {
          o[1 + KP * j] = cat8(lds_read_tr4((const __bf16*)(kT[j][0] + ko)), lds_read_tr4((const __bf16*)(kT[j][1] + ko)));
          if (KP == 2)
            o[2 + 2 * j] = cat8(lds_read_tr4((const __bf16*)(kT[j][0] + ko + KLO)),
                                lds_read_tr4((const __bf16*)(kT[j][1] + ko + KLO)));
        }
      };
      load_ops(ops[0], 0);
#pragma unroll
      for (int ik = 0; ik < NK; ++ik) {
        if (ik + 1 < NK) load_ops(ops[(ik + 1) & 1], ik + 1);
        const bf16x8(&o)[1 + NM] = ops[ik & 1];
#pragma unroll
        for (int j = 0; j < NPH; ++j) {
          S[j] = mfma32(o[1 + KP * j], o[0], S[j]);
          if (KP == 2) S[j] = mfma32(o[2 + 2 * j], o[0], S[j]);
        }
        if (NORM && zw) {
          zc = mfma32(ones, o[1], zc);
          if (KP == 2) zc = mfma32(ones, o[2], zc);
        }
        if (ik + 1 < NK) {
          __builtin_amdgcn_sched_group_barrier(0x100, 2 * (1 + NM), 0);
          __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
        }
      }
      if (NORM && zw && hh == 0) {
        float* const zf = sF + G::F_Z + (NPH * fh + rot) * 32 + n;
        *zf = a * *zf + zc[0];
      }
    }
  }
}

// The output kernel for (C, D, flags): the two-waves-per-SIMD kernel for elu+1 features or a
// denominator at d = 128, else the shared-score kernel (two workgroups per CU where their LDS
// fits). Measured at C = 64, d = 128 on the output pass: identity features with a denominator
// 0.222 ms (eight waves) against 0.234 ms (shared scores, two workgroups) on 8k x 64 heads;
// retention without one 2.22 ms (shared scores) against 2.94 ms (eight waves) on 128k x 64;
// elu+1 with a denominator, both single-rounding, 0.153 ms (eight waves, 2048-token segments)
// against 0.192 ms (shared scores; 0.154 ms with 1024-token segments, two workgroups per CU).
template <int C, int D, bool DECAY, bool NORM, bool ELU, bool OBF>
const void* output_kernel(int& lds, int& threads) {
  if constexpr (W8Geo<C, D, ELU>::FITS && (ELU || NORM)) {
    lds = W8Geo<C, D, ELU>::LDS_BYTES;
    threads = W8Geo<C, D, ELU>::NT;
    return (const void*)k_output_w8<C, D, DECAY, NORM, ELU, OBF>;
  } else {
    using G = ShGeoF<C, D, DECAY, NORM, ELU>;
    static_assert(G::FITS, "LDS budget of the shared-score output kernel");
    lds = G::LDS_BYTES;
    return (const void*)k_output_sh<C, D, DECAY, NORM, ELU, OBF>;
  }
}

template <int C, int D, bool DECAY, bool NORM, bool ELU>
hipError_t launch_flags(const PrefillParams& p, hipStream_t s, bool out) {
  const void* kern = (const void*)k_summary<C, D, DECAY, NORM, ELU>;
  if constexpr (ELU && NORM && !DECAY)
    if (p.sum_rounded) kern = (const void*)k_summary<C, D, DECAY, NORM, ELU, true>;
  int lds = SumGeo<C, D, DECAY && !ELU>::LDS_BYTES;
  int threads = 2 * D;
  if (out)
    kern = p.out_bf16 ? output_kernel<C, D, DECAY, NORM, ELU, true>(lds, threads)
                      : output_kernel<C, D, DECAY, NORM, ELU, false>(lds, threads);
  hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  // x = (batch, head), y = segment: workgroups are dealt to the 8 XCDs round-robin by linear id
  // x + y * B * H, so every XCD gets a share of the sequences with all their segments. With the
  // segment on x, segment s would always land on the same XCDs: for variable-length batches the
  // heavy first segments would pile onto a few of them.
  dim3 grid(p.B * p.H, p.n_seg);
  void* args[] = {(void*)&p};
  e = hipLaunchKernel(kern, grid, dim3(threads), args, lds, s);
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

}  // namespace la
