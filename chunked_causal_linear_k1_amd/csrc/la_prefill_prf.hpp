// la_prefill_prf.hpp -- chunkwise causal linear attention with positive random features,
// bf16 inputs, fp32 state, MFMA 32x32x16 bf16 -> fp32 on gfx950.
//
// Feature map ("Rethinking Attention with Performers" / the positive-random-feature
// estimator of the softmax kernel, as restated on the linear-attention pages):
//   psi(x)_f = exp(w_f . x - |x|^2 / 2) / sqrt(n_psi),   f = 0 .. n_psi - 1,
// one bank W [n_psi, d] per head. The chunkwise method is the one of the identity / elu+1
// kernels (la_prefill_bf16.hpp): per chunk c with L real tokens
//   A_ji = (psi(q_j) . psi(k_i)) gamma^(j-i) [i <= j],
//   o_j  = (gamma^(j+1) psi(q_j) S_prev + sum_i A_ji v_i) / (gamma^(j+1) psi(q_j) . Z_prev + sum_i A_ji + eps),
//   S_next = gamma^L S_prev + sum_i gamma^(L-1-i) psi(k_i) v_i^T   (Z likewise),
// with an n_psi x d_v state. Here the features are computed on chip from the raw tiles:
// psi^T = W X^T is an MFMA GEMM per chunk (M = feature, N = token, k = input dim), with
// W's operand tiles for the wave's features held in registers for the whole segment.
// Computing it transposed leaves each lane with one token and runs of 4 features, so
// |x|^2, the decay Xi and the padding mask are lane scalars, and the features go to LDS
// as 8-byte runs of a [token][feature] tile.
//
// Precision: psi(K) is kept as hi + lo (two bf16 terms) in the scores and in the state
// update, S as hi + lo in psi(Q) S, the score tiles as hi + lo; psi(Q) is rounded to
// bf16 once and the same rounded values feed numerator and denominator.
//
// Work split: wave w owns value columns [32w, 32w + 32) of S and of the outputs (as in the
// other kernels) and feature tiles [w FPW, (w + 1) FPW) of the feature GEMM, so each
// feature's normaliser total is formed inside one wave (a butterfly over its token lanes).
#pragma once
#include "la_prefill_bf16.hpp"

namespace la {
namespace prf {

template <int C, int D, int NP, bool WITH_Q>
struct Geo {
  static constexpr int NW = D / 32;        // waves
  static constexpr int NT = 64 * NW;       // threads
  static constexpr int NJ = C / 32;        // token tiles per chunk
  static constexpr int NFT = NP / 32;      // feature tiles
  static constexpr int FPW = NFT / NW;     // feature tiles per wave
  static constexpr int PR = D + 8;         // raw q / k tiles (row reads)
  static constexpr int PQ = NP + 8;        // psi(Q) (row reads)
  static constexpr int PV = D + 16;        // V (transpose reads)
  static constexpr int PA = 40;            // score tiles, 32 x 32
  static constexpr int NTILE = NJ * (NJ + 1) / 2;
  static constexpr int A_TILE = 2 * 32 * PA * 2;
  static constexpr int RAW = C * PR * 2;   // one raw tile, bytes
  static constexpr int PSIK = C * NP * 2;  // one part (hi or lo) of psi(K), XOR-swizzled, bytes
  static constexpr int OFF_RQ = 0;
  static constexpr int OFF_RK = WITH_Q ? RAW : 0;
  static constexpr int OFF_A = 0;          // score tiles alias the raw tiles, dead once the features exist
  static constexpr int OFF_PQ = OFF_RK + RAW;
  static constexpr int OFF_PK = OFF_PQ + (WITH_Q ? C * PQ * 2 : 0);
  static constexpr int OFF_V = OFF_PK + 2 * PSIK;
  static constexpr int OFF_F = OFF_V + C * PV * 2;
  static constexpr int F_Z = 0;                   // Z [NP]
  static constexpr int F_THETA = NP;              // gamma^(j+1) [C]
  static constexpr int F_R = F_THETA + C;         // score row sums [NTILE][32]
  static constexpr int F_NQ = F_R + NTILE * 32;   // |q_t|^2 [C]
  static constexpr int F_NK = F_NQ + C;           // |k_t|^2 [C]
  static constexpr int F_QMAX = F_NK + C;         // per-wave max_p w_p . q_t [NW][C] (query shift)
  static constexpr int LDS_BYTES = OFF_F + 4 * (F_QMAX + (WITH_Q ? NW * C : 0));
  static_assert(FPW * NW == NFT, "feature tiles split evenly over the waves");
  static_assert(NTILE <= NW, "one score tile per wave");
  static_assert(!WITH_Q || NTILE * A_TILE <= 2 * RAW, "score tiles fit in the raw-tile region");
  static_assert(PSIK <= 32768 && NP <= 256, "psi(K) lo and every row block within a DS immediate of its base");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

// psi(K) tile layout: row t (token), 16-byte chunks XOR-swizzled by swz<128>(t) (the
// pattern of the key tiles of la_prefill_bf16.hpp, valid for any row width of 16-byte
// chunks since the XOR only touches the low 4 chunk-index bits).
template <int NP>
__device__ __forceinline__ int swzp(int row, int col) {
  return row * NP + ((((col >> 3) ^ swz<128>(row)) << 3) | (col & 7));
}

// Sum of x[0..15] over the 32 token lanes of each lane half: a halving butterfly.
// Returns the total of register r = (n >> 1) & 15 (the same in lanes n and n ^ 1).
__device__ __forceinline__ float lane_total16(const float (&x)[16], int n) {
  float v8[8], v4[4], v2[2];
  const bool b16 = n & 16, b8 = n & 8, b4 = n & 4, b2 = n & 2;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float keep = b16 ? x[k + 8] : x[k], send = b16 ? x[k] : x[k + 8];
    v8[k] = keep + __shfl_xor(send, 16);
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float keep = b8 ? v8[k + 4] : v8[k], send = b8 ? v8[k] : v8[k + 4];
    v4[k] = keep + __shfl_xor(send, 8);
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const float keep = b4 ? v4[k + 2] : v4[k], send = b4 ? v4[k] : v4[k + 2];
    v2[k] = keep + __shfl_xor(send, 4);
  }
  float v = (b2 ? v2[1] : v2[0]) + __shfl_xor(b2 ? v2[0] : v2[1], 2);
  return v + __shfl_xor(v, 1);
}

// Commit the raw pieces of one tile to LDS and record each row's squared norm.
template <int C, int D>
__device__ __forceinline__ void commit_raw_norm(const pf::Pieces<C, D>& P, unsigned char* dst, int pitch_bytes,
                                                float* nrm, int prow, int tid) {
  using PG = pf::Geo<C, D, true>;
#pragma unroll
  for (int i = 0; i < PG::NPC; ++i) {
    *(uint4*)(dst + i * 16 * pitch_bytes) = P.r[i];
    const bf16x8 x = __builtin_bit_cast(bf16x8, P.r[i]);
    float sq = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) sq += from_bf16(x[j]) * from_bf16(x[j]);
#pragma unroll
    for (int off = 1; off < PG::PPR; off <<= 1) sq += __shfl_xor(sq, off);
    if (tid % PG::PPR == 0) nrm[prow + 16 * i] = sq;
  }
}

// psi^T tile (M = feature ft*32 + 0..31, N = token jt*32 + 0..31, k = input dim) from a raw
// tile at `raw` (per-lane base: token n, input dims 8 hh + ...).
template <int D>
__device__ __forceinline__ f32x16 feature_gemm(const bf16x8 (&wop)[D / 16], const unsigned char* raw, int jt,
                                               int pitch_bytes) {
  f32x16 acc = f32x16{};
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
    acc = mfma32(wop[kk], *(const bf16x8*)(raw + jt * 32 * pitch_bytes + kk * 32), acc);
  return acc;
}

// Four bf16 as one 8-byte run.
__device__ __forceinline__ uint2 pack4(float a, float b, float c, float d) {
  const bf16x2 lo = __builtin_convertvector((f32x2){a, b}, bf16x2);
  const bf16x2 hi = __builtin_convertvector((f32x2){c, d}, bf16x2);
  return make_uint2(__builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi));
}

// Write 16 feature values of this lane (token t; register r is feature
// ft*32 + 8 (r/4) + 4 hh + r%4) into the swizzled psi(K) tile as hi (at pk) + lo (at pk + LO).
template <int NP, int LO>
__device__ __forceinline__ void write_psik(unsigned char* pk, int t, int ft, int hh, const float (&v)[16]) {
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    bf16x8 h8, l8;
    split8_trunc(v + 8 * q, h8, l8);
    const u32x4 hv = __builtin_bit_cast(u32x4, h8), lv = __builtin_bit_cast(u32x4, l8);
#pragma unroll
    for (int gg = 0; gg < 2; ++gg) {
      const int off = swzp<NP>(t, ft * 32 + 8 * (2 * q + gg) + 4 * hh) * 2;
      *(uint2*)(pk + off) = make_uint2(hv[2 * gg], hv[2 * gg + 1]);
      *(uint2*)(pk + off + LO) = make_uint2(lv[2 * gg], lv[2 * gg + 1]);
    }
  }
}

// Per-lane byte bases of the hot psi(K) reads (pinned, see pin). Score operand: token
// row n, features 16 kk + 8 hh (kk < 8; kk + 8 lies 256 bytes further, as the swizzle
// leaves chunk-index bit 4 alone). State-update operand (transpose reads): rows trow and
// trow + 4, features 32 pt + tcol (pt < 4; pt + 4 lies 256 bytes further).
template <int NP>
struct PsiKBases {
  const unsigned char* rw[8];
  const unsigned char* tr[4][2];
};
template <int NP>
__device__ __forceinline__ PsiKBases<NP> psik_bases(unsigned char* smem, int off_pk, int n, int hh, int trow,
                                                    int tcol) {
  PsiKBases<NP> b;
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) b.rw[kk] = smem + pin(off_pk + swzp<NP>(n, 16 * kk + 8 * hh) * 2);
#pragma unroll
  for (int pt = 0; pt < 4; ++pt) {
    b.tr[pt][0] = smem + pin(off_pk + swzp<NP>(trow, 32 * pt + tcol) * 2);
    b.tr[pt][1] = smem + pin(off_pk + swzp<NP>(trow + 4, 32 * pt + tcol) * 2);
  }
  return b;
}
template <int NP>
__device__ __forceinline__ bf16x8 psik_row(const PsiKBases<NP>& b, int row0, int kk, int extra) {
  return *(const bf16x8*)(b.rw[kk & 7] + (kk >> 3) * 256 + row0 * NP * 2 + extra);
}
template <int NP>
__device__ __forceinline__ bf16x8 psik_tr(const PsiKBases<NP>& b, int row0, int pt, int extra) {
  const int o = (pt >> 2) * 256 + row0 * NP * 2 + extra;
  return cat8(lds_read_tr4((const __bf16*)(b.tr[pt & 3][0] + o)), lds_read_tr4((const __bf16*)(b.tr[pt & 3][1] + o)));
}

// S[pt] += K~^T V over the chunk (M = feature, N = value column, k = token), software-
// pipelined in steps of (16 tokens, up to 4 feature tiles): the operands of the next step
// are read from LDS while the current step's MFMAs run.
template <int C, int D, int NP, int LO, int PV>
__device__ __forceinline__ void state_update_prf(f32x16 (&S)[NP / 32], const PsiKBases<NP>& kb8,
                                                 const unsigned char* vT) {
  constexpr int NFT = NP / 32, PTS = NFT < 4 ? NFT : 4, HALVES = NFT / PTS, NSTEP = (C / 16) * HALVES;
  bf16x8 ops[2][1 + 2 * PTS];  // [buffer][V, then psi(K) hi, lo per feature tile of the step]
  auto load_step = [&](bf16x8 (&o)[1 + 2 * PTS], int st) {
    const int r0 = (st / HALVES) * 16, p0 = (st % HALVES) * PTS;
    o[0] = cat8(lds_read_tr4((const __bf16*)(vT + r0 * PV * 2)), lds_read_tr4((const __bf16*)(vT + (r0 + 4) * PV * 2)));
#pragma unroll
    for (int j = 0; j < PTS; ++j) {
      o[1 + 2 * j] = psik_tr<NP>(kb8, r0, p0 + j, 0);
      o[2 + 2 * j] = psik_tr<NP>(kb8, r0, p0 + j, LO);
    }
  };
  load_step(ops[0], 0);
#pragma unroll
  for (int st = 0; st < NSTEP; ++st) {
    if (st + 1 < NSTEP) load_step(ops[(st + 1) & 1], st + 1);
    const bf16x8(&o)[1 + 2 * PTS] = ops[st & 1];
    const int p0 = (st % HALVES) * PTS;
#pragma unroll
    for (int j = 0; j < PTS; ++j) {
      S[p0 + j] = mfma32(o[1 + 2 * j], o[0], S[p0 + j]);
      S[p0 + j] = mfma32(o[2 + 2 * j], o[0], S[p0 + j]);
    }
    if (st + 1 < NSTEP) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * (1 + 2 * PTS), 0);  // next step's reads
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * PTS, 0);            // this step's MFMAs
    }
  }
}

// ---------------------------------------------------------------------------------------
// Segment summaries: per (sequence, segment), S = sum over the segment's tokens of
// gamma^(seg_end-1-i) psi(k_i) v_i^T and Z likewise, written to the workspace.
template <int C, int D, int NP, bool DECAY, bool NORM>
__global__ __launch_bounds__(2 * D) void k_summary_prf(PrefillParams p) {
  using G = Geo<C, D, NP, false>;
  using PG = pf::Geo<C, D, true>;
  constexpr int NJ = G::NJ, NFT = G::NFT, FPW = G::FPW, NPC = PG::NPC;
  constexpr int PR = G::PR, PV = G::PV, LO = G::PSIK;
  constexpr float LOG2E = 1.4426950408889634f;
  extern __shared__ __align__(16) unsigned char smem[];
  const int bh = blockIdx.x, seg = blockIdx.y, head = bh % p.H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, n = lane & 31, hh = lane >> 5;
  const int L16 = lane & 15, g = lane >> 4;
  const int Ew = 32 * w;
  const float lg = DECAY ? p.log2g[head] : 0.f;
  const float log2_rsqrt = -0.5f * __log2f((float)NP);  // the 1/sqrt(n_psi) factor, as a log2

  const int prow = tid / PG::PPR, pcol = (tid % PG::PPR) * 8;
  const int trow = 8 * (g >> 1) + (L16 >> 2), tcol = 16 * (g & 1) + 4 * (L16 & 3);
  unsigned char* const rkP = smem + pin(G::OFF_RK + (prow * PR + pcol) * 2);
  const unsigned char* const rR = smem + pin(G::OFF_RK + (n * PR + 8 * hh) * 2);
  unsigned char* const pk = smem + pin(G::OFF_PK);
  unsigned char* const vP = smem + pin(G::OFF_V + (prow * PV + pcol) * 2);
  const unsigned char* const vT = smem + pin(G::OFF_V + (trow * PV + Ew + tcol) * 2);
  float* const sF = (float*)(smem + pin(G::OFF_F));
  const PsiKBases<NP> kb8 = psik_bases<NP>(smem, G::OFF_PK, n, hh, trow, tcol);

  // this wave's rows of W as MFMA operands (M = feature, k = input dim)
  const uint16_t* Wh = (const uint16_t*)p.prf_w + (size_t)head * NP * D;
  bf16x8 wop[FPW][D / 16];
#pragma unroll
  for (int f = 0; f < FPW; ++f)
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
      wop[f][kk] = *(const bf16x8*)(Wh + (size_t)((w * FPW + f) * 32 + n) * D + 16 * kk + 8 * hh);

  f32x16 S[NFT];
#pragma unroll
  for (int pt = 0; pt < NFT; ++pt) S[pt] = f32x16{};
  float zacc[FPW][16];  // per-lane partial normaliser sums (this lane's tokens), decayed to the segment end
#pragma unroll
  for (int f = 0; f < FPW; ++f)
#pragma unroll
    for (int r = 0; r < 16; ++r) zacc[f][r] = 0.f;

  const SeqSpan sq = seq_span(p, bh);
  const int T = sq.T, n_chunks = (T + C - 1) / C;
  const uint32_t rse = (uint32_t)p.tok_rows * D, rsb = rse * 2;  // elements / bytes between token rows
  const uint16_t* kg = (const uint16_t*)p.k + sq.row0 * D;
  const uint16_t* vg = (const uint16_t*)p.v + sq.row0 * D;
  const int c0 = seg * p.seg_chunks, c1 = min(min(c0 + p.seg_chunks, n_chunks), p.sum_end);
  pf::Pieces<C, D> pk_, pv_;
  {
    const int L0 = c0 < c1 ? min(C, T - c0 * C) : 0;
    pf::load_pieces<C, D>(pk_, kg + (size_t)c0 * C * rse, L0, rsb);
    pf::load_pieces<C, D>(pv_, vg + (size_t)c0 * C * rse, L0, rsb);
    vm_drain();
  }
  for (int c = c0; c < c1; ++c) {
    const int L = min(C, T - c * C);
    const float a = DECAY ? exp2f((float)L * lg) : 1.f;
    lds_barrier();  // the previous chunk is done with LDS
    commit_raw_norm<C, D>(pk_, rkP, PR * 2, sF + G::F_NK, prow, tid);
#pragma unroll
    for (int i = 0; i < NPC; ++i) *(uint4*)(vP + i * 16 * PV * 2) = pv_.r[i];
    {
      const bool more = c + 1 < c1;
      const int Ln = more ? min(C, T - (c + 1) * C) : 0;
      pf::load_pieces<C, D>(pk_, kg + (size_t)(c + 1) * C * rse, Ln, rsb);
      pf::load_pieces<C, D>(pv_, vg + (size_t)(c + 1) * C * rse, Ln, rsb);
    }
    lds_barrier();
    // K~_t = Xi_t psi(k_t) for this wave's features; padded tokens give exactly zero
#pragma unroll
    for (int f = 0; f < FPW; ++f)
#pragma unroll
      for (int r = 0; r < 16; ++r) zacc[f][r] *= a;
#pragma unroll
    for (int f = 0; f < FPW; ++f) {
      const int ft = w * FPW + f;
#pragma unroll
      for (int jt = 0; jt < NJ; ++jt) {
        const f32x16 acc = feature_gemm<D>(wop[f], rR, jt, PR * 2);
        const int t = jt * 32 + n;
        // exponent offset: |k|^2/2, the 1/sqrt(n_psi) factor and log2 Xi_t; -inf past the end
        const float h = t < L ? 0.5f * sF[G::F_NK + t] * LOG2E - log2_rsqrt - (DECAY ? (float)(L - 1 - t) * lg : 0.f)
                              : __builtin_huge_valf();
        float v[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          v[r] = exp2f(acc[r] * LOG2E - h);
          zacc[f][r] += v[r];
        }
        write_psik<NP, LO>(pk, t, ft, hh, v);
      }
    }
    lds_barrier();
    if (DECAY) {
#pragma unroll
      for (int pt = 0; pt < NFT; ++pt) S[pt] *= a;
    }
    // S[pt] += K~^T V (M = feature, N = value column, k = token)
    state_update_prf<C, D, NP, LO, PV>(S, kb8, vT);
  }
  // segment summary -> workspace [bh][seg][E], E = NP*D + NP
  const size_t E = (size_t)NP * D + NP;
  float* out = p.ws + rec_index(p, bh, seg) * E;
#pragma unroll
  for (int pt = 0; pt < NFT; ++pt)
#pragma unroll
    for (int r = 0; r < 16; ++r) out[(size_t)(pt * 32 + dtile_row(r, lane)) * D + Ew + n] = S[pt][r];
#pragma unroll
  for (int f = 0; f < FPW; ++f) {
    const float z = lane_total16(zacc[f], n);
    const int r = (n >> 1) & 15;
    if ((n & 1) == 0) out[(size_t)NP * D + (w * FPW + f) * 32 + 8 * (r >> 2) + 4 * hh + (r & 3)] = NORM ? z : 0.f;
  }
}

// ---------------------------------------------------------------------------------------
// Output pass: per (sequence, segment), from the segment's exclusive prefix (written by
// the scan), walk the chunks: features, shared score tiles, outputs, state update.
template <int C, int D, int NP, bool DECAY, bool NORM, bool OBF, bool QS>
__global__ __launch_bounds__(2 * D) void k_output_prf(PrefillParams p) {
  using G = Geo<C, D, NP, true>;
  using PG = pf::Geo<C, D, true>;
  constexpr int NJ = G::NJ, NFT = G::NFT, FPW = G::FPW, NPC = PG::NPC;
  constexpr int PR = G::PR, PQ = G::PQ, PV = G::PV, PA = G::PA;
  constexpr int LO = G::PSIK, ALO = 32 * PA * 2;
  constexpr float LOG2E = 1.4426950408889634f;
  extern __shared__ __align__(16) unsigned char smem[];
  const int bh = blockIdx.x, seg = blockIdx.y, head = bh % p.H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, n = lane & 31, hh = lane >> 5;
  const int L16 = lane & 15, g = lane >> 4;
  const int Ew = 32 * w;
  const float lg = DECAY ? p.log2g[head] : 0.f;
  const float log2_rsqrt = -0.5f * __log2f((float)NP);

  const int prow = tid / PG::PPR, pcol = (tid % PG::PPR) * 8;
  const int trow = 8 * (g >> 1) + (L16 >> 2), tcol = 16 * (g & 1) + 4 * (L16 & 3);
  unsigned char* const rqP = smem + pin(G::OFF_RQ + (prow * PR + pcol) * 2);  // raw K at + RAW
  const unsigned char* const rR = smem + pin(G::OFF_RQ + (n * PR + 8 * hh) * 2);
  unsigned char* const pqW = smem + pin(G::OFF_PQ + (n * PQ + 4 * hh) * 2);  // psi(Q) writes / numT operand
  const unsigned char* const pqS = smem + pin(G::OFF_PQ + (n * PQ + 8 * hh) * 2);  // score operand
  const unsigned char* const pqZ = smem + pin(G::OFF_PQ + (n * PQ + hh * (NP / 2)) * 2);  // psi(q) . Z
  unsigned char* const pk = smem + pin(G::OFF_PK);
  unsigned char* const vP = smem + pin(G::OFF_V + (prow * PV + pcol) * 2);
  const unsigned char* const vT = smem + pin(G::OFF_V + (trow * PV + Ew + tcol) * 2);
  unsigned char* const aW = smem + pin(G::OFF_A + (n * PA + 4 * hh) * 2);
  const unsigned char* const aR = smem + pin(G::OFF_A + (n * PA + 8 * hh) * 2);
  float* const sF = (float*)(smem + pin(G::OFF_F));
  float* const fN = (float*)(smem + pin(G::OFF_F + 4 * n));
  const PsiKBases<NP> kb8 = psik_bases<NP>(smem, G::OFF_PK, n, hh, trow, tcol);

  const uint16_t* Wh = (const uint16_t*)p.prf_w + (size_t)head * NP * D;
  bf16x8 wop[FPW][D / 16];
#pragma unroll
  for (int f = 0; f < FPW; ++f)
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
      wop[f][kk] = *(const bf16x8*)(Wh + (size_t)((w * FPW + f) * 32 + n) * D + 16 * kk + 8 * hh);

  // exclusive prefix state of this segment
  const size_t E = (size_t)NP * D + NP;
  const float* pre = p.ws + rec_index(p, bh, seg) * E;
  f32x16 S[NFT];
#pragma unroll
  for (int pt = 0; pt < NFT; ++pt)
#pragma unroll
    for (int r = 0; r < 16; ++r) S[pt][r] = pre[(size_t)(pt * 32 + dtile_row(r, lane)) * D + Ew + n];
  for (int j = tid; j < NP; j += G::NT) sF[G::F_Z + j] = NORM ? pre[(size_t)NP * D + j] : 0.f;
  for (int j = tid; j < C; j += G::NT) sF[G::F_THETA + j] = DECAY ? exp2f((float)(j + 1) * lg) : 1.f;

  // score-tile factors of this lane with decay (see k_output_sh); without decay only the
  // causal mask of the diagonal tile, applied in place
  float fdiag[DECAY ? 16 : 1], foff[DECAY ? 16 : 1];
  if (DECAY) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int ir = dtile_row(r, lane);
      fdiag[r] = ir <= n ? exp2f((float)(n - ir) * lg) : 0.f;
      foff[r] = exp2f((float)(n + 32 - ir) * lg);
    }
  }

  const SeqSpan sq = seq_span(p, bh);
  const int T = sq.T, n_chunks = (T + C - 1) / C;
  const uint32_t rse = (uint32_t)p.tok_rows * D, rsb = rse * 2;  // elements / bytes between token rows
  constexpr int OES = OBF ? 2 : 4;  // output element bytes
  const uint16_t* qg = (const uint16_t*)p.q + sq.row0 * D;
  const uint16_t* kg = (const uint16_t*)p.k + sq.row0 * D;
  const uint16_t* vg = (const uint16_t*)p.v + sq.row0 * D;
  unsigned char* ob = (unsigned char*)p.o + sq.row0 * D * OES;
  const int c0 = seg * p.seg_chunks, c1 = min(c0 + p.seg_chunks, n_chunks);
  if (c0 >= c1) return;  // segment past the end of a shorter sequence: nothing to write
  pf::Pieces<C, D> pq_, pk_, pv_;
  {
    const int L0 = min(C, T - c0 * C);
    pf::load_pieces<C, D>(pq_, qg + (size_t)c0 * C * rse, L0, rsb);
    pf::load_pieces<C, D>(pk_, kg + (size_t)c0 * C * rse, L0, rsb);
    pf::load_pieces<C, D>(pv_, vg + (size_t)c0 * C * rse, L0, rsb);
    vm_drain();
  }
  for (int c = c0; c < c1; ++c) {
    const int t0 = c * C, L = min(C, T - t0);
    const float a = DECAY ? exp2f((float)L * lg) : 1.f;
    lds_barrier();  // the previous chunk is done with LDS (and Z is updated)
    commit_raw_norm<C, D>(pq_, rqP, PR * 2, sF + G::F_NQ, prow, tid);
    commit_raw_norm<C, D>(pk_, rqP + G::RAW, PR * 2, sF + G::F_NK, prow, tid);
#pragma unroll
    for (int i = 0; i < NPC; ++i) *(uint4*)(vP + i * 16 * PV * 2) = pv_.r[i];
    {
      const bool more = c + 1 < c1;
      const int Ln = more ? min(C, T - (c + 1) * C) : 0;
      pf::load_pieces<C, D>(pq_, qg + (size_t)(c + 1) * C * rse, Ln, rsb);
      pf::load_pieces<C, D>(pk_, kg + (size_t)(c + 1) * C * rse, Ln, rsb);
      pf::load_pieces<C, D>(pv_, vg + (size_t)(c + 1) * C * rse, Ln, rsb);
    }
    lds_barrier();

    // ---- QS: the query-row shift. l_p = w_p . q - |q|^2/2 and its maximum differ by the
    // same |q|^2/2, so the shifted feature is exp(w_p . q - max_r w_r . q) / sqrt(m). Each
    // wave takes the maximum over its features (the GEMM is recomputed below), the waves'
    // maxima meet in LDS.
    if (QS) {
#pragma unroll
      for (int jt = 0; jt < NJ; ++jt) {
        float mx = -__builtin_huge_valf();
#pragma unroll
        for (int f = 0; f < FPW; ++f) {
          const f32x16 acc = feature_gemm<D>(wop[f], rR, jt, PR * 2);
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc[r]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32));  // the other half of the lane pair holds the other rows
        if (hh == 0) sF[G::F_QMAX + w * C + jt * 32 + n] = mx;
      }
      lds_barrier();
    }

    // ---- features of this wave's feature tiles: psi(Q) rounded to bf16; psi(K) as hi + lo
    // (zero past the sequence end); zt = sum_i Xi_i psi(k_i) for the feature of register
    // (n >> 1) & 15 (see lane_total16)
    float zt[FPW];
#pragma unroll
    for (int f = 0; f < FPW; ++f) {
      const int ft = w * FPW + f;
      zt[f] = 0.f;
#pragma unroll
      for (int jt = 0; jt < NJ; ++jt) {
        const int t = jt * 32 + n;
        {
          const f32x16 acc = feature_gemm<D>(wop[f], rR, jt, PR * 2);
          float qshift = 0.5f * sF[G::F_NQ + t];  // |q|^2 / 2, or the row's largest w_p . q (QS)
          if (QS) {
            qshift = sF[G::F_QMAX + t];
#pragma unroll
            for (int ww = 1; ww < G::NW; ++ww) qshift = fmaxf(qshift, sF[G::F_QMAX + ww * C + t]);
          }
          const float h = qshift * LOG2E - log2_rsqrt;
          float v[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) v[r] = exp2f(acc[r] * LOG2E - h);
#pragma unroll
          for (int gq = 0; gq < 4; ++gq)
            *(uint2*)(pqW + (jt * 32 * PQ + ft * 32 + 8 * gq) * 2) =
                pack4(v[4 * gq], v[4 * gq + 1], v[4 * gq + 2], v[4 * gq + 3]);
        }
        {
          const f32x16 acc = feature_gemm<D>(wop[f], rR + G::RAW, jt, PR * 2);
          const bool live = t < L;
          const float h = live ? 0.5f * sF[G::F_NK + t] * LOG2E - log2_rsqrt : __builtin_huge_valf();
          const float xi = (DECAY && live) ? exp2f((float)(L - 1 - t) * lg) : 1.f;
          float v[16], vz[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            v[r] = exp2f(acc[r] * LOG2E - h);
            vz[r] = DECAY ? v[r] * xi : v[r];
          }
          if (NORM) zt[f] += lane_total16(vz, n);
          write_psik<NP, LO>(pk, t, ft, hh, v);
        }
      }
    }
    lds_barrier();  // features complete; the raw tiles are dead (the score tiles alias them)

    // ---- score tile w (M = i, N = j, k = feature), masked, decayed, split into hi + lo
    if (w < G::NTILE) {
      const int t = w, jt = pf::tile_jt(t), it = t - jt * (jt + 1) / 2;
      f32x16 acc = f32x16{};
#pragma unroll
      for (int kk = 0; kk < NP / 16; ++kk) {
        const bf16x8 qv = *(const bf16x8*)(pqS + (jt * 32 * PQ + kk * 16) * 2);
        acc = mfma32(psik_row<NP>(kb8, it * 32, kk, 0), qv, acc);
        acc = mfma32(psik_row<NP>(kb8, it * 32, kk, LO), qv, acc);
      }
      const bool diag = it == jt;
      const float tf = (DECAY && !diag) ? exp2f((float)(32 * (jt - it - 1)) * lg) : 1.f;
      float av[16];
      float rs = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if constexpr (DECAY) av[r] = acc[r] * ((diag ? fdiag[r] : foff[r]) * tf);
        else av[r] = (diag && dtile_row(r, lane) > n) ? 0.f : acc[r];
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

    // ---- outputs, transposed as in k_output_sh: numT[e][j] (M = value column, N = token)
    const __amdgpu_buffer_rsrc_t ors = make_rsrc(ob + (size_t)t0 * rse * OES, rows_extent(L, rse * OES, D * OES));
    f32x16 num[NJ];
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt) num[jt] = f32x16{};
#pragma unroll
    for (int pt = 0; pt < NFT; ++pt) {
      bf16x8 sh[2], sl[2];  // S_prev[pt] as hi + lo, k in the D-tile feedback order
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = S[pt][8 * q + j];
        split8_trunc(x, sh[q], sl[q]);
      }
#pragma unroll
      for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const unsigned char* qa = pqW + (jt * 32 * PQ + pt * 32 + 16 * q) * 2;
          const bf16x8 qo = cat8(*(const bf16x4*)qa, *(const bf16x4*)(qa + 16));
          num[jt] = mfma32(sh[q], qo, num[jt]);
          num[jt] = mfma32(sl[q], qo, num[jt]);
        }
    }
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt) {
      if (DECAY) num[jt] *= fN[G::F_THETA + jt * 32];
#pragma unroll
      for (int it = 0; it <= jt; ++it) {
        const unsigned char* at = aR + (jt * (jt + 1) / 2 + it) * G::A_TILE;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int r0 = it * 32 + 16 * q;
          const bf16x8 vv = cat8(lds_read_tr4((const __bf16*)(vT + r0 * PV * 2)),
                                 lds_read_tr4((const __bf16*)(vT + (r0 + 4) * PV * 2)));
          num[jt] = mfma32(vv, *(const bf16x8*)(at + 32 * q), num[jt]);
          num[jt] = mfma32(vv, *(const bf16x8*)(at + 32 * q + ALO), num[jt]);
        }
      }
      float inv = 1.f;
      if (NORM) {
        float qz = 0.f;
        const unsigned char* qr = pqZ + jt * 32 * PQ * 2;
        const f32x4* zr = (const f32x4*)(sF + G::F_Z + hh * (NP / 2));
#pragma unroll
        for (int e8 = 0; e8 < NP / 2; e8 += 8) {
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
      const uint32_t row_el = (uint32_t)(jt * 32 + n) * rse + Ew + 4 * hh;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        store_out4<OBF>(ors, row_el + 8 * q4, num[jt][4 * q4] * inv, num[jt][4 * q4 + 1] * inv,
                        num[jt][4 * q4 + 2] * inv, num[jt][4 * q4 + 3] * inv);
    }

    // ---- state update: S <- gamma^L S + K~^T V, Z <- gamma^L Z + sum_i Xi_i psi(k_i)
    if (DECAY) {
      lds_barrier();  // every wave is done with the score tiles and psi(K)
      // K~ = Xi psi(K): rescale the hi + lo tile in place, rows past L stay zero
      constexpr int NCH = C * NP / 8;  // 8-element chunks of the tile
#pragma unroll
      for (int i = 0; i < NCH / G::NT; ++i) {
        const int ch = tid + i * G::NT, row = ch / (NP / 8), col = (ch % (NP / 8)) * 8;
        const float xi = row < L ? exp2f((float)(L - 1 - row) * lg) : 0.f;
        const int off = swzp<NP>(row, col) * 2;
        const bf16x8 h8 = *(const bf16x8*)(pk + off), l8 = *(const bf16x8*)(pk + off + LO);
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = (from_bf16(h8[j]) + from_bf16(l8[j])) * xi;
        bf16x8 hi, lo;
        split8_trunc(x, hi, lo);
        *(bf16x8*)(pk + off) = hi;
        *(bf16x8*)(pk + off + LO) = lo;
      }
    }
    lds_barrier();  // every wave is done reading Z_prev and psi(Q)
    if (NORM && (n & 1) == 0) {
      const int r = (n >> 1) & 15;
#pragma unroll
      for (int f = 0; f < FPW; ++f) {
        const int fi = (w * FPW + f) * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
        sF[G::F_Z + fi] = a * sF[G::F_Z + fi] + zt[f];
      }
    }
    if (DECAY) {
#pragma unroll
      for (int pt = 0; pt < NFT; ++pt) S[pt] *= a;
    }
    state_update_prf<C, D, NP, LO, PV>(S, kb8, vT);
  }
}

template <int C, int D, int NP, bool DECAY, bool NORM>
hipError_t launch_flags(const PrefillParams& p, hipStream_t s, bool out) {
  const bool qs = p.psi == LA_PSI_PRF_QSHIFT;
  const void* kern = !out ? (const void*)k_summary_prf<C, D, NP, DECAY, NORM>
                     : p.out_bf16 ? (qs ? (const void*)k_output_prf<C, D, NP, DECAY, NORM, true, true>
                                        : (const void*)k_output_prf<C, D, NP, DECAY, NORM, true, false>)
                                  : (qs ? (const void*)k_output_prf<C, D, NP, DECAY, NORM, false, true>
                                        : (const void*)k_output_prf<C, D, NP, DECAY, NORM, false, false>);
  const int lds = out ? Geo<C, D, NP, true>::LDS_BYTES : Geo<C, D, NP, false>::LDS_BYTES;
  hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  // x = (batch, head), y = segment: workgroups are dealt to the 8 XCDs round-robin by linear id
  // x + y * B * H, so every XCD gets a share of the sequences with all their segments. With the
  // segment on x, segment s would always land on the same XCDs: for variable-length batches the
  // heavy first segments would pile onto a few of them.
  dim3 grid(p.B * p.H, p.n_seg);
  void* args[] = {(void*)&p};
  e = hipLaunchKernel(kern, grid, dim3(2 * D), args, lds, s);
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

template <int C, int D, int NP>
hipError_t launch_np(const PrefillParams& p, hipStream_t s, bool out) {
  const bool decay = p.has_decay != 0, norm = p.normalize != 0;
  if (decay) return norm ? launch_flags<C, D, NP, true, true>(p, s, out) : launch_flags<C, D, NP, true, false>(p, s, out);
  return norm ? launch_flags<C, D, NP, false, true>(p, s, out) : launch_flags<C, D, NP, false, false>(p, s, out);
}

}  // namespace prf
}  // namespace la
