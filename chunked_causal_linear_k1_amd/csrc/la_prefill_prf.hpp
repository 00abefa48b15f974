// la_prefill_prf.hpp -- chunkwise causal linear attention with positive random features,
// bf16 inputs, fp32 state, MFMA 32x32x16 bf16 -> fp32 on gfx950.
//
// Feature map ("Linearized 2-Simplicial Attention", section 3.2, positive random features
// for one tensor mode; appendix B.2 for the log-space query shift):
//   psi(x)_f = exp(w_f . x - |x|^2 / 2) / sqrt(n_psi),   f = 0 .. n_psi - 1,
// one bank W [n_psi, d] per head. The chunkwise method is the one of the identity / elu+1
// kernels (la_prefill_bf16.hpp): per chunk c with L real tokens
//   A_ji = (psi(q_j) . psi(k_i)) gamma^(j-i) [i <= j],
//   o_j  = (gamma^(j+1) psi(q_j) S_prev + sum_i A_ji v_i) / (gamma^(j+1) psi(q_j) . Z_prev + sum_i A_ji + eps),
//   S_next = gamma^L S_prev + sum_i gamma^(L-1-i) psi(k_i) v_i^T   (Z likewise),
// with an n_psi x d_v state. The features are computed on chip from the raw tiles:
// psi^T = W X^T is an MFMA GEMM per chunk (M = feature, N = token, k = input dim).
// Computing it transposed leaves each lane with one token and runs of 4 features, so
// |x|^2, the decay Xi and the padding mask are lane scalars, and the features go to LDS
// as 8-byte runs of a [token][feature] tile. The exponentials are the bare hardware 2^x:
// features below the smallest normal float become zero.
//
// Precision: psi(K) is kept as hi + lo (two bf16 terms) in the scores and in the state
// update, S as hi + lo in psi(Q) S, the score tiles as hi + lo; psi(Q) is rounded to
// bf16 once and the same rounded values feed numerator and denominator.
//
// Work split (eight waves, two per SIMD): wave w = (cb, fh) with cb = w % 4, fh = w / 4
// owns value columns [32 cb, 32 cb + 32) and feature half fh of the fp32 state; the feature
// GEMMs are (feature tile, token tile) jobs dealt over the waves; three waves compute the
// three score tiles; the two halves' partial outputs meet through LDS, each half finishing
// one token tile. Z comes from MFMA column sums inside the state update.
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

// Per-lane byte bases of the score operand reads of psi(K) (pinned, see pin): token row n,
// features 16 kk + 8 hh (kk < 8; kk + 8 lies 256 bytes further, as the swizzle leaves
// chunk-index bit 4 alone).
template <int NP>
struct PsiKBases {
  const unsigned char* rw[8];
};
template <int NP>
__device__ __forceinline__ PsiKBases<NP> psik_bases(unsigned char* smem, int off_pk, int n, int hh) {
  PsiKBases<NP> b;
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) b.rw[kk] = smem + pin(off_pk + swzp<NP>(n, 16 * kk + 8 * hh) * 2);
  return b;
}
template <int NP>
__device__ __forceinline__ bf16x8 psik_row(const PsiKBases<NP>& b, int row0, int kk, int extra) {
  return *(const bf16x8*)(b.rw[kk & 7] + (kk >> 3) * 256 + row0 * NP * 2 + extra);
}

// ---------------------------------------------------------------------------------------
// Eight waves, two per SIMD. Wave w = (cb, fh), cb = w % 4, fh = w / 4: value columns
// [32 cb, 32 cb + 32) of the state and of the outputs, and state rows (features) of half fh,
// [fh NP/2, (fh + 1) NP/2). Each wave therefore carries a quarter of the fp32 state's columns
// for half its rows (64 registers at n_psi = 256), the state update is not duplicated, and the
// two halves' partial outputs meet through LDS. The feature GEMMs are split into (feature
// tile, token tile) jobs over the waves.
template <int C, int D, int NP>
struct Geo8 {
  using B = Geo<C, D, NP, true>;
  static constexpr int NWV = 8, NT = 64 * NWV;
  static constexpr int NJ = B::NJ, NFT = B::NFT, NFH = NFT / 2, NTILE = B::NTILE;
  static constexpr int JPW = NFT * NJ / NWV;       // feature jobs per wave
  static constexpr int PPR = D / 8, RSTEP = NT / PPR, NPC = C * PPR / NT;
  static constexpr int OFF_RQ = B::OFF_RQ, OFF_RK = B::OFF_RK, OFF_A = B::OFF_A, OFF_PQ = B::OFF_PQ,
                       OFF_PK = B::OFF_PK, OFF_V = B::OFF_V, OFF_F = B::OFF_F;
  static constexpr int OFF_X = 0;  // half 1's partial outputs: the raw / score / psi(Q) region, dead by then
  static constexpr int F_Z = 0;                    // Z [NP]
  static constexpr int F_THETA = NP;               // gamma^(j+1) [C]
  static constexpr int F_R = F_THETA + C;          // score row sums [NTILE][32]
  static constexpr int F_NQ = F_R + NTILE * 32;    // |q_t|^2 [C]
  static constexpr int F_NK = F_NQ + C;            // |k_t|^2 [C]
  static constexpr int F_QZ = F_NK + C;            // psi(q_t) . Z_prev per feature tile [NFT][C]
  static constexpr int F_QMAX = F_QZ + NFT * C;    // max_p w_p . q_t per feature tile [NFT][C] (query shift)
  static constexpr int LDS_BYTES = OFF_F + 4 * (F_QMAX + NFT * C);
  static constexpr int SUM_LDS_BYTES = Geo<C, D, NP, false>::OFF_F + 4 * F_QMAX;  // no Q tiles, no QMAX
  static_assert(JPW * NWV == NFT * NJ && JPW >= 1 && NJ % JPW == 0,
                "feature jobs split evenly over the waves, one feature tile per wave");
  static_assert(NTILE <= NWV && NPC * NT == C * PPR, "tiling");
  static_assert(4 * (NWV / 2) * NJ * 16 * 64 <= OFF_PK, "partial outputs fit in front of psi(K)");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

// Feature job jb of a wave: feature tile jb / NJ, token tile jb % NJ (with two jobs per wave
// both token tiles of one feature tile, so its W operands serve both).
template <int NJ>
__device__ __forceinline__ int job_ft(int jb) { return jb / NJ; }
template <int NJ>
__device__ __forceinline__ int job_jt8(int jb) { return jb % NJ; }

// The raw pieces of one tile (rows prow + RSTEP i) to LDS with each row's squared norm.
template <int D, int NPC, int RSTEP>
__device__ __forceinline__ void commit_raw_norm8(const pf::PiecesN<NPC>& P, unsigned char* dst, int pitch_bytes,
                                                 float* nrm, int prow, int tid) {
  constexpr int PPR = D / 8;
#pragma unroll
  for (int i = 0; i < NPC; ++i) {
    *(uint4*)(dst + i * RSTEP * pitch_bytes) = P.r[i];
    if (nrm) {
      const bf16x8 x = __builtin_bit_cast(bf16x8, P.r[i]);
      float sq = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) sq += from_bf16(x[j]) * from_bf16(x[j]);
      static_assert(PPR == 16, "one token row per DPP row");
      sq = row16_sum(sq);
      if (tid % PPR == 0) nrm[prow + RSTEP * i] = sq;
    }
  }
}

// Per-lane bases of the state-update operand reads (transpose reads of psi(K): M = feature,
// k = token) for the NFH feature tiles of one wave, its j-th tile being f0 + (j + rot) % NFH:
// rows trow and trow + 4, features 32 tile + tcol. The rotation puts a different tile first
// in each wave of a half, so that the first tile's column sums are spread over the waves.
template <int NFH>
struct StBases {
  const unsigned char* tr[NFH][2];
};
template <int NP, int NFH>
__device__ __forceinline__ StBases<NFH> st_bases(unsigned char* smem, int off_pk, int trow, int tcol, int f0, int rot) {
  StBases<NFH> b;
#pragma unroll
  for (int j = 0; j < NFH; ++j) {
    const int pt = f0 + (j + rot) % NFH;
    b.tr[j][0] = smem + pin(off_pk + swzp<NP>(trow, 32 * pt + tcol) * 2);
    b.tr[j][1] = smem + pin(off_pk + swzp<NP>(trow + 4, 32 * pt + tcol) * 2);
  }
  return b;
}

// S[j] += K~^T V over the chunk for the wave's feature tiles (see StBases), value columns at
// vT (M = feature, N = value column, k = token), software-pipelined in 16-token steps.
// With WZ, also z += 1 K~ for the first tile: an MFMA of an all-ones operand (M) with that
// tile as the N operand, so every row of z holds the tile's column sums sum_i K~_i (lane n:
// feature n of the tile).
template <int C, int NP, int NFH, int LO, int PV, bool WZ>
__device__ __forceinline__ void state_update_half(f32x16 (&S)[NFH], f32x16& z, const StBases<NFH>& sb,
                                                  const unsigned char* vT) {
  constexpr int NK = C / 16;
  bf16x8 ops[2][1 + 2 * NFH];
  auto load_step = [&](bf16x8 (&o)[1 + 2 * NFH], int ik) {
    const int r0 = ik * 16;
    o[0] = cat8(lds_read_tr4((const __bf16*)(vT + r0 * PV * 2)), lds_read_tr4((const __bf16*)(vT + (r0 + 4) * PV * 2)));
#pragma unroll
    for (int j = 0; j < NFH; ++j) {
      const int o0 = r0 * NP * 2;
      o[1 + 2 * j] = cat8(lds_read_tr4((const __bf16*)(sb.tr[j][0] + o0)), lds_read_tr4((const __bf16*)(sb.tr[j][1] + o0)));
      o[2 + 2 * j] =
          cat8(lds_read_tr4((const __bf16*)(sb.tr[j][0] + o0 + LO)), lds_read_tr4((const __bf16*)(sb.tr[j][1] + o0 + LO)));
    }
  };
  const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
  load_step(ops[0], 0);
#pragma unroll
  for (int ik = 0; ik < NK; ++ik) {
    if (ik + 1 < NK) load_step(ops[(ik + 1) & 1], ik + 1);
    const bf16x8(&o)[1 + 2 * NFH] = ops[ik & 1];
#pragma unroll
    for (int j = 0; j < NFH; ++j) {
      S[j] = mfma32(o[1 + 2 * j], o[0], S[j]);
      S[j] = mfma32(o[2 + 2 * j], o[0], S[j]);
    }
    if (WZ) {
      z = mfma32(ones, o[1], z);
      z = mfma32(ones, o[2], z);
    }
    if (ik + 1 < NK) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * (1 + 2 * NFH), 0);     // next step's reads
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * NFH + (WZ ? 2 : 0), 0);  // this step's MFMAs
    }
  }
}

// ---------------------------------------------------------------------------------------
// Segment summaries: per (sequence, segment), S = sum over the segment's tokens of
// gamma^(seg_end-1-i) psi(k_i) v_i^T and Z likewise, written to the workspace.
template <int C, int D, int NP, bool DECAY, bool NORM>
__global__ __launch_bounds__(512) void k_summary_prf(PrefillParams p) {
  using G8 = Geo8<C, D, NP>;
  using G = Geo<C, D, NP, false>;
  constexpr int NJ = G8::NJ, NFH = G8::NFH, JPW = G8::JPW, NPC = G8::NPC, RSTEP = G8::RSTEP;
  constexpr int PR = G::PR, PV = G::PV, LO = G::PSIK;
  constexpr float LOG2E = 1.4426950408889634f;
  extern __shared__ __align__(16) unsigned char smem[];
  const int bh = blockIdx.x, seg = blockIdx.y, head = bh % p.H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, n = lane & 31, hh = lane >> 5;
  const int L16 = lane & 15, g = lane >> 4;
  const int cb = w & 3, fh = w >> 2, Ew = 32 * cb;
  const float lg = DECAY ? p.log2g[head] : 0.f;
  const float log2_rsqrt = -0.5f * __log2f((float)NP);  // the 1/sqrt(n_psi) factor, as a log2

  const int prow = tid / G8::PPR, pcol = (tid % G8::PPR) * 8;
  const int trow = 8 * (g >> 1) + (L16 >> 2), tcol = 16 * (g & 1) + 4 * (L16 & 3);
  unsigned char* const rkP = smem + pin(G::OFF_RK + (prow * PR + pcol) * 2);
  const unsigned char* const rR = smem + pin(G::OFF_RK + (n * PR + 8 * hh) * 2);
  unsigned char* const pk = smem + pin(G::OFF_PK);
  unsigned char* const vP = smem + pin(G::OFF_V + (prow * PV + pcol) * 2);
  const unsigned char* const vT = smem + pin(G::OFF_V + (trow * PV + Ew + tcol) * 2);
  float* const sF = (float*)(smem + pin(G::OFF_F));
  const int rot = cb % NFH;  // this wave's first feature tile is fh NFH + rot (its column sums give Z)
  const StBases<NFH> sb = st_bases<NP, NFH>(smem, G::OFF_PK, trow, tcol, fh * NFH, rot);

  // W rows of this wave's feature tile as MFMA operands (M = feature, k = input dim)
  const uint16_t* Wh = (const uint16_t*)p.prf_w + (size_t)head * NP * D;
  const int ft0 = job_ft<NJ>(w * JPW);
  bf16x8 wop[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) wop[kk] = *(const bf16x8*)(Wh + (size_t)(ft0 * 32 + n) * D + 16 * kk + 8 * hh);

  f32x16 S[NFH];  // S[j]: feature tile fh NFH + (j + rot) % NFH, value columns Ew ..
#pragma unroll
  for (int pt = 0; pt < NFH; ++pt) S[pt] = f32x16{};
  f32x16 Zs = f32x16{};  // column sums of the first tile, decayed to the segment end (every row alike)

  const SeqSpan sq = seq_span(p, bh);
  const int T = sq.T, n_chunks = (T + C - 1) / C;
  const uint32_t rse = (uint32_t)p.tok_rows * D, rsb = rse * 2;  // elements / bytes between token rows
  const uint16_t* kg = (const uint16_t*)p.k + sq.row0 * D;
  const uint16_t* vg = (const uint16_t*)p.v + sq.row0 * D;
  const int c0 = seg * p.seg_chunks, c1 = min(min(c0 + p.seg_chunks, n_chunks), p.sum_end);
  pf::PiecesN<NPC> pk_, pv_;
  {
    const int L0 = c0 < c1 ? min(C, T - c0 * C) : 0;
    pf::load_pieces_n<D, NPC, RSTEP>(pk_, kg + (size_t)c0 * C * rse, L0, prow, pcol, rsb);
    pf::load_pieces_n<D, NPC, RSTEP>(pv_, vg + (size_t)c0 * C * rse, L0, prow, pcol, rsb);
    vm_drain();
  }
  for (int c = c0; c < c1; ++c) {
    const int L = min(C, T - c * C);
    const float a = DECAY ? exp2_hw((float)L * lg) : 1.f;
    lds_barrier();  // the previous chunk is done with LDS
    commit_raw_norm8<D, NPC, RSTEP>(pk_, rkP, PR * 2, sF + G8::F_NK, prow, tid);
#pragma unroll
    for (int i = 0; i < NPC; ++i) *(uint4*)(vP + i * RSTEP * PV * 2) = pv_.r[i];
    {
      const bool more = c + 1 < c1;
      const int Ln = more ? min(C, T - (c + 1) * C) : 0;
      pf::load_pieces_n<D, NPC, RSTEP>(pk_, kg + (size_t)(c + 1) * C * rse, Ln, prow, pcol, rsb);
      pf::load_pieces_n<D, NPC, RSTEP>(pv_, vg + (size_t)(c + 1) * C * rse, Ln, prow, pcol, rsb);
    }
    lds_barrier();
    // K~_t = Xi_t psi(k_t) for this wave's jobs; padded tokens give exactly zero
#pragma unroll
    for (int u = 0; u < JPW; ++u) {
      const int jb = w * JPW + u, ft = job_ft<NJ>(jb), jt = job_jt8<NJ>(jb);
      const f32x16 acc = feature_gemm<D>(wop, rR, jt, PR * 2);
      const int t = jt * 32 + n;
      // exponent offset: |k|^2/2, the 1/sqrt(n_psi) factor and log2 Xi_t; -inf past the end
      const float h = t < L ? 0.5f * sF[G8::F_NK + t] * LOG2E - log2_rsqrt - (DECAY ? (float)(L - 1 - t) * lg : 0.f)
                            : __builtin_huge_valf();
      float v[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) v[r] = exp2_hw(acc[r] * LOG2E - h);
      write_psik<NP, LO>(pk, t, ft, hh, v);
    }
    lds_barrier();
    if (DECAY) {
#pragma unroll
      for (int pt = 0; pt < NFH; ++pt) S[pt] *= a;
      Zs *= a;
    }
    state_update_half<C, NP, NFH, LO, PV, NORM>(S, Zs, sb, vT);
  }
  // segment summary -> workspace [bh][seg][E], E = NP*D + NP
  const size_t E = (size_t)NP * D + NP;
  float* out = p.ws + rec_index(p, bh, seg) * E;
#pragma unroll
  for (int pt = 0; pt < NFH; ++pt) {
    const int tile = fh * NFH + (pt + rot) % NFH;
#pragma unroll
    for (int r = 0; r < 16; ++r) out[(size_t)(tile * 32 + dtile_row(r, lane)) * D + Ew + n] = S[pt][r];
  }
  // normaliser: the column sums of the first tile, from the waves whose first tiles cover the half
  if (cb < NFH && hh == 0) out[(size_t)NP * D + (fh * NFH + rot) * 32 + n] = NORM ? Zs[0] : 0.f;
}

// ---------------------------------------------------------------------------------------
// Output pass: per (sequence, segment), from the segment's exclusive prefix (written by
// the scan), walk the chunks: features, shared score tiles, outputs, state update.
template <int C, int D, int NP, bool DECAY, bool NORM, bool OBF, bool QS>
__global__ __launch_bounds__(512) void k_output_prf(PrefillParams p) {
  using G8 = Geo8<C, D, NP>;
  using G = Geo<C, D, NP, true>;
  constexpr int NJ = G8::NJ, NFH = G8::NFH, NFT = G8::NFT, JPW = G8::JPW, NPC = G8::NPC, RSTEP = G8::RSTEP;
  constexpr int PR = G::PR, PQ = G::PQ, PV = G::PV, PA = G::PA;
  constexpr int LO = G::PSIK, ALO = 32 * PA * 2;
  constexpr float LOG2E = 1.4426950408889634f;
  extern __shared__ __align__(16) unsigned char smem[];
  const int bh = blockIdx.x, seg = blockIdx.y, head = bh % p.H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, n = lane & 31, hh = lane >> 5;
  const int L16 = lane & 15, g = lane >> 4;
  const int cb = w & 3, fh = w >> 2, Ew = 32 * cb;
  const float lg = DECAY ? p.log2g[head] : 0.f;
  const float log2_rsqrt = -0.5f * __log2f((float)NP);

  const int prow = tid / G8::PPR, pcol = (tid % G8::PPR) * 8;
  const int trow = 8 * (g >> 1) + (L16 >> 2), tcol = 16 * (g & 1) + 4 * (L16 & 3);
  unsigned char* const rqP = smem + pin(G::OFF_RQ + (prow * PR + pcol) * 2);  // raw K at + RAW
  const unsigned char* const rR = smem + pin(G::OFF_RQ + (n * PR + 8 * hh) * 2);
  unsigned char* const pqW = smem + pin(G::OFF_PQ + (n * PQ + 4 * hh) * 2);  // psi(Q) writes / numT operand
  const unsigned char* const pqS = smem + pin(G::OFF_PQ + (n * PQ + 8 * hh) * 2);  // score operand
  unsigned char* const pk = smem + pin(G::OFF_PK);
  unsigned char* const vP = smem + pin(G::OFF_V + (prow * PV + pcol) * 2);
  const unsigned char* const vT = smem + pin(G::OFF_V + (trow * PV + Ew + tcol) * 2);
  unsigned char* const aW = smem + pin(G::OFF_A + (n * PA + 4 * hh) * 2);
  const unsigned char* const aR = smem + pin(G::OFF_A + (n * PA + 8 * hh) * 2);
  float* const xch = (float*)(smem + pin(G8::OFF_X)) + 4 * lane;  // [cb][jt][r / 4][lane][r % 4] partial outputs
  float* const sF = (float*)(smem + pin(G::OFF_F));
  float* const fN = (float*)(smem + pin(G::OFF_F + 4 * n));
  const PsiKBases<NP> kb8 = psik_bases<NP>(smem, G::OFF_PK, n, hh);
  const int rot = cb % NFH;  // this wave's first feature tile is fh NFH + rot (its column sums give Z)
  const StBases<NFH> sb = st_bases<NP, NFH>(smem, G::OFF_PK, trow, tcol, fh * NFH, rot);

  // this lane's row of W for the wave's feature tile (M = feature, k = input dim): read again each
  // chunk (the head's bank stays in L2), so that the operands hold registers only until the
  // feature GEMMs are done
  const uint16_t* const wrow =
      (const uint16_t*)p.prf_w + (size_t)head * NP * D + (size_t)(job_ft<NJ>(w * JPW) * 32 + n) * D + 8 * hh;

  // exclusive prefix state of this segment: this wave's rows and columns
  const size_t E = (size_t)NP * D + NP;
  f32x16 S[NFH];  // S[j]: feature tile fh NFH + (j + rot) % NFH, value columns Ew ..
  if (p.fold_records) {
    // no scan ran: fold the summary records before this segment in order (each record's decay
    // gamma^len applied to what came before; all of them are whole sub-segments), one record's
    // loads in flight at a time
    const float* rec = p.ws + (size_t)bh * p.n_rec * E;
    const int nr = seg * p.rec_per_seg;
    const float a = DECAY ? exp2_hw((float)((p.seg_chunks / p.rec_per_seg) * C) * lg) : 1.f;
#pragma unroll
    for (int pt = 0; pt < NFH; ++pt) S[pt] = f32x16{};
    float z = 0.f;
    for (int r0 = 0; r0 < nr; ++r0) {
      const float* x = rec + (size_t)r0 * E;
      f32x16 y[NFH];
#pragma unroll
      for (int pt = 0; pt < NFH; ++pt) {
        const int tile = fh * NFH + (pt + rot) % NFH;
#pragma unroll
        for (int r = 0; r < 16; ++r) y[pt][r] = x[(size_t)(tile * 32 + dtile_row(r, lane)) * D + Ew + n];
      }
      const float zr = (NORM && tid < NP) ? x[(size_t)NP * D + tid] : 0.f;
#pragma unroll
      for (int pt = 0; pt < NFH; ++pt) {
        if (DECAY) S[pt] *= a;
        S[pt] += y[pt];
      }
      z = a * z + zr;
    }
    if (tid < NP) sF[G8::F_Z + tid] = NORM ? z : 0.f;
  } else {
    const float* pre = p.ws + rec_index(p, bh, seg) * E;
#pragma unroll
    for (int pt = 0; pt < NFH; ++pt) {
      const int tile = fh * NFH + (pt + rot) % NFH;
#pragma unroll
      for (int r = 0; r < 16; ++r) S[pt][r] = pre[(size_t)(tile * 32 + dtile_row(r, lane)) * D + Ew + n];
    }
    for (int j = tid; j < NP; j += G8::NT) sF[G8::F_Z + j] = NORM ? pre[(size_t)NP * D + j] : 0.f;
  }
  for (int j = tid; j < C; j += G8::NT) sF[G8::F_THETA + j] = DECAY ? exp2_hw((float)(j + 1) * lg) : 1.f;

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
  pf::PiecesN<NPC> pq_, pk_, pv_;
  {
    const int L0 = min(C, T - c0 * C);
    pf::load_pieces_n<D, NPC, RSTEP>(pq_, qg + (size_t)c0 * C * rse, L0, prow, pcol, rsb);
    pf::load_pieces_n<D, NPC, RSTEP>(pk_, kg + (size_t)c0 * C * rse, L0, prow, pcol, rsb);
    pf::load_pieces_n<D, NPC, RSTEP>(pv_, vg + (size_t)c0 * C * rse, L0, prow, pcol, rsb);
    vm_drain();
  }
  for (int c = c0; c < c1; ++c) {
    const int t0 = c * C, L = min(C, T - t0);
    const float a = DECAY ? exp2_hw((float)L * lg) : 1.f;
    bf16x8 wop[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) wop[kk] = *(const bf16x8*)(wrow + 16 * kk);
    lds_barrier();  // the previous chunk is done with LDS (and Z is updated)
    commit_raw_norm8<D, NPC, RSTEP>(pq_, rqP, PR * 2, sF + G8::F_NQ, prow, tid);
    commit_raw_norm8<D, NPC, RSTEP>(pk_, rqP + G::RAW, PR * 2, sF + G8::F_NK, prow, tid);
#pragma unroll
    for (int i = 0; i < NPC; ++i) *(uint4*)(vP + i * RSTEP * PV * 2) = pv_.r[i];
    {
      const bool more = c + 1 < c1;
      const int Ln = more ? min(C, T - (c + 1) * C) : 0;
      pf::load_pieces_n<D, NPC, RSTEP>(pq_, qg + (size_t)(c + 1) * C * rse, Ln, prow, pcol, rsb);
      pf::load_pieces_n<D, NPC, RSTEP>(pk_, kg + (size_t)(c + 1) * C * rse, Ln, prow, pcol, rsb);
      pf::load_pieces_n<D, NPC, RSTEP>(pv_, vg + (size_t)(c + 1) * C * rse, Ln, prow, pcol, rsb);
    }
    lds_barrier();

    // ---- QS: the query-row shift (see the header): each job's largest logit per token, the
    // feature tiles' maxima meet in LDS
    if (QS) {
#pragma unroll
      for (int u = 0; u < JPW; ++u) {
        const int jb = w * JPW + u, ft = job_ft<NJ>(jb), jt = job_jt8<NJ>(jb);
        const f32x16 acc = feature_gemm<D>(wop, rR, jt, PR * 2);
        float mx = -__builtin_huge_valf();
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc[r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));  // the other lane half holds the tile's other rows
        if (hh == 0) sF[G8::F_QMAX + ft * C + jt * 32 + n] = mx;
      }
      lds_barrier();
    }

    // ---- features of this wave's jobs: psi(Q) rounded to bf16 (and its dot with Z_prev per
    // token); psi(K) as hi + lo, zero past the sequence end
#pragma unroll
    for (int u = 0; u < JPW; ++u) {
      const int jb = w * JPW + u, ft = job_ft<NJ>(jb), jt = job_jt8<NJ>(jb);
      const int t = jt * 32 + n;
      {
        const f32x16 acc = feature_gemm<D>(wop, rR, jt, PR * 2);
        float qshift = 0.5f * sF[G8::F_NQ + t];  // |q|^2 / 2, or the row's largest w_p . q (QS)
        if (QS) {
          qshift = sF[G8::F_QMAX + t];
#pragma unroll
          for (int f = 1; f < NFT; ++f) qshift = fmaxf(qshift, sF[G8::F_QMAX + f * C + t]);
        }
        const float h = qshift * LOG2E - log2_rsqrt;
        float v[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) v[r] = exp2_hw(acc[r] * LOG2E - h);
        float qz = 0.f;
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const uint2 pq4 = pack4(v[4 * gq], v[4 * gq + 1], v[4 * gq + 2], v[4 * gq + 3]);
          *(uint2*)(pqW + (jt * 32 * PQ + ft * 32 + 8 * gq) * 2) = pq4;
          if (NORM) {  // the same rounded features as the numerator reads
            const bf16x4 b4 = __builtin_bit_cast(bf16x4, pq4);
            const f32x4 z4 = *(const f32x4*)(sF + G8::F_Z + ft * 32 + 8 * gq + 4 * hh);
#pragma unroll
            for (int e = 0; e < 4; ++e) qz += from_bf16(b4[e]) * z4[e];
          }
        }
        if (NORM) {
          qz += __shfl_xor(qz, 32);
          if (hh == 0) sF[G8::F_QZ + ft * C + t] = qz;
        }
      }
      {
        const f32x16 acc = feature_gemm<D>(wop, rR + G::RAW, jt, PR * 2);
        const float h = t < L ? 0.5f * sF[G8::F_NK + t] * LOG2E - log2_rsqrt : __builtin_huge_valf();
        float v[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) v[r] = exp2_hw(acc[r] * LOG2E - h);
        write_psik<NP, LO>(pk, t, ft, hh, v);
      }
    }
    lds_barrier();  // features complete; the raw tiles are dead (the score tiles alias them)

    // ---- outputs, transposed: numT[e][j] (M = value column, N = token). The inter-chunk part
    // over this wave's half of the features: S_prev^T psi(Q)^T, S_prev as hi + lo
    f32x16 num[NJ];
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt) num[jt] = f32x16{};
    auto inter = [&]() {
#pragma unroll
      for (int pt = 0; pt < NFH; ++pt) {
        bf16x8 sh[2], sl[2];  // k in the D-tile feedback order
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          float x[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) x[j] = S[pt][8 * q + j];
          split8_trunc(x, sh[q], sl[q]);
        }
        const int fcol = (fh * NFH + (pt + rot) % NFH) * 32;
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const unsigned char* qa = pqW + (jt * 32 * PQ + fcol + 16 * q) * 2;
            const bf16x8 qo = cat8(*(const bf16x4*)qa, *(const bf16x4*)(qa + 16));
            num[jt] = mfma32(sh[q], qo, num[jt]);
            num[jt] = mfma32(sl[q], qo, num[jt]);
          }
      }
    };

    // ---- score tile w (M = i, N = j, k = feature), masked, decayed, split into hi + lo. (The
    // other waves could take their inter-chunk part meanwhile, but holding its accumulators
    // across the score code pushes this kernel past 256 registers.)
    if (w < G8::NTILE) {
      const int tt = w, jt = pf::tile_jt(tt), it = tt - jt * (jt + 1) / 2;
      f32x16 acc = f32x16{};
#pragma unroll
      for (int kk = 0; kk < NP / 16; ++kk) {
        const bf16x8 qv = *(const bf16x8*)(pqS + (jt * 32 * PQ + kk * 16) * 2);
        acc = mfma32(psik_row<NP>(kb8, it * 32, kk, 0), qv, acc);
        acc = mfma32(psik_row<NP>(kb8, it * 32, kk, LO), qv, acc);
      }
      const bool diag = it == jt;
      const float tf = (DECAY && !diag) ? exp2_hw((float)(32 * (jt - it - 1)) * lg) : 1.f;
      float av[16];
      float rs = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ir = dtile_row(r, lane);
        if constexpr (DECAY) {
          const float f = diag ? (ir <= n ? exp2_hw((float)(n - ir) * lg) : 0.f) : exp2_hw((float)(n + 32 - ir) * lg) * tf;
          av[r] = acc[r] * f;
        } else {
          av[r] = (diag && ir > n) ? 0.f : acc[r];
        }
        if (NORM) rs += av[r];
      }
      if (NORM) {
        rs += __shfl_xor(rs, 32);
        if (hh == 0) fN[G8::F_R + tt * 32] = rs;
      }
      unsigned char* at = aW + tt * G::A_TILE;
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

    // ---- the inter-chunk part; theta weights; the intra-chunk term V^T A^T in equal shares:
    // each half adds the diagonal score tile of token tile fh and one 16-key half (k-half fh)
    // of the off-diagonal tile (queries of token tile 1, keys of token tile 0)
    static_assert(NJ == 2, "one token tile per feature half; tiles (0, 0) = 0, (1, 0) = 1, (1, 1) = 2");
    inter();
    if (DECAY) {
#pragma unroll
      for (int jt = 0; jt < NJ; ++jt) num[jt] *= fN[G8::F_THETA + jt * 32];
    }
    {
      auto av_step = [&](f32x16& acc, int t, int it, int q) {
        const unsigned char* at = aR + t * G::A_TILE;
        const int r0 = it * 32 + 16 * q;
        const bf16x8 vv = cat8(lds_read_tr4((const __bf16*)(vT + r0 * PV * 2)),
                               lds_read_tr4((const __bf16*)(vT + (r0 + 4) * PV * 2)));
        acc = mfma32(vv, *(const bf16x8*)(at + 32 * q), acc);
        acc = mfma32(vv, *(const bf16x8*)(at + 32 * q + ALO), acc);
      };
      if (__builtin_amdgcn_readfirstlane(fh)) {
        av_step(num[1], 2, 1, 0);
        av_step(num[1], 2, 1, 1);
        av_step(num[1], 1, 0, 1);
      } else {
        av_step(num[0], 0, 0, 0);
        av_step(num[0], 0, 0, 1);
        av_step(num[1], 1, 0, 0);
      }
    }
    // ---- the halves' partial outputs meet: half h completes token tile jt = h of its value
    // columns, taking the other half's partial of that tile through LDS, so that every wave
    // stores the same number of rows (and the next chunk's loads are not held behind stores)
    lds_barrier();  // every wave is done with psi(Q) and the score tiles: their region takes the partials
    f32x16 mine = fh ? num[1] : num[0];
    {
      const f32x16 give = fh ? num[0] : num[1];
      f32x4* const xo = (f32x4*)(xch + ((cb * NJ + (1 - fh)) * 16) * 64);
#pragma unroll
      for (int q = 0; q < 4; ++q) xo[q * 64] = f32x4{give[4 * q], give[4 * q + 1], give[4 * q + 2], give[4 * q + 3]};
    }
    // K~ = Xi psi(K) with decay: rescale the hi + lo tile in place (every wave is done with the
    // score operands), rows past L stay zero
    if (DECAY) {
      constexpr int NCH = C * NP / 8;  // 8-element chunks of the tile
#pragma unroll
      for (int i = 0; i < NCH / G8::NT; ++i) {
        const int ch = tid + i * G8::NT, row = ch / (NP / 8), col = (ch % (NP / 8)) * 8;
        const float xi = row < L ? exp2_hw((float)(L - 1 - row) * lg) : 0.f;
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
    lds_barrier();
    {
      const int jt = fh;
      const f32x4* const xi4 = (const f32x4*)(xch + ((cb * NJ + jt) * 16) * 64);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 o4 = xi4[q * 64];
#pragma unroll
        for (int e = 0; e < 4; ++e) mine[4 * q + e] += o4[e];
      }
      float inv = 1.f;
      if (NORM) {
        // psi(q_j) . Z_prev (per feature tile, from the feature phase) and the score row sums
        float qz = 0.f;
#pragma unroll
        for (int f = 0; f < NFT; ++f) qz += fN[G8::F_QZ + f * C + jt * 32];
        float rr = fN[G8::F_R + (jt * (jt + 1) / 2) * 32];
        if (jt) rr += fN[G8::F_R + 2 * 32];
        inv = 1.f / (fN[G8::F_THETA + jt * 32] * qz + rr + p.eps);
      }
      const __amdgpu_buffer_rsrc_t ors = make_rsrc(ob + (size_t)t0 * rse * OES, rows_extent(L, rse * OES, D * OES));
      const uint32_t row_el = (uint32_t)(jt * 32 + n) * rse + Ew + 4 * hh;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        store_out4<OBF>(ors, row_el + 8 * q4, mine[4 * q4] * inv, mine[4 * q4 + 1] * inv, mine[4 * q4 + 2] * inv,
                        mine[4 * q4 + 3] * inv);
    }

    // ---- state update: S <- gamma^L S + K~^T V (this wave's rows); Z <- gamma^L Z + 1 K~, from
    // the column sums the waves take of their first tiles (read again only in the next chunk)
    if (DECAY) {
#pragma unroll
      for (int pt = 0; pt < NFH; ++pt) S[pt] *= a;
    }
    f32x16 zc = f32x16{};
    state_update_half<C, NP, NFH, LO, PV, NORM>(S, zc, sb, vT);
    if (NORM && cb < NFH && hh == 0) {
      float* const zf = sF + G8::F_Z + (fh * NFH + rot) * 32 + n;
      *zf = a * *zf + zc[0];
    }
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
  const int lds = out ? Geo8<C, D, NP>::LDS_BYTES : Geo8<C, D, NP>::SUM_LDS_BYTES;
  hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  // x = (batch, head), y = segment: workgroups are dealt to the 8 XCDs round-robin by linear id
  // x + y * B * H, so every XCD gets a share of the sequences with all their segments. With the
  // segment on x, segment s would always land on the same XCDs: for variable-length batches the
  // heavy first segments would pile onto a few of them.
  dim3 grid(p.B * p.H, p.n_seg);
  void* args[] = {(void*)&p};
  e = hipLaunchKernel(kern, grid, dim3(Geo8<C, D, NP>::NT), args, lds, s);
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
