// la_backward_prf.hip -- backward pass of the chunked prefill with positive random features
// ("Linearized 2-Simplicial Attention", 3.2 Positive random features for one tensor mode, and
// 4.2 Custom Triton kernel, Backward, with the appendix's backward query and state sweeps):
// the gradients of L = sum_t dout_t . o_t with respect to q, k, v and the initial state.
//
// With g_t = psi(q_t), f_t = psi(k_t) (n_psi features each) the chain rule of la_backward.hip
// gives, per step of 64 tokens (j, i in the step; theta_j = gamma^(j+1), xi_i = gamma^(L-1-i),
// D_ji = gamma^(j-i) [i <= j]; S_< the state before the step, R_> the adjoint state after it):
//   den_j  = sum_i A_ji + theta_j g_j . Z_< + eps,  A = (G F^T) (.) D
//   dout_j . num_j = sum_i A_ji X_ji + theta_j g_j . Y_j,  X = dout V^T, Y = dout S_<^T
//   dnum_j = dout_j / den_j,  dden_j = -(dout_j . num_j) / den_j^2   (normalize = 0: dout_j, 0)
//   Bm     = (X / den + dden 1^T) (.) D
//   dG     = Bm F + theta (.) (Y / den + dden Z_<^T)
//   dF     = Bm'^T G + xi (.) (V R_>^T + RZ_>),  Bm' = (dNum V^T + dden 1^T) (.) D
//   dV     = A^T dNum + xi (.) (F R_>)
// and the feature map's own Jacobian (psi_p(x) = exp(w_p . x - |x|^2/2) / sqrt(m)):
//   dx = sum_p a_p w_p - (sum_p a_p) x,  a_p = dpsi_p psi_p,
// with the query-row shift (psi_p(q) = exp(w_p . q - max_r w_r . q) / sqrt(m)) the last term
// takes the argmax row w_r* in place of x. The bank is a constant (no gradient).
//
// Decomposition. Unlike the identity / elu+1 sweeps, which carry 128 x 128 states through
// segments of many steps, each workgroup here owns one 64-token step: the forward summary pass
// (one record per step) and the scan give every step its prefix S_< directly, and the reverse
// scan of the query kernel's per-step adjoint records gives R_>. A 256 x 128 fp32 state is 128
// KiB; reading it per step costs state traffic, but no state is carried on chip and the n_psi
// features are processed in quarters of 64, which keeps the LDS image under 150 KiB.
//
// Precision as in the other sweeps: every operand that is not exact in bf16 (features, dout,
// dNum, the states, the C x C tiles, the Jacobian weights) is a two-term hi + lo bf16 expansion
// on MFMA 32x32x16 with fp32 accumulation; q, k, v and the bank are exact bf16 operands.
#include "la_device.hpp"
#include "la_kernels.hpp"

namespace la {

hipError_t launch_prefill_prf_bf16(const PrefillParams& p, hipStream_t s, bool out);

namespace {

constexpr int PC = 64;      // tokens per step (one workgroup)
constexpr int PD = 128;     // d_k = d_v
constexpr int PNT = 256;    // four waves
constexpr int PR = PD + 8;  // pitch (elements) of the 64 x 128 bf16 tiles
constexpr int PQW = 64;     // features per quarter
constexpr int PF = PQW + 8; // pitch of the 64 x 64 bf16 tiles (feature quarters, C x C tiles)
constexpr float LOG2E = 1.4426950408889634f;

// LDS image: bf16 element offsets, then float tables.
struct PG {
  static constexpr int RAW = PC * PR, SQT = PC * PF;
  static constexpr int QR = 0, KR = RAW, VR = 2 * RAW;
  static constexpr int BH = 3 * RAW, BL = BH + RAW;        // dout (query) / dNum then R_> quarter (key), hi + lo
  static constexpr int GH = BL + RAW, GL = GH + SQT;       // G quarter (then A, then the key Jacobian weights)
  static constexpr int FH = GL + SQT, FL = FH + SQT;       // F quarter (then the query Jacobian weights)
  static constexpr int MH = FL + SQT, ML = MH + SQT;       // Bm
  static constexpr int HALVES = ML + SQT;
  static constexpr int F0 = HALVES / 2;
  // per-token tables [PC]
  static constexpr int NQ = F0, NK = NQ + PC, HQ = NK + PC, HK = HQ + PC, QA = HK + PC, TH = QA + PC, XI = TH + PC,
                       DM = XI + PC, IV = DM + PC, DD = IV + PC, WI = DD + PC, WT = WI + PC, AS = WT + PC,
                       AX = AS + 2 * PC, GZ = AX + 2 * PC, GY = GZ + 2 * PC, CJ = GY + 2 * PC, MX = CJ + 2 * PC;
  static constexpr int ZQ = MX + 2 * 2 * 4 * PC;  // per (quarter, ft) max partials [4][2][PC] values then indices
  static constexpr int FEND = ZQ + 256;            // Z_< / RZ_> of all features (<= 256)
  static constexpr int BYTES = FEND * 4;
};
static_assert(PG::HALVES % 8 == 0, "float tables 16-byte aligned");
static_assert(PG::BYTES <= 160 * 1024, "LDS image fits a CU");

// ---- loads -------------------------------------------------------------------------------

// A step's 64 token rows of 128 bf16 as 16-byte pieces: thread t holds rows t / 16 + 16 i, columns 8 (t % 16).
struct Raw {
  uint4 r[PC * PD / 8 / PNT];
};
__device__ __forceinline__ void load_raw(Raw& P, const void* base, int valid, uint32_t rsb) {
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, rows_extent(valid, rsb, PD * 2));
  const int t = threadIdx.x;
  const uint32_t v0 = (uint32_t)(t >> 4) * rsb + (uint32_t)(t & 15) * 16;
#pragma unroll
  for (int i = 0; i < 4; ++i) P.r[i] = buf_load16(rs, v0, (uint32_t)(16 * i) * rsb);
}
__device__ __forceinline__ void commit_raw_rows(const Raw& P, __bf16* dst, float* norm) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = (t >> 4) + 16 * i, col = (t & 15) * 8;
    *(uint4*)(dst + row * PR + col) = P.r[i];
    if (norm) {
      const bf16x8 x = __builtin_bit_cast(bf16x8, P.r[i]);
      float sq = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) sq += from_bf16(x[j]) * from_bf16(x[j]);
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) sq += __shfl_xor(sq, off);
      if ((t & 15) == 0) norm[row] = sq;
    }
  }
}

// dout (fp32 or bf16) of the step, times s_j per token, as hi + lo: thread t holds token t / 4,
// columns 4 (t % 4) + 16 i.
template <bool DBF>
__device__ __forceinline__ void commit_dout(const void* base, int valid, uint32_t rsbd, const float* scale,
                                            __bf16* hi, __bf16* lo) {
  constexpr int ES = DBF ? 2 : 4;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, rows_extent(valid, rsbd, PD * ES));
  const int t = threadIdx.x, j = t >> 2, c0 = 4 * (t & 3);
  const float s = scale ? scale[j] : 1.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int col = c0 + 16 * i;
    f32x4 x;
    if (DBF) {
      const u32x2 w = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, (uint32_t)j * rsbd + col * 2, 0, 0));
      x = f32x4{__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u), __uint_as_float(w[1] << 16),
                __uint_as_float(w[1] & 0xffff0000u)};
    } else {
      x = __builtin_bit_cast(f32x4, buf_load16(rs, (uint32_t)j * rsbd + col * 4));
    }
    bf16x4 h, l;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bf16_pair pr = split_bf16(s * x[e]);
      h[e] = pr.hi;
      l[e] = pr.lo;
    }
    *(bf16x4*)(hi + j * PR + col) = h;
    *(bf16x4*)(lo + j * PR + col) = l;
  }
}

// ---- tile helpers ------------------------------------------------------------------------

__device__ __forceinline__ f32x16 zero16p() {
  f32x16 z;
#pragma unroll
  for (int r = 0; r < 16; ++r) z[r] = 0.f;
  return z;
}

// Eight fp32 values at p (16-byte aligned) as hi + lo.
__device__ __forceinline__ void split_g8(const float* p, bf16x8& hi, bf16x8& lo) {
  const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
  float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  split8_trunc(x, hi, lo);
}

// Row sums over the 32 columns of a D-tile (lane l ends with row dtile_row((l >> 1) & 15, l)).
__device__ __forceinline__ float rsum16(const f32x16& v, int lane) {
  float a[8], b[4], c[2];
  const bool b4 = lane & 16, b3 = lane & 8, b2 = lane & 4, b1 = lane & 2;
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = (b4 ? v[8 + i] : v[i]) + __shfl_xor(b4 ? v[i] : v[8 + i], 16);
#pragma unroll
  for (int i = 0; i < 4; ++i) b[i] = (b3 ? a[4 + i] : a[i]) + __shfl_xor(b3 ? a[i] : a[4 + i], 8);
#pragma unroll
  for (int i = 0; i < 2; ++i) c[i] = (b2 ? b[2 + i] : b[i]) + __shfl_xor(b2 ? b[i] : b[2 + i], 4);
  const float d = (b1 ? c[1] : c[0]) + __shfl_xor(b1 ? c[0] : c[1], 2);
  return d + __shfl_xor(d, 1);
}
__device__ __forceinline__ int rsum16_row(int lane) { return dtile_row((lane >> 1) & 15, lane); }

// The larger of (v, i) and (w, j); on equal values the smaller index (the first maximum).
__device__ __forceinline__ void vmax_pair(float& v, int& i, float w, int j) {
  if (w > v || (w == v && j < i)) {
    v = w;
    i = j;
  }
}
// Row maximum and its column over the 32 columns of a D-tile whose columns are c0 + lane % 32;
// the same lane mapping as rsum16.
__device__ __forceinline__ void rmax16(const f32x16& v, int c0, int lane, float& mv, int& mi) {
  const int col = c0 + (lane & 31);
  float a[8], b[4], c[2];
  int ai[8], bi[4], ci[2];
  const bool b4 = lane & 16, b3 = lane & 8, b2 = lane & 4, b1 = lane & 2;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = b4 ? v[8 + i] : v[i];
    ai[i] = col;
    vmax_pair(a[i], ai[i], __shfl_xor(b4 ? v[i] : v[8 + i], 16), col ^ 16);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    b[i] = b3 ? a[4 + i] : a[i];
    bi[i] = b3 ? ai[4 + i] : ai[i];
    vmax_pair(b[i], bi[i], __shfl_xor(b3 ? a[i] : a[4 + i], 8), __shfl_xor(b3 ? ai[i] : ai[4 + i], 8));
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    c[i] = b2 ? b[2 + i] : b[i];
    ci[i] = b2 ? bi[2 + i] : bi[i];
    vmax_pair(c[i], ci[i], __shfl_xor(b2 ? b[i] : b[2 + i], 4), __shfl_xor(b2 ? bi[i] : bi[2 + i], 4));
  }
  mv = b1 ? c[1] : c[0];
  mi = b1 ? ci[1] : ci[0];
  vmax_pair(mv, mi, __shfl_xor(b1 ? c[0] : c[1], 2), __shfl_xor(b1 ? ci[0] : ci[1], 2));
  vmax_pair(mv, mi, __shfl_xor(mv, 1), __shfl_xor(mi, 1));
}

// Logits w_p . x for the tile (tokens 32 jt.., features p0 + 0..31) of the raw tile at X:
// A[m=j][k=d] = x_j[d], B[k=d][n=p] = W[p][d] read straight from the bank.
__device__ __forceinline__ f32x16 logit_tile(const __bf16* X, const uint16_t* Wh, int jt, int p0, int lane) {
  f32x16 acc = zero16p();
  const uint16_t* wr = Wh + (size_t)(p0 + (lane & 31)) * PD + 8 * (lane >> 5);
#pragma unroll
  for (int k0 = 0; k0 < PD; k0 += 16)
    acc = mfma32(ld_cols8(X, PR, 32 * jt, k0, lane), *(const bf16x8*)(wr + k0), acc);
  return acc;
}

// Feature tile (tokens 32 jt.., features of quarter qi, tile ft) into a quarter image (pitch PF)
// as hi + lo: psi = exp2(logit log2e - h_j), h_j from the per-token table (+inf: zero row).
__device__ __forceinline__ void feature_tile(const __bf16* X, const uint16_t* Wh, const float* h, int qi, int jt,
                                             int ft, __bf16* dh, __bf16* dl, int lane) {
  const f32x16 acc = logit_tile(X, Wh, jt, PQW * qi + 32 * ft, lane);
  const int col = 32 * ft + (lane & 31);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int j = 32 * jt + dtile_row(r, lane);
    const bf16_pair pr = split_bf16(exp2f(acc[r] * LOG2E - h[j]));
    dh[j * PF + col] = pr.hi;
    dl[j * PF + col] = pr.lo;
  }
}

// acc += A B over k in [0, K) for operands in LDS; *_T: the operand is stored with its k
// index along the storage column (transpose reads), else along the storage row. LO_*: a lo part
// exists (at the hi pointer's offset `lo_*`). Three products when both have lo parts.
template <bool A_T, bool A_LO, bool B_T, bool B_LO, int K>
__device__ __forceinline__ f32x16 tile_mma(f32x16 acc, const __bf16* a, int pa, int lo_a, int am0, const __bf16* b,
                                           int pb, int lo_b, int bn0, int lane) {
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += 16) {
    const bf16x8 ah = A_T ? ld_rows8(a, pa, k0, am0, lane) : ld_cols8(a, pa, am0, k0, lane);
    const bf16x8 bh = B_T ? ld_rows8(b, pb, k0, bn0, lane) : ld_cols8(b, pb, bn0, k0, lane);
    acc = mfma32(ah, bh, acc);
    if (B_LO) acc = mfma32(ah, B_T ? ld_rows8(b + lo_b, pb, k0, bn0, lane) : ld_cols8(b + lo_b, pb, bn0, k0, lane), acc);
    if (A_LO) acc = mfma32(A_T ? ld_rows8(a + lo_a, pa, k0, am0, lane) : ld_cols8(a + lo_a, pa, am0, k0, lane), bh, acc);
  }
  return acc;
}

// (hi + lo) * f per element, 8 values, re-split as hi + lo.
__device__ __forceinline__ void scale_split_prf(const bf16x8& xh, const bf16x8& xl, const float* f, bf16x8& hi,
                                                bf16x8& lo) {
  float y[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) y[j] = (from_bf16(xh[j]) + from_bf16(xl[j])) * f[j];
  split8_trunc(y, hi, lo);
}

// A D-tile's values as hi + lo into a 64 x 64 image (pitch PF) at rows 32 rt.., columns 32 ct..
__device__ __forceinline__ void store_sq(__bf16* h, __bf16* l, const f32x16& v, int rt, int ct, int lane) {
  const int c = 32 * ct + (lane & 31);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const bf16_pair pr = split_bf16(v[r]);
    const int row = 32 * rt + dtile_row(r, lane);
    h[row * PF + c] = pr.hi;
    l[row * PF + c] = pr.lo;
  }
}

// Per-token tables of a step: theta, xi, the decay mask by lag, the feature exponents' offsets.
template <bool DECAY>
__device__ __forceinline__ void step_tables(float* sf, int L, float lg, float log2_rsqrt, bool qs) {
  const int j = threadIdx.x;
  if (j < PC) {
    sf[PG::TH + j] = DECAY ? exp2f((float)(j + 1) * lg) : 1.f;
    sf[PG::XI + j] = j < L ? (DECAY ? exp2f((float)(L - 1 - j) * lg) : 1.f) : 0.f;
    sf[PG::DM + j] = DECAY ? exp2f((float)j * lg) : 1.f;
    if (!qs) sf[PG::HQ + j] = 0.5f * sf[PG::NQ + j] * LOG2E - log2_rsqrt;
    // keys past the step's end are the monoid identity: zero features
    sf[PG::HK + j] = j < L ? 0.5f * sf[PG::NK + j] * LOG2E - log2_rsqrt : __builtin_huge_valf();
  }
}

// The query-row shift: each token's largest logit and its feature index (first maximum).
template <int NP>
__device__ __forceinline__ void query_shift(float* sf, const __bf16* sh, const uint16_t* Wh, float log2_rsqrt,
                                            int w, int lane) {
  const int jt = w >> 1, ft = w & 1;
#pragma unroll
  for (int qi = 0; qi < NP / PQW; ++qi) {
    const int p0 = PQW * qi + 32 * ft;
    float mv;
    int mi;
    rmax16(logit_tile(sh + PG::QR, Wh, jt, p0, lane), p0, lane, mv, mi);
    if ((lane & 1) == 0) {
      const int j = 32 * jt + rsum16_row(lane);
      sf[PG::MX + (qi * 2 + ft) * PC + j] = mv;
      ((int*)sf)[PG::MX + 8 * PC + (qi * 2 + ft) * PC + j] = mi;
    }
  }
  lds_barrier();
  if (threadIdx.x < PC) {
    const int j = threadIdx.x;
    float mv = sf[PG::MX + j];
    int mi = ((const int*)sf)[PG::MX + 8 * PC + j];
    for (int s = 1; s < 2 * (NP / PQW); ++s)
      vmax_pair(mv, mi, sf[PG::MX + s * PC + j], ((const int*)sf)[PG::MX + 8 * PC + s * PC + j]);
    sf[PG::HQ + j] = mv * LOG2E - log2_rsqrt;
    ((int*)sf)[PG::QA + j] = mi;
  }
}

// Y = dout S_<^T tile (tokens 32 jt.., features of quarter qi, tile ft): A[m=j][k=e] = dout
// (hi + lo in the B image), B[k=e][n=p] = S_<[p][e] read from the step's forward record.
__device__ __forceinline__ f32x16 y_tile(const __bf16* sh, const float* pre, int qi, int jt, int ft, int lane) {
  f32x16 y = zero16p();
  const float* srow = pre + (size_t)(PQW * qi + 32 * ft + (lane & 31)) * PD + 8 * (lane >> 5);
#pragma unroll
  for (int k0 = 0; k0 < PD; k0 += 16) {
    bf16x8 sbh, sbl;
    split_g8(srow + k0, sbh, sbl);
    const bf16x8 nh = ld_cols8(sh + PG::BH, PR, 32 * jt, k0, lane);
    y = mfma32(nh, sbh, y);
    y = mfma32(nh, sbl, y);
    y = mfma32(ld_cols8(sh + PG::BL, PR, 32 * jt, k0, lane), sbh, y);
  }
  return y;
}

// G and F quarter qi: each wave one (token tile, feature tile) of each.
__device__ __forceinline__ void features_quarter(__bf16* sh, const float* sf, const uint16_t* Wh, int qi, int w,
                                                 int lane) {
  const int jt = w >> 1, ft = w & 1;
  feature_tile(sh + PG::QR, Wh, sf + PG::HQ, qi, jt, ft, sh + PG::GH, sh + PG::GL, lane);
  feature_tile(sh + PG::KR, Wh, sf + PG::HK, qi, jt, ft, sh + PG::FH, sh + PG::FL, lane);
}

// Tile (jt, it) of the lower block triangle for waves 0..2.
__device__ __forceinline__ int jobj(int job) { return job == 0 ? 0 : 1; }
__device__ __forceinline__ int jobi(int job) { return job == 2 ? 1 : 0; }

// ---- query kernel ------------------------------------------------------------------------

template <int NP, bool DECAY, bool NORM, bool DBF, bool QS>
__global__ __launch_bounds__(PNT) void k_bwd_prf_query(BackwardParams bp) {
  const PrefillParams& p = bp.f;
  constexpr int NQT = NP / PQW;
  extern __shared__ __align__(16) unsigned char smem[];
  __bf16* sh = (__bf16*)smem;
  float* sf = (float*)smem;
  const int bh = blockIdx.x, seg = blockIdx.y, tid = threadIdx.x, lane0 = tid & 63, w = tid >> 6;
  const int head = bh % p.H;
  int lane = lane0;
  const SeqSpan sq = seq_span(p, bh);
  const int t0 = seg * PC, L = max(0, min(PC, sq.T - t0));
  const size_t E = (size_t)NP * PD + NP;
  float* rrec = bp.rev + ((size_t)bh * p.n_seg + seg) * E;
  if (L == 0) {  // a step past the end of a shorter sequence: an empty adjoint record
    for (int i = tid; i < (int)E; i += PNT) rrec[i] = 0.f;
    return;
  }
  const float* pre = p.ws + ((size_t)bh * p.n_seg + seg) * E;  // S_< [p][e], Z_< [p]
  const float lg = DECAY ? p.log2g[head] : 0.f;
  const float log2_rsqrt = -0.5f * __log2f((float)NP);
  const uint16_t* Wh = (const uint16_t*)p.prf_w + (size_t)head * NP * PD;
  const uint16_t* Wt = bp.wt + (size_t)head * NP * PD;  // [d][p]
  const long long r0 = sq.row0 + (long long)t0 * p.tok_rows;
  const uint32_t rsb = (uint32_t)p.tok_rows * PD * 2, rsb4 = (uint32_t)p.tok_rows * PD * 4;
  const uint32_t rsbd = (uint32_t)p.tok_rows * PD * (DBF ? 2 : 4);
  const int jt = w >> 1, ft = w & 1;

  {
    Raw tq, tk, tv;
    load_raw(tq, (const uint16_t*)p.q + r0 * PD, L, rsb);
    load_raw(tk, (const uint16_t*)p.k + r0 * PD, L, rsb);
    load_raw(tv, (const uint16_t*)p.v + r0 * PD, L, rsb);
    commit_raw_rows(tq, sh + PG::QR, sf + PG::NQ);
    commit_raw_rows(tk, sh + PG::KR, sf + PG::NK);
    commit_raw_rows(tv, sh + PG::VR, nullptr);
  }
  commit_dout<DBF>((const unsigned char*)bp.dout + r0 * PD * (DBF ? 2 : 4), L, rsbd, nullptr, sh + PG::BH, sh + PG::BL);
  for (int i = tid; i < NP; i += PNT) sf[PG::ZQ + i] = NORM ? pre[(size_t)NP * PD + i] : 0.f;
  lds_barrier();
  step_tables<DECAY>(sf, L, lg, log2_rsqrt, QS);
  if (QS) query_shift<NP>(sf, sh, Wh, log2_rsqrt, w, lane);
  lds_barrier();

  // X = dout V^T for the lower block triangle (waves 0..2)
  f32x16 X = zero16p(), A = zero16p();
  if (w < 3)
    X = tile_mma<false, true, false, false, PD>(X, sh + PG::BH, PR, PG::BL - PG::BH, 32 * jobj(w), sh + PG::VR, PR,
                                                0, 32 * jobi(w), lane);
  // pass 1 over feature quarters (with a denominator): A, g . Z_< and g . Y
  float gz = 0.f, gy = 0.f;
#pragma unroll 1
  for (int qi = 0; NORM && qi < NQT; ++qi) {
    // the lane index, opaque once per quarter: per-lane LDS addresses are then formed inside the
    // loop from a few bases, not hoisted out of it as one live register per access
    const int lane = pin(lane0);
    features_quarter(sh, sf, Wh, qi, w, lane);
    const f32x16 y = y_tile(sh, pre, qi, jt, ft, lane);
    lds_barrier();  // the quarter's features are complete
    {
      if (w < 3)
        A = tile_mma<false, true, false, true, PQW>(A, sh + PG::GH, PF, PG::GL - PG::GH, 32 * jobj(w), sh + PG::FH,
                                                    PF, PG::FL - PG::FH, 32 * jobi(w), lane);
      f32x16 a1, a2;
      const int col = 32 * ft + (lane & 31);
      const float z = sf[PG::ZQ + PQW * qi + col];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = 32 * jt + dtile_row(r, lane);
        const float g = from_bf16(sh[PG::GH + j * PF + col]) + from_bf16(sh[PG::GL + j * PF + col]);
        a1[r] = g * z;
        a2[r] = g * y[r];
      }
      gz += rsum16(a1, lane);
      gy += rsum16(a2, lane);
    }
    lds_barrier();  // before the next quarter's features
  }
  if (NORM) {
    if ((lane & 1) == 0) {
      const int j = 32 * jt + rsum16_row(lane);
      sf[PG::GZ + ft * PC + j] = gz;
      sf[PG::GY + ft * PC + j] = gy;
    }
    if (w < 3) {  // row sums of A (.) D and of A (.) D (.) X
      const int it = jobi(w), jtt = jobj(w), i = 32 * it + (lane & 31);
      f32x16 Am, AX;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = 32 * jtt + dtile_row(r, lane);
        Am[r] = i <= j ? A[r] * (DECAY ? sf[PG::DM + j - i] : 1.f) : 0.f;
        AX[r] = Am[r] * X[r];
      }
      const float sa = rsum16(Am, lane), sx = rsum16(AX, lane);
      if ((lane & 1) == 0) {
        const int j = 32 * jtt + rsum16_row(lane);
        sf[PG::AS + it * PC + j] = sa;
        sf[PG::AX + it * PC + j] = sx;
      }
    } else if (lane < 32) {  // the upper tile (0, 1) is zero
      sf[PG::AS + PC + lane] = 0.f;
      sf[PG::AX + PC + lane] = 0.f;
    }
    lds_barrier();
  }
  if (tid < PC) {  // per token: 1/den, dden and the adjoint record's weights
    const int j = tid;
    float inv = 1.f, dden = 0.f;
    if (NORM) {
      const float th = sf[PG::TH + j];
      const float den = sf[PG::AS + j] + sf[PG::AS + PC + j] + th * (sf[PG::GZ + j] + sf[PG::GZ + PC + j]) + p.eps;
      const float dn = sf[PG::AX + j] + sf[PG::AX + PC + j] + th * (sf[PG::GY + j] + sf[PG::GY + PC + j]);
      inv = j < L ? 1.f / den : 0.f;  // padded rows: no gradient flows (their den may be 0)
      dden = -dn * inv * inv;
      if (j < L) {
        float* tk2 = bp.tok + (size_t)(sq.row0 + (long long)(t0 + j) * p.tok_rows) * 2;
        tk2[0] = inv;
        tk2[1] = dden;
      }
    }
    sf[PG::IV + j] = inv;
    sf[PG::DD + j] = dden;
    sf[PG::WT + j] = sf[PG::TH + j];
    sf[PG::WI + j] = sf[PG::TH + j] * inv;
  }
  lds_barrier();
  // Bm = (X / den + dden) (.) D, columns past the step's end zero (waves 0..2)
  if (w < 3) {
    const int it = jobi(w), jtt = jobj(w), i = 32 * it + (lane & 31);
    f32x16 bm;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = 32 * jtt + dtile_row(r, lane);
      const float x = X[r] * sf[PG::IV + j] + sf[PG::DD + j];
      bm[r] = (i <= j && i < L) ? x * (DECAY ? sf[PG::DM + j - i] : 1.f) : 0.f;
    }
    store_sq(sh + PG::MH, sh + PG::ML, bm, jtt, it, lane);
  } else {  // wave 3: the upper tile (0, 1)
    const f32x16 z = zero16p();
    store_sq(sh + PG::MH, sh + PG::ML, z, 0, 1, lane);
  }

  // pass 2 over feature quarters: dG, the Jacobian weights a = dG g, dq += a W, the adjoint record
  f32x16 dqa[2] = {zero16p(), zero16p()};
  float cj = 0.f;
  const __amdgpu_buffer_rsrc_t rrs = make_rsrc(rrec, (uint32_t)(E * 4));
#pragma unroll 1
  for (int qi = 0; qi < NQT; ++qi) {
    const int lane = pin(lane0);
    lds_barrier();  // Bm complete; the previous quarter is done with G, F and the weights
    features_quarter(sh, sf, Wh, qi, w, lane);
    const f32x16 yq = y_tile(sh, pre, qi, jt, ft, lane);
    lds_barrier();
    // dG tile (jt, ft): A[m=j][k=i] = Bm (zero for i > j), B[k=i][n=p] = F[i][p]
    f32x16 dg = tile_mma<false, true, true, true, PC>(zero16p(), sh + PG::MH, PF, PG::ML - PG::MH, 32 * jt,
                                                      sh + PG::FH, PF, PG::FL - PG::FH, 32 * ft, lane);
    f32x16 aw;
    {
      const int col = 32 * ft + (lane & 31);
      const float z = sf[PG::ZQ + PQW * qi + col];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = 32 * jt + dtile_row(r, lane);
        const float d = dg[r] + sf[PG::TH + j] * (sf[PG::IV + j] * yq[r] + sf[PG::DD + j] * z);
        const float g = from_bf16(sh[PG::GH + j * PF + col]) + from_bf16(sh[PG::GL + j * PF + col]);
        aw[r] = d * g;
      }
      cj += rsum16(aw, lane);
    }
    lds_barrier();  // every wave is done with F
    store_sq(sh + PG::FH, sh + PG::FL, aw, jt, ft, lane);  // the weights take F's place
    // adjoint record of this quarter's features: [p][e] = sum_j (W_j inv_j G[j][p]) dout[j][e]
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int pt = jt, et = 2 * ft + u;  // feature tile pt of the quarter, value tile et
      f32x16 acc = zero16p();
#pragma unroll
      for (int k0 = 0; k0 < PC; k0 += 16) {
        const bf16x8 gh = ld_rows8(sh + PG::GH, PF, k0, 32 * pt, lane);  // A[m=p][k=j] = G[j][p]
        const bf16x8 gl = ld_rows8(sh + PG::GL, PF, k0, 32 * pt, lane);
        bf16x8 s_h, s_l;
        scale_split_prf(gh, gl, sf + PG::WI + k0 + 8 * (lane >> 5), s_h, s_l);
        const bf16x8 nh = ld_rows8(sh + PG::BH, PR, k0, 32 * et, lane);  // B[k=j][n=e] = dout[j][e]
        const bf16x8 nl = ld_rows8(sh + PG::BL, PR, k0, 32 * et, lane);
        acc = mfma32(s_h, nh, acc);
        acc = mfma32(s_h, nl, acc);
        acc = mfma32(s_l, nh, acc);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r)
        __builtin_amdgcn_raw_buffer_store_b32(
            __float_as_uint(acc[r]), rrs,
            (uint32_t)((PQW * qi + 32 * pt + dtile_row(r, lane)) * PD + 32 * et + (lane & 31)) * 4, 0, 0);
    }
    if (tid < PQW) {  // its normaliser part: sum_j W_j G[j][p] dden_j
      float rz = 0.f;
      if (NORM)
        for (int j = 0; j < L; ++j)
          rz += sf[PG::WT + j] * (from_bf16(sh[PG::GH + j * PF + tid]) + from_bf16(sh[PG::GL + j * PF + tid])) *
                sf[PG::DD + j];
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(rz), rrs, (uint32_t)(NP * PD + PQW * qi + tid) * 4, 0, 0);
    }
    lds_barrier();  // the weights are complete
    // dq tiles (jt, 2 ft + u) += a W: A[m=j][k=p] = a, B[k=p][n=d] = W^T[d][p]
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int dt = 2 * ft + u;
      const uint16_t* wr = Wt + (size_t)(32 * dt + (lane & 31)) * NP + PQW * qi + 8 * (lane >> 5);
#pragma unroll
      for (int k0 = 0; k0 < PQW; k0 += 16) {
        const bf16x8 wb = *(const bf16x8*)(wr + k0);
        dqa[u] = mfma32(ld_cols8(sh + PG::FH, PF, 32 * jt, k0, lane), wb, dqa[u]);
        dqa[u] = mfma32(ld_cols8(sh + PG::FL, PF, 32 * jt, k0, lane), wb, dqa[u]);
      }
    }
  }
  if ((lane & 1) == 0) sf[PG::CJ + ft * PC + 32 * jt + rsum16_row(lane)] = cj;
  lds_barrier();
  // dq = sum_p a_p w_p - (sum_p a_p) x, x = q (or the argmax row of the bank with the shift)
  const __amdgpu_buffer_rsrc_t rdq = make_rsrc(bp.dq + r0 * PD, rows_extent(L, rsb4, PD * 4));
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int d = 32 * (2 * ft + u) + (lane & 31);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = 32 * jt + dtile_row(r, lane);
      const float c = sf[PG::CJ + j] + sf[PG::CJ + PC + j];
      const float x = QS ? bf16_bits_to_f32(Wh[(size_t)((const int*)sf)[PG::QA + j] * PD + d])
                         : from_bf16(sh[PG::QR + j * PR + d]);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(dqa[u][r] - c * x), rdq, (uint32_t)j * rsb4 + d * 4, 0, 0);
    }
  }
}

// ---- key kernel --------------------------------------------------------------------------

template <int NP, bool DECAY, bool NORM, bool DBF, bool QS>
__global__ __launch_bounds__(PNT) void k_bwd_prf_key(BackwardParams bp) {
  const PrefillParams& p = bp.f;
  constexpr int NQT = NP / PQW;
  extern __shared__ __align__(16) unsigned char smem[];
  __bf16* sh = (__bf16*)smem;
  float* sf = (float*)smem;
  const int bh = blockIdx.x, seg = blockIdx.y, tid = threadIdx.x, lane0 = tid & 63, w = tid >> 6;
  const int head = bh % p.H;
  int lane = lane0;
  const SeqSpan sq = seq_span(p, bh);
  const int t0 = seg * PC, L = max(0, min(PC, sq.T - t0));
  if (L == 0) return;
  const size_t E = (size_t)NP * PD + NP;
  const float* rpre = bp.rev + ((size_t)bh * p.n_seg + seg) * E;  // R_> [p][e], RZ_> [p]
  const float lg = DECAY ? p.log2g[head] : 0.f;
  const float log2_rsqrt = -0.5f * __log2f((float)NP);
  const uint16_t* Wh = (const uint16_t*)p.prf_w + (size_t)head * NP * PD;
  const uint16_t* Wt = bp.wt + (size_t)head * NP * PD;
  const long long r0 = sq.row0 + (long long)t0 * p.tok_rows;
  const uint32_t rsb = (uint32_t)p.tok_rows * PD * 2, rsb4 = (uint32_t)p.tok_rows * PD * 4;
  const uint32_t rsbd = (uint32_t)p.tok_rows * PD * (DBF ? 2 : 4);
  const int jt = w >> 1, ft = w & 1;

  {
    Raw tq, tk, tv;
    load_raw(tq, (const uint16_t*)p.q + r0 * PD, L, rsb);
    load_raw(tk, (const uint16_t*)p.k + r0 * PD, L, rsb);
    load_raw(tv, (const uint16_t*)p.v + r0 * PD, L, rsb);
    commit_raw_rows(tq, sh + PG::QR, sf + PG::NQ);
    commit_raw_rows(tk, sh + PG::KR, sf + PG::NK);
    commit_raw_rows(tv, sh + PG::VR, nullptr);
  }
  if (tid < PC) {
    const int j = tid;
    float inv = 1.f, dden = 0.f;
    if (NORM && j < L) {
      const float* tk2 = bp.tok + (size_t)(sq.row0 + (long long)(t0 + j) * p.tok_rows) * 2;
      inv = tk2[0];
      dden = tk2[1];
    }
    sf[PG::IV + j] = (NORM && j >= L) ? 0.f : inv;
    sf[PG::DD + j] = dden;
  }
  lds_barrier();
  // dNum = dout / den as hi + lo
  commit_dout<DBF>((const unsigned char*)bp.dout + r0 * PD * (DBF ? 2 : 4), L, rsbd, sf + PG::IV, sh + PG::BH,
                   sh + PG::BL);
  step_tables<DECAY>(sf, L, lg, log2_rsqrt, QS);
  if (QS) query_shift<NP>(sf, sh, Wh, log2_rsqrt, w, lane);
  lds_barrier();

  // pass 1 over feature quarters: A = G F^T (waves 0..2)
  f32x16 A = zero16p();
#pragma unroll 1
  for (int qi = 0; qi < NQT; ++qi) {
    const int lane = pin(lane0);
    features_quarter(sh, sf, Wh, qi, w, lane);
    lds_barrier();
    if (w < 3)
      A = tile_mma<false, true, false, true, PQW>(A, sh + PG::GH, PF, PG::GL - PG::GH, 32 * jobj(w), sh + PG::FH, PF,
                                                  PG::FL - PG::FH, 32 * jobi(w), lane);
    lds_barrier();
  }
  // A (.) D into the G image; Bm' = (dNum V^T + dden) (.) D (waves 0..2)
  if (w < 3) {
    const int it = jobi(w), jtt = jobj(w), i = 32 * it + (lane & 31);
    const f32x16 X = tile_mma<false, true, false, false, PD>(zero16p(), sh + PG::BH, PR, PG::BL - PG::BH, 32 * jtt,
                                                             sh + PG::VR, PR, 0, 32 * it, lane);
    f32x16 am, bm;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = 32 * jtt + dtile_row(r, lane);
      const float dm = i <= j ? (DECAY ? sf[PG::DM + j - i] : 1.f) : 0.f;
      am[r] = A[r] * dm;
      bm[r] = i < L ? (X[r] + sf[PG::DD + j]) * dm : 0.f;
    }
    store_sq(sh + PG::GH, sh + PG::GL, am, jtt, it, lane);
    store_sq(sh + PG::MH, sh + PG::ML, bm, jtt, it, lane);
  } else {  // wave 3: the upper tiles (0, 1)
    const f32x16 z = zero16p();
    store_sq(sh + PG::GH, sh + PG::GL, z, 0, 1, lane);
    store_sq(sh + PG::MH, sh + PG::ML, z, 0, 1, lane);
  }
  lds_barrier();
  // dV tiles (it = jt, value tiles 2 ft + u): A^T dNum, A[m=i][k=j] = A[j][i] (zero for j < i), B[k=j][n=e] = dNum
  f32x16 dva[2], dvf[2] = {zero16p(), zero16p()};
#pragma unroll
  for (int u = 0; u < 2; ++u)
    dva[u] = tile_mma<true, true, true, true, PC>(zero16p(), sh + PG::GH, PF, PG::GL - PG::GH, 32 * jt, sh + PG::BH,
                                                  PR, PG::BL - PG::BH, 32 * (2 * ft + u), lane);
  lds_barrier();  // dNum and A are dead: R_> quarters take dNum's place

  f32x16 dka[2] = {zero16p(), zero16p()};
  float ci = 0.f;
#pragma unroll 1
  for (int qi = 0; qi < NQT; ++qi) {
    const int lane = pin(lane0);
    // R_> rows of this quarter's features as hi + lo (pitch PR), RZ_> of them
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int idx = tid + PNT * i, row = idx >> 5, col = 4 * (idx & 31);
      const f32x4 x = *(const f32x4*)(rpre + (size_t)(PQW * qi + row) * PD + col);
      bf16x4 h, l;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bf16_pair pr = split_bf16(x[e]);
        h[e] = pr.hi;
        l[e] = pr.lo;
      }
      *(bf16x4*)(sh + PG::BH + row * PR + col) = h;
      *(bf16x4*)(sh + PG::BL + row * PR + col) = l;
    }
    if (tid < PQW) sf[PG::ZQ + tid] = NORM ? rpre[(size_t)NP * PD + PQW * qi + tid] : 0.f;
    features_quarter(sh, sf, Wh, qi, w, lane);
    lds_barrier();
    // dF tile (it = jt, ft): Bm'^T G (Bm' zero for j < i) + xi (V R_>^T + RZ_>)
    const int it = jt;
    f32x16 d1 = tile_mma<true, true, true, true, PC>(zero16p(), sh + PG::MH, PF, PG::ML - PG::MH, 32 * it,
                                                     sh + PG::GH, PF, PG::GL - PG::GH, 32 * ft, lane);
    f32x16 d2 = tile_mma<false, false, false, true, PD>(zero16p(), sh + PG::VR, PR, 0, 32 * it, sh + PG::BH, PR,
                                                        PG::BL - PG::BH, 32 * ft, lane);
    f32x16 aw;
    {
      const int col = 32 * ft + (lane & 31);
      const float rz = sf[PG::ZQ + col];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = 32 * it + dtile_row(r, lane);
        const float d = d1[r] + sf[PG::XI + i] * (d2[r] + rz);
        const float f = from_bf16(sh[PG::FH + i * PF + col]) + from_bf16(sh[PG::FL + i * PF + col]);
        aw[r] = d * f;
      }
      ci += rsum16(aw, lane);
    }
    // dV tiles += F R_> over this quarter's features: A[m=i][k=p] = F, B[k=p][n=e] = R_>[p][e]
#pragma unroll
    for (int u = 0; u < 2; ++u)
      dvf[u] = tile_mma<false, true, true, true, PQW>(dvf[u], sh + PG::FH, PF, PG::FL - PG::FH, 32 * it, sh + PG::BH,
                                                      PR, PG::BL - PG::BH, 32 * (2 * ft + u), lane);
    lds_barrier();  // every wave is done with G (and F, R_>)
    store_sq(sh + PG::GH, sh + PG::GL, aw, it, ft, lane);  // the weights take G's place
    lds_barrier();
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int dt = 2 * ft + u;
      const uint16_t* wr = Wt + (size_t)(32 * dt + (lane & 31)) * NP + PQW * qi + 8 * (lane >> 5);
#pragma unroll
      for (int k0 = 0; k0 < PQW; k0 += 16) {
        const bf16x8 wb = *(const bf16x8*)(wr + k0);
        dka[u] = mfma32(ld_cols8(sh + PG::GH, PF, 32 * it, k0, lane), wb, dka[u]);
        dka[u] = mfma32(ld_cols8(sh + PG::GL, PF, 32 * it, k0, lane), wb, dka[u]);
      }
    }
    lds_barrier();  // before the next quarter overwrites R_>, G and F
  }
  if ((lane & 1) == 0) sf[PG::CJ + ft * PC + 32 * jt + rsum16_row(lane)] = ci;
  lds_barrier();
  const __amdgpu_buffer_rsrc_t rdk = make_rsrc(bp.dk + r0 * PD, rows_extent(L, rsb4, PD * 4));
  const __amdgpu_buffer_rsrc_t rdv = make_rsrc(bp.dv + r0 * PD, rows_extent(L, rsb4, PD * 4));
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int d = 32 * (2 * ft + u) + (lane & 31);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = 32 * jt + dtile_row(r, lane);
      const float c = sf[PG::CJ + i] + sf[PG::CJ + PC + i];
      const float dkv = dka[u][r] - c * from_bf16(sh[PG::KR + i * PR + d]);  // keys take no shift
      const float dvv = dva[u][r] + sf[PG::XI + i] * dvf[u][r];
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(dkv), rdk, (uint32_t)i * rsb4 + d * 4, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(dvv), rdv, (uint32_t)i * rsb4 + d * 4, 0, 0);
    }
  }
}

// The bank transposed per head, [H][d][n_psi] bf16: the Jacobians contract over features, so
// their operand reads are 16-byte rows of this copy.
__global__ __launch_bounds__(256) void k_bank_transpose(const uint16_t* __restrict__ w, uint16_t* __restrict__ wt,
                                                        int np) {
  // one 32 x 32 tile per workgroup, through LDS, so that both the reads and the writes are rows
  __shared__ uint16_t t[32][34];
  constexpr int NTD = PD / 32;
  const int h = blockIdx.x, p0 = (blockIdx.y / NTD) * 32, d0 = (blockIdx.y % NTD) * 32;
  const uint16_t* src = w + (size_t)h * np * PD;
  uint16_t* dst = wt + (size_t)h * np * PD;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int r = ty; r < 32; r += 8) t[r][tx] = src[(size_t)(p0 + r) * PD + d0 + tx];
  __syncthreads();
  for (int r = ty; r < 32; r += 8) dst[(size_t)(d0 + r) * np + p0 + tx] = t[tx][r];
}

template <int NP, bool DECAY, bool NORM, bool DBF, bool QS>
hipError_t launch_k(const BackwardParams& bp, hipStream_t s, bool key) {
  const void* kern = key ? (const void*)k_bwd_prf_key<NP, DECAY, NORM, DBF, QS>
                         : (const void*)k_bwd_prf_query<NP, DECAY, NORM, DBF, QS>;
  hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, PG::BYTES);
  if (e != hipSuccess) return e;
  dim3 grid(bp.f.B * bp.f.H, bp.f.n_seg);
  void* args[] = {(void*)&bp};
  e = hipLaunchKernel(kern, grid, dim3(PNT), args, PG::BYTES, s);
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

template <int NP>
hipError_t launch_np_b(const BackwardParams& bp, hipStream_t s, bool key) {
  const bool decay = bp.f.has_decay != 0, norm = bp.f.normalize != 0, dbf = bp.dout_bf16 != 0;
  const bool qs = bp.f.psi == LA_PSI_PRF_QSHIFT;
  // the query-row shift comes with a denominator (it is refused without one)
  if (qs) {
    if (decay) return dbf ? launch_k<NP, true, true, true, true>(bp, s, key) : launch_k<NP, true, true, false, true>(bp, s, key);
    return dbf ? launch_k<NP, false, true, true, true>(bp, s, key) : launch_k<NP, false, true, false, true>(bp, s, key);
  }
  if (decay) {
    if (norm) return dbf ? launch_k<NP, true, true, true, false>(bp, s, key) : launch_k<NP, true, true, false, false>(bp, s, key);
    return dbf ? launch_k<NP, true, false, true, false>(bp, s, key) : launch_k<NP, true, false, false, false>(bp, s, key);
  }
  if (norm) return dbf ? launch_k<NP, false, true, true, false>(bp, s, key) : launch_k<NP, false, true, false, false>(bp, s, key);
  return dbf ? launch_k<NP, false, false, true, false>(bp, s, key) : launch_k<NP, false, false, false, false>(bp, s, key);
}

}  // namespace

bool prefill_backward_prf_supported(int C, int d_k, int d_v, int n_psi) {
  return d_k == PD && d_v == PD && (n_psi == 128 || n_psi == 256) && (C == 32 || C == 64 || C == 128);
}

hipError_t launch_bank_transpose(const void* w, uint16_t* wt, int H, int n_psi, hipStream_t s) {
  if (n_psi % 32 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_bank_transpose, dim3(H, (n_psi / 32) * (PD / 32)), dim3(256), 0, s, (const uint16_t*)w, wt,
                     n_psi);
  return hipGetLastError();
}

hipError_t launch_prefill_backward_prf(const BackwardParams& bp, hipStream_t s, bool key_sweep) {
  if (bp.f.n_psi == 256) return launch_np_b<256>(bp, s, key_sweep);
  if (bp.f.n_psi == 128) return launch_np_b<128>(bp, s, key_sweep);
  return hipErrorInvalidValue;
}

}  // namespace la
