// la_backward.hip -- backward pass of the chunked prefill: the gradients of
// L = sum_t dout_t . o_t with respect to q, k, v (and, through the scan, the initial state).
//
// Two sweeps, as in "Linearized 2-Simplicial Attention" (4.2 Custom Triton kernel, Backward;
// appendix "Backward query sweep" and "Backward state sweep"): a query sweep that recomputes
// the prefix state and produces dq, and a state sweep that produces the key and value
// gradients from the adjoint state. With g_t = psi(q_t), f_t = psi(k_t) and the read
// o_t = g_t^T S_t / (g_t . Z_t + eps) of the inclusive state ("Log-Depth Chunked
// Linear-Attention Scan", Mathematical statement), the chain rule gives
//   dnum_t = dout_t / den_t,  dden_t = -(dout_t . num_t) / den_t^2   (normalize = 0: dout_t, 0)
//   dg_t   = S_t dnum_t + Z_t dden_t
//   R_t    = sum_{u >= t} gamma^(u-t) g_u dnum_u^T,  RZ_t likewise with dden_u  (adjoint state)
//   df_t   = R_t v_t + RZ_t,  dv_t = R_t^T f_t.
// Per step of BC tokens (j, i inside the step; theta_j = gamma^(j+1), xi_i = gamma^(L-1-i),
// D_ji = gamma^(j-i) [i <= j]; the chunk algebra of the same page's Implementation notes and of
// "Linear Attention and Retentive Networks", Retentive Networks, representation C):
//   Bm  = (dNum V^T + dden 1^T) (.) D                       C x C
//   dG  = Bm F + theta (.) (dNum S_<^T + dden Z_<^T)        query sweep; S_< the state before the step
//   A   = (G F^T) (.) D
//   dV  = A^T dNum + xi (.) (F R_>)                         state sweep; R_> the adjoint after the step
//   dF  = Bm^T G + xi (.) (V R_>^T + RZ_>)
//   R_> of the previous step = gamma^L R_> + (theta (.) G)^T dNum
// The query sweep recomputes dout_t . num_t from the same tiles (X = dout V^T, Y = dout S_<^T):
//   dout_j . num_j = sum_i A_ji X_ji + theta_j g_j . Y_j,  den_j = sum_i A_ji + theta_j g_j . Z_< + eps,
// so only the inputs are needed (no saved output), and dden does not inherit the rounding of a
// stored o: the terms S dnum and Z dden nearly cancel for a normalised average, which would
// amplify it. Segments: the query sweep starts from the forward scan's prefix and accumulates
// each segment's adjoint summary sum_t gamma^(t - start + 1) g_t dnum_t^T; the segment scan
// run in reverse order turns those into the adjoint state after each segment.
//
// Both kernels: one workgroup of eight waves per (sequence, segment), split into two
// groups of four with different roles (see each kernel), d_k = d_v = n_psi = 128, bf16
// operands on MFMA 32x32x16 with fp32 accumulation; every operand that is not
// exact in bf16 (the states, scaled features, dNum, the C x C tiles, elu+1 keys) is a
// two-term hi + lo expansion (psi(q) included, unlike the forward output pass: the adjoint
// state sums psi(q) against signed upstream gradients without averaging the rounding out).
// Wave w of a group owns the 32 columns [32w, 32w + 32) of the outputs that group produces.
#include "la_device.hpp"
#include "la_kernels.hpp"

namespace la {
namespace {

constexpr int BC = 64;    // tokens per step
constexpr int BD = 128;   // d_k = d_v = n_psi
constexpr int TP = BD + 8;  // pitch (elements) of the C x D bf16 tiles
constexpr int SQ = BC + 8;  // pitch of the C x C bf16 tiles

// LDS image (bf16 element offsets, then float tables).
struct BG {
  static constexpr int TILE = BC * TP, STILE = BC * SQ;
  static constexpr int QH = 0, QL = TILE, KH = 2 * TILE, KL = 3 * TILE, V = 4 * TILE, NH = 5 * TILE, NL = 6 * TILE;
  static constexpr int AH = 7 * TILE, AL = AH + STILE, BH = AL + STILE, BL = BH + STILE;
  static constexpr int HALVES = BL + STILE;
  static constexpr int F0 = HALVES / 2;      // first float
  static constexpr int TH = F0, XI = TH + BC, DD = XI + BC, IV = DD + BC, WT = IV + BC, ZV = WT + BC;
  static constexpr int DM = ZV + BD;  // gamma^n, n = 0..BC-1 (the causal decay mask by lag)
  static constexpr int FEND = DM + BC;
  static constexpr int BYTES = FEND * 4;
};
static_assert(BG::HALVES % 8 == 0, "float tables 16-byte aligned");
static_assert(BG::BYTES <= 160 * 1024, "LDS image fits a CU");
// the query sweep's row partials (8 x BC floats) sit in the AH region, unused there
static_assert(9 * BC * 2 <= BG::STILE, "row partials and weights fit one bf16 C x C tile");

// ---- global tiles ----------------------------------------------------------------------

// A step of BC token rows x BD bf16 over NT threads: BC*BD/8/NT pieces of 8 elements per
// thread (row t/16 + (NT/16) i).
template <int NT>
struct Tile16 {
  static constexpr int N = BC * BD / 8 / NT;
  uint4 r[N];
};
template <int NT>
__device__ __forceinline__ void load_tile16(Tile16<NT>& P, const void* base, int valid, uint32_t rsb) {
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, rows_extent(valid, rsb, BD * 2));
  const int t = threadIdx.x;
  const uint32_t v0 = (uint32_t)(t >> 4) * rsb + (uint32_t)(t & 15) * 16;
#pragma unroll
  for (int i = 0; i < Tile16<NT>::N; ++i) P.r[i] = buf_load16(rs, v0, (uint32_t)((NT / 16) * i) * rsb);
}
template <int NT>
__device__ __forceinline__ int t16_row(int i) { return (threadIdx.x >> 4) + (NT / 16) * i; }
__device__ __forceinline__ int t16_col() { return (threadIdx.x & 15) * 8; }

// A step of BC token rows x BD fp32 (or bf16) values over NT threads: TPT = NT / BC threads per
// token; thread t holds token t / TPT, columns 4 (t % TPT) + 4 TPT i + 0..3.
template <int NT>
struct TileF {
  static constexpr int TPT = NT / BC, N = BD / (4 * TPT);
  f32x4 r[N];
};
template <int NT, bool BF>
__device__ __forceinline__ void load_tileF(TileF<NT>& P, const void* base, int valid, uint32_t rsb) {
  constexpr int ES = BF ? 2 : 4, TPT = TileF<NT>::TPT;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, rows_extent(valid, rsb, BD * ES));
  const int t = threadIdx.x;
  const uint32_t v0 = (uint32_t)(t / TPT) * rsb + (uint32_t)(4 * (t % TPT)) * ES;
#pragma unroll
  for (int i = 0; i < TileF<NT>::N; ++i) {
    if (BF) {
      const u32x2 w = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, v0, 4 * TPT * i * ES, 0));
      P.r[i] = f32x4{__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u), __uint_as_float(w[1] << 16),
                     __uint_as_float(w[1] & 0xffff0000u)};
    } else {
      P.r[i] = __builtin_bit_cast(f32x4, buf_load16(rs, v0, 4 * TPT * i * ES));
    }
  }
}
template <int NT>
__device__ __forceinline__ int tf_tok() { return threadIdx.x / TileF<NT>::TPT; }
template <int NT>
__device__ __forceinline__ int tf_col(int i) { return 4 * (threadIdx.x % TileF<NT>::TPT) + 4 * TileF<NT>::TPT * i; }

// Sum over the threads of a token (TPT adjacent lanes of one wave).
template <int NT>
__device__ __forceinline__ float token_sum(float x) {
#pragma unroll
  for (int o = 1; o < TileF<NT>::TPT; o <<= 1) x += __shfl_xor(x, o);
  return x;
}

// ---- commits ---------------------------------------------------------------------------

// psi(x) of a bf16 tile to LDS as hi (+ lo when LO): rows >= L are zero (padded positions
// are the monoid identity). ELU: elu+1.
template <int NT, bool ELU, bool LO>
__device__ __forceinline__ void commit_feat(const Tile16<NT>& P, __bf16* hi, __bf16* lo, int L) {
#pragma unroll
  for (int i = 0; i < Tile16<NT>::N; ++i) {
    const int row = t16_row<NT>(i), col = t16_col();
    const bf16x8 x = __builtin_bit_cast(bf16x8, P.r[i]);
    bf16x8 h, l;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float xf = from_bf16(x[j]);
      const float f = row < L ? (ELU ? elu1(xf) : xf) : 0.f;
      const bf16_pair pr = split_bf16(f);
      h[j] = pr.hi;
      l[j] = pr.lo;
    }
    *(bf16x8*)(hi + row * TP + col) = h;
    if (LO) *(bf16x8*)(lo + row * TP + col) = l;
  }
}

template <int NT>
__device__ __forceinline__ void commit_raw(const Tile16<NT>& P, __bf16* dst) {
#pragma unroll
  for (int i = 0; i < Tile16<NT>::N; ++i) *(uint4*)(dst + t16_row<NT>(i) * TP + t16_col()) = P.r[i];
}

// s * x (x from a TileF, s the token's scale) as hi + lo.
template <int NT>
__device__ __forceinline__ void commit_scaled(const TileF<NT>& P, float s, __bf16* hi, __bf16* lo) {
  const int j = tf_tok<NT>();
#pragma unroll
  for (int i = 0; i < TileF<NT>::N; ++i) {
    const int col = tf_col<NT>(i);
    bf16x4 h, l;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bf16_pair pr = split_bf16(s * P.r[i][e]);
      h[e] = pr.hi;
      l[e] = pr.lo;
    }
    *(bf16x4*)(hi + j * TP + col) = h;
    *(bf16x4*)(lo + j * TP + col) = l;
  }
}

// ---- helpers ---------------------------------------------------------------------------

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int r = 0; r < 16; ++r) z[r] = 0.f;
  return z;
}

// (hi + lo) * f per element, 8 values, re-split as hi + lo (LO false: lo ignored).
template <bool LO>
__device__ __forceinline__ void scale_split(const bf16x8& xh, const bf16x8& xl, const float* f, bf16x8& hi,
                                            bf16x8& lo) {
  float y[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) y[j] = (from_bf16(xh[j]) + (LO ? from_bf16(xl[j]) : 0.f)) * f[j];
  split8_trunc(y, hi, lo);
}

// Registers 8q..8q+7 of a D-tile (rows in the feedback order of k-half q) as hi + lo operands.
__device__ __forceinline__ void split_dtile(const f32x16& D, bf16x8 (&hi)[2], bf16x8 (&lo)[2]) {
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = D[8 * q + j];
    split8_trunc(x, hi[q], lo[q]);
  }
}

// Row sums of a D-tile over its 32 columns (the 32 lanes of each half-wave), by recursive
// halving (16 exchanges): lane l ends with the sum of row dtile_row((l >> 1) & 15, l).
__device__ __forceinline__ float rowsum16(const f32x16& v, int lane) {
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
__device__ __forceinline__ int rowsum16_row(int lane) { return dtile_row((lane >> 1) & 15, lane); }

// The causal decay mask D_ji (0 above the diagonal), gamma^(j-i) read from the step's table:
// read from LDS rather than recomputed, so the compiler cannot hoist one live value per
// element out of the step loop.
template <bool DECAY>
__device__ __forceinline__ float dmask(int j, int i, const float* sf) {
  return i <= j ? (DECAY ? sf[BG::DM + j - i] : 1.f) : 0.f;
}

// Tile (jt, it) of the lower block triangle of a C x C matrix: job 0 -> (0,0), 1 -> (1,0), 2 -> (1,1).
__device__ __forceinline__ int job_jt(int job) { return job == 0 ? 0 : 1; }
__device__ __forceinline__ int job_it(int job) { return job == 2 ? 1 : 0; }

// A = G F^T tile (jt, it), unmasked: G and F as hi + lo (lo only for elu+1).
template <bool ELU>
__device__ __forceinline__ f32x16 a_tile_acc(const __bf16* sh, int jt, int it, int lane) {
  f32x16 acc = zero16();
#pragma unroll 2
  for (int k0 = 0; k0 < BD; k0 += 16) {
    const bf16x8 gh = ld_cols8(sh + BG::QH, TP, 32 * jt, k0, lane);  // A[m=j][k=p] = G[j][p]
    const bf16x8 fh = ld_cols8(sh + BG::KH, TP, 32 * it, k0, lane);  // B[k=p][n=i] = F[i][p]
    acc = mfma32(gh, fh, acc);
    if (ELU) {
      acc = mfma32(gh, ld_cols8(sh + BG::KL, TP, 32 * it, k0, lane), acc);
      acc = mfma32(ld_cols8(sh + BG::QL, TP, 32 * jt, k0, lane), fh, acc);
    }
  }
  return acc;
}

// X = N V^T tile (jt, it), N = the hi + lo tile in NH/NL (unmasked).
__device__ __forceinline__ f32x16 x_tile_acc(const __bf16* sh, int jt, int it, int lane) {
  f32x16 acc = zero16();
#pragma unroll 2
  for (int k0 = 0; k0 < BD; k0 += 16) {
    const bf16x8 b = ld_cols8(sh + BG::V, TP, 32 * it, k0, lane);  // B[k=e][n=i] = V[i][e]
    acc = mfma32(ld_cols8(sh + BG::NH, TP, 32 * jt, k0, lane), b, acc);
    acc = mfma32(ld_cols8(sh + BG::NL, TP, 32 * jt, k0, lane), b, acc);
  }
  return acc;
}

// Bm tile (jt, it) = (X inv_j + dden_j) (.) D, split hi + lo into LDS. INV: X was formed
// from dout (query sweep) and takes inv_j here; otherwise from dNum (state sweep).
template <bool DECAY, bool NORM, bool INV>
__device__ __forceinline__ void store_bm(__bf16* sh, const float* sf, const f32x16& X, int jt, int it, int L,
                                         float lg, int lane) {
  const int i = 32 * it + (lane & 31);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int j = 32 * jt + dtile_row(r, lane);
    const float x = NORM ? (INV ? X[r] * sf[BG::IV + j] : X[r]) + sf[BG::DD + j] : X[r];
    const bf16_pair pr = split_bf16(i < L ? x * dmask<DECAY>(j, i, sf) : 0.f);
    sh[BG::BH + j * SQ + i] = pr.hi;
    sh[BG::BL + j * SQ + i] = pr.lo;
  }
}

// psi'(x) from psi(x) for elu+1: 1 where x > 0 (psi > 1), exp(x) = psi where x <= 0.
__device__ __forceinline__ float dpsi_from_feat(float f) { return fminf(f, 1.f); }

// ---- query sweep -----------------------------------------------------------------------

// Eight waves, specialised like the state sweep's: waves 0..3 hold S_<^T (feature columns
// 32 cw..) and produce Y = dout S_<^T, dG and the state update; waves 4..7 hold the segment's
// adjoint summary (value columns 32 cw..) and produce the X = dout V^T and A tiles, Bm and the
// summary's update.
constexpr int QNT = 512;

template <bool ELU, bool DECAY, bool NORM, bool DBF>
__global__ __launch_bounds__(QNT) void k_bwd_query(BackwardParams bp) {
  const PrefillParams& p = bp.f;
  extern __shared__ __align__(16) unsigned char smem[];
  __bf16* sh = (__bf16*)smem;
  float* sf = (float*)smem;
  float* part = sf + BG::AH / 2;  // row partials: A sums [2][BC], A.X sums [2][BC], g.Y sums [4][BC]
  float* wi = part + 8 * BC;      // W_j / den_j, the adjoint summary's token weights
  const int bh = blockIdx.x, seg = blockIdx.y, tid = threadIdx.x, lane0 = tid & 63, w = tid >> 6;
  const int role = w >> 2, cw = w & 3;
  const SeqSpan sq = seq_span(p, bh);
  const int T = sq.T;
  const int seg_tok = p.seg_chunks * p.C;
  const int tb = seg * seg_tok, te = min(tb + seg_tok, T);
  const size_t E = (size_t)BD * BD + BD;
  float* rrec = bp.rev + ((size_t)bh * p.n_seg + seg) * E;
  const int col0 = 32 * cw + (lane0 & 31);
  // role 0: St[t] = S_<^T[e][p], rows e in tile t, column p = col
  // role 1: St[t] = adjoint summary [p][e], rows p in tile t, column e = col
  f32x16 St[4];
  const float* pre = p.ws + ((size_t)bh * p.n_seg + seg) * E;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) St[t][r] = role == 0 && tb < te ? pre[(size_t)col0 * BD + 32 * t + dtile_row(r, lane0)] : 0.f;
  const int zp = tid - QNT / 2;                                          // role-1 thread zp < BD: RZ[zp]
  float zreg = (NORM && tid < BD && tb < te) ? pre[(size_t)BD * BD + tid] : 0.f;  // role-0 thread p: Z_<[p]
  float rz = 0.f;
  if (tb < te) {
    const float lg = DECAY ? p.log2g[bh % p.H] : 0.f;
    const uint32_t rsb = (uint32_t)p.tok_rows * BD * 2, rsb4 = (uint32_t)p.tok_rows * BD * 4;
    const uint32_t rsbd = (uint32_t)p.tok_rows * BD * (DBF ? 2 : 4);

    for (int t0 = tb; t0 < te; t0 += BC) {
      // the lane index, opaque once per step (see the state sweep)
      const int lane = pin(lane0), col = 32 * cw + (lane & 31);
      const int L = min(BC, te - t0);
      const long long r0 = sq.row0 + (long long)t0 * p.tok_rows;
      Tile16<QNT> tq, tk, tv;
      load_tile16<QNT>(tq, (const uint16_t*)p.q + r0 * BD, L, rsb);
      load_tile16<QNT>(tk, (const uint16_t*)p.k + r0 * BD, L, rsb);
      load_tile16<QNT>(tv, (const uint16_t*)p.v + r0 * BD, L, rsb);
      TileF<QNT> tdo;
      load_tileF<QNT, DBF>(tdo, (const unsigned char*)bp.dout + r0 * BD * (DBF ? 2 : 4), L, rsbd);
      lds_barrier();  // the previous step is done with LDS
      commit_feat<QNT, ELU, ELU>(tq, sh + BG::QH, sh + BG::QL, L);
      commit_feat<QNT, ELU, ELU>(tk, sh + BG::KH, sh + BG::KL, L);
      commit_raw<QNT>(tv, sh + BG::V);
      commit_scaled<QNT>(tdo, 1.f, sh + BG::NH, sh + BG::NL);  // dout as hi + lo
      if (tid < BC) {
        const int j = tid;
        sf[BG::TH + j] = DECAY ? exp2f((float)(j + 1) * lg) : 1.f;
        sf[BG::XI + j] = j < L ? (DECAY ? exp2f((float)(L - 1 - j) * lg) : 1.f) : 0.f;
        sf[BG::WT + j] = DECAY ? exp2f((float)(t0 - tb + j + 1) * lg) : 1.f;
        sf[BG::DM + j] = DECAY ? exp2f((float)j * lg) : 1.f;
        if (!NORM) {
          sf[BG::IV + j] = 1.f;
          sf[BG::DD + j] = 0.f;
          wi[j] = sf[BG::WT + j];
        }
      }
      if (NORM && tid < BD) sf[BG::ZV + tid] = zreg;
      lds_barrier();

      f32x16 X = zero16();  // role 1, cw < 3: the X = dout V^T tile of the lower block triangle
      f32x16 Y[2];          // role 0: Y = dout S_<^T, rows j, column p = col
      if (role == 1) {
        if (cw < 3) {
          const int jt = job_jt(cw), it = job_it(cw);
          X = x_tile_acc(sh, jt, it, lane);
          if (NORM) {  // A = G F^T and the row partials sum_i A_ji, sum_i A_ji X_ji
            const f32x16 A = a_tile_acc<ELU>(sh, jt, it, lane);
            f32x16 Am, AX;
            const int i = 32 * it + (lane & 31);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              Am[r] = A[r] * dmask<DECAY>(32 * jt + dtile_row(r, lane), i, sf);
              AX[r] = Am[r] * X[r];
            }
            const float sa = rowsum16(Am, lane), sx = rowsum16(AX, lane);
            if ((lane & 1) == 0) {
              const int j = 32 * jt + rowsum16_row(lane);
              part[it * BC + j] = sa;
              part[2 * BC + it * BC + j] = sx;
            }
          }
        } else if (NORM && lane < 32) {  // the upper tile (0, 1) is zero
          part[BC + lane] = 0.f;
          part[3 * BC + lane] = 0.f;
        }
      } else {
        Y[0] = zero16();
        Y[1] = zero16();
#pragma unroll
        for (int et = 0; et < 4; ++et) {
          bf16x8 sth[2], stl[2];
          split_dtile(St[et], sth, stl);
#pragma unroll
          for (int qq = 0; qq < 2; ++qq)
#pragma unroll
            for (int jt = 0; jt < 2; ++jt) {
              const bf16x8 nh = ld_cols8_perm(sh + BG::NH, TP, 32 * jt, 32 * et, qq, lane);
              const bf16x8 nl = ld_cols8_perm(sh + BG::NL, TP, 32 * jt, 32 * et, qq, lane);
              Y[jt] = mfma32(nh, sth[qq], Y[jt]);
              Y[jt] = mfma32(nh, stl[qq], Y[jt]);
              Y[jt] = mfma32(nl, sth[qq], Y[jt]);
            }
          __builtin_amdgcn_sched_barrier(0);
        }
        if (NORM) {  // row partials of g_j . Y_j over this wave's 32 features
#pragma unroll
          for (int jt = 0; jt < 2; ++jt) {
            f32x16 gy;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int j = 32 * jt + dtile_row(r, lane);
              const float g = from_bf16(sh[BG::QH + j * TP + col]) + (ELU ? from_bf16(sh[BG::QL + j * TP + col]) : 0.f);
              gy[r] = g * Y[jt][r];
            }
            const float sy = rowsum16(gy, lane);
            if ((lane & 1) == 0) part[(4 + cw) * BC + 32 * jt + rowsum16_row(lane)] = sy;
          }
        }
      }
      if (NORM) {
        lds_barrier();
        // per token: den, dout . num, 1/den and dden = -(dout . num) / den^2
        constexpr int TPT = TileF<QNT>::TPT, FW = BD / TPT;
        const int j = tf_tok<QNT>(), qq = tid % TPT;
        float zs = 0.f;
        for (int pp = FW * qq; pp < FW * qq + FW; ++pp) {
          const float g = from_bf16(sh[BG::QH + j * TP + pp]) + (ELU ? from_bf16(sh[BG::QL + j * TP + pp]) : 0.f);
          zs += g * sf[BG::ZV + pp];
        }
        zs = token_sum<QNT>(zs);
        if (qq == 0) {
          const float th = sf[BG::TH + j];
          const float den = part[j] + part[BC + j] + th * zs + p.eps;
          const float dn = part[2 * BC + j] + part[3 * BC + j] +
                           th * (part[4 * BC + j] + part[5 * BC + j] + part[6 * BC + j] + part[7 * BC + j]);
          // padded rows: dnum = dden = 0 (their den may be 0 when eps is)
          const float inv = j < L ? 1.f / den : 0.f;
          const float dden = -dn * inv * inv;
          sf[BG::IV + j] = inv;
          sf[BG::DD + j] = dden;
          wi[j] = sf[BG::WT + j] * inv;
          if (j < L) {
            float* tk2 = bp.tok + (size_t)(sq.row0 + (long long)(t0 + j) * p.tok_rows) * 2;  // by token row
            tk2[0] = inv;
            tk2[1] = dden;
          }
        }
        lds_barrier();
      }

      // Bm tiles as hi + lo
      if (role == 1 && cw < 3) store_bm<DECAY, NORM, true>(sh, sf, X, job_jt(cw), job_it(cw), L, lg, lane);
      lds_barrier();

      if (role == 0) {
        // dG = Bm F + theta (inv Y + dden Z_<): rows j, column p = col
        const __amdgpu_buffer_rsrc_t rdq = make_rsrc(bp.dq + r0 * BD, rows_extent(L, rsb4, BD * 4));
        const float zpv = NORM ? sf[BG::ZV + col] : 0.f;
#pragma unroll
        for (int jt = 0; jt < 2; ++jt) {
          f32x16 a1 = zero16();
#pragma unroll
          for (int k0 = 0; k0 < 32 * (jt + 1); k0 += 16) {
            const bf16x8 kh = ld_rows8(sh + BG::KH, TP, k0, 32 * cw, lane);  // B[k=i][n=p] = F[i][p]
            const bf16x8 bmh = ld_cols8(sh + BG::BH, SQ, 32 * jt, k0, lane);  // A[m=j][k=i] = Bm[j][i]
            const bf16x8 bml = ld_cols8(sh + BG::BL, SQ, 32 * jt, k0, lane);
            a1 = mfma32(bmh, kh, a1);
            a1 = mfma32(bml, kh, a1);
            if (ELU) a1 = mfma32(bmh, ld_rows8(sh + BG::KL, TP, k0, 32 * cw, lane), a1);
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = 32 * jt + dtile_row(r, lane);
            const float st = NORM ? sf[BG::IV + j] * Y[jt][r] + sf[BG::DD + j] * zpv : Y[jt][r];
            float g = a1[r] + sf[BG::TH + j] * st;
            if (ELU)
              g *= dpsi_from_feat(from_bf16(sh[BG::QH + j * TP + col]) + from_bf16(sh[BG::QL + j * TP + col]));
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(g), rdq, (uint32_t)j * rsb4 + (uint32_t)col * 4, 0, 0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        // state: S_< <- gamma^L S_< + F^T (xi V), held transposed: S^T[e][p] += sum_i (xi_i V[i][e]) F[i][p]
        // (token step outermost: the F operands are read once per step for all four tiles; each
        // tile's MFMAs keep their order)
        const float a = DECAY ? exp2f((float)L * lg) : 1.f;
        if (DECAY) {
#pragma unroll
          for (int et = 0; et < 4; ++et) St[et] *= a;
        }
#pragma unroll
        for (int k0 = 0; k0 < BC; k0 += 16) {
          const bf16x8 kh = ld_rows8(sh + BG::KH, TP, k0, 32 * cw, lane);  // B[k=i][n=p] = F[i][p]
          const bf16x8 kl = ELU ? ld_rows8(sh + BG::KL, TP, k0, 32 * cw, lane) : kh;
#pragma unroll
          for (int et = 0; et < 4; ++et) {
            const bf16x8 va = ld_rows8(sh + BG::V, TP, k0, 32 * et, lane);  // A[m=e][k=i] = V[i][e]
            if (DECAY) {
              bf16x8 vh, vl;
              scale_split<false>(va, va, sf + BG::XI + k0 + 8 * (lane >> 5), vh, vl);
              St[et] = mfma32(vh, kh, St[et]);
              St[et] = mfma32(vl, kh, St[et]);
              if (ELU) St[et] = mfma32(vh, kl, St[et]);
            } else {
              St[et] = mfma32(va, kh, St[et]);  // rows past L are zero in F
              if (ELU) St[et] = mfma32(va, kl, St[et]);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        if (NORM && tid < BD) {
          float zn = a * zreg;
          for (int i = 0; i < L; ++i)
            zn += sf[BG::XI + i] *
                  (from_bf16(sh[BG::KH + i * TP + tid]) + (ELU ? from_bf16(sh[BG::KL + i * TP + tid]) : 0.f));
          zreg = zn;
        }
      } else {
        // adjoint summary: [p][e] += sum_j (W_j inv_j G[j][p]) dout[j][e] (token step outermost:
        // the dout operands are read once per step for all four tiles)
#pragma unroll
        for (int k0 = 0; k0 < BC; k0 += 16) {
          const bf16x8 nh = ld_rows8(sh + BG::NH, TP, k0, 32 * cw, lane);  // B[k=j][n=e]
          const bf16x8 nl = ld_rows8(sh + BG::NL, TP, k0, 32 * cw, lane);
#pragma unroll
          for (int pt = 0; pt < 4; ++pt) {
            const bf16x8 gh = ld_rows8(sh + BG::QH, TP, k0, 32 * pt, lane);  // A[m=p][k=j] = G[j][p]
            if (DECAY || NORM) {
              bf16x8 sh2, sl2;
              const bf16x8 gl = ELU ? ld_rows8(sh + BG::QL, TP, k0, 32 * pt, lane) : gh;
              scale_split<ELU>(gh, gl, wi + k0 + 8 * (lane >> 5), sh2, sl2);
              St[pt] = mfma32(sh2, nh, St[pt]);
              St[pt] = mfma32(sh2, nl, St[pt]);
              St[pt] = mfma32(sl2, nh, St[pt]);
            } else {
              St[pt] = mfma32(gh, nh, St[pt]);
              St[pt] = mfma32(gh, nl, St[pt]);
              if (ELU) St[pt] = mfma32(ld_rows8(sh + BG::QL, TP, k0, 32 * pt, lane), nh, St[pt]);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        if (NORM && zp < BD) {
          for (int j = 0; j < L; ++j) {
            const float g = from_bf16(sh[BG::QH + j * TP + zp]) + (ELU ? from_bf16(sh[BG::QL + j * TP + zp]) : 0.f);
            rz += sf[BG::WT + j] * g * sf[BG::DD + j];
          }
        }
      }
    }
  }
  // the segment's adjoint summary [S (p, e)][Z (p)] (role 1; zero for an empty segment)
  if (role == 1) {
#pragma unroll
    for (int pt = 0; pt < 4; ++pt)
#pragma unroll
      for (int r = 0; r < 16; ++r) rrec[(size_t)(32 * pt + dtile_row(r, lane0)) * BD + col0] = St[pt][r];
    if (zp < BD) rrec[(size_t)BD * BD + zp] = rz;
  }
}

// ---- state sweep -----------------------------------------------------------------------

// Eight waves, specialised by the state they hold (two waves per SIMD): waves 0..3 hold R
// (value columns 32 cw..) and produce dv, waves 4..7 hold R^T (feature columns 32 cw..) and
// produce dk. Each wave then carries one 128 x 32 state instead of two, and the second wave
// on each SIMD hides the other's LDS and MFMA latencies.
constexpr int KNT = 512;

template <bool ELU, bool DECAY, bool NORM, bool DBF>
__global__ __launch_bounds__(KNT) void k_bwd_key(BackwardParams bp) {
  const PrefillParams& p = bp.f;
  extern __shared__ __align__(16) unsigned char smem[];
  __bf16* sh = (__bf16*)smem;
  float* sf = (float*)smem;
  const int bh = blockIdx.x, seg = blockIdx.y, tid = threadIdx.x, lane0 = tid & 63, w = tid >> 6;
  const int role = w >> 2, cw = w & 3;  // role 0: R and dv; role 1: R^T and dk
  const SeqSpan sq = seq_span(p, bh);
  const int T = sq.T;
  const int seg_tok = p.seg_chunks * p.C;
  const int tb = seg * seg_tok, te = min(tb + seg_tok, T);
  if (tb >= te) return;
  const size_t E = (size_t)BD * BD + BD;
  const float* rpre = bp.rev + ((size_t)bh * p.n_seg + seg) * E;  // the adjoint state after this segment
  const float lg = DECAY ? p.log2g[bh % p.H] : 0.f;
  const uint32_t rsb = (uint32_t)p.tok_rows * BD * 2, rsb4 = (uint32_t)p.tok_rows * BD * 4;
  const uint32_t rsbd = (uint32_t)p.tok_rows * BD * (DBF ? 2 : 4);
  const int col0 = 32 * cw + (lane0 & 31);
  // role 0: St[t] = R[p][e], rows p in tile t, column e = col
  // role 1: St[t] = R^T[e][p], rows e in tile t, column p = col
  f32x16 St[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      St[t][r] = role == 0 ? rpre[(size_t)(32 * t + dtile_row(r, lane0)) * BD + col0]
                           : rpre[(size_t)col0 * BD + 32 * t + dtile_row(r, lane0)];
  const int zp = tid - KNT / 2;  // role-1 thread zp < BD holds RZ[zp]
  float rz = (NORM && role == 1 && zp < BD) ? rpre[(size_t)BD * BD + zp] : 0.f;

  const int nsteps = (te - tb + BC - 1) / BC;
  for (int s = nsteps - 1; s >= 0; --s) {
    // the lane index, opaque to the optimiser once per step: every per-lane LDS address is then
    // formed inside the step (a few bases plus immediates) rather than hoisted out of the loop
    // as one live register per access
    const int lane = pin(lane0), col = 32 * cw + (lane & 31);
    const int t0 = tb + s * BC, L = min(BC, te - t0);
    const long long r0 = sq.row0 + (long long)t0 * p.tok_rows;
    Tile16<KNT> tq, tk, tv;
    load_tile16<KNT>(tq, (const uint16_t*)p.q + r0 * BD, L, rsb);
    load_tile16<KNT>(tk, (const uint16_t*)p.k + r0 * BD, L, rsb);
    load_tile16<KNT>(tv, (const uint16_t*)p.v + r0 * BD, L, rsb);
    TileF<KNT> tdo;
    load_tileF<KNT, DBF>(tdo, (const unsigned char*)bp.dout + r0 * BD * (DBF ? 2 : 4), L, rsbd);
    float inv = 1.f, dden = 0.f;
    if (NORM) {
      const int j = tf_tok<KNT>();
      if (j < L) {
        const float* tk2 = bp.tok + (size_t)(sq.row0 + (long long)(t0 + j) * p.tok_rows) * 2;
        inv = tk2[0];
        dden = tk2[1];
      }
    }
    lds_barrier();
    commit_feat<KNT, ELU, ELU>(tq, sh + BG::QH, sh + BG::QL, L);
    commit_feat<KNT, ELU, ELU>(tk, sh + BG::KH, sh + BG::KL, L);
    commit_raw<KNT>(tv, sh + BG::V);
    commit_scaled<KNT>(tdo, inv, sh + BG::NH, sh + BG::NL);
    if (tid < BC) {
      const int j = tid;
      sf[BG::TH + j] = DECAY ? exp2f((float)(j + 1) * lg) : 1.f;
      sf[BG::XI + j] = j < L ? (DECAY ? exp2f((float)(L - 1 - j) * lg) : 1.f) : 0.f;
      sf[BG::DM + j] = DECAY ? exp2f((float)j * lg) : 1.f;
    }
    if (NORM && (tid % TileF<KNT>::TPT) == 0) sf[BG::DD + tf_tok<KNT>()] = dden;
    if (NORM && role == 1 && zp < BD) sf[BG::ZV + zp] = rz;
    lds_barrier();

    // A tiles (role 0) and Bm tiles (role 1) of the lower block triangle, hi + lo
    if (cw < 3) {
      const int jt = job_jt(cw), it = job_it(cw);
      if (role == 0) {
        const f32x16 acc = a_tile_acc<ELU>(sh, jt, it, lane);
        const int i = 32 * it + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = 32 * jt + dtile_row(r, lane);
          const bf16_pair pr = split_bf16(acc[r] * dmask<DECAY>(j, i, sf));
          sh[BG::AH + j * SQ + i] = pr.hi;
          sh[BG::AL + j * SQ + i] = pr.lo;
        }
      } else {
        store_bm<DECAY, NORM, false>(sh, sf, x_tile_acc(sh, jt, it, lane), jt, it, L, lg, lane);
      }
    }
    lds_barrier();
    const float a = DECAY ? exp2f((float)L * lg) : 1.f;
    __builtin_amdgcn_sched_barrier(0);

    if (role == 0) {
      // dV = A^T dNum + xi (F R), computed transposed: dV^T[e][i], rows e (this wave's columns),
      // column i = 32 it + lane % 32. Operand registers serve either side of an MFMA, so swapping
      // them transposes the product; each lane then holds four consecutive columns of one token
      // and stores them with one 16-byte store (a quarter of the store instructions).
      f32x16 a2[2] = {zero16(), zero16()};
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        bf16x8 rh[2], rl[2];
        split_dtile(St[pt], rh, rl);
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
          for (int it = 0; it < 2; ++it) {
            const bf16x8 kh = ld_cols8_perm(sh + BG::KH, TP, 32 * it, 32 * pt, q, lane);  // B[k=p][n=i] = F[i][p]
            a2[it] = mfma32(rh[q], kh, a2[it]);  // A[m=e][k=p] = R[p][e] (the D-tile, transposed)
            a2[it] = mfma32(rl[q], kh, a2[it]);
            if (ELU) a2[it] = mfma32(rh[q], ld_cols8_perm(sh + BG::KL, TP, 32 * it, 32 * pt, q, lane), a2[it]);
          }
        __builtin_amdgcn_sched_barrier(0);
      }
      const __amdgpu_buffer_rsrc_t rdv = make_rsrc(bp.dv + r0 * BD, rows_extent(L, rsb4, BD * 4));
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        f32x16 a1 = zero16();
#pragma unroll
        for (int k0 = 32 * it; k0 < BC; k0 += 16) {
          const bf16x8 ah = ld_rows8(sh + BG::AH, SQ, k0, 32 * it, lane);  // B[k=j][n=i] = A[j][i]
          const bf16x8 al = ld_rows8(sh + BG::AL, SQ, k0, 32 * it, lane);
          const bf16x8 nh = ld_rows8(sh + BG::NH, TP, k0, 32 * cw, lane);  // A[m=e][k=j] = dNum[j][e]
          const bf16x8 nl = ld_rows8(sh + BG::NL, TP, k0, 32 * cw, lane);
          a1 = mfma32(nh, ah, a1);
          a1 = mfma32(nl, ah, a1);
          a1 = mfma32(nh, al, a1);
        }
        const int i = 32 * it + (lane & 31);
        const float xi = sf[BG::XI + i];
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {  // registers 4 g4 .. 4 g4 + 3: columns 32 cw + 8 g4 + 4 hh + 0..3
          f32x4 o;
#pragma unroll
          for (int u = 0; u < 4; ++u) o[u] = a1[4 * g4 + u] + xi * a2[it][4 * g4 + u];
          const uint32_t e = 32 * cw + 8 * g4 + 4 * (lane >> 5);
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o), rdv, (uint32_t)i * rsb4 + e * 4, 0, 0);
        }
      }
      // R <- gamma^L R + (theta G)^T dNum: R[p][e] += sum_j (theta_j G[j][p]) dNum[j][e], token
      // step outermost so that the dNum operands are read once per step (each tile's MFMAs keep
      // their order)
      if (DECAY) {
#pragma unroll
        for (int t = 0; t < 4; ++t) St[t] *= a;
      }
#pragma unroll
      for (int k0 = 0; k0 < BC; k0 += 16) {
        const float* th = sf + BG::TH + k0 + 8 * (lane >> 5);
        const bf16x8 nh = ld_rows8(sh + BG::NH, TP, k0, 32 * cw, lane);
        const bf16x8 nl = ld_rows8(sh + BG::NL, TP, k0, 32 * cw, lane);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const bf16x8 ga = ld_rows8(sh + BG::QH, TP, k0, 32 * t, lane);  // A[m=p][k=j]
          if (DECAY) {
            bf16x8 gh, gl;
            scale_split<ELU>(ga, ELU ? ld_rows8(sh + BG::QL, TP, k0, 32 * t, lane) : ga, th, gh, gl);
            St[t] = mfma32(gh, nh, St[t]);
            St[t] = mfma32(gh, nl, St[t]);
            St[t] = mfma32(gl, nh, St[t]);
          } else {
            St[t] = mfma32(ga, nh, St[t]);
            St[t] = mfma32(ga, nl, St[t]);
            if (ELU) St[t] = mfma32(ld_rows8(sh + BG::QL, TP, k0, 32 * t, lane), nh, St[t]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      // dF = Bm^T G + xi (V R^T + RZ), computed transposed like dV: dF^T[p][i], rows p (this
      // wave's features), column i = 32 it + lane % 32, stored 16 bytes at a time
      f32x16 a2[2] = {zero16(), zero16()};
#pragma unroll
      for (int et = 0; et < 4; ++et) {
        bf16x8 th2[2], tl2[2];
        split_dtile(St[et], th2, tl2);
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
          for (int it = 0; it < 2; ++it) {
            const bf16x8 va = ld_cols8_perm(sh + BG::V, TP, 32 * it, 32 * et, q, lane);  // B[k=e][n=i] = V[i][e]
            a2[it] = mfma32(th2[q], va, a2[it]);  // A[m=p][k=e] = R^T[e][p] (the D-tile, transposed)
            a2[it] = mfma32(tl2[q], va, a2[it]);
          }
        __builtin_amdgcn_sched_barrier(0);
      }
      const __amdgpu_buffer_rsrc_t rdk = make_rsrc(bp.dk + r0 * BD, rows_extent(L, rsb4, BD * 4));
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        f32x16 a1 = zero16();
#pragma unroll
        for (int k0 = 32 * it; k0 < BC; k0 += 16) {
          const bf16x8 bmh = ld_rows8(sh + BG::BH, SQ, k0, 32 * it, lane);  // B[k=j][n=i] = Bm[j][i]
          const bf16x8 bml = ld_rows8(sh + BG::BL, SQ, k0, 32 * it, lane);
          const bf16x8 gq = ld_rows8(sh + BG::QH, TP, k0, 32 * cw, lane);  // A[m=p][k=j] = G[j][p]
          a1 = mfma32(gq, bmh, a1);
          a1 = mfma32(gq, bml, a1);
          if (ELU) a1 = mfma32(ld_rows8(sh + BG::QL, TP, k0, 32 * cw, lane), bmh, a1);
        }
        const int i = 32 * it + (lane & 31);
        const float xi = sf[BG::XI + i];
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {  // registers 4 g4 .. 4 g4 + 3: features 32 cw + 8 g4 + 4 hh + 0..3
          const int p0 = 32 * cw + 8 * g4 + 4 * (lane >> 5);
          const f32x4 rz4 = NORM ? *(const f32x4*)(sf + BG::ZV + p0) : f32x4{0.f, 0.f, 0.f, 0.f};
          f32x4 o;
#pragma unroll
          for (int u = 0; u < 4; ++u) o[u] = a1[4 * g4 + u] + xi * (a2[it][4 * g4 + u] + rz4[u]);
          if (ELU) {
            const bf16x4 kh4 = *(const bf16x4*)(sh + BG::KH + i * TP + p0);
            const bf16x4 kl4 = *(const bf16x4*)(sh + BG::KL + i * TP + p0);
#pragma unroll
            for (int u = 0; u < 4; ++u) o[u] *= dpsi_from_feat(from_bf16(kh4[u]) + from_bf16(kl4[u]));
          }
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o), rdk, (uint32_t)i * rsb4 + (uint32_t)p0 * 4,
                                                 0, 0);
        }
      }
      // R^T <- gamma^L R^T + dNum^T (theta G): R^T[e][p] += sum_j dNum[j][e] (theta_j G[j][p]), token
      // step outermost so that theta G (read, scaled and split) is formed once per step for all
      // four tiles (each tile's MFMAs keep their order)
      if (DECAY) {
#pragma unroll
        for (int t = 0; t < 4; ++t) St[t] *= a;
      }
#pragma unroll
      for (int k0 = 0; k0 < BC; k0 += 16) {
        const float* th = sf + BG::TH + k0 + 8 * (lane >> 5);
        const bf16x8 gb = ld_rows8(sh + BG::QH, TP, k0, 32 * cw, lane);  // B[k=j][n=p]
        bf16x8 gh, gl;
        if (DECAY) scale_split<ELU>(gb, ELU ? ld_rows8(sh + BG::QL, TP, k0, 32 * cw, lane) : gb, th, gh, gl);
        else gh = gb, gl = ELU ? ld_rows8(sh + BG::QL, TP, k0, 32 * cw, lane) : gb;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const bf16x8 nh = ld_rows8(sh + BG::NH, TP, k0, 32 * t, lane);  // A[m=e][k=j] = dNum[j][e]
          const bf16x8 nl = ld_rows8(sh + BG::NL, TP, k0, 32 * t, lane);
          if (DECAY) {
            St[t] = mfma32(nh, gh, St[t]);
            St[t] = mfma32(nl, gh, St[t]);
            St[t] = mfma32(nh, gl, St[t]);
          } else {
            St[t] = mfma32(nh, gh, St[t]);
            St[t] = mfma32(nl, gh, St[t]);
            if (ELU) St[t] = mfma32(nh, gl, St[t]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (NORM && zp < BD) {
        float zn = a * rz;
        for (int j = 0; j < L; ++j) {
          const float g = from_bf16(sh[BG::QH + j * TP + zp]) + (ELU ? from_bf16(sh[BG::QL + j * TP + zp]) : 0.f);
          zn += sf[BG::TH + j] * g * sf[BG::DD + j];
        }
        rz = zn;
      }
    }
  }
}

template <bool ELU, bool DECAY, bool NORM, bool DBF>
hipError_t launch4(const BackwardParams& p, hipStream_t s, bool key_sweep) {
  const void* kern = key_sweep ? (const void*)k_bwd_key<ELU, DECAY, NORM, DBF>
                               : (const void*)k_bwd_query<ELU, DECAY, NORM, DBF>;
  hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, BG::BYTES);
  if (e != hipSuccess) return e;
  dim3 grid(p.f.B * p.f.H, p.f.n_seg);  // sequences on x: every XCD gets all segments of its sequences
  void* args[] = {(void*)&p};
  e = hipLaunchKernel(kern, grid, dim3(key_sweep ? KNT : QNT), args, BG::BYTES, s);
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

template <bool ELU, bool DECAY>
hipError_t launch2(const BackwardParams& p, hipStream_t s, bool key_sweep) {
  const bool norm = p.f.normalize != 0, dbf = p.dout_bf16 != 0;
  if (norm) return dbf ? launch4<ELU, DECAY, true, true>(p, s, key_sweep) : launch4<ELU, DECAY, true, false>(p, s, key_sweep);
  return dbf ? launch4<ELU, DECAY, false, true>(p, s, key_sweep) : launch4<ELU, DECAY, false, false>(p, s, key_sweep);
}

}  // namespace

bool prefill_backward_supported(int C, int d_k, int d_v, int n_psi, int psi) {
  if (psi != LA_PSI_IDENTITY && psi != LA_PSI_ELU1) return false;
  if (d_k != BD || d_v != BD || n_psi != BD) return false;
  return C == 32 || C == 64 || C == 128;  // segments are whole multiples of the 64-token step
}

hipError_t launch_prefill_backward(const BackwardParams& p, hipStream_t s, bool key_sweep) {
  const bool elu = p.f.psi == LA_PSI_ELU1, decay = p.f.has_decay != 0;
  if (elu) return decay ? launch2<true, true>(p, s, key_sweep) : launch2<true, false>(p, s, key_sweep);
  return decay ? launch2<false, true>(p, s, key_sweep) : launch2<false, false>(p, s, key_sweep);
}

}  // namespace la
