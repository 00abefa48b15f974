// la_scan.hip -- exclusive scan of segment summaries under the decayed monoid.
//
// Each (batch, head) sequence has n_seg segment summaries X_s = (a_s, S_s, Z_s) in
// the workspace, a_s = gamma^(L_s) for a segment of L_s tokens. Summaries combine
// as (a1, X1) (+) (a2, X2) = (a1 a2, a2 X1 + X2) -- the additive monoid of
// "Log-Depth Chunked Linear-Attention Scan" (Mathematical statement) when
// gamma = 1, and the chunkwise decay of "Linear Attention and Retentive
// Networks" (Retentive Networks, representation C) otherwise. The scan replaces
// X_s with init (+) X_0 (+) ... (+) X_{s-1} and writes init (+) X_0 (+) ... as the
// final state.
//
// With `reverse` the segment order is reversed: segment s receives the fold of segments
// n_seg-1, ..., s+1 (each decayed by the segments between it and s) and the final state is
// the fold of all of them. This is the adjoint state of the backward pass, which gathers
// every later read of a state and decays the same way on its way back.
//
// The state elements (n_psi*d_v + n_psi per sequence) are independent. A workgroup
// takes 256 consecutive elements (4 per lane, 16-byte accesses) and spreads the segment
// axis over W waves: each wave folds its run of segments (holding the run in registers
// when it is at most RUN long, so every element is read once and written once), the W
// wave totals are scanned with a Blelloch up-sweep/down-sweep in LDS (log2 W levels
// each; the down-sweep combines parent-prefix (+) left-sum in that order because the
// monoid does not commute), and each wave then writes its run's exclusive prefixes.
// With few segments (W below 4) a workgroup holds several such groups of W waves, each on
// its own 256 elements, so that short scans still run four waves per workgroup.
// The order of all floating-point operations is fixed: results are deterministic.
#include "la_device.hpp"
#include "la_kernels.hpp"

namespace la {
namespace {

constexpr int kMaxWaves = 16;
constexpr int kMinGroupWaves = 4;  // waves per workgroup at least (W times the element groups)

// Waves over the segment axis: a power of two, runs of ~4 segments per wave.
__host__ __device__ inline int scan_seg_waves(int n_seg) {
  int W = 1;
  while (W < kMaxWaves && W * 4 < n_seg) W <<= 1;
  return W;
}

__device__ __forceinline__ f32x4 ld4(const float* p) { return *(const f32x4*)p; }
__device__ __forceinline__ void st4(float* p, const f32x4& v) { *(f32x4*)p = v; }

// RUN > 0: runs of up to RUN segments are kept in registers between the fold and the
// rewrite; RUN == 0: the rewrite reads the run again (any run length).
template <int RUN>
__global__ __launch_bounds__(64 * kMaxWaves) void k_segment_scan(ScanParams p) {
  __shared__ f32x4 sx[kMaxWaves][64];
  __shared__ f32x4 sa[kMaxWaves][64];  // decays per element: rows differ under per-row gates
  const int W = scan_seg_waves(p.n_seg);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int w = wid % W, grp = wid / W, n_grp = (blockDim.x >> 6) / W;
  const int o = grp * W;  // this element group's LDS slots
  const int bh = blockIdx.x, head = bh % p.H;  // sequences on x (no 65535 cap), element blocks on y
  const size_t SE = (size_t)p.n_psi * p.d_v;
  const size_t E = SE + p.n_psi;  // scanned elements; a multiple of 4 (n_psi and d_v are)
  // segment record: S, Z, then (gated) the segment's per-row decay vector
  const size_t REC = E + (p.gated ? p.n_psi : 0);
  const size_t e = (((size_t)blockIdx.y * n_grp + grp) * 64 + lane) * 4;
  const bool live = e < E;
  const float lg = p.has_decay ? p.log2g[head] : 0.f;
  // scan position i is segment seg_of(i): the same segment in forward order, mirrored in reverse
  auto seg_of = [&](int i) -> int { return p.reverse ? p.n_seg - 1 - i : i; };
  float* base = p.ws + (size_t)bh * p.n_seg * REC + e;
  // the state rows of this lane's 4 elements: one row (S part, d_v a multiple of 4) or four
  // consecutive rows (Z part); their decays under per-row gates
  const bool zpart = e >= SE;
  const size_t row = zpart ? e - SE : e / p.d_v;
  const float* gvec = p.ws + (size_t)bh * p.n_seg * REC + E + (live ? row : 0);
  int T = p.T;  // this sequence's length
  if (p.cu_seqlens) {
    int start;
    T = packed_len(p.cu_seqlens, bh / p.H, p.total, p.T, &start);
  }

  // this wave's run of segments
  const int per = (p.n_seg + W - 1) / W;
  const int s0 = min(w * per, p.n_seg), s1 = min(s0 + per, p.n_seg);
  auto seg_decay = [&](int s) -> f32x4 {
    if (p.gated) {  // products of the segment's gates for these rows
      if (!live) return f32x4{1.f, 1.f, 1.f, 1.f};
      if (zpart) return ld4(gvec + (size_t)s * REC);
      const float a = gvec[(size_t)s * REC];
      return f32x4{a, a, a, a};
    }
    const int len = max(0, min(p.seg_len, T - s * p.seg_len));  // 0 past a shorter sequence's end
    const float a = gpow(lg, (float)len);
    return f32x4{a, a, a, a};
  };

  // Length of this wave's chain of dependent (+) steps, for the diagnostic record: its run's
  // fold, the tree's levels up and down, the carry of the initial state, the run's rewrite.
  int chain = 2 * max(0, s1 - s0) + 1;

  // 1. fold the run: total = X_s0 (+) ... (+) X_{s1-1}
  f32x4 run[RUN > 0 ? RUN : 1];
  f32x4 tx = {0.f, 0.f, 0.f, 0.f};
  f32x4 ta = {1.f, 1.f, 1.f, 1.f};
  if (RUN > 0) {
#pragma unroll
    for (int i = 0; i < (RUN > 0 ? RUN : 1); ++i)
      run[i] = (live && s0 + i < s1) ? ld4(base + (size_t)seg_of(s0 + i) * REC) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < (RUN > 0 ? RUN : 1); ++i) {
      if (s0 + i < s1) {
        const f32x4 as = seg_decay(seg_of(s0 + i));
        tx = as * tx + run[i];
        ta *= as;
      }
    }
  } else {
    for (int s = s0; s < s1; ++s) {
      const f32x4 as = seg_decay(seg_of(s));
      if (live) tx = as * tx + ld4(base + (size_t)seg_of(s) * REC);
      ta *= as;
    }
  }
  sx[o + w][lane] = tx;
  sa[o + w][lane] = ta;
  __syncthreads();

  // 2. Blelloch over the W wave totals (W is a power of two)
  for (int d = 1; d < W; d <<= 1) {  // up-sweep: node right <- left (+) right
    ++chain;
    const int right = (w + 1) * 2 * d - 1;
    const bool act = right < W;
    f32x4 nx = {0.f, 0.f, 0.f, 0.f};
    f32x4 na = {1.f, 1.f, 1.f, 1.f};
    if (act) {
      const int left = right - d;
      nx = sa[o + right][lane] * sx[o + left][lane] + sx[o + right][lane];
      na = sa[o + left][lane] * sa[o + right][lane];
    }
    __syncthreads();
    if (act) {
      sx[o + right][lane] = nx;
      sa[o + right][lane] = na;
    }
    __syncthreads();
  }
  if (w == W - 1) {
    sx[o + W - 1][lane] = f32x4{0.f, 0.f, 0.f, 0.f};
    sa[o + W - 1][lane] = f32x4{1.f, 1.f, 1.f, 1.f};
  }
  __syncthreads();
  for (int d = W >> 1; d >= 1; d >>= 1) {  // down-sweep
    ++chain;
    const int right = (w + 1) * 2 * d - 1;
    f32x4 lx = {0.f, 0.f, 0.f, 0.f}, px = {0.f, 0.f, 0.f, 0.f};
    f32x4 la_ = {1.f, 1.f, 1.f, 1.f}, pa = {1.f, 1.f, 1.f, 1.f};
    const bool act = right < W;
    if (act) {
      const int left = right - d;
      lx = sx[o + left][lane];
      la_ = sa[o + left][lane];
      px = sx[o + right][lane];
      pa = sa[o + right][lane];
    }
    __syncthreads();
    if (act) {
      const int left = right - d;
      sx[o + left][lane] = px;              // left child gets the parent's prefix
      sx[o + right][lane] = la_ * px + lx;  // right child: prefix (+) left sum
      sa[o + left][lane] = pa;
      sa[o + right][lane] = pa * la_;
    }
    __syncthreads();
  }

  // 3. carry into this run: init (+) prefix_w
  f32x4 cx = sx[o + w][lane];
  const f32x4 ca = sa[o + w][lane];
  if (live) {
    f32x4 init = {0.f, 0.f, 0.f, 0.f};
    if (e < SE) {
      if (p.init_S) init = ld4(p.init_S + (size_t)bh * SE + e);
    } else if (p.init_Z) {
      init = ld4(p.init_Z + (size_t)bh * p.n_psi + (e - SE));
    }
    cx = ca * init + cx;
  }
  // 4. rewrite the run with exclusive prefixes
  if (RUN > 0) {
#pragma unroll
    for (int i = 0; i < (RUN > 0 ? RUN : 1); ++i) {
      if (s0 + i < s1) {
        const f32x4 as = seg_decay(seg_of(s0 + i));
        if (live) st4(base + (size_t)seg_of(s0 + i) * REC, cx);
        cx = as * cx + run[i];
      }
    }
  } else {
    for (int s = s0; s < s1; ++s) {
      const f32x4 as = seg_decay(seg_of(s));
      if (live) {
        const f32x4 xs = ld4(base + (size_t)seg_of(s) * REC);
        st4(base + (size_t)seg_of(s) * REC, cx);
        cx = as * cx + xs;
      }
    }
  }
  if (p.rounds && lane == 0 && grp == 0 && blockIdx.y == 0) atomicMax(p.rounds, chain);
  // 5. the wave holding the last segment writes the final state
  if (live && s1 == p.n_seg && s0 < s1) {
    if (e < SE) {
      if (p.final_S) st4(p.final_S + (size_t)bh * SE + e, cx);
    } else if (p.final_Z) {
      st4(p.final_Z + (size_t)bh * p.n_psi + (e - SE), cx);
    }
  }
}

}  // namespace

hipError_t scan_depth_probe(int n_seg, float* ws, int* rounds, hipStream_t s) {
  ScanParams p{};
  p.ws = ws;
  p.init_S = p.init_Z = nullptr;
  p.final_S = p.final_Z = nullptr;
  p.cu_seqlens = nullptr;
  p.BH = p.H = 1;
  p.T = p.n_seg = n_seg;
  p.seg_len = 1;
  p.n_psi = p.d_v = 4;
  p.rounds = rounds;
  return launch_segment_scan(p, s);
}

hipError_t launch_segment_scan(const ScanParams& p, hipStream_t s) {
  const int W = scan_seg_waves(p.n_seg);
  const int G = W < kMinGroupWaves ? kMinGroupWaves / W : 1;  // element groups per workgroup
  const int per = (p.n_seg + W - 1) / W;
  const size_t E = (size_t)p.n_psi * p.d_v + p.n_psi;
  dim3 grid(p.BH, (unsigned)((E + 256 * G - 1) / (256 * G)));
  const dim3 block(64 * W * G);
  if (per <= 4)
    hipLaunchKernelGGL(k_segment_scan<4>, grid, block, 0, s, p);
  else if (per <= 8)
    hipLaunchKernelGGL(k_segment_scan<8>, grid, block, 0, s, p);
  else
    hipLaunchKernelGGL(k_segment_scan<0>, grid, block, 0, s, p);
  return hipGetLastError();
}

}  // namespace la
