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
// The state elements (n_psi*d_v + n_psi per sequence) are independent. Up to 128 segments,
// a workgroup takes 256 consecutive elements (4 per lane, 16-byte accesses) and spreads the
// segment axis over W waves: each wave folds its run of at most 8 segments in registers (so
// every element is read once and written once), the W wave totals are scanned with a
// Blelloch up-sweep/down-sweep in LDS (log2 W levels each; the down-sweep combines
// parent-prefix (+) left-sum in that order because the monoid does not commute), and each
// wave then writes its run's exclusive prefixes. With few segments (W below 4) a workgroup
// holds several such groups of W waves, each on its own 256 elements, so that short scans
// still run four waves per workgroup. Beyond 128 segments the lanes hold segments instead
// (k_segment_scan_lanes): a Hillis-Steele scan across each wavefront's 64 lanes, a Blelloch
// scan across its waves, and a carried prefix across blocks of up to 1024 segments.
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

// Runs of up to RUN segments are kept in registers between the fold and the rewrite.
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
  f32x4 run[RUN];
  f32x4 tx = {0.f, 0.f, 0.f, 0.f};
  f32x4 ta = {1.f, 1.f, 1.f, 1.f};
#pragma unroll
  for (int i = 0; i < RUN; ++i)
    run[i] = (live && s0 + i < s1 && (p.n_read <= 0 || seg_of(s0 + i) < p.n_read))
                 ? ld4(base + (size_t)seg_of(s0 + i) * REC)
                 : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < RUN; ++i) {
    if (s0 + i < s1) {
      const f32x4 as = seg_decay(seg_of(s0 + i));
      tx = as * tx + run[i];
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
#pragma unroll
  for (int i = 0; i < RUN; ++i) {
    if (s0 + i < s1) {
      const f32x4 as = seg_decay(seg_of(s0 + i));
      if (live && (p.write_every <= 1 || seg_of(s0 + i) % p.write_every == 0))
        st4(base + (size_t)seg_of(s0 + i) * REC, cx);
      cx = as * cx + run[i];
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

// Many segments: lanes hold consecutive segments. A workgroup takes one 16-byte element
// group (4 state elements) of one sequence; wave w holds segments [blk + 64 w, blk + 64 w + 64)
// of a block of 64 NW. Inside a wavefront, an inclusive Hillis-Steele scan across the lanes
// (log2 64 = 6 rounds of lane shifts); across the wavefronts, a Blelloch up-sweep/down-sweep
// over the NW wave totals in LDS (log2 NW levels each); across blocks, the prefix of the
// blocks before, carried in registers (one combine per block). Every lane of a wave reads
// its segment's 16 bytes of one record; the element groups of neighbouring workgroups share
// those lines in L2.
template <int NW>
__global__ __launch_bounds__(64 * NW) void k_segment_scan_lanes(ScanParams p) {
  __shared__ f32x4 tx[NW], ta[NW];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int bh = blockIdx.x, head = bh % p.H;
  const size_t SE = (size_t)p.n_psi * p.d_v;
  const size_t E = SE + p.n_psi;
  const size_t REC = E + (p.gated ? p.n_psi : 0);
  const size_t e = (size_t)blockIdx.y * 4;  // E is a multiple of 4: every group is whole
  const float lg = p.has_decay ? p.log2g[head] : 0.f;
  auto seg_of = [&](int i) -> int { return p.reverse ? p.n_seg - 1 - i : i; };
  float* base = p.ws + (size_t)bh * p.n_seg * REC + e;
  const bool zpart = e >= SE;
  const size_t row = zpart ? e - SE : e / p.d_v;
  const float* gvec = p.ws + (size_t)bh * p.n_seg * REC + E + row;
  int T = p.T;
  if (p.cu_seqlens) {
    int start;
    T = packed_len(p.cu_seqlens, bh / p.H, p.total, p.T, &start);
  }
  auto seg_decay = [&](int s) -> f32x4 {
    if (p.gated) {
      if (zpart) return ld4(gvec + (size_t)s * REC);
      const float a = gvec[(size_t)s * REC];
      return f32x4{a, a, a, a};
    }
    const int len = max(0, min(p.seg_len, T - s * p.seg_len));
    const float a = gpow(lg, (float)len);
    return f32x4{a, a, a, a};
  };
  auto shfl_up4 = [&](const f32x4& v, int d) {
    return f32x4{__shfl_up(v[0], d), __shfl_up(v[1], d), __shfl_up(v[2], d), __shfl_up(v[3], d)};
  };

  // the prefix of everything before the current block: init (+) X_0 (+) ...
  f32x4 cx = {0.f, 0.f, 0.f, 0.f}, ca = {1.f, 1.f, 1.f, 1.f};
  if (e < SE) {
    if (p.init_S) cx = ld4(p.init_S + (size_t)bh * SE + e);
  } else if (p.init_Z) {
    cx = ld4(p.init_Z + (size_t)bh * p.n_psi + (e - SE));
  }
  int chain = 0;  // dependent (+) levels, for the diagnostic record
  for (int blk = 0; blk < p.n_seg; blk += 64 * NW) {
    const int s = blk + 64 * w + lane;
    const bool in = s < p.n_seg;
    f32x4 x = in ? ld4(base + (size_t)seg_of(s) * REC) : f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 a = in ? seg_decay(seg_of(s)) : f32x4{1.f, 1.f, 1.f, 1.f};
    // 1. inclusive scan across the wavefront's lanes: lane l <- (lane l - d) (+) lane l
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const f32x4 xp = shfl_up4(x, d), ap = shfl_up4(a, d);
      if (lane >= d) {
        x = a * xp + x;
        a = ap * a;
      }
    }
    chain += 6;
    // the lane's exclusive prefix within its wave
    f32x4 lx = shfl_up4(x, 1), la = shfl_up4(a, 1);
    if (lane == 0) {
      lx = f32x4{0.f, 0.f, 0.f, 0.f};
      la = f32x4{1.f, 1.f, 1.f, 1.f};
    }
    if (lane == 63) {
      tx[w] = x;
      ta[w] = a;
    }
    __syncthreads();
    // 2. Blelloch over the NW wave totals (node w held by lane 0 of wave w)
    for (int d = 1; d < NW; d <<= 1) {
      ++chain;
      const int right = (w + 1) * 2 * d - 1;
      const bool act = lane == 0 && right < NW;
      f32x4 nx = {0.f, 0.f, 0.f, 0.f}, na = {1.f, 1.f, 1.f, 1.f};
      if (act) {
        const int left = right - d;
        nx = ta[right] * tx[left] + tx[right];
        na = ta[left] * ta[right];
      }
      __syncthreads();
      if (act) {
        tx[right] = nx;
        ta[right] = na;
      }
      __syncthreads();
    }
    const f32x4 bx = tx[NW - 1], ba = ta[NW - 1];  // the block's total
    __syncthreads();
    if (w == NW - 1 && lane == 0) {
      tx[NW - 1] = f32x4{0.f, 0.f, 0.f, 0.f};
      ta[NW - 1] = f32x4{1.f, 1.f, 1.f, 1.f};
    }
    __syncthreads();
    for (int d = NW >> 1; d >= 1; d >>= 1) {
      ++chain;
      const int right = (w + 1) * 2 * d - 1;
      const bool act = lane == 0 && right < NW;
      f32x4 lx2 = {0.f, 0.f, 0.f, 0.f}, px = {0.f, 0.f, 0.f, 0.f};
      f32x4 la2 = {1.f, 1.f, 1.f, 1.f}, pa = {1.f, 1.f, 1.f, 1.f};
      if (act) {
        const int left = right - d;
        lx2 = tx[left];
        la2 = ta[left];
        px = tx[right];
        pa = ta[right];
      }
      __syncthreads();
      if (act) {
        const int left = right - d;
        tx[left] = px;
        tx[right] = la2 * px + lx2;
        ta[left] = pa;
        ta[right] = pa * la2;
      }
      __syncthreads();
    }
    // 3. the segment's exclusive prefix: carry (+) wave prefix (+) lane prefix
    const f32x4 wx = tx[w], wa = ta[w];
    const f32x4 px = wa * cx + wx, pa = ca * wa;
    if (in) st4(base + (size_t)seg_of(s) * REC, la * px + lx);
    chain += 2;
    (void)pa;
    // 4. carry the block's total
    cx = ba * cx + bx;
    ca = ca * ba;
    __syncthreads();  // the wave totals are rewritten by the next block
  }
  if (p.rounds && threadIdx.x == 0 && blockIdx.y == 0) atomicMax(p.rounds, chain);
  // 5. the final state: the prefix of all segments
  if (threadIdx.x == 0) {
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
  if (per > 8) {  // many segments: lanes over segments (log-depth within each block of 64 NW)
    const dim3 lgrid(p.BH, (unsigned)(E / 4));
    if (p.n_seg <= 256)
      hipLaunchKernelGGL(k_segment_scan_lanes<4>, lgrid, dim3(256), 0, s, p);
    else if (p.n_seg <= 512)
      hipLaunchKernelGGL(k_segment_scan_lanes<8>, lgrid, dim3(512), 0, s, p);
    else
      hipLaunchKernelGGL(k_segment_scan_lanes<16>, lgrid, dim3(1024), 0, s, p);
    return hipGetLastError();
  }
  if (per <= 4)
    hipLaunchKernelGGL(k_segment_scan<4>, grid, block, 0, s, p);
  else
    hipLaunchKernelGGL(k_segment_scan<8>, grid, block, 0, s, p);
  return hipGetLastError();
}

}  // namespace la
