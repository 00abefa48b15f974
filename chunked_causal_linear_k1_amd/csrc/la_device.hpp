// la_device.hpp -- device-side building blocks for gfx950 (CDNA4), wave64.
//
// MFMA operand layouts used throughout (v_mfma_f32_32x32x16_bf16):
//   A (32 x 16): lane l holds row m = l%32, k = 8*(l/32) + 0..7
//   B (16 x 32): lane l holds col n = l%32, k = 8*(l/32) + 0..7
//   D (32 x 32): lane l holds col n = l%32, rows m = 8*(r/4) + 4*(l/32) + r%4, r = 0..15
// A D-tile can be fed back as an operand whose k runs over the tile's rows: for
// k-half q (rows 16q..16q+15) lane (n, h=l/32) supplies registers 8q..8q+7, i.e.
// rows 16q + perm(h, j) with perm(h, j) = 4h + j for j < 4 and 8 + 4h + (j-4) for
// j >= 4; the partner operand then reads its k values in that same order.
//
// ds_read_b64_tr_b16 (transpose read), per 16-lane group: lane L receives element
// L%4 of the 4-element chunks addressed by lanes L/4, L/4+4, L/4+8, L/4+12. If lane
// L' addresses X[r0 + L'/4][c0 + 4*(L'%4)], lane L receives X[r0..r0+3][c0 + L]:
// four consecutive rows of one column, which is what an operand with k running
// over rows needs.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace la {

// Calls f(std::integral_constant<int, I>()) for I = B .. E-1 in order: a loop whose index is a
// constant expression in the body (for builtins that take constant arguments, such as the
// schedule-group barriers).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>());
    static_for<B + 1, E>(f);
  }
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

#define LA_LDS __attribute__((address_space(3)))

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// fp32 -> bf16, round to nearest even (hardware conversion on gfx950).
__device__ __forceinline__ __bf16 to_bf16(float x) { return (__bf16)x; }
__device__ __forceinline__ float from_bf16(__bf16 x) { return (float)x; }

// x = hi + lo with hi = bf16(x), lo = bf16(x - hi): a two-term bf16 expansion whose
// sum carries about 16 significant bits.
struct bf16_pair {
  __bf16 hi, lo;
};
__device__ __forceinline__ bf16_pair split_bf16(float x) {
  const __bf16 hi = to_bf16(x);
  return {hi, to_bf16(x - from_bf16(hi))};
}

// Eight fp32 values as two bf16x8 MFMA operands hi + lo, cheaply: hi keeps the top 16
// bits of each value (truncation, exact as a bf16), the residual x - hi is exact in
// fp32 and is rounded once to bf16. hi + lo carries about 16 significant bits.
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void split8_trunc(const float* x, bf16x8& hi, bf16x8& lo) {
  u32x4v h, l;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const unsigned a = __float_as_uint(x[2 * k]), b = __float_as_uint(x[2 * k + 1]);
    const float ra = x[2 * k] - __uint_as_float(a & 0xffff0000u);
    const float rb = x[2 * k + 1] - __uint_as_float(b & 0xffff0000u);
    h[k] = __builtin_amdgcn_perm(b, a, 0x07060302u);  // {hi16(b), hi16(a)}
    // one packed round-to-nearest-even conversion, element 0 in the low half
    const bf16x2 lp = __builtin_convertvector((f32x2){ra, rb}, bf16x2);
    l[k] = __builtin_bit_cast(unsigned, lp);
  }
  hi = __builtin_bit_cast(bf16x8, h);
  lo = __builtin_bit_cast(bf16x8, l);
}

// The same hi + lo split with hi rounded to nearest even (lo = RNE(x - hi), x - hi exact
// in fp32): for operands whose hi part also serves alone, where truncation would bias it
// toward zero by about a quarter of a bf16 ulp on average.
__device__ __forceinline__ void split8_rne(const float* x, bf16x8& hi, bf16x8& lo) {
  u32x4v h, l;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const bf16x2 hp = __builtin_convertvector((f32x2){x[2 * k], x[2 * k + 1]}, bf16x2);
    const unsigned hb = __builtin_bit_cast(unsigned, hp);
    const float ra = x[2 * k] - __uint_as_float(hb << 16);
    const float rb = x[2 * k + 1] - __uint_as_float(hb & 0xffff0000u);
    h[k] = hb;
    const bf16x2 lp = __builtin_convertvector((f32x2){ra, rb}, bf16x2);
    l[k] = __builtin_bit_cast(unsigned, lp);
  }
  hi = __builtin_bit_cast(bf16x8, h);
  lo = __builtin_bit_cast(bf16x8, l);
}

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Transpose read of four bf16 from LDS (see the header comment for the lane mapping).
__device__ __forceinline__ bf16x4 lds_read_tr4(const __bf16* p) {
  i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LA_LDS i16x4*)(p));
  return __builtin_bit_cast(bf16x4, r);
}

__device__ __forceinline__ bf16x8 cat8(const bf16x4& a, const bf16x4& b) {
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}

// Operand with k running over 8 consecutive rows of a row-major LDS tile X (pitch in
// elements): lane (c = l%32, h = l/32) receives X[r0 + 8h + 0..7][c0 + c].
__device__ __forceinline__ bf16x8 ld_rows8(const __bf16* X, int pitch, int r0, int c0, int lane) {
  const int L = lane & 15, g = lane >> 4;            // 16-lane group g = 0..3
  const int col = c0 + 16 * (g & 1) + 4 * (L & 3);
  const int row = r0 + 8 * (g >> 1) + (L >> 2);
  bf16x4 lo = lds_read_tr4(X + row * pitch + col);
  bf16x4 hi = lds_read_tr4(X + (row + 4) * pitch + col);
  return cat8(lo, hi);
}

// Same, but the 8 rows follow the D-tile feedback order of k-half q:
// rows r0 + 16q + {4h..4h+3, 8+4h..8+4h+3}.
__device__ __forceinline__ bf16x8 ld_rows8_perm(const __bf16* X, int pitch, int r0, int q, int c0, int lane) {
  const int L = lane & 15, g = lane >> 4;
  const int col = c0 + 16 * (g & 1) + 4 * (L & 3);
  const int row = r0 + 16 * q + 4 * (g >> 1) + (L >> 2);
  bf16x4 a = lds_read_tr4(X + row * pitch + col);
  bf16x4 b = lds_read_tr4(X + (row + 8) * pitch + col);
  return cat8(a, b);
}

// Operand with k running along a row: lane (m = l%32, h) receives X[r0 + m][k0 + 8h + 0..7].
__device__ __forceinline__ bf16x8 ld_cols8(const __bf16* X, int pitch, int r0, int k0, int lane) {
  const int m = lane & 31, h = lane >> 5;
  return *(const bf16x8*)(X + (r0 + m) * pitch + k0 + 8 * h);
}

// Same in the D-tile feedback order of k-half q: X[r0 + m][k0 + 16q + {4h..4h+3, 8+4h..8+4h+3}].
__device__ __forceinline__ bf16x8 ld_cols8_perm(const __bf16* X, int pitch, int r0, int k0, int q, int lane) {
  const int m = lane & 31, h = lane >> 5;
  const __bf16* p = X + (r0 + m) * pitch + k0 + 16 * q + 4 * h;
  bf16x4 a = *(const bf16x4*)(p);
  bf16x4 b = *(const bf16x4*)(p + 8);
  return cat8(a, b);
}

// Buffer resource over [p, p + bytes) (gfx9 family: raw buffer, no stride). A buffer
// load at an offset past `bytes` returns zeros instead of touching memory, which is
// how ragged tails are read without branches. Token tiles are read once per pass and not
// reused by the workgroup that loads them, so their loads carry the non-temporal bit
// (cache-policy operand 2): the 128k retention call went 3.07 -> 3.03 ms.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2));
}
// Same with a wave-uniform part of the offset in the scalar offset operand, so loads
// that differ only by a constant stride share one offset register.
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 2));
}

// Bound of a buffer resource over `rows` token rows spaced `stride` bytes apart, each
// `row_bytes` long: 0 when rows <= 0, so every load reads zero and no store lands. A row
// at or past `rows` starts at or beyond the bound (stride >= row_bytes).
__device__ __forceinline__ uint32_t rows_extent(int rows, uint32_t stride, uint32_t row_bytes) {
  return rows > 0 ? (uint32_t)(rows - 1) * stride + row_bytes : 0u;
}

// Four consecutive outputs at element offset `elem` of an fp32 (OBF false) or bf16 (OBF
// true, each value rounded to nearest even) output tensor.
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
template <bool OBF>
__device__ __forceinline__ void store_out4(__amdgpu_buffer_rsrc_t r, uint32_t elem, float a, float b, float c,
                                           float d) {
  if (OBF) {
    const bf16x2 ab = __builtin_convertvector((f32x2){a, b}, bf16x2);
    const bf16x2 cd = __builtin_convertvector((f32x2){c, d}, bf16x2);
    const u32x2 w = {__builtin_bit_cast(uint32_t, ab), __builtin_bit_cast(uint32_t, cd)};
    __builtin_amdgcn_raw_buffer_store_b64(w, r, elem * 2, 0, 0);
  } else {
    const u32x4 w = {__float_as_uint(a), __float_as_uint(b), __float_as_uint(c), __float_as_uint(d)};
    __builtin_amdgcn_raw_buffer_store_b128(w, r, elem * 4, 0, 0);
  }
}
template <bool OBF>
__device__ __forceinline__ void store_out1(__amdgpu_buffer_rsrc_t r, uint32_t elem, float x) {
  if (OBF)
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, (__bf16)x), r, elem * 2, 0, 0);
  else
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, elem * 4, 0, 0);
}

// An integer the optimiser must treat as unknown. Used for per-lane LDS base addresses:
// kept in one register each, with every access a base plus an immediate offset, rather
// than the constant parts folded back in and a register materialised per access (the
// DS immediate only reaches 64 KiB, less than the LDS image of the prefill kernels).
__device__ __forceinline__ int pin(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// XOR-swizzled row-major tiles (no padding, pitch = D elements): the 16-byte chunk c of
// row r is stored at chunk c ^ swz<D>(r). The pattern keeps both access kinds free of
// LDS bank conflicts -- 16 rows read at one chunk (row operands) and 4 consecutive rows
// read at one 32-byte pair of chunks (transpose reads).
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return ((r & 7) << 1) | ((r >> 3) & 1);
  else return (((r >> 1) & 3) << 1) | ((r >> 3) & 1);
}
template <int D>
__device__ __forceinline__ int swz_off(int row, int col) {
  return row * D + ((((col >> 3) ^ swz<D>(row)) << 3) | (col & 7));
}
// Swizzled-tile versions of the operand loaders above.
template <int D>
__device__ __forceinline__ bf16x8 ld_cols8_swz(const __bf16* X, int r0, int k0, int lane) {
  const int m = lane & 31, h = lane >> 5;
  return *(const bf16x8*)(X + swz_off<D>(r0 + m, k0 + 8 * h));
}
template <int D>
__device__ __forceinline__ bf16x8 ld_rows8_swz(const __bf16* X, int r0, int c0, int lane) {
  const int L = lane & 15, g = lane >> 4;
  const int col = c0 + 16 * (g & 1) + 4 * (L & 3);
  const int row = r0 + 8 * (g >> 1) + (L >> 2);
  bf16x4 lo = lds_read_tr4(X + swz_off<D>(row, col));
  bf16x4 hi = lds_read_tr4(X + swz_off<D>(row + 4, col));
  return cat8(lo, hi);
}

// Workgroup barrier for LDS hand-offs only. __syncthreads() also orders global memory,
// which makes every wave wait for all of its outstanding global loads and stores
// (s_waitcnt vmcnt(0)) -- including the next chunk's prefetched tiles and this chunk's
// output stores, which would serialise memory traffic with the matrix work. Here each
// wave only waits for its own LDS operations (lgkmcnt(0); vmcnt and expcnt left at
// their maxima) before the hardware barrier; the empty asm statements keep the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Wait for every outstanding vector-memory access of this wave (vmcnt 0; lgkmcnt and
// expcnt left at their maxima). Used where a loop is entered with loads in flight, so the
// wait the compiler inserts at the loop header only has to cover the loop's own accesses.
__device__ __forceinline__ void vm_drain() { __builtin_amdgcn_s_waitcnt(0x0f70); }

// Row index (within a 32x32 D-tile) of accumulator register r in lane l.
__device__ __forceinline__ int dtile_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// gamma^n for n >= 0 from log2(gamma) (<= 0); exactly 1 when log2g == 0.
__device__ __forceinline__ float gpow(float log2g, float n) { return log2g == 0.f ? 1.f : exp2f(n * log2g); }

__device__ __forceinline__ float elu1(float x) { return x > 0.f ? x + 1.f : __expf(x); }

// Sum over each DPP row of 16 lanes (lanes 16r .. 16r + 15), left in every lane of the row:
// adds whose second operand is a DPP view (quad permutations, then the half-row and row
// mirrors), so no LDS-routed lane permutes.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_mov<0x141>(v);  // row_half_mirror: lane i of 8 <- lane 7 - i
  v += dpp_mov<0x140>(v);  // row_mirror: lane i of 16 <- lane 15 - i
  return v;
}

// 2^x by the hardware instruction alone (about 1 ulp), without the library's rescaling of
// arguments below -126: results under the smallest normal float flush to zero. Used for
// feature values and for decay factors gamma^n (n >= 0), where such a value is lost against the
// fp32 rounding of any sum it enters; the library form spends four more VALU instructions per
// value on that range.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace la
