// Streaming reference kernels for bench.py: the byte patterns of the two prefill passes with
// none of the method's arithmetic, as a measured practical ceiling for the memory-bound
// kernels on the same box. Measurement only; not part of liblinattn.
//
//   ccl_stream_mix:   o[i] = q[i] + k[i] * v[i], bf16 in, fp32 out (the output pass's mix:
//                     6 bytes read and 4 written per element)
//   ccl_stream_read2: sum over i of k[i] * v[i], one partial per wave (the summary pass's
//                     reads: 4 bytes per element, a negligible write)
//
// Both take n (elements, a multiple of 8, 16-byte aligned pointers) and a stream; grid-stride
// loops over 16-byte pieces, 8192 workgroups of 512 threads. Return 0 or a hipError_t.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kGrid = 8192, kBlock = 512;

__device__ __forceinline__ float bf_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

__global__ __launch_bounds__(kBlock) void k_stream_mix(const uint4* __restrict__ q, const uint4* __restrict__ k,
                                                       const uint4* __restrict__ v, f32x4* __restrict__ o,
                                                       size_t n8) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n8; i += stride) {
    const uint4 a = q[i], b = k[i], c = v[i];
    const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w}, cw[4] = {c.x, c.y, c.z, c.w};
    f32x4 r[2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      r[j / 2][2 * (j % 2)] = bf_lo(aw[j]) + bf_lo(bw[j]) * bf_lo(cw[j]);
      r[j / 2][2 * (j % 2) + 1] = bf_hi(aw[j]) + bf_hi(bw[j]) * bf_hi(cw[j]);
    }
    o[2 * i] = r[0];
    o[2 * i + 1] = r[1];
  }
}

__global__ __launch_bounds__(kBlock) void k_stream_read2(const uint4* __restrict__ k, const uint4* __restrict__ v,
                                                         float* __restrict__ part, size_t n8) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  float acc = 0.f;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n8; i += stride) {
    const uint4 b = k[i], c = v[i];
    const uint32_t bw[4] = {b.x, b.y, b.z, b.w}, cw[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) acc += bf_lo(bw[j]) * bf_lo(cw[j]) + bf_hi(bw[j]) * bf_hi(cw[j]);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if ((threadIdx.x & 63) == 0) part[(blockIdx.x * (size_t)blockDim.x + threadIdx.x) / 64] = acc;
}

bool ok16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" {

// partial sums written by ccl_stream_read2 (floats)
size_t ccl_stream_read2_parts(void) { return (size_t)kGrid * kBlock / 64; }

int ccl_stream_mix(const void* q, const void* k, const void* v, float* o, size_t n, hipStream_t stream) {
  if (n % 8 || !ok16(q) || !ok16(k) || !ok16(v) || !ok16(o)) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(k_stream_mix, dim3(kGrid), dim3(kBlock), 0, stream, (const uint4*)q, (const uint4*)k,
                     (const uint4*)v, (f32x4*)o, n / 8);
  return (int)hipGetLastError();
}

int ccl_stream_read2(const void* k, const void* v, float* part, size_t n, hipStream_t stream) {
  if (n % 8 || !ok16(k) || !ok16(v)) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(k_stream_read2, dim3(kGrid), dim3(kBlock), 0, stream, (const uint4*)k, (const uint4*)v, part,
                     n / 8);
  return (int)hipGetLastError();
}

}  // extern "C"
