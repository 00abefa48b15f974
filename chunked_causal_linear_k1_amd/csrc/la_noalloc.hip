// la_noalloc.hip -- lin_attn_prefill_noalloc: the prefill of lin_attn_prefill for callers that
// cannot allocate device memory (work under HIP graph capture, serving loops and harnesses that
// forbid allocation).
//
// The one device buffer the prefill needs beyond its inputs and outputs is the workspace of
// segment summary records (written by the summary pass, turned into exclusive prefixes by the
// scan, read by the output pass). Here it is a file-scope device array, `scratch`, which every
// device the library runs on holds (one copy per device) from when the library's code object
// is loaded there until the process ends. In host code `scratch` only names the symbol: its
// device address on the current device comes from hipGetSymbolAddress, looked up once per
// device and kept in g_scratch, and only that address is ever handed to a kernel.
//
// Nothing in the records needs to start at zero: the summary pass writes every record the scan
// reads. Calls on one device share the array, so calls that overlap in time there race.
#include <mutex>

#include "la_kernels.hpp"

namespace {

static __device__ __align__(256) unsigned char scratch[LA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // scratch's address on each device, once looked up

la_status scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return LA_ERR_HIP;
  if (dev >= kMaxDevices) return LA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return LA_ERR_HIP;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return LA_OK;
}

}  // namespace

extern "C" la_status lin_attn_prefill_noalloc(const la_prefill_desc* d, const void* q, const void* k,
                                              const void* v, const float* gamma, const void* prf_w,
                                              const float* init_S, const float* init_Z, void* o, float* final_S,
                                              float* final_Z, hipStream_t stream) {
  // host-only checks first: a call the scratch cannot serve is refused before the device is touched
  la_status st = la::prefill_capped_check(d, LA_NOALLOC_SCRATCH_BYTES);
  if (st != LA_OK) return st;
  void* ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st != LA_OK) return st;
  return la::prefill_capped(d, q, k, v, gamma, prf_w, init_S, init_Z, o, final_S, final_Z, ws,
                            LA_NOALLOC_SCRATCH_BYTES, stream);
}
