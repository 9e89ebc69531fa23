// noalloc.hip -- ssd_chunk_bwd_noalloc: the chunked backward with its workspace
// in a device array of fixed size that the library owns, for callers that
// cannot allocate device memory (code under HIP graph capture, serving loops,
// harnesses that forbid hipMalloc).
//
// The array lives in this translation unit's code object, so its device memory
// is taken when the code object is first loaded on a device (the first call of
// this entry point there) and held until the process ends.  Each device has
// its own copy at its own address: the address is looked up once per device
// with hipGetSymbolAddress and only that address is handed to the kernels (the
// array's name in host code is a host-side stand-in, not a device address).
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "../../include/ssmvjp.h"

namespace {

static_assert(SSMVJP_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size must keep 256-byte alignment");
static __device__ __align__(256) unsigned char scratch[SSMVJP_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_setup;

// The device address of `scratch` on the current device (looked up on first use).
ssmvjp_status scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return SSMVJP_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return SSMVJP_EUNSUPPORTED;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_setup);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      void* q = nullptr;
      if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr) return SSMVJP_EHIP;
      g_scratch[dev].store(q, std::memory_order_release);
      p = q;
    }
  }
  *out = p;
  return SSMVJP_OK;
}

}  // namespace

extern "C" ssmvjp_status ssd_chunk_bwd_noalloc(const ssmvjp_ssd_desc* desc, const void* x_or_v,
                                               const float* dt_or_da, const float* A, const void* B, const void* C,
                                               const float* s0, const void* dy, const float* ds_final,
                                               void* dx_or_dv, float* d_dt_or_dda, void* dB, void* dC, float* d_s0,
                                               void* stream) {
  // sizes beyond the array are refused before anything else happens
  size_t need = 0;
  ssmvjp_status s = ssd_chunk_bwd_workspace(desc, &need);
  if (s != SSMVJP_OK) return s;
  if (need > (size_t)SSMVJP_NOALLOC_SCRATCH_BYTES) return SSMVJP_EWORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    s = scratch_ptr(&ws);
    if (s != SSMVJP_OK) return s;
  }
  // every region of the chunked workspace is written before it is read within
  // one call, so nothing needs clearing between calls
  return ssd_chunk_bwd(desc, x_or_v, dt_or_da, A, B, C, s0, dy, ds_final, dx_or_dv, d_dt_or_dda, dB, dC, d_s0, ws,
                       need > 0 ? (size_t)SSMVJP_NOALLOC_SCRATCH_BYTES : 0, stream);
}
