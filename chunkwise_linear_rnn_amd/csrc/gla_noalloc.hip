// Allocation-free variant of the layer forward, for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that forbid it):
// gla_chunk_fwd with its scratch space taken from a fixed device array of this library
// instead of a caller workspace.  It launches exactly the kernels of gla_chunk_fwd.
//
// The array lives in this source file's code object, so it is placed on a device only
// when this entry point first runs there, and stays until the process ends.  Its device
// address comes from hipGetSymbolAddress once per device (with that device current);
// host code never uses the array's own name as an address.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <mutex>

#include "gla.h"

namespace {

constexpr size_t kScratchBytes = size_t(128) << 20;   // GLA_NOALLOC_SCRATCH_BYTES
static_assert(kScratchBytes == GLA_NOALLOC_SCRATCH_BYTES, "header and library agree");

__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// The scratch array's address on the current device, looked up on first use there.
gla_status_t scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return GLA_ERR_DEVICE;
  if (dev >= kMaxDevices) return GLA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return GLA_ERR_DEVICE;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return GLA_OK;
}

}  // namespace

extern "C" gla_status_t gla_chunk_fwd_noalloc(const gla_desc_t* d, const void* q, const void* k,
                                              const void* v, const void* log_alpha,
                                              const float* S0, void* o, float* S_T,
                                              void* stream) {
  // everything that can be refused is refused before the device is touched
  size_t need = 0;
  gla_status_t st = gla_workspace_bytes(d, GLA_PASS_FWD, &need);
  if (st != GLA_OK) return st;
  if (need > kScratchBytes) return GLA_ERR_WORKSPACE;
  const long long bh = (long long)d->B * d->H;
  if (bh == 0 || d->T == 0 || need == 0)   // nothing uses scratch: the plain entry point
    return gla_chunk_fwd(d, q, k, v, log_alpha, S0, o, S_T, nullptr, 0, stream);
  if (!q || !k || !v || !log_alpha || !o) return GLA_ERR_INVALID_ARG;
  void* ws = nullptr;
  if ((st = scratch_on_current_device(&ws)) != GLA_OK) return st;
  return gla_chunk_fwd(d, q, k, v, log_alpha, S0, o, S_T, ws, kScratchBytes, stream);
}
