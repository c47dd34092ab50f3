// The per-GPU buffer behind kvq_attn_decode_noalloc: decode-step attention
// for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid allocation).
//
// The buffer is file-scope device memory: every GPU the library runs on
// holds its own copy, at its own address, until the process ends.  Host code
// never passes the array's name to a kernel (on the host it is only a
// handle); it looks the device address up once per device with
// hipGetSymbolAddress and passes that, exactly as a caller's workspace.
// Every call on one GPU shares that GPU's copy: calls that overlap on one
// GPU race.  Nothing in it needs to start at zero (each split writes its
// whole partial result before the combine reads it).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "kvq_internal.hpp"

namespace kvq {

namespace {

__device__ __attribute__((aligned(256))) uint8_t scratch[kAttnScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};

}  // namespace

hipError_t attn_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace kvq
