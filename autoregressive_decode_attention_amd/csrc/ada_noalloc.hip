// ada_noalloc.hip -- the library's static scratch buffer, for the decode
// entry point that allocates nothing (ada_decode_attn_gqa_noalloc).
//
// A split decode call keeps its per-split partial results in device scratch
// memory. The regular entry points take that scratch from the caller (a
// workspace argument); callers that cannot allocate -- code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc -- use this
// file-scope array instead. Each device that loads the library holds its own
// copy, at its own address, until the process ends. In host code the array's
// name is not a device address: the address is fetched once per device with
// hipGetSymbolAddress (with that device current) and only that pointer is
// handed to kernels.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "ada_internal.h"

namespace ada {
namespace {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxScratchDevices];
std::mutex g_scratch_mutex;

}  // namespace

hipError_t scratch_buffer(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (p == nullptr) return hipErrorInvalidSymbol;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace ada
