// ada_measure.hip -- a measurement kernel of libada: a plain streaming read
// of a device buffer, the floor a decode call's K/V stream is measured
// against.
//
// [DECODE-FASTPATH] (Cuda-Compute-OSS issue #343, "Current limitation") puts
// the whole cost of a one-token decode in reading K and V once. The peak of
// the memory is a published figure; what one launch can stream on this
// device at a given size is measured here with the loads the decode kernel
// uses (16-byte nontemporal loads, fully coalesced) and nothing else.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ada_internal.h"

namespace ada {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 8;  // 16-byte loads in flight per lane

// Workgroup w reads the 16-byte chunks w * 256 + tid, then every
// gridDim.x * 256 chunks after that, kReadUnroll loads issued before any is
// used; the xor of everything read is reduced per wavefront and written to
// sink[w * 4 + wave], so no load can be dropped.
__global__ __launch_bounds__(kReadThreads) void hbm_read_kernel(const u32x4* __restrict__ src, size_t chunks,
                                                                uint32_t* __restrict__ sink) {
  const size_t stride = static_cast<size_t>(gridDim.x) * kReadThreads;
  size_t i = static_cast<size_t>(blockIdx.x) * kReadThreads + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + (kReadUnroll - 1) * stride < chunks; i += kReadUnroll * stride) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u];
  }
  for (; i < chunks; i += stride) acc ^= __builtin_nontemporal_load(src + i);
  uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
  for (int off = 32; off > 0; off >>= 1) x ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(x), off));
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * (kReadThreads / 64) + threadIdx.x / 64] = x;
}

}  // namespace

hipError_t launch_hbm_read(const void* src, size_t bytes, uint32_t* sink, int workgroups, hipStream_t stream) {
  hipLaunchKernelGGL(hbm_read_kernel, dim3(workgroups), dim3(kReadThreads), 0, stream,
                     static_cast<const u32x4*>(src), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace ada
