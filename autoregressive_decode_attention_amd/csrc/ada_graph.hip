// ada_graph.hip -- the one kernel of the graph-captured decode step: the
// device-side advance of the token positions between two steps.
//
// Decode step i after a T-token prompt attends over T + i + 1 slots, so the
// position grows by one per generated token ([ACTIVE-PREFIX] section 2, which
// keeps it a host integer so that no step reads it back from the device).
// Here the positions stay on the device and this kernel advances them, so a
// whole multi-layer step replays as one graph with no host work at all.
#include <hip/hip_runtime.h>

#include "ada_internal.h"

namespace ada {
namespace {

// pos[b] += delta for b < batch; one thread per row.
__global__ __launch_bounds__(256) void advance_positions_kernel(int32_t* __restrict__ pos, int batch, int delta) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < batch) pos[b] += delta;
}

}  // namespace

hipError_t launch_advance_positions(int32_t* pos, int batch, int delta, hipStream_t stream) {
  const int blocks = (batch + 255) / 256;
  hipLaunchKernelGGL(advance_positions_kernel, dim3(blocks), dim3(256), 0, stream, pos, batch, delta);
  return hipGetLastError();
}

}  // namespace ada
