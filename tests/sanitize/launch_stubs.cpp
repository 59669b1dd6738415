// Host-only stand-ins for the gfx950 kernel launchers of libada, so that the
// C ABI layer (ada_api.cpp) can be built with a host compiler under
// AddressSanitizer and UndefinedBehaviorSanitizer and driven without a GPU.
// A stub enqueues nothing; it checks the launch description the ABI layer
// built against what every launch must satisfy and aborts otherwise (the
// sanitizer run then fails).
#include <cstdio>
#include <cstdint>
#include <cstdlib>

#include "ada_internal.h"

namespace {
void require(bool ok, const char* what) {
  if (!ok) {
    std::fprintf(stderr, "launch stub: %s\n", what);
    std::abort();
  }
}
}  // namespace

namespace ada {

int prefill_rows_per_workgroup(int, int, int, int, int) { return 64; }

hipError_t launch_prefill(const PrefillLaunch& p) {
  require(p.batch > 0 && p.q_len > 0 && p.n_head % p.n_kv_head == 0, "prefill shape");
  require(p.q && p.k_cache && p.v_cache && p.out, "prefill pointers");
  return hipSuccess;
}

hipError_t launch_prefill_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache, const int32_t*,
                                 int batch, int n_kv_head, int q_len, int capacity, hipStream_t) {
  require(k_new && v_new && k_cache && v_cache && batch > 0 && n_kv_head > 0 && q_len > 0 && capacity > 0,
          "prefill append arguments");
  return hipSuccess;
}

hipError_t launch_partial(const DecodeLaunch& p) {
  require(p.batch > 0 && p.n_kv_head > 0 && p.n_head % p.n_kv_head == 0, "partial shape");
  require(p.splits >= 1 && p.splits <= kMaxSplits && p.chunk >= 0, "partial plan");
  require(p.max_kv_len >= 1 && p.max_kv_len <= p.capacity, "partial length bound");
  require(p.chunk == 0 || static_cast<long>(p.splits) * p.chunk >= p.max_kv_len, "partial plan covers the prefix");
  require(p.direct ? p.out != nullptr : p.workspace != nullptr, "partial destination");
  return hipSuccess;
}

hipError_t launch_combine(const CombineLaunch& p) {
  require(p.workspace && p.out && p.batch > 0 && p.splits >= 1 && p.splits <= kMaxSplits, "combine arguments");
  return hipSuccess;
}

hipError_t launch_rope_kv_append(const void*, void*, const void* k_new, const void* v_new, const void* cos,
                                 const void* sin, void* k_cache, void* v_cache, const int32_t* pos, int batch, int,
                                 int n_kv_head, int capacity, int, hipStream_t) {
  require(k_new && v_new && cos && sin && k_cache && v_cache && pos && batch > 0 && n_kv_head > 0 && capacity > 0,
          "rope append arguments");
  return hipSuccess;
}

hipError_t launch_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache, const int32_t* pos,
                            int batch, int n_kv_head, int capacity, hipStream_t) {
  require(k_new && v_new && k_cache && v_cache && pos && batch > 0 && n_kv_head > 0 && capacity > 0,
          "append arguments");
  return hipSuccess;
}

hipError_t launch_advance_positions(int32_t* pos, int batch, int, hipStream_t) {
  require(pos && batch > 0, "advance arguments");
  return hipSuccess;
}

// Stand-in for the static scratch buffer: a fixed, never dereferenced address.
hipError_t scratch_buffer(void** ptr) {
  *ptr = reinterpret_cast<void*>(uintptr_t{0x7f0000000000});
  return hipSuccess;
}

hipError_t launch_hbm_read(const void* src, size_t bytes, uint32_t* sink, int workgroups, hipStream_t) {
  require(src && sink && bytes > 0 && bytes % 16 == 0 && workgroups > 0, "read probe arguments");
  return hipSuccess;
}

}  // namespace ada
