// ada_internal.h -- launchers shared between the C ABI layer (ada_api.cpp)
// and the kernels (ada_kernels.hip). Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ada {

constexpr int kHeadDim = 128;
constexpr int kMaxGroup = 8;
constexpr int kThreads = 256;    // 4 wavefronts of 64
constexpr int kTileRows = 64;    // slot granularity the heuristic rounds split ranges to
constexpr int kMaxSplits = 256;  // equals ADA_MAX_SPLITS
// Bytes of the static per-device scratch buffer of the allocation-free
// decode entry point (equals ADA_NOALLOC_SCRATCH_BYTES).
constexpr size_t kScratchBytes = size_t(4) << 20;

// Workspace layout for `splits` splits, split-major (the partials of one
// split are contiguous, so partials computed on separate key ranges can be
// concatenated along the split axis and combined together):
//   [ml_offset, +ml_bytes)       float2 (running max in log2 units, sum) per
//                                (split, batch row, query head); m = -inf
//                                marks an empty split
//   [acc_offset, +acc_bytes)     float[head_dim] unnormalised accumulator per
//                                (split, batch row, query head)
struct WorkspaceLayout {
  size_t ml_offset;
  size_t acc_offset;
  size_t total;
};

WorkspaceLayout workspace_layout(int batch, int n_head, int n_kv_head, int head_dim, int splits);

struct DecodeLaunch {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* kv_len;
  const void* k_new;    // decode step: new rows appended at pos (else NULL)
  const void* v_new;
  const int32_t* pos;   // decode step: device slots, or NULL (slot max_kv_len - 1)
  const void* cos;      // decode step with rotary embedding: [B, D] tables (else NULL)
  const void* sin;
  void* out;        // written when direct
  void* workspace;  // partials written when !direct
  int batch, n_head, n_kv_head, capacity, max_kv_len;
  int splits, chunk;  // chunk 0: balanced plan derived on the device from the row lengths
  bool direct;       // one split: write the output, no partials
  float scale_log2;  // scale * log2(e)
  int dtype;         // 0 fp16, 1 bf16
  hipStream_t stream;
};

struct CombineLaunch {
  const void* workspace;
  void* out;
  int batch, n_head, n_kv_head, splits;
  int dtype;
  hipStream_t stream;
  // Balanced plan (the partial launch had chunk == 0): the row lengths it
  // was derived from, so the combine derives the same plan.
  bool balanced = false;
  const int32_t* kv_len = nullptr;
  const int32_t* pos = nullptr;
  bool step = false;  // lengths are pos + 1 (decode step)
  int max_kv_len = 0;
};

struct PrefillLaunch {
  const void* q;        // [B, H_q, T, D]
  const void* k_cache;  // [B, H_kv, S, D]
  const void* v_cache;
  const int32_t* start;  // device [B] first position of each row, or NULL (0)
  void* out;             // [B, H_q, T, D]
  int batch, n_head, n_kv_head, q_len, capacity;
  float scale_log2;
  int dtype;
  int rows_per_workgroup;  // 64 or 128, from prefill_rows_per_workgroup
  hipStream_t stream;
};

// Query rows per prefill workgroup (64 or 128) for a call on a device with
// num_cus compute units; pure host arithmetic.
int prefill_rows_per_workgroup(int batch, int n_head, int n_kv_head, int q_len, int num_cus);

hipError_t launch_prefill(const PrefillLaunch& p);
hipError_t launch_prefill_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                                 const int32_t* start, int batch, int n_kv_head, int q_len, int capacity,
                                 hipStream_t stream);

hipError_t launch_partial(const DecodeLaunch& p);
hipError_t launch_combine(const CombineLaunch& p);

hipError_t launch_rope_kv_append(const void* q, void* q_out, const void* k_new, const void* v_new,
                                 const void* cos, const void* sin, void* k_cache, void* v_cache,
                                 const int32_t* pos, int batch, int n_head, int n_kv_head, int capacity,
                                 int dtype, hipStream_t stream);

hipError_t launch_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                            const int32_t* pos, int batch, int n_kv_head, int capacity,
                            hipStream_t stream);

hipError_t launch_advance_positions(int32_t* pos, int batch, int delta, hipStream_t stream);

// Device address of the current device's static scratch buffer
// (kScratchBytes, 256-byte aligned), fetched once per device.
hipError_t scratch_buffer(void** ptr);

// Streaming read of `bytes` (a multiple of 16) from src by `workgroups`
// 256-thread workgroups; one 32-bit xor per wavefront to sink.
hipError_t launch_hbm_read(const void* src, size_t bytes, uint32_t* sink, int workgroups, hipStream_t stream);

}  // namespace ada
