// ada_api.cpp -- the C ABI of libada: host-side validation, the split
// heuristic, workspace arithmetic and dispatch to the gfx950 kernels.
//
// Every argument is checked before the first HIP call, so a rejected call
// has no effect and the checks run without a GPU. The ABI itself is
// documented in include/ada.h.
#include "ada.h"

#include <atomic>
#include <cmath>
#include <climits>
#include <cstdint>
#include <initializer_list>
#include <vector>

#include "ada_internal.h"

namespace {

thread_local int g_last_hip_error = 0;

// Compute-unit count per HIP device, filled on first use (0 = not yet known).
constexpr int kMaxDevices = 64;
std::atomic<int> g_num_cus[kMaxDevices];

int hip_fail(hipError_t e) {
  g_last_hip_error = static_cast<int>(e);
  return ADA_ERR_HIP;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Product of non-negative factors, saturated at INT64_MAX: size checks on
// arguments of any magnitude never overflow.
int64_t sat_mul(std::initializer_list<int64_t> factors) {
  __int128 p = 1;
  for (int64_t f : factors) {
    p *= f;
    if (p > INT64_MAX) return INT64_MAX;
  }
  return static_cast<int64_t>(p);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int current_device_cus(int* cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev >= 0 && dev < kMaxDevices) {
    int cached = g_num_cus[dev].load(std::memory_order_relaxed);
    if (cached > 0) {
      *cus = cached;
      return ADA_OK;
    }
  }
  int n = 0;
  e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e);
  if (n <= 0) n = 1;
  if (dev >= 0 && dev < kMaxDevices) g_num_cus[dev].store(n, std::memory_order_relaxed);
  *cus = n;
  return ADA_OK;
}

// Split plan: chunk = slots per split; splits = number of split workgroups
// per (batch row, KV head) actually launched.
struct Plan {
  int splits;
  int chunk;
};

// Forced split count: near-equal ranges, no rounding beyond one slot.
Plan forced_plan(int max_kv_len, int requested) {
  if (max_kv_len <= 0) return {1, 1};
  int chunk = static_cast<int>(ceil_div(max_kv_len, requested));
  if (chunk < 1) chunk = 1;
  return {static_cast<int>(ceil_div(max_kv_len, chunk)), chunk};
}

// Heuristic (measured on MI355X, cold HBM): one 4-wave workgroup per compute
// unit (a streaming read on this device is fastest with one workgroup per
// compute unit, and two per unit only add partials); splits never shorter
// than 64 slots (one workgroup tile); while a split would exceed 8192 slots,
// double the split count so long rows still spread over every compute unit.
// Ranges are rounded up to whole 64-slot tiles.
Plan heuristic_plan(int batch, int n_head, int n_kv_head, int max_kv_len, int num_cus) {
  if (batch <= 0 || n_head <= 0 || n_kv_head <= 0 || max_kv_len <= 0 || num_cus <= 0)
    return {1, max_kv_len > 0 ? max_kv_len : 1};
  // A prefix of at most four 64-slot tiles: one workgroup per (row, KV head)
  // streams it faster than a split call pays for its combine launch
  // (measured on MI355X for 8-32 units at 235-256 slots).
  if (max_kv_len <= 4 * ada::kTileRows)
    return {1, static_cast<int>(ceil_div(max_kv_len, ada::kTileRows) * ada::kTileRows)};
  const int64_t units = static_cast<int64_t>(batch) * n_kv_head;
  int64_t splits = ceil_div(num_cus, units);
  const int64_t by_len = ceil_div(max_kv_len, ada::kTileRows);
  if (splits > by_len) splits = by_len;
  if (splits < 1) splits = 1;
  while (ceil_div(max_kv_len, splits) > 8192 && splits * 2 <= by_len) splits *= 2;
  if (splits > ADA_MAX_SPLITS) splits = ADA_MAX_SPLITS;
  int64_t chunk = ceil_div(ceil_div(max_kv_len, splits), ada::kTileRows) * ada::kTileRows;
  return {static_cast<int>(ceil_div(max_kv_len, chunk)), static_cast<int>(chunk)};
}

}  // namespace

namespace ada {

WorkspaceLayout workspace_layout(int batch, int n_head, int n_kv_head, int head_dim, int splits) {
  WorkspaceLayout w{};
  auto round256 = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  const size_t rows = static_cast<size_t>(batch) * n_head * splits;
  (void)n_kv_head;
  w.ml_offset = 0;
  w.acc_offset = w.ml_offset + round256(rows * 2 * sizeof(float));
  w.total = w.acc_offset + round256(rows * static_cast<size_t>(head_dim) * sizeof(float));
  return w;
}

}  // namespace ada

extern "C" {

int ada_abi_version(void) { return ADA_ABI_VERSION; }

const char* ada_status_string(int status) {
  switch (status) {
    case ADA_OK: return "ok";
    case ADA_ERR_NULL: return "a required pointer is NULL";
    case ADA_ERR_SHAPE: return "batch, head count, capacity or max_kv_len out of range";
    case ADA_ERR_GQA: return "n_head must be a multiple of n_kv_head with group size 1..8";
    case ADA_ERR_DTYPE: return "dtype must be ADA_F16 or ADA_BF16";
    case ADA_ERR_HEAD_DIM: return "head_dim must be 128";
    case ADA_ERR_SCALE: return "scale must be finite";
    case ADA_ERR_WORKSPACE: return "workspace missing or too small for the split count";
    case ADA_ERR_SPLITS: return "num_splits out of range";
    case ADA_ERR_ALIGN: return "device pointers must be 16-byte aligned";
    case ADA_ERR_HIP: return "HIP runtime error (see ada_last_hip_error)";
    case ADA_ERR_DEVICE: return "step graph launched on another device than the one it was created on";
    case ADA_ERR_SCRATCH: return "the call needs more split scratch than the library's static buffer holds";
    default: return "unknown status";
  }
}

int ada_last_hip_error(void) { return g_last_hip_error; }

int ada_device_num_cus(int device, int* num_cus) {
  if (!num_cus) return ADA_ERR_NULL;
  int n = 0;
  hipError_t e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, device);
  if (e != hipSuccess) return hip_fail(e);
  *num_cus = n;
  return ADA_OK;
}

int ada_prefill_rows_per_workgroup(int batch, int n_head, int n_kv_head, int q_len, int num_cus) {
  return ada::prefill_rows_per_workgroup(batch, n_head, n_kv_head, q_len, num_cus);
}

int ada_decode_num_splits(int batch, int n_head, int n_kv_head, int max_kv_len, int num_cus) {
  return heuristic_plan(batch, n_head, n_kv_head, max_kv_len, num_cus).splits;
}

int ada_decode_plan(int batch, int n_head, int n_kv_head, int max_kv_len, int num_splits, int num_cus, int* splits,
                    int* chunk) {
  if (!splits || !chunk) return ADA_ERR_NULL;
  if (num_splits < 0 || num_splits > ADA_MAX_SPLITS) return ADA_ERR_SPLITS;
  const Plan p = num_splits > 0 ? forced_plan(max_kv_len, num_splits)
                                : heuristic_plan(batch, n_head, n_kv_head, max_kv_len, num_cus);
  *splits = p.splits;
  *chunk = p.chunk;
  return ADA_OK;
}

size_t ada_decode_workspace_bytes(int batch, int n_head, int n_kv_head, int head_dim, int num_splits) {
  if (num_splits < 1 || batch <= 0 || n_head <= 0 || n_kv_head <= 0 || head_dim <= 0) return 0;
  // sizes no call could use (and that would wrap size_t) report 0
  if (sat_mul({batch, n_head, num_splits, static_cast<int64_t>(head_dim) + 2, 4}) > (int64_t(1) << 56)) return 0;
  return ada::workspace_layout(batch, n_head, n_kv_head, head_dim, num_splits).total;
}

int ada_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                  const int32_t* pos, int batch, int n_kv_head, int capacity, int head_dim,
                  int dtype, void* stream) {
  if (dtype != ADA_F16 && dtype != ADA_BF16) return ADA_ERR_DTYPE;
  if (batch < 0 || n_kv_head <= 0 || capacity <= 0) return ADA_ERR_SHAPE;
  if (head_dim != ada::kHeadDim) return ADA_ERR_HEAD_DIM;
  // the launch indexes the rows' 16-byte chunks with 32-bit ints
  if (sat_mul({batch, n_kv_head, ada::kHeadDim * 2 / 16}) > INT32_MAX - 255) return ADA_ERR_SHAPE;
  if (batch == 0) return ADA_OK;
  if (!k_new || !v_new || !k_cache || !v_cache || !pos) return ADA_ERR_NULL;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache))
    return ADA_ERR_ALIGN;
  hipError_t e = ada::launch_kv_append(k_new, v_new, k_cache, v_cache, pos, batch, n_kv_head,
                                       capacity, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ADA_OK : hip_fail(e);
}

int ada_rope_kv_append(const void* q, void* q_out, const void* k_new, const void* v_new, const void* cos,
                       const void* sin, void* k_cache, void* v_cache, const int32_t* pos, int batch,
                       int n_head, int n_kv_head, int capacity, int head_dim, int dtype, void* stream) {
  if (dtype != ADA_F16 && dtype != ADA_BF16) return ADA_ERR_DTYPE;
  if (batch < 0 || n_kv_head <= 0 || capacity <= 0 || n_head < 0) return ADA_ERR_SHAPE;
  if (head_dim != ada::kHeadDim) return ADA_ERR_HEAD_DIM;
  if ((q == nullptr) != (q_out == nullptr)) return ADA_ERR_NULL;
  if (q != nullptr && n_head <= 0) return ADA_ERR_SHAPE;
  const int64_t heads = (q ? static_cast<int64_t>(n_head) : 0) + n_kv_head;
  if (sat_mul({batch, heads, 16}) > INT32_MAX - 255) return ADA_ERR_SHAPE;
  if (batch == 0) return ADA_OK;
  if (!k_new || !v_new || !cos || !sin || !k_cache || !v_cache || !pos) return ADA_ERR_NULL;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(cos) || !aligned16(sin) ||
      !aligned16(k_cache) || !aligned16(v_cache) || (q && (!aligned16(q) || !aligned16(q_out))))
    return ADA_ERR_ALIGN;
  hipError_t e = ada::launch_rope_kv_append(q, q_out, k_new, v_new, cos, sin, k_cache, v_cache, pos, batch,
                                            n_head, n_kv_head, capacity, dtype,
                                            static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ADA_OK : hip_fail(e);
}

}  // extern "C"

namespace {

// Checks shared by the decode entry points; fills the launch description
// except out/workspace/direct. Returns ADA_OK or the status to report.
int prepare_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* kv_len,
                   int batch, int n_head, int n_kv_head, int head_dim, int capacity,
                   int max_kv_len, float scale, int dtype, int num_splits, void* stream,
                   ada::DecodeLaunch* p) {
  if (dtype != ADA_F16 && dtype != ADA_BF16) return ADA_ERR_DTYPE;
  if (batch < 0 || n_head <= 0 || n_kv_head <= 0 || capacity <= 0) return ADA_ERR_SHAPE;
  if (n_head % n_kv_head != 0 || n_head / n_kv_head > ada::kMaxGroup) return ADA_ERR_GQA;
  if (head_dim != ada::kHeadDim) return ADA_ERR_HEAD_DIM;
  if (!std::isfinite(scale)) return ADA_ERR_SCALE;
  if (max_kv_len <= 0) max_kv_len = capacity;
  if (max_kv_len > capacity) return ADA_ERR_SHAPE;
  if (num_splits < 0 || num_splits > ADA_MAX_SPLITS) return ADA_ERR_SPLITS;
  if (batch > 65535 || n_kv_head > 65535) return ADA_ERR_SHAPE;  // grid limits
  if (batch == 0) return ADA_OK;
  if (!q || !k_cache || !v_cache) return ADA_ERR_NULL;  // kv_len may be NULL (lockstep rows)
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) return ADA_ERR_ALIGN;

  Plan plan{};
  if (num_splits > 0) {
    plan = forced_plan(max_kv_len, num_splits);
  } else {
    int cus = 0;
    int rc = current_device_cus(&cus);
    if (rc != ADA_OK) return rc;
    plan = heuristic_plan(batch, n_head, n_kv_head, max_kv_len, cus);
  }
  *p = ada::DecodeLaunch{};
  p->q = q;
  p->k_cache = k_cache;
  p->v_cache = v_cache;
  p->kv_len = kv_len;
  p->batch = batch;
  p->n_head = n_head;
  p->n_kv_head = n_kv_head;
  p->capacity = capacity;
  p->max_kv_len = max_kv_len;
  p->splits = plan.splits;
  p->chunk = plan.chunk;
  p->scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  p->dtype = dtype;
  p->stream = static_cast<hipStream_t>(stream);
  return ADA_OK;
}

// Rows per call up to which a call with device-side lengths uses the
// balanced plan (each workgroup reads every row's length to find its range).
constexpr int kBalancedMaxBatch = 64;

// Prefixes up to which the balanced plan is used: the kernels sum the rows'
// lengths in 32 bits (64 rows of at most 2^25 slots).
constexpr int kBalancedMaxLen = 1 << 25;

// Use the balanced split plan? Only for heuristic split counts (a forced
// count keeps the per-row ranges it asks for), lengths that only the device
// knows, more than one row and at least two splits per row.
bool use_balanced(const ada::DecodeLaunch& p, bool device_lengths, int num_splits) {
  return device_lengths && num_splits == 0 && p.batch >= 2 && p.batch <= kBalancedMaxBatch && p.splits >= 2 &&
         p.max_kv_len <= kBalancedMaxLen;
}

int check_workspace(const void* workspace, size_t workspace_bytes, int batch, int n_head,
                    int n_kv_head, int splits) {
  const ada::WorkspaceLayout w = ada::workspace_layout(batch, n_head, n_kv_head, ada::kHeadDim, splits);
  if (w.total - w.acc_offset > static_cast<size_t>(INT32_MAX)) return ADA_ERR_SHAPE;  // 32-bit offsets
  const size_t need = w.total;
  if (!workspace || workspace_bytes < need) return ADA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return ADA_ERR_ALIGN;
  return ADA_OK;
}

}  // namespace

extern "C" {

int ada_decode_attn_gqa_ex(const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* kv_len, int batch, int n_head, int n_kv_head,
                           int head_dim, int capacity, int max_kv_len, float scale, int dtype,
                           void* out, void* workspace, size_t workspace_bytes, void* stream,
                           int num_splits) {
  ada::DecodeLaunch p{};
  int rc = prepare_decode(q, k_cache, v_cache, kv_len, batch, n_head, n_kv_head, head_dim, capacity,
                          max_kv_len, scale, dtype, num_splits, stream, &p);
  if (rc != ADA_OK || batch == 0) return rc;
  if (!out) return ADA_ERR_NULL;
  if (!aligned16(out)) return ADA_ERR_ALIGN;
  p.out = out;
  p.direct = p.splits == 1;
  if (!p.direct) {
    rc = check_workspace(workspace, workspace_bytes, batch, n_head, n_kv_head, p.splits);
    if (rc != ADA_OK) return rc;
    p.workspace = workspace;
  }
  const bool balanced = use_balanced(p, kv_len != nullptr, num_splits);
  if (balanced) p.chunk = 0;
  hipError_t e = ada::launch_partial(p);
  if (e != hipSuccess) return hip_fail(e);
  if (p.direct) return ADA_OK;
  ada::CombineLaunch c{workspace, out, batch, n_head, n_kv_head, p.splits, dtype, p.stream};
  c.balanced = balanced;
  c.kv_len = kv_len;
  c.max_kv_len = p.max_kv_len;
  e = ada::launch_combine(c);
  return e == hipSuccess ? ADA_OK : hip_fail(e);
}

int ada_decode_attn_gqa(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* kv_len, int batch, int n_head, int n_kv_head, int head_dim,
                        int capacity, int max_kv_len, float scale, int dtype, void* out,
                        void* workspace, size_t workspace_bytes, void* stream) {
  return ada_decode_attn_gqa_ex(q, k_cache, v_cache, kv_len, batch, n_head, n_kv_head, head_dim,
                                capacity, max_kv_len, scale, dtype, out, workspace,
                                workspace_bytes, stream, 0);
}

int ada_decode_attn_gqa_noalloc(const void* q, const void* k_cache, const void* v_cache, const int32_t* kv_len,
                                int batch, int n_head, int n_kv_head, int head_dim, int capacity, int max_kv_len,
                                float scale, int dtype, void* out, void* stream, int num_splits) {
  ada::DecodeLaunch p{};
  int rc = prepare_decode(q, k_cache, v_cache, kv_len, batch, n_head, n_kv_head, head_dim, capacity,
                          max_kv_len, scale, dtype, num_splits, stream, &p);
  if (rc != ADA_OK || batch == 0) return rc;
  if (!out) return ADA_ERR_NULL;
  if (!aligned16(out)) return ADA_ERR_ALIGN;
  void* scratch = nullptr;
  size_t scratch_bytes = 0;
  if (p.splits > 1) {
    if (ada::workspace_layout(batch, n_head, n_kv_head, ada::kHeadDim, p.splits).total > ada::kScratchBytes)
      return ADA_ERR_SCRATCH;
    hipError_t e = ada::scratch_buffer(&scratch);
    if (e != hipSuccess) return hip_fail(e);
    scratch_bytes = ada::kScratchBytes;
  }
  return ada_decode_attn_gqa_ex(q, k_cache, v_cache, kv_len, batch, n_head, n_kv_head, head_dim, capacity,
                                max_kv_len, scale, dtype, out, scratch, scratch_bytes, stream, num_splits);
}

}  // extern "C"

namespace {

// A validated decode step: the launch description and whether it uses the
// balanced plan.
struct StepLaunch {
  ada::DecodeLaunch p;
  bool balanced;
};

// Checks of a decode step (with rotary tables when cos/sin are given) and
// its launch plan; nothing is enqueued. batch == 0 leaves s->p.batch == 0.
int prepare_step(const void* q, const void* k_new, const void* v_new, const void* cos, const void* sin,
                 void* k_cache, void* v_cache, const int32_t* pos, int batch, int n_head, int n_kv_head,
                 int head_dim, int capacity, int max_pos, float scale, int dtype, void* out, void* workspace,
                 size_t workspace_bytes, void* stream, int num_splits, StepLaunch* s) {
  if (max_pos < 0 || max_pos >= capacity) {
    if (dtype != ADA_F16 && dtype != ADA_BF16) return ADA_ERR_DTYPE;
    return ADA_ERR_SHAPE;
  }
  ada::DecodeLaunch& p = s->p;
  s->balanced = false;
  int rc = prepare_decode(q, k_cache, v_cache, nullptr, batch, n_head, n_kv_head, head_dim, capacity,
                          max_pos + 1, scale, dtype, num_splits, stream, &p);
  if (rc != ADA_OK) return rc;
  if (batch == 0) {
    p.batch = 0;
    return ADA_OK;
  }
  if (!k_new || !v_new || !out) return ADA_ERR_NULL;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(out)) return ADA_ERR_ALIGN;
  if ((cos == nullptr) != (sin == nullptr)) return ADA_ERR_NULL;
  if (cos && (!aligned16(cos) || !aligned16(sin))) return ADA_ERR_ALIGN;
  p.k_new = k_new;
  p.v_new = v_new;
  p.pos = pos;
  p.cos = cos;
  p.sin = sin;
  p.out = out;
  p.direct = p.splits == 1;
  if (!p.direct) {
    rc = check_workspace(workspace, workspace_bytes, batch, n_head, n_kv_head, p.splits);
    if (rc != ADA_OK) return rc;
    p.workspace = workspace;
  }
  s->balanced = use_balanced(p, pos != nullptr, num_splits);
  if (s->balanced) p.chunk = 0;
  return ADA_OK;
}

// Enqueues a prepared step on `stream`: the partial kernel, then the combine
// kernel when the step has more than one split.
int launch_step(const StepLaunch& s, hipStream_t stream) {
  ada::DecodeLaunch p = s.p;
  if (p.batch == 0) return ADA_OK;
  p.stream = stream;
  hipError_t e = ada::launch_partial(p);
  if (e != hipSuccess) return hip_fail(e);
  if (p.direct) return ADA_OK;
  ada::CombineLaunch c{p.workspace, p.out, p.batch, p.n_head, p.n_kv_head, p.splits, p.dtype, stream};
  c.balanced = s.balanced;
  c.pos = p.pos;
  c.step = true;
  c.max_kv_len = p.max_kv_len;
  e = ada::launch_combine(c);
  return e == hipSuccess ? ADA_OK : hip_fail(e);
}

int decode_step_impl(const void* q, const void* k_new, const void* v_new, const void* cos, const void* sin,
                     void* k_cache, void* v_cache, const int32_t* pos, int batch, int n_head, int n_kv_head,
                     int head_dim, int capacity, int max_pos, float scale, int dtype, void* out,
                     void* workspace, size_t workspace_bytes, void* stream, int num_splits) {
  StepLaunch s{};
  int rc = prepare_step(q, k_new, v_new, cos, sin, k_cache, v_cache, pos, batch, n_head, n_kv_head, head_dim,
                        capacity, max_pos, scale, dtype, out, workspace, workspace_bytes, stream, num_splits, &s);
  if (rc != ADA_OK) return rc;
  return launch_step(s, static_cast<hipStream_t>(stream));
}

}  // namespace

extern "C" {

int ada_decode_step(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                    const int32_t* pos, int batch, int n_head, int n_kv_head, int head_dim,
                    int capacity, int max_pos, float scale, int dtype, void* out, void* workspace,
                    size_t workspace_bytes, void* stream, int num_splits) {
  return decode_step_impl(q, k_new, v_new, nullptr, nullptr, k_cache, v_cache, pos, batch, n_head, n_kv_head,
                          head_dim, capacity, max_pos, scale, dtype, out, workspace, workspace_bytes, stream,
                          num_splits);
}

int ada_decode_step_rope(const void* q, const void* k_new, const void* v_new, const void* cos, const void* sin,
                         void* k_cache, void* v_cache, const int32_t* pos, int batch, int n_head, int n_kv_head,
                         int head_dim, int capacity, int max_pos, float scale, int dtype, void* out,
                         void* workspace, size_t workspace_bytes, void* stream, int num_splits) {
  if (!cos || !sin) {
    if (dtype != ADA_F16 && dtype != ADA_BF16) return ADA_ERR_DTYPE;
    if (batch > 0) return ADA_ERR_NULL;
  }
  return decode_step_impl(q, k_new, v_new, cos, sin, k_cache, v_cache, pos, batch, n_head, n_kv_head, head_dim,
                          capacity, max_pos, scale, dtype, out, workspace, workspace_bytes, stream, num_splits);
}

int ada_prefill_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache, const int32_t* start,
                       int batch, int n_kv_head, int q_len, int capacity, int head_dim, int dtype, void* stream) {
  if (dtype != ADA_F16 && dtype != ADA_BF16) return ADA_ERR_DTYPE;
  if (batch < 0 || n_kv_head <= 0 || q_len < 0 || capacity <= 0) return ADA_ERR_SHAPE;
  if (head_dim != ada::kHeadDim) return ADA_ERR_HEAD_DIM;
  const int64_t chunks = sat_mul({batch, n_kv_head, q_len, ada::kHeadDim * 2 / 16});
  if ((chunks + 255) / 256 > INT32_MAX) return ADA_ERR_SHAPE;
  if (batch == 0 || q_len == 0) return ADA_OK;
  if (!k_new || !v_new || !k_cache || !v_cache) return ADA_ERR_NULL;  // start may be NULL (slot 0)
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache)) return ADA_ERR_ALIGN;
  hipError_t e = ada::launch_prefill_append(k_new, v_new, k_cache, v_cache, start, batch, n_kv_head, q_len, capacity,
                                            static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ADA_OK : hip_fail(e);
}

int ada_prefill_attn_gqa(const void* q, const void* k_cache, const void* v_cache, const int32_t* start, int batch,
                         int n_head, int n_kv_head, int q_len, int head_dim, int capacity, float scale, int dtype,
                         void* out, void* stream) {
  if (dtype != ADA_F16 && dtype != ADA_BF16) return ADA_ERR_DTYPE;
  if (batch < 0 || n_head <= 0 || n_kv_head <= 0 || q_len < 0 || capacity <= 0) return ADA_ERR_SHAPE;
  if (n_head % n_kv_head != 0 || n_head / n_kv_head > ada::kMaxGroup) return ADA_ERR_GQA;
  if (head_dim != ada::kHeadDim) return ADA_ERR_HEAD_DIM;
  if (!std::isfinite(scale)) return ADA_ERR_SCALE;
  // the kernel addresses one KV head's slab with 32-bit byte offsets
  if (static_cast<int64_t>(capacity) * head_dim * 2 > INT32_MAX) return ADA_ERR_SHAPE;
  const int64_t row_tiles = ceil_div(sat_mul({n_head / n_kv_head, q_len}), 64);
  if (sat_mul({row_tiles, batch, n_kv_head}) > INT32_MAX) return ADA_ERR_SHAPE;
  if (sat_mul({batch, n_head, q_len, head_dim}) > (int64_t(1) << 40)) return ADA_ERR_SHAPE;
  if (batch == 0 || q_len == 0) return ADA_OK;
  if (!q || !k_cache || !v_cache || !out) return ADA_ERR_NULL;  // start may be NULL (slot 0)
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out)) return ADA_ERR_ALIGN;
  ada::PrefillLaunch p{};
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.start = start;
  p.out = out;
  p.batch = batch;
  p.n_head = n_head;
  p.n_kv_head = n_kv_head;
  p.q_len = q_len;
  p.capacity = capacity;
  p.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  p.dtype = dtype;
  int cus = 0;
  int rc = current_device_cus(&cus);
  if (rc != ADA_OK) return rc;
  p.rows_per_workgroup = ada::prefill_rows_per_workgroup(batch, n_head, n_kv_head, q_len, cus);
  p.stream = static_cast<hipStream_t>(stream);
  hipError_t e = ada::launch_prefill(p);
  return e == hipSuccess ? ADA_OK : hip_fail(e);
}

int ada_decode_partial(const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* kv_len, int batch, int n_head, int n_kv_head, int head_dim,
                       int capacity, int max_kv_len, float scale, int dtype, int num_splits,
                       void* workspace, size_t workspace_bytes, int* splits_used, void* stream) {
  ada::DecodeLaunch p{};
  int rc = prepare_decode(q, k_cache, v_cache, kv_len, batch, n_head, n_kv_head, head_dim, capacity,
                          max_kv_len, scale, dtype, num_splits, stream, &p);
  if (rc != ADA_OK) return rc;
  if (splits_used) *splits_used = batch == 0 ? 0 : p.splits;
  if (batch == 0) return ADA_OK;
  rc = check_workspace(workspace, workspace_bytes, batch, n_head, n_kv_head, p.splits);
  if (rc != ADA_OK) return rc;
  p.workspace = workspace;
  p.direct = false;
  hipError_t e = ada::launch_partial(p);
  return e == hipSuccess ? ADA_OK : hip_fail(e);
}

int ada_decode_combine(const void* workspace, size_t workspace_bytes, int batch, int n_head,
                       int n_kv_head, int head_dim, int num_splits, int dtype, void* out,
                       void* stream) {
  if (dtype != ADA_F16 && dtype != ADA_BF16) return ADA_ERR_DTYPE;
  if (batch < 0 || n_head <= 0 || n_kv_head <= 0) return ADA_ERR_SHAPE;
  if (n_head % n_kv_head != 0 || n_head / n_kv_head > ada::kMaxGroup) return ADA_ERR_GQA;
  if (head_dim != ada::kHeadDim) return ADA_ERR_HEAD_DIM;
  if (num_splits < 1 || num_splits > ADA_MAX_SPLITS) return ADA_ERR_SPLITS;
  if (batch > 65535 || n_kv_head > 65535) return ADA_ERR_SHAPE;
  if (batch == 0) return ADA_OK;
  if (!out) return ADA_ERR_NULL;
  if (!aligned16(out)) return ADA_ERR_ALIGN;
  int rc = check_workspace(workspace, workspace_bytes, batch, n_head, n_kv_head, num_splits);
  if (rc != ADA_OK) return rc;
  ada::CombineLaunch c{workspace, out, batch, n_head, n_kv_head, num_splits, dtype,
                       static_cast<hipStream_t>(stream)};
  hipError_t e = ada::launch_combine(c);
  return e == hipSuccess ? ADA_OK : hip_fail(e);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Graph-captured multi-layer decode step.

struct ada_step_graph {
  hipGraphExec_t exec;  // NULL when the step has no work (batch 0)
  int device;
};

namespace {

// Records the prepared layers and the position advance on a private stream
// and instantiates the graph.
int capture_step(const std::vector<StepLaunch>& steps, int32_t* pos, int batch, int advance,
                 hipGraphExec_t* exec) {
  hipStream_t s = nullptr;
  hipError_t e = hipStreamCreateWithFlags(&s, hipStreamNonBlocking);
  if (e != hipSuccess) return hip_fail(e);
  e = hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) {
    (void)hipStreamDestroy(s);
    return hip_fail(e);
  }
  int rc = ADA_OK;
  for (const StepLaunch& st : steps) {
    rc = launch_step(st, s);
    if (rc != ADA_OK) break;
  }
  if (rc == ADA_OK && advance) {
    e = ada::launch_advance_positions(pos, batch, 1, s);
    if (e != hipSuccess) rc = hip_fail(e);
  }
  hipGraph_t graph = nullptr;
  e = hipStreamEndCapture(s, &graph);
  if (rc == ADA_OK && e != hipSuccess) rc = hip_fail(e);
  if (rc == ADA_OK) {
    e = hipGraphInstantiate(exec, graph, nullptr, nullptr, 0);
    if (e != hipSuccess) rc = hip_fail(e);
  }
  if (graph) (void)hipGraphDestroy(graph);
  (void)hipStreamDestroy(s);
  return rc;
}

}  // namespace

extern "C" {

int ada_step_graph_create(const ada_step_layer* layers, int n_layers, int32_t* pos, int batch, int n_head,
                          int n_kv_head, int head_dim, int capacity, int max_pos, float scale, int dtype,
                          int advance, void* workspace, size_t workspace_bytes, ada_step_graph** graph) {
  if (!graph) return ADA_ERR_NULL;
  *graph = nullptr;
  if (n_layers <= 0) return ADA_ERR_SHAPE;
  if (!layers) return ADA_ERR_NULL;
  if (batch > 0 && !pos) return ADA_ERR_NULL;
  if (pos && (reinterpret_cast<uintptr_t>(pos) & 3u) != 0) return ADA_ERR_ALIGN;
  std::vector<StepLaunch> steps(static_cast<size_t>(n_layers));
  // First every layer's arguments (a one-split plan needs no device query),
  // then the real plans, which read the device's compute-unit count.
  for (int i = 0; i < n_layers; ++i) {
    const ada_step_layer& L = layers[i];
    int rc = prepare_step(L.q, L.k_new, L.v_new, L.cos, L.sin, L.k_cache, L.v_cache, pos, batch, n_head,
                          n_kv_head, head_dim, capacity, max_pos, scale, dtype, L.out, workspace, workspace_bytes,
                          nullptr, 1, &steps[i]);
    if (rc != ADA_OK) return rc;
  }
  for (int i = 0; i < n_layers; ++i) {
    const ada_step_layer& L = layers[i];
    int rc = prepare_step(L.q, L.k_new, L.v_new, L.cos, L.sin, L.k_cache, L.v_cache, pos, batch, n_head,
                          n_kv_head, head_dim, capacity, max_pos, scale, dtype, L.out, workspace, workspace_bytes,
                          nullptr, 0, &steps[i]);
    if (rc != ADA_OK) return rc;
  }
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  hipGraphExec_t exec = nullptr;
  if (batch > 0) {
    int rc = capture_step(steps, pos, batch, advance, &exec);
    if (rc != ADA_OK) return rc;
  }
  *graph = new ada_step_graph{exec, dev};
  return ADA_OK;
}

int ada_step_graph_launch(ada_step_graph* graph, void* stream) {
  if (!graph) return ADA_ERR_NULL;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev != graph->device) return ADA_ERR_DEVICE;
  if (!graph->exec) return ADA_OK;
  e = hipGraphLaunch(graph->exec, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ADA_OK : hip_fail(e);
}

void ada_step_graph_destroy(ada_step_graph* graph) {
  if (!graph) return;
  if (graph->exec) (void)hipGraphExecDestroy(graph->exec);
  delete graph;
}

}  // extern "C"

extern "C" {

int ada_hbm_read(const void* src, size_t bytes, uint32_t* sink, int workgroups, void* stream) {
  if (workgroups <= 0 || workgroups > (1 << 20) || bytes % 16 != 0) return ADA_ERR_SHAPE;
  if (bytes == 0) return ADA_OK;
  if (!src || !sink) return ADA_ERR_NULL;
  if (!aligned16(src) || (reinterpret_cast<uintptr_t>(sink) & 3u) != 0) return ADA_ERR_ALIGN;
  hipError_t e = ada::launch_hbm_read(src, bytes, sink, workgroups, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ADA_OK : hip_fail(e);
}

}  // extern "C"
