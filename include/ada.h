/*
 * ada.h -- C ABI of the single-token decode-attention library for AMD
 * Instinct MI355X (gfx950).
 *
 * The library does one job: the decode step of grouped-query attention for
 * one new token per sequence,
 *
 *     out[b, h, :] = softmax_j( scale * q[b, h, :] . K[b, g, j, :] ) V[b, g, j, :]
 *     over the active prefix j < kv_len[b] only, with g = h / (n_head / n_kv_head),
 *
 * plus the in-place cache append that precedes it. The cache stays
 * preallocated at its full capacity; only the live prefix is read, in place,
 * and KV heads are never expanded to the query-head count.
 *
 * Pages cited (by title and section):
 *   [DECODE-FASTPATH] Cuda-Compute-OSS issue #343, "one-token decode fast
 *                     path: skip FlashAttention's prefill-tuned tiling for
 *                     q_len=1".
 *   [ACTIVE-PREFIX]   fish-speech issue #1310, "Optimize native AR decoding
 *                     by attending only to the active KV-cache prefix".
 *   [FORWARD-STEP]    VoxCPM issue #395, "MiniCPM4
 *                     MiniCPMAttention.forward_step Attention Performance
 *                     Fix".
 *
 * Conventions for every entry point:
 *   - All tensors are dense and row-major (last index fastest); element types
 *     are IEEE binary16 (ADA_F16) or bfloat16 (ADA_BF16), one type per call.
 *   - Pointers named as device pointers must point to device memory of the
 *     current HIP device and be 16-byte aligned. The caller owns every buffer;
 *     the library allocates no device memory, keeps no per-call state,
 *     never synchronises, and only enqueues work on `stream` (a hipStream_t;
 *     NULL is the default stream).
 *   - Arguments are validated on the host before any HIP call, so a rejected
 *     call has no effect and needs no GPU. Return value: ADA_OK or a negative
 *     ada_status. HIP launch failures return ADA_ERR_HIP; the HIP error code
 *     is then available from ada_last_hip_error() on the calling thread.
 *   - A call with batch == 0 is a valid no-op (pointers may then be NULL).
 *   - Only head_dim == 128 is supported (every page uses it).
 */
#ifndef ADA_H
#define ADA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ADA_ABI_VERSION 3

/* Element type of q, caches, new rows and output. */
typedef enum ada_dtype { ADA_F16 = 0, ADA_BF16 = 1 } ada_dtype;

typedef enum ada_status {
  ADA_OK = 0,
  ADA_ERR_NULL = -1,      /* a required pointer is NULL                      */
  ADA_ERR_SHAPE = -2,     /* batch/heads/capacity/max_kv_len out of range     */
  ADA_ERR_GQA = -3,       /* n_head not a multiple of n_kv_head, or the group
                             size n_head / n_kv_head is not 1..8             */
  ADA_ERR_DTYPE = -4,     /* dtype is not ADA_F16 or ADA_BF16                 */
  ADA_ERR_HEAD_DIM = -5,  /* head_dim != 128                                  */
  ADA_ERR_SCALE = -6,     /* scale is not finite                              */
  ADA_ERR_WORKSPACE = -7, /* workspace NULL or smaller than required          */
  ADA_ERR_SPLITS = -8,    /* num_splits outside [0, ADA_MAX_SPLITS]           */
  ADA_ERR_ALIGN = -9,     /* a device pointer is not 16-byte aligned          */
  ADA_ERR_HIP = -10,      /* a HIP runtime call failed                        */
  ADA_ERR_DEVICE = -11,   /* a step graph launched on another device than the
                             one current when it was created                 */
  ADA_ERR_SCRATCH = -12   /* ada_decode_attn_gqa_noalloc: the call's split
                             partials exceed ADA_NOALLOC_SCRATCH_BYTES        */
} ada_status;

/* Upper bound on the number of key-range splits of one decode call. */
#define ADA_MAX_SPLITS 256

/* Library ABI version (ADA_ABI_VERSION of the build). */
int ada_abi_version(void);

/* Static, NUL-terminated description of a status code. */
const char* ada_status_string(int status);

/* hipError_t of the last call on this thread that returned ADA_ERR_HIP. */
int ada_last_hip_error(void);

/* Number of compute units of HIP device `device`, written to *num_cus.
 * Returns ADA_ERR_NULL, ADA_ERR_HIP or ADA_OK. */
int ada_device_num_cus(int device, int* num_cus);

/*
 * In-place KV-cache append ([FORWARD-STEP] section 4: the new key and value
 * rows are written at slot position_id of the preallocated cache;
 * [ACTIVE-PREFIX] section 2: allocation and in-place update are unchanged).
 *
 *   k_new, v_new  device, [batch, n_kv_head, head_dim]  (the memory order of
 *                 the [batch, n_kv_head, 1, head_dim] projection view)
 *   k_cache,      device, [batch, n_kv_head, capacity, head_dim], updated in
 *   v_cache       place: row pos[b] of every KV head of batch row b.
 *   pos           device int32 [batch]. A row with pos[b] outside
 *                 [0, capacity) is skipped (nothing written), on the device.
 *
 * Values are copied bit for bit. k_new/v_new must not overlap the caches.
 * ADA_ERR_SHAPE when batch * n_kv_head rows are too many to index with the
 * launch's 32-bit thread indices (more than about 2^27).
 */
int ada_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                  const int32_t* pos, int batch, int n_kv_head, int capacity,
                  int head_dim, int dtype, void* stream);

/*
 * Rotary embedding of the new token, then the append: [FORWARD-STEP] section
 * 4 applies apply_rotary_pos_emb(query, key, cos, sin) to the step's query
 * and key just before the key and value rows are written at position_id. The
 * page names the function without printing it; it is read as the rotate-half
 * form, per head of D values with h = D / 2:
 *   out[i] = x[i] cos[i] - x[i + h] sin[i]    (i <  h)
 *   out[i] = x[i] cos[i] + x[i - h] sin[i]    (i >= h)
 * computed exactly from the stored 16-bit values and rounded once to the
 * dtype (nearest, ties to even; a zero result is +0). Exact for inputs whose
 * products x * cos, x * sin stay within fp32's normal range (always for
 * fp16; bf16 magnitudes below about 1e-19 may round differently). Inputs
 * must be finite.
 *
 *   q, q_out      device, [batch, n_head, head_dim]: q_out = rotated q. q_out
 *                 may equal q (in place). Both NULL: keys only (n_head is
 *                 then ignored); one NULL alone is ADA_ERR_NULL.
 *   k_new, v_new  device, [batch, n_kv_head, head_dim]; k_new is rotated
 *                 before the write, v_new is copied.
 *   cos, sin      device, [batch, head_dim] in dtype: row b is the table of
 *                 batch row b's position (the caller computes it, with any
 *                 frequency scaling of its model).
 *   k_cache,      device, [batch, n_kv_head, capacity, head_dim]; row pos[b]
 *   v_cache       of every KV head of batch row b is written when
 *                 0 <= pos[b] < capacity, else nothing is.
 *   pos           device int32 [batch].
 * All buffers 16-byte aligned (ADA_ERR_ALIGN); head_dim 128. Returns
 * ADA_ERR_SHAPE for negative sizes or a launch too large to index, ADA_OK
 * without work for batch == 0. One kernel launch on `stream`.
 */
int ada_rope_kv_append(const void* q, void* q_out, const void* k_new, const void* v_new, const void* cos,
                       const void* sin, void* k_cache, void* v_cache, const int32_t* pos, int batch,
                       int n_head, int n_kv_head, int capacity, int head_dim, int dtype, void* stream);

/*
 * Split heuristic: number of key-range splits for a decode call over
 * batch * n_kv_head (batch row, KV head) units whose live prefixes are at
 * most max_kv_len slots, on a device with num_cus compute units. Prefixes of
 * at most 256 slots take one split (no combine launch). Otherwise it aims at
 * one 4-wave workgroup per compute unit, never splits below 64 slots, and
 * doubles the split count while a split would exceed 8192 slots; the
 * per-split range is rounded up to a multiple of 64 and the count returned
 * is the one that rounding yields. Pure host arithmetic; returns 1..256
 * (1 for non-positive inputs).
 */
int ada_decode_num_splits(int batch, int n_head, int n_kv_head, int max_kv_len, int num_cus);

/*
 * The launch plan a decode call over max_kv_len slots uses: *splits key-range
 * splits per (batch row, KV head) of *chunk slots each (the last may be
 * shorter). num_splits == 0 gives the heuristic of ada_decode_num_splits for
 * num_cus compute units; 1..ADA_MAX_SPLITS forces near-equal ranges of
 * ceil(max_kv_len / num_splits) slots, as ada_decode_attn_gqa_ex does (fewer
 * splits when the prefix is shorter; num_cus is then unused). Callers size
 * workspaces with *splits (ada_decode_workspace_bytes). Pure host
 * arithmetic: ADA_ERR_NULL for NULL outputs, ADA_ERR_SPLITS for num_splits
 * outside [0, ADA_MAX_SPLITS], else ADA_OK (max_kv_len <= 0 gives 1 split).
 */
int ada_decode_plan(int batch, int n_head, int n_kv_head, int max_kv_len, int num_splits, int num_cus, int* splits,
                    int* chunk);

/*
 * Bytes of device workspace that holds num_splits (>= 1) per-split partial
 * results: a running maximum and sum (2 floats) and an unnormalised
 * accumulator (head_dim floats) per (split, batch row, query head), stored
 * split-major, each array rounded up to 256 bytes. Returns 0 for
 * num_splits < 1, non-positive sizes, or a size beyond 2^56 bytes (no call
 * can use it). ada_decode_attn_gqa needs this much
 * only when it uses 2 or more splits. n_kv_head is accepted for symmetry
 * with the decode calls. Pure host arithmetic.
 */
size_t ada_decode_workspace_bytes(int batch, int n_head, int n_kv_head, int head_dim,
                                  int num_splits);

/*
 * Single-token decode attention with grouped-query heads, over the active
 * prefix of a preallocated cache, read in place.
 *
 * Definition ([DECODE-FASTPATH] "Proposed implementation": softmax of the
 * scaled q.K row times V, softmax accumulated in fp32, output cast back to
 * the input type; [ACTIVE-PREFIX] section 2 and [FORWARD-STEP] sections 3-4:
 * attend over slots [0, kv_len) only, kv_len = position_id + 1 after the
 * append; [ACTIVE-PREFIX] section 1: query head h reads KV head
 * h / (n_head / n_kv_head), the repeat_interleave order).
 *
 *   q          device, [batch, n_head, head_dim]  (the [B, H, 1, D] query)
 *   k_cache,   device, [batch, n_kv_head, capacity, head_dim]; only slots
 *   v_cache    j < n_b are read, n_b = min(max(kv_len[b], 0), max_kv_len).
 *              Slots at and beyond n_b may hold anything (NaN included).
 *   kv_len     device int32 [batch], live prefix length per batch row, or
 *              NULL: every row then holds max_kv_len live slots (one host-side
 *              position for the whole batch, as the pages' decode loops pass
 *              it, [ACTIVE-PREFIX] section 2), and the kernels read no length
 *              from the device.
 *   max_kv_len host upper bound on kv_len[b], sizes the launch; <= 0 means
 *              capacity; > capacity is ADA_ERR_SHAPE. Device values above it
 *              are clamped to it.
 *   scale      finite; the pages use 1/sqrt(head_dim). 0 gives equal weights.
 *   out        device, [batch, n_head, head_dim] (= [B, H*D] as the output
 *              projection consumes it, [FORWARD-STEP] section 4); must not
 *              overlap the inputs. Rounded to the element type
 *              round-to-nearest-even. A row with n_b == 0 is all zeros.
 *   workspace  device scratch, at least ada_decode_workspace_bytes(...)
 *              bytes for the split count the call uses (ada_decode_num_splits
 *              on the current device); may be NULL when that count is 1. Its
 *              contents need no preparation. Calls that share a workspace
 *              must be ordered (same stream, or synchronised).
 *
 * With one split a single kernel writes the output; with more, a partial
 * kernel writes per-split results to the workspace and a combine kernel
 * merges them (log-sum-exp weights, split order). Scores, softmax
 * statistics and accumulators are fp32. The result is bitwise deterministic
 * for a given split count and given lengths.
 *
 * Balanced plan: with device lengths (kv_len != NULL), 2..64 batch rows and
 * two or more heuristic splits, the splits * batch workgroups of each KV head
 * are shared among the rows in proportion to their lengths rather than
 * `splits` per row: both kernels derive one common range length from
 * kv_len on the device (no host synchronisation) and row b takes
 * ceil(n_b / range) consecutive workgroups. Ragged batches then spread their
 * keys over all workgroups; the workspace size is unchanged. A forced split
 * count (ada_decode_attn_gqa_ex with num_splits > 0) and ada_decode_partial
 * keep the per-row plan.
 */
int ada_decode_attn_gqa(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* kv_len, int batch, int n_head, int n_kv_head,
                        int head_dim, int capacity, int max_kv_len, float scale, int dtype,
                        void* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * As ada_decode_attn_gqa, with the split count forced: num_splits == 0 uses
 * the heuristic; 1..ADA_MAX_SPLITS splits the key range into that many
 * near-equal ranges (fewer when max_kv_len is smaller). For tests and tuning.
 */
int ada_decode_attn_gqa_ex(const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* kv_len, int batch, int n_head, int n_kv_head,
                           int head_dim, int capacity, int max_kv_len, float scale, int dtype,
                           void* out, void* workspace, size_t workspace_bytes, void* stream,
                           int num_splits);

/*
 * ada_decode_attn_gqa_ex without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc. The split partials go to a static
 * scratch array of ADA_NOALLOC_SCRATCH_BYTES that the library holds on every
 * device it runs on until the process ends; the call allocates nothing
 * (no hipMalloc, no hipFree). Same kernels, plan and results as
 * ada_decode_attn_gqa_ex with the same num_splits (0 = heuristic).
 *
 * Limit: ADA_ERR_SCRATCH when the call uses two or more splits and
 * ada_decode_workspace_bytes(batch, n_head, n_kv_head, head_dim, splits)
 * exceeds ADA_NOALLOC_SCRATCH_BYTES (about 8000 (batch row, query head,
 * split) partials: e.g. batch 8 x 32 heads x 8 splits uses 1.06 MB).
 * The scratch array is shared by every call on a device and keeps the last
 * call's contents (nothing in it needs clearing: each call writes every
 * partial it reads). Calls that may overlap on one device -- on different
 * streams without synchronisation, or from several threads -- race on it;
 * order them. The first call on a device fetches the array's address
 * (hipGetSymbolAddress), so it is ADA_ERR_HIP if that fails.
 */
#define ADA_NOALLOC_SCRATCH_BYTES (4u << 20)

int ada_decode_attn_gqa_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* kv_len, int batch, int n_head, int n_kv_head,
                                int head_dim, int capacity, int max_kv_len, float scale, int dtype,
                                void* out, void* stream, int num_splits);

/*
 * One whole decode step in one call: append the new key/value rows, then
 * attend over the prefix that ends with them ([FORWARD-STEP] section 4: the
 * cache write at position_id followed by attention over slots
 * 0..position_id). Equivalent to ada_kv_append(k_new, v_new, k_cache, v_cache,
 * pos) followed by ada_decode_attn_gqa with kv_len[b] = pos[b] + 1, with
 * one kernel launch fewer: the kernel that attends reads the new rows from
 * k_new/v_new while another workgroup of the same launch writes them into
 * the cache.
 *
 *   k_new, v_new  device, [batch, n_kv_head, head_dim].
 *   k_cache,      device, [batch, n_kv_head, capacity, head_dim], updated in
 *   v_cache       place at slot pos[b] (when 0 <= pos[b] < capacity).
 *   pos           device int32 [batch], or NULL: every row at slot max_pos.
 *   max_pos       host upper bound on pos[b], 0 <= max_pos < capacity (else
 *                 ADA_ERR_SHAPE); sizes the launch. A row attends over
 *                 min(pos[b], max_pos) + 1 slots; pos[b] < 0 gives a zero row
 *                 and writes nothing.
 *   num_splits    0 = heuristic, else forced as in ada_decode_attn_gqa_ex.
 * Other arguments as ada_decode_attn_gqa_ex. k_new/v_new must not overlap
 * the caches or out.
 */
int ada_decode_step(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                    const int32_t* pos, int batch, int n_head, int n_kv_head, int head_dim,
                    int capacity, int max_pos, float scale, int dtype, void* out, void* workspace,
                    size_t workspace_bytes, void* stream, int num_splits);

/*
 * ada_decode_step with the rotary embedding of ada_rope_kv_append applied to
 * q and k_new first ([FORWARD-STEP] section 4: rotate, write the cache row at
 * position_id, attend over slots 0..position_id with the rotated query).
 * Equivalent to ada_rope_kv_append into a temporary rotated query, then
 * ada_decode_attn_gqa with kv_len[b] = pos[b] + 1, in the launches of
 * ada_decode_step: every workgroup rotates its own copy of the query, the
 * workgroup of the first split writes the rotated key, and the workgroup
 * whose key range holds slot pos[b] uses the rotated key it computed itself.
 * q is not modified.
 *
 *   cos, sin  device, [batch, head_dim] in dtype, 16-byte aligned, both
 *             required (ADA_ERR_NULL).
 * Other arguments as ada_decode_step.
 */
int ada_decode_step_rope(const void* q, const void* k_new, const void* v_new, const void* cos, const void* sin,
                         void* k_cache, void* v_cache, const int32_t* pos, int batch, int n_head, int n_kv_head,
                         int head_dim, int capacity, int max_pos, float scale, int dtype, void* out,
                         void* workspace, size_t workspace_bytes, void* stream, int num_splits);

/*
 * Prompt append: the T prompt rows of every (batch row, KV head) written into
 * slots start[b] .. start[b] + T - 1 of the preallocated caches, bit for bit
 * ([ACTIVE-PREFIX] section 2: after the prompt prefill the cache holds
 * kv_len = T slots; the allocation never changes). Slots outside
 * [0, capacity) are skipped.
 *
 *   k_new, v_new  device, [batch, n_kv_head, q_len, head_dim].
 *   k_cache,      device, [batch, n_kv_head, capacity, head_dim], updated in
 *   v_cache       place.
 *   start         device int32 [batch], or NULL: every row starts at slot 0.
 * All buffers 16-byte aligned (ADA_ERR_ALIGN); head_dim 128. ADA_OK without
 * work for batch == 0 or q_len == 0. One kernel launch on `stream`.
 */
int ada_prefill_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache, const int32_t* start,
                       int batch, int n_kv_head, int q_len, int capacity, int head_dim, int dtype, void* stream);

/*
 * Causal prefill attention over the cache: q_len query tokens per batch row,
 * token t at position start[b] + t attending cache slots 0 .. start[b] + t
 * ([FORWARD-STEP] section 5: the batch prefill path runs attention with
 * is_causal=True; with start = 0 this is that square causal mask over the
 * prompt, and start > 0 continues a prompt after earlier tokens). The prompt's
 * own rows must already be in the cache (ada_prefill_append). For token t of
 * row b and query head h (KV head h / G, G = n_head / n_kv_head),
 * n = clamp(start[b] + t + 1, 0, capacity):
 *   out[b,h,t,:] = softmax_j(scale * q[b,h,t,:] . K[b,g,j,:]) V[b,g,j,:], j < n
 * and n == 0 gives zeros. Scores and softmax statistics in fp32 (16-bit
 * products are exact; [DECODE-FASTPATH] "Proposed implementation" asks for
 * fp32 softmax accumulation). The weighted sum runs on the matrix cores with
 * each fp32 weight split into two 16-bit values, hi = rnd(p) and
 * lo = rnd(p - hi), so the weights keep 16 (bf16) or 22 (fp16) significant
 * bits; the row sums add the same pairs. Output rounded to nearest even.
 *
 *   q, out     device, [batch, n_head, q_len, head_dim] (the head-major query
 *              of an SDPA call); out must not overlap the inputs.
 *   k_cache,   device, [batch, n_kv_head, capacity, head_dim], read in place.
 *   v_cache
 *   start      device int32 [batch], or NULL: every row starts at slot 0.
 *   scale      finite float (1/sqrt(head_dim) is SDPA's default).
 * n_head a multiple of n_kv_head with n_head / n_kv_head in 1..8 (ADA_ERR_GQA);
 * head_dim 128; capacity below 2^23 slots (one KV head's slab under 2 GiB,
 * addressed with 32-bit offsets; else ADA_ERR_SHAPE); buffers 16-byte
 * aligned; ADA_OK without work for batch == 0 or q_len == 0. One kernel
 * launch on `stream`, no workspace.
 */
int ada_prefill_attn_gqa(const void* q, const void* k_cache, const void* v_cache, const int32_t* start, int batch,
                         int n_head, int n_kv_head, int q_len, int head_dim, int capacity, float scale, int dtype,
                         void* out, void* stream);

/*
 * Query rows per workgroup of ada_prefill_attn_gqa on a device with num_cus
 * compute units: 128 (each wavefront takes two 16-row blocks, so every key
 * and value operand read from LDS serves both) when that still launches at
 * least 2 workgroups per compute unit, i.e.
 *   ceil((n_head / n_kv_head) * q_len / 128) * batch * n_kv_head >= 2 * num_cus,
 * else 64 (one block per wavefront). 64 for invalid arguments.
 * The choice changes the launch only, not the result beyond rounding order.
 * Pure host arithmetic.
 */
int ada_prefill_rows_per_workgroup(int batch, int n_head, int n_kv_head, int q_len, int num_cus);

/*
 * The two halves of a decode call, for callers that merge partial results
 * themselves -- e.g. key ranges held by different devices, whose partials are
 * concatenated along the split axis and combined once.
 *
 * ada_decode_partial: arguments as ada_decode_attn_gqa_ex without `out`;
 * always writes partials (never the output) for every split, the split count
 * it used going to *splits_used (may be NULL). Split s covers slots
 * [s*c, min((s+1)*c, n_b)) with c = ceil(max_kv_len / splits) (the
 * heuristic rounds c up to a multiple of 64); with scores
 * x = scale*log2(e)*q.k, its entry holds a reference m (max x - 8 <= m <=
 * max x over the range), l = sum of exp2(x - m) and acc = sum of
 * exp2(x - m) * v (fp32, unnormalised); an empty range holds m = -inf, l = 0
 * and an accumulator that must not be read. This is the online (running max and sum) softmax of
 * [DECODE-FASTPATH], "Current limitation", applied per key range.
 *
 * ada_decode_combine: merges num_splits partials per (batch row, query head)
 * in split order: M = max m_s, out = sum exp2(m_s - M) acc_s /
 * sum exp2(m_s - M) l_s, rounded to `dtype` round-to-nearest-even; all-empty
 * rows give zeros. `workspace` holds num_splits partials laid out as
 * ada_decode_partial writes them (split-major).
 */
int ada_decode_partial(const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* kv_len, int batch, int n_head, int n_kv_head, int head_dim,
                       int capacity, int max_kv_len, float scale, int dtype, int num_splits,
                       void* workspace, size_t workspace_bytes, int* splits_used, void* stream);

int ada_decode_combine(const void* workspace, size_t workspace_bytes, int batch, int n_head,
                       int n_kv_head, int head_dim, int num_splits, int dtype, void* out,
                       void* stream);

/*
 * Graph-captured multi-layer decode step.
 *
 * Decode step i after a T-token prompt writes the new key/value rows at slot
 * T + i and attends over T + i + 1 slots ([ACTIVE-PREFIX] section 2; section
 * 4 of [FORWARD-STEP] does the same per layer with position_id). For a model
 * with n_layers attention layers that share batch, head counts and cache
 * capacity, ada_step_graph_create records, once, the launches of
 * ada_decode_step (or ada_decode_step_rope for a layer with rotary tables)
 * for every layer in order, followed by a kernel that adds one to every
 * pos[b], into one HIP graph. Each ada_step_graph_launch then runs a whole
 * step -- all layers and the position advance -- as a single graph launch
 * with no host work and no device-to-host read: the positions live on the
 * device and the kernels read them there.
 *
 * The graph holds the buffer addresses given at creation, not their
 * contents: per step the caller writes the new q, k_new, v_new (and cos,
 * sin) into the same buffers and reads out after the launch. Every layer
 * uses the launch plan of ada_decode_step with the given max_pos (the split
 * count for max_pos + 1 live slots on the device current at creation), so a
 * replay gives bit for bit what those ada_decode_step calls would give.
 *
 *   layers    host array of n_layers (>= 1) layer descriptions, read only
 *             during the call. Per layer: q [batch, n_head, head_dim],
 *             k_new and v_new [batch, n_kv_head, head_dim], k_cache and
 *             v_cache [batch, n_kv_head, capacity, head_dim], out
 *             [batch, n_head, head_dim]; cos and sin [batch, head_dim] or
 *             both NULL (no rotary embedding for that layer). Device
 *             pointers, 16-byte aligned, with the no-overlap rules of
 *             ada_decode_step.
 *   pos       device int32 [batch], required: the slot each row appends at
 *             in the next launch. A launch advances it by one when
 *             `advance` is non-zero.
 *   max_pos   host upper bound on pos[b] over every launch the caller will
 *             make, 0 <= max_pos < capacity; sizes the launches. A row whose
 *             pos[b] exceeds max_pos attends over max_pos + 1 slots only
 *             (as in ada_decode_step).
 *   workspace device scratch shared by the layers (they run in order), at
 *             least ada_decode_workspace_bytes for the split count of
 *             max_pos + 1 slots (may be NULL when that count is 1); it must
 *             stay allocated, and untouched by other work that can overlap
 *             a launch, for the life of the graph.
 *   graph     receives the handle; set to NULL on any error.
 * Other arguments as ada_decode_step. Every layer is validated before
 * anything is recorded; an invalid layer returns its ada_decode_step status
 * and creates nothing. Creation records on a private stream of its own and
 * runs no kernel, so it must not be called while the calling thread is
 * itself capturing a stream; it is ADA_ERR_HIP if graph capture or
 * instantiation fails.
 */
typedef struct ada_step_layer {
  const void* q;
  const void* k_new;
  const void* v_new;
  void* k_cache;
  void* v_cache;
  void* out;
  const void* cos; /* rotary tables for this layer, or NULL */
  const void* sin;
} ada_step_layer;

typedef struct ada_step_graph ada_step_graph;

int ada_step_graph_create(const ada_step_layer* layers, int n_layers, int32_t* pos, int batch, int n_head,
                          int n_kv_head, int head_dim, int capacity, int max_pos, float scale, int dtype,
                          int advance, void* workspace, size_t workspace_bytes, ada_step_graph** graph);

/*
 * One step: launches the graph on `stream` (ordered after earlier work on
 * it, like any kernel launch). Launches of one graph share its workspace and
 * positions and must be ordered. ADA_ERR_NULL for a NULL graph,
 * ADA_ERR_DEVICE when the current device is not the one of its creation.
 */
int ada_step_graph_launch(ada_step_graph* graph, void* stream);

/* Frees the graph (NULL is a no-op). No launch of it may still be pending:
 * synchronise the streams it was launched on first. */
void ada_step_graph_destroy(ada_step_graph* graph);

/*
 * Measurement: a plain streaming read, the floor a decode call's K/V stream
 * is measured against. [DECODE-FASTPATH] "Current limitation" puts the whole
 * cost of a one-token decode in reading K and V once; this reads `bytes`
 * bytes of `src` once, with the 16-byte nontemporal loads the decode kernel
 * uses and no arithmetic, spread over `workgroups` 256-thread workgroups
 * (chunk i of 16 bytes to workgroup (i / 256) mod workgroups), and writes
 * the xor of what each wavefront read to sink[4 * workgroup + wavefront]
 * (so that no load can be dropped). Time it with events on `stream`.
 *
 *   src     device, 16-byte aligned, `bytes` (a multiple of 16) readable.
 *   sink    device uint32 [4 * workgroups], 4-byte aligned, overwritten.
 * ADA_ERR_SHAPE for workgroups outside 1..2^20 or bytes not a multiple of
 * 16; ADA_OK without work for bytes == 0. One kernel launch.
 */
int ada_hbm_read(const void* src, size_t bytes, uint32_t* sink, int workgroups, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ADA_H */
