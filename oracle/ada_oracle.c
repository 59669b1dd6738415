/*
 * ada_oracle.c -- plain, slow CPU reference for single-token decode attention
 * over the active prefix of a preallocated KV cache, and for the in-place
 * cache append that precedes it.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg load this file's library. The GPU library
 * never includes, links or calls it, and this file includes nothing of the
 * GPU library: the two share no code, header, table or helper.
 *
 * Everything is computed in IEEE double from the stored 16-bit values, with
 * no blocking, splitting or reordering beyond the plain definition, so that
 * a reader can check each function against the pages by eye.
 *
 * Pages cited (by title and section; the reader has the pages):
 *   [DECODE-FASTPATH]  Cuda-Compute-OSS issue #343, "one-token decode fast
 *                      path: skip FlashAttention's prefill-tuned tiling for
 *                      q_len=1".
 *   [ACTIVE-PREFIX]    fish-speech issue #1310, "Optimize native AR decoding
 *                      by attending only to the active KV-cache prefix".
 *   [FORWARD-STEP]     VoxCPM issue #395, "MiniCPM4
 *                      MiniCPMAttention.forward_step Attention Performance
 *                      Fix".
 *
 * Every function here is pinned by the CPU tests to results obtained another
 * way (an independent library implementation of attention, closed forms,
 * invariants and exhaustive decoding checks); see the test files named
 * test_oracle_*.py.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_F16 = 0, ORACLE_BF16 = 1 };

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction
 * bits. Exponent 0 encodes zero and subnormals (fraction * 2^-24); exponent
 * 31 encodes infinities (fraction 0) and NaNs. */
double ada_oracle_f16_to_f64(uint16_t bits) {
  int sign = (bits >> 15) & 1;
  int expo = (bits >> 10) & 0x1f;
  int frac = bits & 0x3ff;
  double mag;
  if (expo == 0) {
    mag = ldexp((double)frac, -24);
  } else if (expo == 31) {
    mag = frac ? NAN : INFINITY;
  } else {
    mag = ldexp(1.0 + (double)frac / 1024.0, expo - 15);
  }
  return sign ? -mag : mag;
}

/* bfloat16: the upper half of an IEEE binary32, i.e. 1 sign bit, 8 exponent
 * bits (bias 127), 7 fraction bits. Exponent 0 encodes zero and subnormals
 * (fraction * 2^-133); exponent 255 encodes infinities and NaNs. */
double ada_oracle_bf16_to_f64(uint16_t bits) {
  int sign = (bits >> 15) & 1;
  int expo = (bits >> 7) & 0xff;
  int frac = bits & 0x7f;
  double mag;
  if (expo == 0) {
    mag = ldexp((double)frac, -133);
  } else if (expo == 255) {
    mag = frac ? NAN : INFINITY;
  } else {
    mag = ldexp(1.0 + (double)frac / 128.0, expo - 127);
  }
  return sign ? -mag : mag;
}

static double decode16(uint16_t bits, int dtype) {
  return dtype == ORACLE_BF16 ? ada_oracle_bf16_to_f64(bits)
                              : ada_oracle_f16_to_f64(bits);
}

/* Number of threads the parallel loop below may use. */
int ada_oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Sets the number of threads later calls may use (n >= 1); the results do
 * not depend on it (each output row is computed by one thread). */
void ada_oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n >= 1) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/*
 * Single-token decode attention, grouped-query heads read in place.
 *
 *   q        [batch, n_head, head_dim]                 16-bit values
 *   k_cache  [batch, n_kv_head, capacity, head_dim]    16-bit values
 *   v_cache  [batch, n_kv_head, capacity, head_dim]    16-bit values
 *   kv_len   [batch]  number of valid leading cache slots per batch row
 *   out      [batch, n_head, head_dim]                 double, unrounded
 *
 * For batch row b and query head h:
 *   - Grouped-query sharing: query heads come in n_kv_head consecutive groups
 *     of G = n_head / n_kv_head, and head h reads KV head g = h / G. This is
 *     the head order produced by repeat_interleave of the KV heads along the
 *     head axis ([ACTIVE-PREFIX] section 1; the enable_gqa call of
 *     [FORWARD-STEP] section 4 follows the same order).
 *   - Active prefix: only slots j < n, n = clamp(kv_len[b], 0, capacity),
 *     take part; the tail is never read ([ACTIVE-PREFIX] section 2;
 *     [FORWARD-STEP] sections 3 and 4, where n = position_id + 1).
 *   - Attention of one query row ([DECODE-FASTPATH], "Proposed
 *     implementation" and the max-subtracted softmax of "Correctness
 *     risks"):
 *       x_j = scale * sum_d q[b,h,d] * K[b,g,j,d]
 *       m   = max_j x_j
 *       out[b,h,:] = sum_j exp(x_j - m) * V[b,g,j,:] / sum_j exp(x_j - m)
 *   - n == 0 (never reached on the pages) gives a zero row: an empty sum.
 *
 * Returns 0, or -1 on a bad argument (nothing written), -2 on allocation
 * failure.
 */
int ada_oracle_decode(const uint16_t* q, const uint16_t* k_cache,
                      const uint16_t* v_cache, const int32_t* kv_len,
                      int batch, int n_head, int n_kv_head, int head_dim,
                      int capacity, double scale, int dtype, double* out) {
  if (batch < 0 || n_head <= 0 || n_kv_head <= 0 || head_dim <= 0 ||
      capacity <= 0 || n_head % n_kv_head != 0 ||
      (dtype != ORACLE_F16 && dtype != ORACLE_BF16))
    return -1;
  if (batch == 0) return 0;
  if (!q || !k_cache || !v_cache || !kv_len || !out) return -1;

  const int group = n_head / n_kv_head;
  const long rows = (long)batch * n_head;
  int failed = 0;

#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
  for (long bh = 0; bh < rows; ++bh) {
    const int b = (int)(bh / n_head);
    const int h = (int)(bh % n_head);
    const int g = h / group;
    int n = kv_len[b];
    if (n < 0) n = 0;
    if (n > capacity) n = capacity;

    double* o = out + bh * head_dim;
    for (int d = 0; d < head_dim; ++d) o[d] = 0.0;
    if (n == 0) continue;

    const uint16_t* qrow = q + bh * head_dim;
    const uint16_t* kbase =
        k_cache + ((size_t)b * n_kv_head + g) * (size_t)capacity * head_dim;
    const uint16_t* vbase =
        v_cache + ((size_t)b * n_kv_head + g) * (size_t)capacity * head_dim;

    double* qd = (double*)malloc(sizeof(double) * head_dim);
    double* x = (double*)malloc(sizeof(double) * n);
    if (!qd || !x) {
      free(qd);
      free(x);
      failed = 1;
      continue;
    }
    for (int d = 0; d < head_dim; ++d) qd[d] = decode16(qrow[d], dtype);

    /* scores */
    for (int j = 0; j < n; ++j) {
      const uint16_t* krow = kbase + (size_t)j * head_dim;
      double dot = 0.0;
      for (int d = 0; d < head_dim; ++d) dot += qd[d] * decode16(krow[d], dtype);
      x[j] = scale * dot;
    }
    /* max-subtracted softmax weights and their sum */
    double m = x[0];
    for (int j = 1; j < n; ++j)
      if (x[j] > m) m = x[j];
    double wsum = 0.0;
    for (int j = 0; j < n; ++j) {
      x[j] = exp(x[j] - m);
      wsum += x[j];
    }
    /* weighted sum of value rows */
    for (int j = 0; j < n; ++j) {
      const uint16_t* vrow = vbase + (size_t)j * head_dim;
      for (int d = 0; d < head_dim; ++d) o[d] += x[j] * decode16(vrow[d], dtype);
    }
    for (int d = 0; d < head_dim; ++d) o[d] /= wsum;

    free(qd);
    free(x);
  }
  return failed ? -2 : 0;
}

/*
 * In-place cache append: the new key and value rows of every (batch row,
 * KV head) are written into slot pos[b] of the preallocated caches; the
 * allocation itself never changes ([FORWARD-STEP] section 4, the cache write
 * at position_id; [ACTIVE-PREFIX] section 2, in-place update unchanged).
 * A batch row whose pos[b] lies outside [0, capacity) writes nothing.
 *
 *   k_new, v_new [batch, n_kv_head, head_dim]; caches [batch, n_kv_head,
 *   capacity, head_dim]. Values are copied bit for bit.
 */
int ada_oracle_kv_append(const uint16_t* k_new, const uint16_t* v_new,
                         uint16_t* k_cache, uint16_t* v_cache,
                         const int32_t* pos, int batch, int n_kv_head,
                         int capacity, int head_dim) {
  if (batch < 0 || n_kv_head <= 0 || capacity <= 0 || head_dim <= 0) return -1;
  if (batch == 0) return 0;
  if (!k_new || !v_new || !k_cache || !v_cache || !pos) return -1;
  for (int b = 0; b < batch; ++b) {
    int p = pos[b];
    if (p < 0 || p >= capacity) continue;
    for (int g = 0; g < n_kv_head; ++g) {
      size_t src = ((size_t)b * n_kv_head + g) * head_dim;
      size_t dst = (((size_t)b * n_kv_head + g) * capacity + p) * head_dim;
      memcpy(k_cache + dst, k_new + src, sizeof(uint16_t) * head_dim);
      memcpy(v_cache + dst, v_new + src, sizeof(uint16_t) * head_dim);
    }
  }
  return 0;
}

/*
 * Causal prefill attention over the cache: T query tokens per batch row at
 * positions start[b] .. start[b] + T - 1, each attending to every cache slot
 * up to and including its own position. The prompt's keys and values are
 * already in the cache (ada_oracle_prefill_append below).
 *
 *   q        [batch, n_head, T, head_dim]     16-bit values (the head-major
 *                                             query of an SDPA call)
 *   k_cache, v_cache [batch, n_kv_head, capacity, head_dim]
 *   start    [batch]  position of the first query token of each row
 *   out      [batch, n_head, T, head_dim]     double, unrounded
 *
 * The pages run prompt prefill as SDPA with is_causal=True over the prompt
 * ([FORWARD-STEP] section 5, forward() keeps is_causal=True), with the cache
 * holding kv_len = T slots after it ([ACTIVE-PREFIX] section 2). Query token
 * t of batch row b, head h (KV head g = h / G as in the decode):
 *   n = clamp(start[b] + t + 1, 0, capacity)
 *   x_j = scale * sum_d q[b,h,t,d] * K[b,g,j,d]      for j < n
 *   out[b,h,t,:] = sum_j exp(x_j - m) V[b,g,j,:] / sum_j exp(x_j - m),  m = max_j x_j
 * With start = 0 this is the causal (lower-triangular) mask of a square
 * score matrix; with start > 0 (a prompt continued after earlier tokens) each
 * token still sees exactly the slots up to its own position. n == 0 gives a
 * zero row.
 */
int ada_oracle_prefill(const uint16_t* q, const uint16_t* k_cache,
                       const uint16_t* v_cache, const int32_t* start,
                       int batch, int n_head, int n_kv_head, int q_len,
                       int head_dim, int capacity, double scale, int dtype,
                       double* out) {
  if (batch < 0 || n_head <= 0 || n_kv_head <= 0 || q_len < 0 ||
      head_dim <= 0 || capacity <= 0 || n_head % n_kv_head != 0 ||
      (dtype != ORACLE_F16 && dtype != ORACLE_BF16))
    return -1;
  if (batch == 0 || q_len == 0) return 0;
  if (!q || !k_cache || !v_cache || !start || !out) return -1;

  const int group = n_head / n_kv_head;
  const long rows = (long)batch * n_head * q_len;
  int failed = 0;

#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
  for (long r = 0; r < rows; ++r) {
    const int t = (int)(r % q_len);
    const int h = (int)((r / q_len) % n_head);
    const int b = (int)(r / ((long)q_len * n_head));
    const int g = h / group;
    long nl = (long)start[b] + t + 1;
    if (nl < 0) nl = 0;
    if (nl > capacity) nl = capacity;
    const int n = (int)nl;

    double* o = out + r * head_dim;
    for (int d = 0; d < head_dim; ++d) o[d] = 0.0;
    if (n == 0) continue;

    const uint16_t* qrow = q + r * head_dim;
    const uint16_t* kbase =
        k_cache + ((size_t)b * n_kv_head + g) * (size_t)capacity * head_dim;
    const uint16_t* vbase =
        v_cache + ((size_t)b * n_kv_head + g) * (size_t)capacity * head_dim;

    double* qd = (double*)malloc(sizeof(double) * head_dim);
    double* x = (double*)malloc(sizeof(double) * n);
    if (!qd || !x) {
      free(qd);
      free(x);
      failed = 1;
      continue;
    }
    for (int d = 0; d < head_dim; ++d) qd[d] = decode16(qrow[d], dtype);
    for (int j = 0; j < n; ++j) {
      const uint16_t* krow = kbase + (size_t)j * head_dim;
      double dot = 0.0;
      for (int d = 0; d < head_dim; ++d) dot += qd[d] * decode16(krow[d], dtype);
      x[j] = scale * dot;
    }
    double m = x[0];
    for (int j = 1; j < n; ++j)
      if (x[j] > m) m = x[j];
    double wsum = 0.0;
    for (int j = 0; j < n; ++j) {
      x[j] = exp(x[j] - m);
      wsum += x[j];
    }
    for (int j = 0; j < n; ++j) {
      const uint16_t* vrow = vbase + (size_t)j * head_dim;
      for (int d = 0; d < head_dim; ++d) o[d] += x[j] * decode16(vrow[d], dtype);
    }
    for (int d = 0; d < head_dim; ++d) o[d] /= wsum;
    free(qd);
    free(x);
  }
  return failed ? -2 : 0;
}

/*
 * Prompt append: the T new key and value rows of every (batch row, KV head)
 * go to slots start[b] .. start[b] + T - 1 of the preallocated caches, bit
 * for bit ([ACTIVE-PREFIX] section 2: prefill fills the first kv_len = T
 * slots, the allocation is unchanged). Rows whose slot falls outside
 * [0, capacity) are not written.
 *
 *   k_new, v_new [batch, n_kv_head, T, head_dim]
 */
int ada_oracle_prefill_append(const uint16_t* k_new, const uint16_t* v_new,
                              uint16_t* k_cache, uint16_t* v_cache,
                              const int32_t* start, int batch, int n_kv_head,
                              int q_len, int capacity, int head_dim) {
  if (batch < 0 || n_kv_head <= 0 || q_len < 0 || capacity <= 0 || head_dim <= 0)
    return -1;
  if (batch == 0 || q_len == 0) return 0;
  if (!k_new || !v_new || !k_cache || !v_cache || !start) return -1;
  for (int b = 0; b < batch; ++b) {
    for (int g = 0; g < n_kv_head; ++g) {
      for (int t = 0; t < q_len; ++t) {
        long p = (long)start[b] + t;
        if (p < 0 || p >= capacity) continue;
        size_t src = (((size_t)b * n_kv_head + g) * q_len + t) * head_dim;
        size_t dst = (((size_t)b * n_kv_head + g) * capacity + (size_t)p) * head_dim;
        memcpy(k_cache + dst, k_new + src, sizeof(uint16_t) * head_dim);
        memcpy(v_cache + dst, v_new + src, sizeof(uint16_t) * head_dim);
      }
    }
  }
  return 0;
}
