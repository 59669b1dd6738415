/* Drives the CPU oracle (oracle/ada_oracle.c) on seeded small inputs and its
 * edge cases -- empty, negative, clamped and ragged lengths, NaN-filled cache
 * tails, continued prompts, appends outside the cache, rejected arguments --
 * for a build under AddressSanitizer and UndefinedBehaviorSanitizer. Outputs
 * must be finite wherever the slots they attend to are. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int ada_oracle_decode(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache, const int32_t* kv_len,
                      int batch, int n_head, int n_kv_head, int head_dim, int capacity, double scale, int dtype,
                      double* out);
int ada_oracle_kv_append(const uint16_t* k_new, const uint16_t* v_new, uint16_t* k_cache, uint16_t* v_cache,
                         const int32_t* pos, int batch, int n_kv_head, int capacity, int head_dim);
int ada_oracle_prefill(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache, const int32_t* start,
                       int batch, int n_head, int n_kv_head, int q_len, int head_dim, int capacity, double scale,
                       int dtype, double* out);
int ada_oracle_prefill_append(const uint16_t* k_new, const uint16_t* v_new, uint16_t* k_cache, uint16_t* v_cache,
                              const int32_t* start, int batch, int n_kv_head, int q_len, int capacity, int head_dim);

static uint64_t state = 20261202u;
static uint32_t next(void) {
  state = state * 6364136223846793005ull + 1442695040888963407ull;
  return (uint32_t)(state >> 33);
}
/* A random finite 16-bit value of magnitude below 4 in either format. */
static uint16_t rand16(int dtype) {
  const uint32_t sign = (next() & 1u) << 15;
  if (dtype == 0) return (uint16_t)(sign | ((uint32_t)(next() % 17u) << 10) | (next() & 0x3ffu)); /* exp 0..16 */
  return (uint16_t)(sign | ((uint32_t)(100u + next() % 28u) << 7) | (next() & 0x7fu));          /* exp 100..127 */
}
static int failures = 0, checks = 0;
static void expect(int ok, const char* what) {
  ++checks;
  if (!ok) {
    printf("FAIL %s\n", what);
    ++failures;
  }
}

int main(void) {
  for (int it = 0; it < 400; ++it) {
    const int dtype = (int)(next() % 2);
    const int B = 1 + (int)(next() % 3), Hkv = 1 + (int)(next() % 3), G = 1 + (int)(next() % 4), Hq = Hkv * G;
    const int D = (int)(next() % 3) == 0 ? 128 : 1 + (int)(next() % 9);
    const int S = 1 + (int)(next() % 40);
    const size_t cache = (size_t)B * Hkv * S * D;
    uint16_t* q = malloc(sizeof(uint16_t) * (size_t)B * Hq * S * D);
    uint16_t* k = malloc(sizeof(uint16_t) * cache);
    uint16_t* v = malloc(sizeof(uint16_t) * cache);
    double* out = malloc(sizeof(double) * (size_t)B * Hq * S * D);
    int32_t len[3], start[3];
    for (size_t i = 0; i < (size_t)B * Hq * S * D; ++i) q[i] = rand16(dtype);
    for (int b = 0; b < B; ++b) {
      const int r = (int)(next() % 6);
      len[b] = r == 0 ? 0 : r == 1 ? -5 : r == 2 ? S + 7 : (int)(1 + next() % (unsigned)S);
      start[b] = r == 0 ? S : r == 1 ? -3 : (int)(next() % (unsigned)S);
    }
    /* finite values in the attended slots, NaN beyond */
    for (int b = 0; b < B; ++b) {
      const int n = len[b] < 0 ? 0 : (len[b] > S ? S : len[b]);
      for (int h = 0; h < Hkv; ++h)
        for (int j = 0; j < S; ++j)
          for (int d = 0; d < D; ++d) {
            const size_t i = (((size_t)b * Hkv + h) * S + j) * D + d;
            k[i] = j < n ? rand16(dtype) : (dtype == 0 ? 0x7e00 : 0x7fc0);
            v[i] = j < n ? rand16(dtype) : (dtype == 0 ? 0x7e00 : 0x7fc0);
          }
    }
    const double scale = (next() % 4) == 0 ? 0.0 : 1.0 / sqrt((double)D);
    expect(ada_oracle_decode(q, k, v, len, B, Hq, Hkv, D, S, scale, dtype, out) == 0, "decode status");
    int finite = 1;
    for (size_t i = 0; i < (size_t)B * Hq * D; ++i) finite &= isfinite(out[i]) != 0;
    expect(finite, "decode finite over the attended prefix");
    /* rejected arguments leave nothing written and return -1 */
    expect(ada_oracle_decode(q, k, v, len, B, Hq, Hq + 1, D, S, scale, dtype, out) == -1,
           "decode rejects a bad head map");
    expect(ada_oracle_decode(q, k, v, len, B, Hq, Hkv, D, S, scale, 7, out) == -1, "decode rejects dtype");
    /* appends inside and outside the cache */
    uint16_t kn[3 * 3 * 128], vn[3 * 3 * 128];
    for (int i = 0; i < B * Hkv * D; ++i) kn[i] = rand16(dtype), vn[i] = rand16(dtype);
    int32_t pos[3];
    for (int b = 0; b < B; ++b) pos[b] = (int)(next() % (unsigned)(S + 4)) - 2;
    expect(ada_oracle_kv_append(kn, vn, k, v, pos, B, Hkv, S, D) == 0, "append status");
    /* prefill over the whole cache (every slot finite now), continued prompts */
    for (size_t i = 0; i < cache; ++i) k[i] = rand16(dtype), v[i] = rand16(dtype);
    const int T = 1 + (int)(next() % (unsigned)S);
    expect(ada_oracle_prefill(q, k, v, start, B, Hq, Hkv, T, D, S, scale, dtype, out) == 0, "prefill status");
    finite = 1;
    for (size_t i = 0; i < (size_t)B * Hq * T * D; ++i) finite &= isfinite(out[i]) != 0;
    expect(finite, "prefill finite");
    uint16_t* kp = malloc(sizeof(uint16_t) * (size_t)B * Hkv * T * D);
    uint16_t* vp = malloc(sizeof(uint16_t) * (size_t)B * Hkv * T * D);
    for (size_t i = 0; i < (size_t)B * Hkv * T * D; ++i) kp[i] = rand16(dtype), vp[i] = rand16(dtype);
    expect(ada_oracle_prefill_append(kp, vp, k, v, start, B, Hkv, T, S, D) == 0, "prefill append status");
    free(kp);
    free(vp);
    free(q);
    free(k);
    free(v);
    free(out);
  }
  printf("oracle driver: %d checks, %d failures\n", checks, failures);
  return failures ? 1 : 0;
}
