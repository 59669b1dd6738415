// Drives every entry point of libada's C ABI through its host-side paths
// (validation, split planning, workspace arithmetic, dispatch to the launch
// stubs) with fixed edge cases and a seeded fuzz of argument values, for a
// build under AddressSanitizer and UndefinedBehaviorSanitizer. Device
// pointers are fake aligned addresses: the host side never dereferences
// them. Without a GPU, calls that need the device's compute-unit count end
// in ADA_ERR_HIP; forced split counts reach the stubs.
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <random>

#include "ada.h"

namespace {
int failures = 0, checks = 0;
void expect(int got, int want, const char* what) {
  ++checks;
  if (got != want) {
    std::printf("FAIL %s: got %d want %d\n", what, got, want);
    ++failures;
  }
}
bool known_status(int s) { return s <= 0 && s >= -12; }
void* dev(uintptr_t k) { return reinterpret_cast<void*>(0x100000 + 256 * k); }
int32_t* dev_i(uintptr_t k) { return static_cast<int32_t*>(dev(k)); }
void* misaligned() { return reinterpret_cast<void*>(0x100008); }
}  // namespace

int main() {
  // Fixed cases, one per status of each entry point.
  const size_t big = size_t(1) << 40;
  expect(ada_abi_version(), ADA_ABI_VERSION, "abi version");
  for (int s = 1; s >= -12; --s) ++checks, (void)ada_status_string(s);
  expect(ada_kv_append(dev(1), dev(2), dev(3), dev(4), dev_i(5), 2, 8, 1024, 128, ADA_F16, nullptr), ADA_OK, "append");
  expect(ada_kv_append(dev(1), dev(2), dev(3), dev(4), dev_i(5), 2, 8, 1024, 64, ADA_F16, nullptr), ADA_ERR_HEAD_DIM,
         "append head_dim");
  expect(ada_kv_append(misaligned(), dev(2), dev(3), dev(4), dev_i(5), 2, 8, 1024, 128, ADA_BF16, nullptr),
         ADA_ERR_ALIGN, "append align");
  expect(ada_decode_attn_gqa_ex(dev(1), dev(2), dev(3), dev_i(4), 4, 32, 8, 128, 8192, 8192, 0.088f, ADA_BF16, dev(5),
                                dev(6), big, nullptr, 7),
         ADA_OK, "decode forced splits");
  expect(ada_decode_attn_gqa_ex(dev(1), dev(2), dev(3), dev_i(4), 4, 32, 8, 128, 8192, 8192, NAN, ADA_BF16, dev(5),
                                dev(6), big, nullptr, 7),
         ADA_ERR_SCALE, "decode scale");
  expect(ada_decode_attn_gqa_ex(dev(1), dev(2), dev(3), dev_i(4), 4, 32, 8, 128, 8192, 8192, 0.088f, ADA_BF16, dev(5),
                                dev(6), 16, nullptr, 7),
         ADA_ERR_WORKSPACE, "decode workspace");
  expect(ada_decode_attn_gqa_ex(dev(1), dev(2), dev(3), dev_i(4), 4, 36, 8, 128, 8192, 8192, 0.088f, ADA_BF16, dev(5),
                                dev(6), big, nullptr, 7),
         ADA_ERR_GQA, "decode gqa");
  expect(ada_decode_step(dev(1), dev(2), dev(3), dev(4), dev(5), dev_i(6), 1, 32, 8, 128, 32768, 1257, 0.088f, ADA_F16,
                         dev(7), dev(8), big, nullptr, 20),
         ADA_OK, "decode step forced splits");
  expect(ada_decode_step_rope(dev(1), dev(2), dev(3), dev(9), dev(10), dev(4), dev(5), dev_i(6), 1, 32, 8, 128, 32768,
                              1257, 0.088f, ADA_F16, dev(7), dev(8), big, nullptr, 1),
         ADA_OK, "decode step rope");
  expect(ada_rope_kv_append(dev(1), dev(1), dev(2), dev(3), dev(4), dev(5), dev(6), dev(7), dev_i(8), 4, 32, 8, 8192,
                            128, ADA_BF16, nullptr),
         ADA_OK, "rope append");
  expect(ada_prefill_append(dev(1), dev(2), dev(3), dev(4), nullptr, 1, 8, 4096, 8192, 128, ADA_BF16, nullptr), ADA_OK,
         "prefill append");
  expect(ada_decode_combine(dev(1), big, 8, 32, 8, 128, 8, ADA_BF16, dev(2), nullptr), ADA_OK, "combine");
  int used = -1;
  expect(ada_decode_partial(dev(1), dev(2), dev(3), nullptr, 8, 32, 8, 128, 32768, 32768, 0.088f, ADA_BF16, 8, dev(4),
                            big, &used, nullptr),
         ADA_OK, "partial");
  expect(used, 8, "partial splits used");
  ada_step_graph* g = nullptr;
  expect(ada_step_graph_create(nullptr, 1, dev_i(1), 1, 32, 8, 128, 32768, 10, 0.088f, ADA_F16, 1, dev(2), big, &g),
         ADA_ERR_NULL, "graph layers");
  expect(ada_step_graph_launch(nullptr, nullptr), ADA_ERR_NULL, "graph launch");
  ada_step_graph_destroy(nullptr);

  // Seeded fuzz: every entry point with arguments drawn from interesting
  // values; every call must return a known status (and the sanitizers stay
  // quiet).
  std::mt19937_64 rng(20261202);
  const int ints[] = {INT_MIN, -65536, -3, -1, 0, 1, 2, 3, 4, 7, 8, 9, 16, 17, 31, 32, 63, 64, 65, 127, 128, 129, 255,
                      256, 257, 1000, 1024, 4096, 8191, 8192, 32768, 65535, 65536, 1 << 20, 1 << 23, 1 << 25,
                      (1 << 25) + 1, INT_MAX / 256, INT_MAX / 2, INT_MAX};
  auto pick = [&]() { return ints[rng() % (sizeof(ints) / sizeof(ints[0]))]; };
  auto ptr = [&]() -> void* {
    switch (rng() % 8) {
      case 0: return nullptr;
      case 1: return misaligned();
      default: return dev(rng() % 64);
    }
  };
  const float scales[] = {0.088f, 0.0f, -1.0f, 1e30f, INFINITY, -INFINITY, NAN};
  for (int it = 0; it < 20000; ++it) {
    const int B = pick(), Hq = pick(), Hkv = pick(), D = (rng() % 4) ? 128 : pick(), S = pick(), n = pick(),
              splits = (rng() % 3) ? static_cast<int>(rng() % 300) : pick(), dt = static_cast<int>(rng() % 3);
    const float sc = scales[rng() % 7];
    const size_t ws = (rng() % 2) ? big : static_cast<size_t>(rng() % 100000);
    int s;
    s = ada_decode_attn_gqa_ex(ptr(), ptr(), ptr(), static_cast<const int32_t*>(ptr()), B, Hq, Hkv, D, S, n, sc, dt,
                               ptr(), ptr(), ws, nullptr, splits);
    expect(known_status(s), true, "fuzz decode");
    s = ada_decode_step(ptr(), ptr(), ptr(), ptr(), ptr(), static_cast<const int32_t*>(ptr()), B, Hq, Hkv, D, S, n, sc,
                        dt, ptr(), ptr(), ws, nullptr, splits);
    expect(known_status(s), true, "fuzz step");
    s = ada_decode_step_rope(ptr(), ptr(), ptr(), ptr(), ptr(), ptr(), ptr(), static_cast<const int32_t*>(ptr()), B, Hq,
                             Hkv, D, S, n, sc, dt, ptr(), ptr(), ws, nullptr, splits);
    expect(known_status(s), true, "fuzz step rope");
    int u = 0;
    s = ada_decode_partial(ptr(), ptr(), ptr(), static_cast<const int32_t*>(ptr()), B, Hq, Hkv, D, S, n, sc, dt, splits,
                           ptr(), ws, &u, nullptr);
    expect(known_status(s), true, "fuzz partial");
    s = ada_decode_combine(ptr(), ws, B, Hq, Hkv, D, splits, dt, ptr(), nullptr);
    expect(known_status(s), true, "fuzz combine");
    s = ada_kv_append(ptr(), ptr(), ptr(), ptr(), static_cast<const int32_t*>(ptr()), B, Hkv, S, D, dt, nullptr);
    expect(known_status(s), true, "fuzz append");
    s = ada_rope_kv_append(ptr(), ptr(), ptr(), ptr(), ptr(), ptr(), ptr(), ptr(), static_cast<const int32_t*>(ptr()),
                           B, Hq, Hkv, S, D, dt, nullptr);
    expect(known_status(s), true, "fuzz rope append");
    s = ada_prefill_append(ptr(), ptr(), ptr(), ptr(), static_cast<const int32_t*>(ptr()), B, Hkv, n, S, D, dt,
                           nullptr);
    expect(known_status(s), true, "fuzz prefill append");
    s = ada_prefill_attn_gqa(ptr(), ptr(), ptr(), static_cast<const int32_t*>(ptr()), B, Hq, Hkv, n, D, S, sc, dt,
                             ptr(), nullptr);
    expect(known_status(s), true, "fuzz prefill");
    (void)ada_decode_num_splits(B, Hq, Hkv, n, pick());
    {
      int ps = 0, pc = 0;
      s = ada_decode_plan(B, Hq, Hkv, n, splits, pick(), &ps, &pc);
      expect(known_status(s), true, "fuzz plan");
      if (s == ADA_OK) expect(ps >= 1 && ps <= ADA_MAX_SPLITS && pc >= 1, true, "fuzz plan range");
    }
    (void)ada_decode_workspace_bytes(B, Hq, Hkv, D, splits);
    s = ada_decode_attn_gqa_noalloc(ptr(), ptr(), ptr(), static_cast<const int32_t*>(ptr()), B, Hq, Hkv, D, S, n,
                                    sc, dt, ptr(), nullptr, splits);
    expect(known_status(s), true, "fuzz noalloc");
    s = ada_hbm_read(ptr(), static_cast<size_t>(n) * 16 + (rng() % 4 == 0 ? 8 : 0), static_cast<uint32_t*>(ptr()),
                     pick(), nullptr);
    expect(known_status(s), true, "fuzz read probe");
    (void)ada_prefill_rows_per_workgroup(B, Hq, Hkv, n, pick());
    ada_step_layer layers[2];
    for (ada_step_layer& l : layers) l = {ptr(), ptr(), ptr(), ptr(), ptr(), ptr(), (rng() % 2) ? ptr() : nullptr, nullptr};
    ada_step_graph* gr = nullptr;
    s = ada_step_graph_create(layers, static_cast<int>(rng() % 3), static_cast<int32_t*>(ptr()), B, Hq, Hkv, D, S, n,
                              sc, dt, static_cast<int>(rng() % 2), ptr(), ws, &gr);
    expect(known_status(s), true, "fuzz graph");
    if (s == ADA_OK) ada_step_graph_destroy(gr);
  }
  // Split plans over a grid of shapes: the plan covers the prefix, stays
  // within ADA_MAX_SPLITS and its workspace size is consistent.
  for (int B : {1, 2, 4, 8, 64, 65, 1000})
    for (int Hkv : {1, 2, 8, 16})
      for (int n : {1, 63, 64, 65, 255, 256, 257, 400, 1024, 1258, 4096, 8192, 32768, 1 << 20, 1 << 25})
        for (int cus : {1, 80, 256, 304}) {
          const int sp = ada_decode_num_splits(B, 4 * Hkv, Hkv, n, cus);
          expect(sp >= 1 && sp <= ADA_MAX_SPLITS, true, "plan range");
          int ps = 0, pc = 0;
          expect(ada_decode_plan(B, 4 * Hkv, Hkv, n, 0, cus, &ps, &pc), ADA_OK, "plan call");
          expect(ps == sp && static_cast<long>(ps) * pc >= n && static_cast<long>(ps - 1) * pc < n, true,
                 "plan covers the prefix");
          expect(ada_decode_workspace_bytes(B, 4 * Hkv, Hkv, 128, sp) > 0, true, "plan workspace");
        }
  std::printf("abi driver: %d checks, %d failures\n", checks, failures);
  return failures ? 1 : 0;
}
