// ada_kernels.hip -- gfx950 kernels of libada: single-token decode attention
// over the active prefix of a preallocated KV cache, and the in-place append.
//
// Pages cited (by title and section):
//   [DECODE-FASTPATH] Cuda-Compute-OSS issue #343, "one-token decode fast
//                     path: skip FlashAttention's prefill-tuned tiling for
//                     q_len=1".
//   [ACTIVE-PREFIX]   fish-speech issue #1310, "Optimize native AR decoding
//                     by attending only to the active KV-cache prefix".
//   [FORWARD-STEP]    VoxCPM issue #395, "MiniCPM4
//                     MiniCPMAttention.forward_step Attention Performance Fix".
//
// The decode step reads every live K and V row once per KV head and does a
// few flops per byte, so it is bound by HBM bandwidth ([DECODE-FASTPATH],
// "Current limitation"). The design follows from that:
//
//   * Partial kernel: one workgroup (4 wavefronts) per (key-range split, KV
//     head, batch row). Each K/V row it loads serves all G = n_head /
//     n_kv_head query heads of the group: KV heads are never expanded
//     ([ACTIVE-PREFIX] section 1).
//   * Lane layout: L lanes per key row (8 for G <= 4, 16 above), each lane
//     holding 8 or 16 head dims in 16-byte chunks, so one 16-byte load per
//     lane covers 64 / L consecutive rows in contiguous 128- or 256-byte
//     runs: fully coalesced, with the nontemporal cache policy (each byte is
//     read once). Loads run P tiles ahead of the compute through a register
//     ring.
//   * q.k in fp32 with the packed 16-bit dot instructions (products of two
//     16-bit values are exact in fp32), summed over the L lanes of a row with
//     DPP butterfly adds; scale*log2(e) is applied to the sum.
//   * Online softmax in base 2 with one reference m per head for the whole
//     wavefront (sum l and fp32 accumulator per lane), rescaling only when a
//     score exceeds the reference by more than 2^8 (so almost never after
//     the first rows). At the end the lane groups' sums are added by a
//     butterfly of 32/16-lane permlane swaps and a DPP rotate that carries
//     two accumulators per exchange; wavefronts merge through LDS.
//   * Rotary decode step: the query heads and the new key are rotated once
//     per workgroup (rotate-half form, correctly rounded to 16 bits) and
//     shared through LDS ([FORWARD-STEP] section 4).
//   * With one split the workgroup writes the output directly. With several
//     splits each workgroup stores its (m, l, acc) partial and a second,
//     small kernel merges a row's partials in split order (log-sum-exp
//     weights), so the result does not depend on scheduling. The kernel
//     boundary publishes the partials once per launch; a per-workgroup
//     device-scope release (which writes back the L2 of the workgroup's XCD)
//     measured far slower on this chip once workgroups number in the hundreds.
//   * Slots at and beyond kv_len[b] are never loaded: the tail may hold
//     anything ([ACTIVE-PREFIX] section 2; [FORWARD-STEP] section 3).
//   * fp32 -> fp16/bf16 output conversion rounds to nearest even
//     ([DECODE-FASTPATH], "Proposed implementation": cast back to the input
//     type).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ada_internal.h"

namespace ada {
namespace {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = kThreads / 64;
constexpr float kNegInf = -__builtin_inff();
// Largest base-2 exponent a softmax weight may reach before the accumulator
// is rescaled (weights stay <= 256, sums stay far inside fp32 range).
constexpr float kRescaleSlack = 8.0f;

struct F16 {
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c,
                                  false);
  }
  static __device__ __forceinline__ void unpack(uint32_t u, float& lo, float& hi) {
    f16x2 h = __builtin_bit_cast(f16x2, u);
    lo = static_cast<float>(h.x);
    hi = static_cast<float>(h.y);
  }
  static __device__ __forceinline__ uint16_t round(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
  }
};

struct BF16 {
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), c, false);
  }
  static __device__ __forceinline__ void unpack(uint32_t u, float& lo, float& hi) {
    lo = __uint_as_float(u << 16);
    hi = __uint_as_float(u & 0xffff0000u);
  }
  static __device__ __forceinline__ uint16_t round(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
  }
};

// ---------------------------------------------------------------------------
// Cross-lane reductions. A "row" of the hardware is 16 lanes; DPP moves data
// within a row, the permlane swaps exchange rows 16 and 32 lanes apart.

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <- lane 7-i within each 8
constexpr int kDppRor8 = 0x128;       // lane i <- lane i^8 within each 16
constexpr int kDppRowShr1 = 0x111;    // lane i <- lane i-1 within each 16 (none for the first)
constexpr int kDppRowShr2 = 0x112;
constexpr int kDppRowShr4 = 0x114;
constexpr int kDppRowShr8 = 0x118;

struct Sum {
  static __device__ __forceinline__ float op(float a, float b) { return a + b; }
};
struct Max {
  static __device__ __forceinline__ float op(float a, float b) { return fmaxf(a, b); }
};

template <class Op>
__device__ __forceinline__ float xor16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return Op::op(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
template <class Op>
__device__ __forceinline__ float xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return Op::op(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Reduce over the L consecutive lanes of a lane group (L = 8 or 16).
template <int L>
__device__ __forceinline__ float lane_group_sum(float x) {
  x += dpp<kDppXor1>(x);
  x += dpp<kDppXor2>(x);
  x += dpp<kDppHalfMirror>(x);
  if constexpr (L == 16) x += dpp<kDppRor8>(x);
  return x;
}

// Reduce over the 64 / L lane groups of a wavefront (lanes equal modulo L).
template <int L, class Op>
__device__ __forceinline__ float across_groups(float x) {
  if constexpr (L == 8) x = Op::op(x, dpp<kDppRor8>(x));
  x = xor16<Op>(x);
  return xor32<Op>(x);
}

// Reduce over all 64 lanes.
template <class Op>
__device__ __forceinline__ float wave_reduce(float x) {
  x = Op::op(x, dpp<kDppXor1>(x));
  x = Op::op(x, dpp<kDppXor2>(x));
  x = Op::op(x, dpp<kDppHalfMirror>(x));
  x = Op::op(x, dpp<kDppRor8>(x));
  x = xor16<Op>(x);
  return xor32<Op>(x);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Reference for exp2(m - ref): the running maximum itself, or 0 while it is
// still -inf (nothing seen yet), so that an empty state weighs exp2(-inf) = 0.
__device__ __forceinline__ float finite_ref(float m) { return m == kNegInf ? 0.0f : m; }

__device__ __forceinline__ uint4 load16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// K/V rows are read exactly once: nontemporal loads (the `nt` cache policy)
// stream them past the caches. On MI355X a plain read kernel reaches about
// 6.4 TB/s with ordinary loads and about 7.2 TB/s with nontemporal ones.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load16_stream(const uint16_t* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <class E>
__device__ __forceinline__ void unpack8(const uint4& u, float* f) {
  E::unpack(u.x, f[0], f[1]);
  E::unpack(u.y, f[2], f[3]);
  E::unpack(u.z, f[4], f[5]);
  E::unpack(u.w, f[6], f[7]);
}

template <class E>
__device__ __forceinline__ float dot8(const uint4& k, const uint4& q, float s) {
  s = E::dot2(k.x, q.x, s);
  s = E::dot2(k.y, q.y, s);
  s = E::dot2(k.z, q.z, s);
  return E::dot2(k.w, q.w, s);
}

// ---------------------------------------------------------------------------
// Rotary embedding of the new token's query and key before the cache write
// ([FORWARD-STEP] section 4 applies apply_rotary_pos_emb there; it is read
// as the rotate-half form): with h = D / 2,
//   out[i] = x[i] cos[i] - x[i + h] sin[i]    (i <  h)
//   out[i] = x[i] cos[i] + x[i - h] sin[i]    (i >= h)
// over the stored 16-bit values, rounded once to the 16-bit format (nearest,
// ties to even; a zero result is +0).
//
// Both products are exact in fp32 (two 8- or 11-bit significands; inputs
// whose products fall below fp32's normal range are the exception). The sum
// is formed with its exact rounding error (Knuth's two-sum), and the fp32
// result is then rounded to odd: an inexact sum moves to the neighbour with
// an odd last bit on the side of the exact value. An fp32 value rounded to
// odd keeps enough information for the final round-to-nearest-even to 16
// bits (13 or 16 fewer significand bits) to give the correctly rounded
// result of the exact sum.
template <class E>
__device__ __forceinline__ uint32_t round_sum(float a, float b) {
  const float s = a + b;
  const float bv = s - a;
  const float av = s - bv;
  const float err = (a - av) + (b - bv);
  uint32_t bits = __float_as_uint(s);
  if (err != 0.0f && __builtin_isfinite(s)) {
    if ((err < 0.0f) != (s < 0.0f)) bits -= 1u;  // truncate toward zero...
    bits |= 1u;                                  // ...then force the last bit odd
  }
  const uint32_t r = E::round(__uint_as_float(bits));
  return (r & 0x7fffu) == 0 ? 0u : r;
}

// Rotate 8 consecutive dims [d0, d0 + 8) of a head: x holds them, partner the
// dims h away (d0 +- h), c and s the table entries of [d0, d0 + 8).
template <class E>
__device__ __forceinline__ uint4 rope8(const uint4& x, const uint4& partner, const uint4& c, const uint4& s,
                                       bool first_half) {
  float xf[8], pf[8], cf[8], sf[8];
  unpack8<E>(x, xf);
  unpack8<E>(partner, pf);
  unpack8<E>(c, cf);
  unpack8<E>(s, sf);
  uint32_t w[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float p0 = pf[2 * k] * sf[2 * k];
    const float p1 = pf[2 * k + 1] * sf[2 * k + 1];
    const uint32_t lo = round_sum<E>(xf[2 * k] * cf[2 * k], first_half ? -p0 : p0);
    const uint32_t hi = round_sum<E>(xf[2 * k + 1] * cf[2 * k + 1], first_half ? -p1 : p1);
    w[k] = lo | (hi << 16);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Rotated 16-byte chunk at dims [d0, d0 + 8) of the head starting at `row`,
// with the table row `cs` / `sn` (D entries each).
template <class E>
__device__ __forceinline__ uint4 rope_chunk(const uint16_t* row, const uint16_t* cs, const uint16_t* sn, int d0) {
  constexpr int H = kHeadDim / 2;
  const int partner = d0 < H ? d0 + H : d0 - H;
  return rope8<E>(load16(row + d0), load16(row + partner), load16(cs + d0), load16(sn + d0), d0 < H);
}

// ---------------------------------------------------------------------------
// Partial kernels: shared prologue and epilogue.

// Where one workgroup stands: its split's live slot range and the indices of
// its outputs. With k_new != NULL the call is a whole decode step: the new
// key/value rows (k_new, v_new: [B, H_kv, D]) belong at slot p = pos[b] (or
// max_kv_len - 1 when pos is NULL), the workgroup of split 0 writes them
// into the cache, the workgroup whose range holds slot p reads that row from
// k_new/v_new instead of the cache (no launch waits for the write), and the
// live prefix is p + 1 slots. Otherwise lengths come from kv_len, or are
// max_kv_len for every row when kv_len is NULL (one position for the whole
// batch: nothing is read before the K/V stream starts).
// Live slots of a decode step whose new row sits at slot p: p + 1 clamped
// to [0, max_kv_len], written so that p = INT_MAX does not overflow.
__device__ __forceinline__ int step_length(int p, int max_kv_len) {
  return p < 0 ? 0 : (p >= max_kv_len ? max_kv_len : p + 1);
}

// Live slots of batch row b: pos[b] + 1 for a decode step (pos NULL: all
// rows at slot max_kv_len - 1), else kv_len[b] (NULL: max_kv_len), clamped
// to [0, max_kv_len].
__device__ __forceinline__ int row_length(const int32_t* kv_len, const int32_t* pos, bool step, int max_kv_len,
                                          int b) {
  if (step) return step_length(pos != nullptr ? pos[b] : max_kv_len - 1, max_kv_len);
  const int n = kv_len != nullptr ? kv_len[b] : max_kv_len;
  return n < 0 ? 0 : (n > max_kv_len ? max_kv_len : n);
}

// Integer sum over the 64 lanes of a wavefront (every lane gets it); all
// lanes must be active.
__device__ __forceinline__ unsigned wave_sum_u32(unsigned x) {
  x += static_cast<unsigned>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), kDppXor1, 0xF, 0xF, false));
  x += static_cast<unsigned>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), kDppXor2, 0xF, 0xF, false));
  x += static_cast<unsigned>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), kDppHalfMirror, 0xF, 0xF, false));
  x += static_cast<unsigned>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), kDppRor8, 0xF, 0xF, false));
  auto r16 = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = r16[0] + r16[1];
  auto r32 = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return r32[0] + r32[1];
}

// Inclusive prefix sum over the lanes of a wavefront; all lanes active.
// Row shifts scan each 16-lane row (a lane with no source lane d below it in
// its row adds 0), then every row adds the totals of the rows before it,
// read from their last lanes into scalars. No LDS round trip.
__device__ __forceinline__ unsigned wave_inclusive_scan(unsigned x, int lane) {
  x += static_cast<unsigned>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), kDppRowShr1, 0xF, 0xF, false));
  x += static_cast<unsigned>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), kDppRowShr2, 0xF, 0xF, false));
  x += static_cast<unsigned>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), kDppRowShr4, 0xF, 0xF, false));
  x += static_cast<unsigned>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), kDppRowShr8, 0xF, 0xF, false));
  const unsigned r0 = static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(x), 15));
  const unsigned r1 = static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(x), 31));
  const unsigned r2 = static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(x), 47));
  const int row = lane >> 4;
  return x + (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
}

// Balanced split plan for batches whose lengths live on the device (so the
// host cannot size the splits per row): the `slots` workgroups of a KV head
// are shared by all rows with one common chunk c (a multiple of the 64-slot
// tile), row b taking ceil(n_b / c) consecutive slots. c is the smallest
// multiple of 64 from ceil(total / slots) on for which the rows fit (tried 8
// times), else ceil(total / (slots - batch)) rounded up, which always fits
// (each row wastes less than one chunk). Every kernel of a call derives the
// same plan from the same lengths.
//
// Evaluated by a whole wavefront, one batch row per lane (batch <= 64, all
// lanes active): lane-parallel divisions and cross-lane sums instead of a
// serial walk over the rows. The host keeps max_kv_len <= 2^25 on this path,
// so every sum fits in 32 bits. Returns, for the lane's row (zeros for lanes
// past the batch), its first slot and slot count, and for a decode step the
// slot of its new row; the chunk is the same in every lane.
struct BalancedRows {
  int chunk;
  int first;  // first workgroup slot of this lane's row
  int count;  // slots of this lane's row
  int p;      // decode step: pos[lane] (pos NULL: max_kv_len - 1)
};

__device__ __forceinline__ BalancedRows balanced_rows(const int32_t* kv_len, const int32_t* pos, bool step,
                                                      int max_kv_len, int batch, int slots, int lane) {
  int p = max_kv_len - 1;
  unsigned n = 0;
  if (lane < batch) {
    if (step && pos != nullptr) p = pos[lane];
    n = static_cast<unsigned>(step ? step_length(p, max_kv_len) : row_length(kv_len, pos, false, max_kv_len, lane));
  }
  const unsigned total = wave_sum_u32(n);
  const unsigned tile = kTileRows;
  auto round_tile = [&](unsigned c) { return c < tile ? tile : (c + tile - 1) / tile * tile; };
  unsigned c = round_tile((total + slots - 1) / slots);
  bool fits = false;
  for (int tries = 0; tries < 8; ++tries, c += tile) {
    if (wave_sum_u32((n + c - 1) / c) <= static_cast<unsigned>(slots)) {
      fits = true;
      break;
    }
  }
  if (!fits) {
    const unsigned free = slots - batch;  // >= batch: the host asks for >= 2 slots per row
    c = round_tile((total + free - 1) / free);
  }
  const unsigned count = (n + c - 1) / c;
  const unsigned incl = wave_inclusive_scan(count, lane);
  return {static_cast<int>(c), static_cast<int>(incl - count), static_cast<int>(count), p};
}

struct SplitRange {
  int n;          // live slots of this batch row
  int row_begin;  // this split's first slot
  int last_row;   // this split's last live slot
  int p_new;      // slot appended by this call, or -1
  int split;      // this workgroup's split of its row (0 writes the appended row)
  int b;          // batch row (not the grid's z index under the balanced plan)
  size_t head_off;   // (b, g) head of the caches, in elements
  size_t new_row;    // (b, g) row of k_new / v_new, in elements
  size_t out_row0;   // first output element of the group's query heads
  size_t part_row0;  // first partial entry of the group's query heads
};

// Returns false when the split holds no live slot; it has then written what
// an empty split owes (a zero row when writing the output directly, an
// "empty" mark for the combine otherwise).
template <int G, bool R>
__device__ __forceinline__ bool begin_split(SplitRange& r, uint16_t* k_cache, uint16_t* v_cache,
                                            const int32_t* kv_len, const uint16_t* k_new,
                                            const uint16_t* v_new, const int32_t* pos, uint16_t* out,
                                            float2* part_ml, int n_kv_head, int capacity, int max_kv_len,
                                            int chunk, int direct) {
  constexpr int D = kHeadDim;
  const int g = blockIdx.y;
  const int tid = threadIdx.x;
  const int n_head = n_kv_head * G;
  int split = blockIdx.x;
  int b = blockIdx.z;
  size_t slot = static_cast<size_t>(split) * gridDim.z + b;  // partial slot (split-major)
  int p_dev = 0;  // under the balanced plan: pos[b], already read by lane b
  const bool balanced = chunk == 0;
  if (balanced) {
    // Balanced plan: this workgroup is slot z * splits + x of its KV head;
    // its row is the one whose slot range holds it.
    const int idx = blockIdx.z * gridDim.x + blockIdx.x;
    const int lane = tid & 63;
    const BalancedRows rows = balanced_rows(kv_len, pos, k_new != nullptr, max_kv_len, gridDim.z,
                                            gridDim.x * gridDim.z, lane);
    chunk = rows.chunk;
    const unsigned long long hit =
        __ballot(lane < static_cast<int>(gridDim.z) && idx >= rows.first && idx < rows.first + rows.count);
    if (hit == 0) return false;  // a slot no row needs: nothing to write
    b = __ffsll(hit) - 1;  // uniform: lane reads below need no LDS round trip
    split = idx - __builtin_amdgcn_readlane(rows.first, b);
    p_dev = __builtin_amdgcn_readlane(rows.p, b);
    slot = idx;
  }
  r.head_off = (static_cast<size_t>(b) * n_kv_head + g) * static_cast<size_t>(capacity) * D;
  r.new_row = (static_cast<size_t>(b) * n_kv_head + g) * D;
  r.p_new = -1;
  if (k_new != nullptr) {
    r.p_new = pos == nullptr ? max_kv_len - 1 : (balanced ? p_dev : pos[b]);
    if (split == 0 && tid < 32 && r.p_new >= 0 && r.p_new < capacity) {
      const int c = 8 * (tid & 15);  // one 16-byte chunk of the key (tid < 16) or value row
      const size_t dst = r.head_off + static_cast<size_t>(r.p_new) * D + c;
      if (tid < 16) {
        // with rotary tables the rotated key is written once it is computed
        if constexpr (!R) *reinterpret_cast<uint4*>(k_cache + dst) = load16(k_new + r.new_row + c);
      } else {
        *reinterpret_cast<uint4*>(v_cache + dst) = load16(v_new + r.new_row + c);
      }
    }
  }
  if (k_new != nullptr) {
    r.n = step_length(r.p_new, max_kv_len);
  } else {
    const int n = kv_len != nullptr ? kv_len[b] : max_kv_len;
    r.n = n < 0 ? 0 : (n > max_kv_len ? max_kv_len : n);
  }
  const int nsplit = (r.n + chunk - 1) / chunk;  // splits holding live slots
  const size_t head_row0 = static_cast<size_t>(b) * n_head + static_cast<size_t>(g) * G;
  r.out_row0 = head_row0 * D;
  r.part_row0 = slot * n_head + static_cast<size_t>(g) * G;  // slot-major partials
  if (split >= nsplit) {
    if (direct) {
      for (int idx = tid; idx < G * D; idx += kThreads) out[r.out_row0 + idx] = 0;
    } else if (tid < G) {
      part_ml[r.part_row0 + tid] = make_float2(kNegInf, 0.0f);
    }
    return false;
  }
  r.split = split;
  r.b = b;
  r.row_begin = split * chunk;
  r.last_row = min(r.row_begin + chunk, r.n) - 1;
  return true;
}

// Sum V per-lane values over the 64 / L lane groups of a wavefront (lanes
// equal modulo L), two values per exchange: a lane swap of registers a and b
// followed by an add leaves a's pair sum in the lanes whose exchange bit is
// clear and b's in the others, so each step halves the live registers. At
// the end lane l holds, in x[0 .. V / (64 / L)), the sums of values
// u + (V / (64 / L)) * (l / L).
template <int L, int V>
__device__ __forceinline__ void sum_lane_groups(float (&x)[V], int lane) {
  constexpr int NG = 64 / L;
  static_assert(V % NG == 0, "values must split evenly over the lane groups");
#pragma unroll
  for (int r = 0; r < V / 2; ++r) {  // lanes 32 apart
    auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x[r]), __float_as_uint(x[r + V / 2]), false, false);
    x[r] = __uint_as_float(s[0]) + __uint_as_float(s[1]);
  }
#pragma unroll
  for (int r = 0; r < V / 4; ++r) {  // lanes 16 apart
    auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x[r]), __float_as_uint(x[r + V / 4]), false, false);
    x[r] = __uint_as_float(s[0]) + __uint_as_float(s[1]);
  }
  if constexpr (L == 8) {  // lanes 8 apart, within a 16-lane row
    const bool hi = (lane & 8) != 0;
#pragma unroll
    for (int r = 0; r < V / 8; ++r) {
      const float mine = hi ? x[r + V / 8] : x[r];
      const float send = hi ? x[r] : x[r + V / 8];
      x[r] = mine + dpp<kDppRor8>(send);
    }
  }
}

// Merge the 4 wavefronts' states through LDS and write either the output
// (one split) or this split's partial. Each wave passes its state: m[i] and
// l[i] (the same in every lane) and the accumulator sums as left by
// sum_lane_groups over acc[G][128 / L] flattened head-major, where lane
// group g's sub-lane s held dims [8*s + 64*c, +8) in slots 8*c .. 8*c + 7.
template <class E, int G, int L>
__device__ __forceinline__ void finish_split(const SplitRange& r, const float (&m)[G], const float (&l)[G],
                                             const float (&red)[G * (128 / L)], uint16_t* out,
                                             float2* part_ml, float* part_acc, int direct) {
  constexpr int D = kHeadDim;
  constexpr int DPL = 128 / L;
  constexpr int V = G * DPL;
  constexpr int PER = V / (64 / L);  // sums held per lane
  __shared__ float s_acc[kWaves][G][D];
  __shared__ float2 s_ml[kWaves][G];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int sub = lane % L;
  const int v0 = PER * (lane / L);
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int v = v0 + u;
    const int i = v / DPL;
    const int slot = v % DPL;
    s_acc[wave][i][8 * sub + 64 * (slot / 8) + slot % 8] = red[u];
  }
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < G; ++i) s_ml[wave][i] = make_float2(m[i], l[i]);
  }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += kThreads) {
    const int i = idx / D;
    const int d = idx % D;
    float mw = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mw = fmaxf(mw, s_ml[w][i].x);
    const float ref = finite_ref(mw);
    float lsum = 0.0f, o = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float wt = fast_exp2(s_ml[w][i].x - ref);
      lsum += s_ml[w][i].y * wt;
      o += s_acc[w][i][d] * wt;
    }
    if (direct) {
      out[r.out_row0 + idx] = E::round(o / lsum);
    } else {
      const size_t pr = r.part_row0 + i;
      part_acc[pr * D + d] = o;
      if (d == 0) part_ml[pr] = make_float2(mw, lsum);
    }
  }
}

// ---------------------------------------------------------------------------
// Partial kernel.
//
// Template parameters:
//   G  query heads per KV head
//   L  lanes per key row (8: 16 dims per lane; 16: 8 dims per lane)
//   T  rows per lane group per tile
//   P  tiles in flight ahead of the one being computed (register ring of
//      P + 1 tiles; the ring is unrolled so buffers never move)
template <class E, int G, int L, int T, int P, bool R>
__global__ __launch_bounds__(kThreads) void partial_kernel(
    const uint16_t* __restrict__ q, uint16_t* k_cache, uint16_t* v_cache,
    const int32_t* __restrict__ kv_len, const uint16_t* __restrict__ k_new,
    const uint16_t* __restrict__ v_new, const int32_t* __restrict__ pos,
    const uint16_t* __restrict__ cs, const uint16_t* __restrict__ sn,
    uint16_t* __restrict__ out, float2* __restrict__ part_ml, float* __restrict__ part_acc,
    int n_kv_head, int capacity, int max_kv_len, int chunk, int direct, float scale_log2) {
  constexpr int D = kHeadDim;
  constexpr int CH = 16 / L;             // 16-byte chunks per lane per row
  constexpr int DPL = 8 * CH;            // dims per lane
  constexpr int kRows = 64 / L;          // rows covered by one wave-wide load
  constexpr int kWaveRows = kRows * T;   // rows per wave per tile
  constexpr int kTile = kWaveRows * kWaves;
  constexpr int NB = P + 1;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int grp = lane / L;   // row of this lane within a wave-wide load
  const int sub = lane % L;   // dims [8*sub, +8) (and [64 + 8*sub, +8) when L == 8)

  SplitRange r;
  if (!begin_split<G, R>(r, k_cache, v_cache, kv_len, k_new, v_new, pos, out, part_ml, n_kv_head, capacity,
                         max_kv_len, chunk, direct))
    return;
  const int last_row = r.last_row;
  const int p_new = r.p_new;

  uint4 qv[G][CH];
  uint4 krot[R ? CH : 1];  // rotated new key (rotary tables only)
  if constexpr (!R) {
#pragma unroll
    for (int i = 0; i < G; ++i) {
#pragma unroll
      for (int c = 0; c < CH; ++c) qv[i][c] = load16(q + r.out_row0 + static_cast<size_t>(i) * D + 8 * sub + 64 * c);
    }
  }

  float m[G], l[G], acc[G][DPL];
#pragma unroll
  for (int i = 0; i < G; ++i) {
    m[i] = kNegInf;
    l[i] = 0.0f;
#pragma unroll
    for (int d = 0; d < DPL; ++d) acc[i][d] = 0.0f;
  }

  const uint16_t* kbase = k_cache + r.head_off + 8 * sub;
  const uint16_t* vbase = v_cache + r.head_off + 8 * sub;
  const uint16_t* knew = k_new != nullptr ? k_new + r.new_row + 8 * sub : kbase;
  const uint16_t* vnew = v_new != nullptr ? v_new + r.new_row + 8 * sub : vbase;

  const int wave_first = r.row_begin + wave * kWaveRows;
  const int span = last_row + 1 - wave_first;
  const int ntiles = span > 0 ? (span + kTile - 1) / kTile : 0;  // same for the whole wave
  const int my_first = wave_first + grp;

  // Rows past the split's end are loaded from its last live row (always in
  // bounds and finite) and given zero weight, so no branch guards the loads.
  uint4 kb[NB][T][CH], vb[NB][T][CH];
  auto load_tile = [&](int base, uint4 (&kr)[T][CH], uint4 (&vr)[T][CH]) {
    // Only the tile holding the appended slot (the last live row) reads a row
    // from k_new / v_new; the test is uniform across the wave.
    const int tile_row0 = base - grp;
    const bool has_new = p_new >= tile_row0 && p_new < tile_row0 + kWaveRows;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int row = min(base + t * kRows, last_row);
      const size_t off = static_cast<size_t>(row) * D;
      const uint16_t* kp = kbase + off;
      const uint16_t* vp = vbase + off;
      if (has_new && row == p_new) {
        kp = knew;
        vp = vnew;
      }
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        kr[t][c] = load16_stream(kp + 64 * c);
        vr[t][c] = load16_stream(vp + 64 * c);
      }
    }
  };

  auto process = [&](int base, const uint4 (&kr_in)[T][CH], const uint4 (&vr)[T][CH]) {
    uint4 kr[T][CH];
#pragma unroll
    for (int t = 0; t < T; ++t) {
#pragma unroll
      for (int c = 0; c < CH; ++c) kr[t][c] = kr_in[t][c];
    }
    if constexpr (R) {
      const int tile_row0 = base - grp;
      if (p_new >= tile_row0 && p_new < tile_row0 + kWaveRows) {  // uniform across the wave
#pragma unroll
        for (int t = 0; t < T; ++t) {
          if (min(base + t * kRows, last_row) == p_new) {
#pragma unroll
            for (int c = 0; c < CH; ++c) kr[t][c] = krot[c];
          }
        }
      }
    }
    float x[T][G];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const bool valid = base + t * kRows <= last_row;
#pragma unroll
      for (int i = 0; i < G; ++i) {
        float sc = 0.0f;
#pragma unroll
        for (int c = 0; c < CH; ++c) sc = dot8<E>(kr[t][c], qv[i][c], sc);
        sc = lane_group_sum<L>(sc);
        x[t][i] = valid ? sc * scale_log2 : kNegInf;
      }
    }
    // The reference m is one value per head for the whole wavefront, and it
    // need not be the exact running maximum: weights exp2(x - m) up to
    // 2^kRescaleSlack are harmless in fp32, so the accumulator is rescaled
    // only when some row scores more than kRescaleSlack above the reference
    // (always on the wave's first live rows). Only then is the tile maximum
    // reduced across the lane groups.
    float mt[G];
    bool grow = false;
#pragma unroll
    for (int i = 0; i < G; ++i) {
      mt[i] = x[0][i];
#pragma unroll
      for (int t = 1; t < T; ++t) mt[i] = fmaxf(mt[i], x[t][i]);
      grow |= mt[i] > m[i] + kRescaleSlack;
    }
    if (__any(grow)) {
#pragma unroll
      for (int i = 0; i < G; ++i) {
        const float m_new = fmaxf(m[i], across_groups<L, Max>(mt[i]));
        const float alpha = fast_exp2(m[i] - finite_ref(m_new));
        l[i] *= alpha;
#pragma unroll
        for (int d = 0; d < DPL; ++d) acc[i][d] *= alpha;
        m[i] = m_new;
      }
    }
    float p[T][G];
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const float ref = finite_ref(m[i]);
#pragma unroll
      for (int t = 0; t < T; ++t) {
        p[t][i] = fast_exp2(x[t][i] - ref);
        l[i] += p[t][i];
      }
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
      float vf[DPL];
#pragma unroll
      for (int c = 0; c < CH; ++c) unpack8<E>(vr[t][c], vf + 8 * c);
#pragma unroll
      for (int i = 0; i < G; ++i) {
#pragma unroll
        for (int d = 0; d < DPL; ++d) acc[i][d] = fmaf(p[t][i], vf[d], acc[i][d]);
      }
    }
  };

  // Every load below is issued unconditionally (rows past the split clamp
  // to its last live row, so they stay in bounds; tiles past the end are
  // loaded but never processed). The number of loads between a tile's
  // issue and its use is then the same on every path, so the compiler waits
  // for that tile only (vmcnt of the P tiles issued after it) instead of
  // draining every load in flight at the top of each unrolled group.
#pragma unroll
  for (int pf = 0; pf < P; ++pf) load_tile(my_first + pf * kTile, kb[pf], vb[pf]);

  // With rotary tables (a decode step with rotary embedding) the G query
  // heads and the new key are rotated once per workgroup, one 16-byte chunk
  // per thread, after the first tiles are on their way; the first split
  // writes the rotated key into the cache, and the rotated key replaces the
  // loaded row in the tile that holds slot p_new.
  if constexpr (R) {
    __shared__ uint4 s_rot[G + 1][16];  // [query heads..., new key][chunk]
    if (tid < (G + 1) * 16) {
      const int h = tid / 16;
      const int c = tid % 16;
      const uint16_t* row = h < G ? q + r.out_row0 + static_cast<size_t>(h) * D : k_new + r.new_row;
      const uint4 v = rope_chunk<E>(row, cs + static_cast<size_t>(r.b) * D, sn + static_cast<size_t>(r.b) * D, 8 * c);
      s_rot[h][c] = v;
      if (h == G && r.split == 0 && p_new >= 0 && p_new < capacity)
        *reinterpret_cast<uint4*>(k_cache + r.head_off + static_cast<size_t>(p_new) * D + 8 * c) = v;
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < CH; ++c) {
#pragma unroll
      for (int i = 0; i < G; ++i) qv[i][c] = s_rot[i][sub + 8 * c];
      krot[c] = s_rot[G][sub + 8 * c];
    }
  }

  // Whole groups of NB tiles: tile t sits in ring slot t % NB.
  int t0 = 0;
  for (; t0 + NB <= ntiles; t0 += NB) {
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      load_tile(my_first + (t0 + u + P) * kTile, kb[(u + P) % NB], vb[(u + P) % NB]);
      process(my_first + (t0 + u) * kTile, kb[u], vb[u]);
    }
  }
  // The last ntiles - t0 < NB tiles (at most P, all loaded already).
#pragma unroll
  for (int u = 0; u < NB - 1; ++u) {
    if (t0 + u < ntiles) process(my_first + (t0 + u) * kTile, kb[u], vb[u]);
  }

  // Lanes equal modulo L hold the same dims of different rows, all relative
  // to the same reference m: the wave's state is their plain sum.
#pragma unroll
  for (int i = 0; i < G; ++i) l[i] = across_groups<L, Sum>(l[i]);
  constexpr int V = G * DPL;
  float red[V];
#pragma unroll
  for (int i = 0; i < G; ++i) {
#pragma unroll
    for (int d = 0; d < DPL; ++d) red[i * DPL + d] = acc[i][d];
  }
  sum_lane_groups<L, V>(red, lane);
  finish_split<E, G, L>(r, m, l, red, out, part_ml, part_acc, direct);
}

// Buffer resource over a workspace array: 32-bit byte offsets instead of
// 64-bit addresses keep one register per in-flight load. Word 3 is the gfx9
// raw-buffer format (32-bit data format); the host keeps every offset below
// 2^31.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t workspace_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), 0x7fffffff,
                                           0x00020000);
}

__device__ __forceinline__ float2 buffer_load_f2(__amdgpu_buffer_rsrc_t r, uint32_t byte_offset) {
  return __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(r, byte_offset, 0, 0));
}

// Combine kernel: one workgroup per (KV head, batch row), one wavefront per
// query head of the group, two dims per lane. It merges the num_splits
// partials of its head in split order with log-sum-exp weights,
//   M = max_s m_s,  out = sum_s exp2(m_s - M) acc_s / sum_s exp2(m_s - M) l_s,
// then rounds to the output type. Empty splits carry m = -inf and weigh 0
// (their accumulators are never used); a head whose splits are all empty
// (kv_len 0) gets zeros.
//
// Splits are taken in batches of kBatch whose loads are all issued before
// any is used, and batches are merged online (running max, rescaled sums),
// so a call waits for memory once per batch and needs no LDS or barrier.
template <class E>
__global__ __launch_bounds__(64 * kMaxGroup) void combine_kernel(
    uint16_t* __restrict__ out, const float2* __restrict__ part_ml,
    const float* __restrict__ part_acc, int n_kv_head, int group, int num_splits,
    const int32_t* __restrict__ kv_len, const int32_t* __restrict__ pos, int step, int max_kv_len,
    int balanced) {
  constexpr int D = kHeadDim;
  constexpr int kBatch = 32;  // the heuristic rarely asks for more: one memory wait
  const int g = blockIdx.x;
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int i = threadIdx.x >> 6;  // query head within the group
  const int n_head = n_kv_head * group;
  const uint32_t head_row = static_cast<uint32_t>(b) * n_head + static_cast<uint32_t>(g) * group + i;
  // Partial entry of split s: slot * n_head + g * group + i, where the slot
  // is s * batch + b (split-major), or first_slot(b) + s under the balanced
  // plan (the row's consecutive slots).
  uint32_t row0 = head_row;
  uint32_t split_stride = static_cast<uint32_t>(gridDim.y) * n_head;
  if (balanced) {
    const int slots = num_splits * static_cast<int>(gridDim.y);
    const BalancedRows rows = balanced_rows(kv_len, pos, step != 0, max_kv_len, gridDim.y, slots, lane);
    const int first = __builtin_amdgcn_readlane(rows.first, b);
    num_splits = __builtin_amdgcn_readlane(rows.count, b);
    row0 = static_cast<uint32_t>(first) * n_head + static_cast<uint32_t>(g) * group + i;
    split_stride = n_head;
  }
  const __amdgpu_buffer_rsrc_t ml_r = workspace_rsrc(part_ml);
  const __amdgpu_buffer_rsrc_t acc_r = workspace_rsrc(part_acc);

  float m_run = kNegInf, l_run = 0.0f;
  float2 o = make_float2(0.0f, 0.0f);
  for (int s0 = 0; s0 < num_splits; s0 += kBatch) {
    float2 ml[kBatch], a[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int s = s0 + k;
      if (s < num_splits) {
        const uint32_t row = row0 + static_cast<uint32_t>(s) * split_stride;
        ml[k] = buffer_load_f2(ml_r, row * 8u);
        a[k] = buffer_load_f2(acc_r, row * (D * 4u) + lane * 8u);
      } else {
        ml[k] = make_float2(kNegInf, 0.0f);
        a[k] = make_float2(0.0f, 0.0f);
      }
    }
    float mb = m_run;
#pragma unroll
    for (int k = 0; k < kBatch; ++k) mb = fmaxf(mb, ml[k].x);
    const float ref = finite_ref(mb);
    const float c = fast_exp2(m_run - ref);  // rescale what earlier batches summed
    l_run *= c;
    o.x *= c;
    o.y *= c;
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const float w = fast_exp2(ml[k].x - ref);
      if (w > 0.0f) {  // empty splits (w == 0) hold stale accumulators: skip, never multiply
        l_run = fmaf(w, ml[k].y, l_run);
        o.x = fmaf(w, a[k].x, o.x);
        o.y = fmaf(w, a[k].y, o.y);
      }
    }
    m_run = mb;
  }
  const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
  const uint32_t packed = static_cast<uint32_t>(E::round(o.x * inv)) |
                          (static_cast<uint32_t>(E::round(o.y * inv)) << 16);
  reinterpret_cast<uint32_t*>(out + static_cast<size_t>(head_row) * D)[lane] = packed;
}

// In-place append: row pos[b] of every KV head of batch row b, K and V, as
// 16 sixteen-byte chunks per 128-element row ([FORWARD-STEP] section 4).
__global__ __launch_bounds__(256) void kv_append_kernel(const uint4* __restrict__ k_new,
                                                        const uint4* __restrict__ v_new,
                                                        uint4* __restrict__ k_cache,
                                                        uint4* __restrict__ v_cache,
                                                        const int32_t* __restrict__ pos,
                                                        int n_kv_head, int capacity, int rows) {
  constexpr int kChunks = kHeadDim * 2 / 16;  // 16-byte chunks per row
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= rows * kChunks) return;
  const int row = idx / kChunks;  // b * n_kv_head + h
  const int c = idx % kChunks;
  const int b = row / n_kv_head;
  const int p = pos[b];
  if (p < 0 || p >= capacity) return;
  const size_t dst = (static_cast<size_t>(row) * capacity + p) * kChunks + c;
  k_cache[dst] = k_new[static_cast<size_t>(row) * kChunks + c];
  v_cache[dst] = v_new[static_cast<size_t>(row) * kChunks + c];
}

// Rotary embedding of the new token's query and key, and the append of the
// rotated key and the value at slot pos[b] ([FORWARD-STEP] section 4): 16
// lanes per 128-element row, one 16-byte chunk each. Rows [0, B*Hq) are query
// heads (q -> q_out, which may be q itself: a lane reads both chunks it needs
// before the wave writes), rows [B*Hq, B*Hq + B*Hkv) are KV heads. A slot
// outside [0, capacity) writes nothing to the cache.
template <class E>
__global__ __launch_bounds__(256) void rope_append_kernel(
    const uint16_t* q, uint16_t* q_out, const uint16_t* __restrict__ k_new,
    const uint16_t* __restrict__ v_new, const uint16_t* __restrict__ cs, const uint16_t* __restrict__ sn,
    uint16_t* __restrict__ k_cache, uint16_t* __restrict__ v_cache, const int32_t* __restrict__ pos,
    int n_head, int n_kv_head, int capacity, int q_rows, int rows) {
  constexpr int D = kHeadDim;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  const int row = idx / 16;
  const int d0 = 8 * (idx % 16);
  if (row >= rows) return;
  if (row < q_rows) {
    const int b = row / n_head;
    const size_t off = static_cast<size_t>(row) * D;
    const uint4 v = rope_chunk<E>(q + off, cs + static_cast<size_t>(b) * D, sn + static_cast<size_t>(b) * D, d0);
    *reinterpret_cast<uint4*>(q_out + off + d0) = v;
    return;
  }
  const int kr = row - q_rows;  // b * n_kv_head + h
  const int b = kr / n_kv_head;
  const int p = pos[b];
  if (p < 0 || p >= capacity) return;
  const size_t src = static_cast<size_t>(kr) * D;
  const size_t dst = (static_cast<size_t>(kr) * capacity + p) * D + d0;
  const uint4 k = rope_chunk<E>(k_new + src, cs + static_cast<size_t>(b) * D, sn + static_cast<size_t>(b) * D, d0);
  *reinterpret_cast<uint4*>(k_cache + dst) = k;
  *reinterpret_cast<uint4*>(v_cache + dst) = load16(v_new + src + d0);
}

// Per group size: lanes per row L, rows per lane group per tile T, tiles in
// flight P. Every choice gives 64-row workgroup tiles, the granularity the
// split heuristic rounds to.
template <int G> struct TileConfig;
// With the ring's loads unconditional, one tile in flight ahead of the one
// being computed is enough for grouped heads (their per-row work covers the
// latency; a deeper ring only costs registers), two for MHA (measured on
// MI355X: MiniCPM shape 27.7 -> 26.0 us at kv 8192, G = 8 44.4 -> 42.1 us,
// MHA kv 8192 15.7 -> 15.3 us).
template <> struct TileConfig<1> { static constexpr int L = 8, T = 2, P = 2; };
template <> struct TileConfig<2> { static constexpr int L = 8, T = 2, P = 1; };
template <> struct TileConfig<3> { static constexpr int L = 8, T = 2, P = 1; };
template <> struct TileConfig<4> { static constexpr int L = 8, T = 2, P = 1; };
template <> struct TileConfig<5> { static constexpr int L = 16, T = 4, P = 1; };
template <> struct TileConfig<6> { static constexpr int L = 16, T = 4, P = 1; };
template <> struct TileConfig<7> { static constexpr int L = 16, T = 4, P = 1; };
template <> struct TileConfig<8> { static constexpr int L = 16, T = 4, P = 1; };

template <class E, int G>
hipError_t launch_partial_g(const DecodeLaunch& p) {
  using C = TileConfig<G>;
  static_assert(kWaves * (64 / C::L) * C::T == kTileRows, "workgroup tile must be kTileRows rows");
  float2* part_ml = nullptr;
  float* part_acc = nullptr;
  if (!p.direct) {
    const WorkspaceLayout w = workspace_layout(p.batch, p.n_head, p.n_kv_head, kHeadDim, p.splits);
    char* base = static_cast<char*>(p.workspace);
    part_ml = reinterpret_cast<float2*>(base + w.ml_offset);
    part_acc = reinterpret_cast<float*>(base + w.acc_offset);
  }
  const dim3 grid(p.splits, p.n_kv_head, p.batch);
  const uint16_t* q = static_cast<const uint16_t*>(p.q);
  uint16_t* k_cache = static_cast<uint16_t*>(const_cast<void*>(p.k_cache));
  uint16_t* v_cache = static_cast<uint16_t*>(const_cast<void*>(p.v_cache));
  const uint16_t* k_new = static_cast<const uint16_t*>(p.k_new);
  const uint16_t* v_new = static_cast<const uint16_t*>(p.v_new);
  uint16_t* out = static_cast<uint16_t*>(p.out);
  const uint16_t* cs = static_cast<const uint16_t*>(p.cos);
  const uint16_t* sn = static_cast<const uint16_t*>(p.sin);
  if (cs != nullptr) {
    hipLaunchKernelGGL((partial_kernel<E, G, C::L, C::T, C::P, true>), grid, dim3(kThreads), 0, p.stream, q,
                       k_cache, v_cache, p.kv_len, k_new, v_new, p.pos, cs, sn, out, part_ml, part_acc,
                       p.n_kv_head, p.capacity, p.max_kv_len, p.chunk, p.direct ? 1 : 0, p.scale_log2);
  } else {
    hipLaunchKernelGGL((partial_kernel<E, G, C::L, C::T, C::P, false>), grid, dim3(kThreads), 0, p.stream, q,
                       k_cache, v_cache, p.kv_len, k_new, v_new, p.pos, cs, sn, out, part_ml, part_acc,
                       p.n_kv_head, p.capacity, p.max_kv_len, p.chunk, p.direct ? 1 : 0, p.scale_log2);
  }
  return hipGetLastError();
}

hipError_t launch_combine_impl(const CombineLaunch& p) {
  const WorkspaceLayout w = workspace_layout(p.batch, p.n_head, p.n_kv_head, kHeadDim, p.splits);
  const char* base = static_cast<const char*>(p.workspace);
  const int group = p.n_head / p.n_kv_head;
  const float2* ml = reinterpret_cast<const float2*>(base + w.ml_offset);
  const float* acc = reinterpret_cast<const float*>(base + w.acc_offset);
  uint16_t* out = static_cast<uint16_t*>(p.out);
  const dim3 grid(p.n_kv_head, p.batch), block(64 * group);
  if (p.dtype == 1) {
    hipLaunchKernelGGL(combine_kernel<BF16>, grid, block, 0, p.stream, out, ml, acc, p.n_kv_head, group, p.splits,
                       p.kv_len, p.pos, p.step ? 1 : 0, p.max_kv_len, p.balanced ? 1 : 0);
  } else {
    hipLaunchKernelGGL(combine_kernel<F16>, grid, block, 0, p.stream, out, ml, acc, p.n_kv_head, group, p.splits,
                       p.kv_len, p.pos, p.step ? 1 : 0, p.max_kv_len, p.balanced ? 1 : 0);
  }
  return hipGetLastError();
}

#define ADA_DISPATCH_GROUP(FN, P)                                   \
  switch ((P).n_head / (P).n_kv_head) {                             \
    case 1: return (P).dtype == 1 ? FN<BF16, 1>(P) : FN<F16, 1>(P); \
    case 2: return (P).dtype == 1 ? FN<BF16, 2>(P) : FN<F16, 2>(P); \
    case 3: return (P).dtype == 1 ? FN<BF16, 3>(P) : FN<F16, 3>(P); \
    case 4: return (P).dtype == 1 ? FN<BF16, 4>(P) : FN<F16, 4>(P); \
    case 5: return (P).dtype == 1 ? FN<BF16, 5>(P) : FN<F16, 5>(P); \
    case 6: return (P).dtype == 1 ? FN<BF16, 6>(P) : FN<F16, 6>(P); \
    case 7: return (P).dtype == 1 ? FN<BF16, 7>(P) : FN<F16, 7>(P); \
    case 8: return (P).dtype == 1 ? FN<BF16, 8>(P) : FN<F16, 8>(P); \
    default: return hipErrorInvalidValue;                           \
  }

}  // namespace

hipError_t launch_partial(const DecodeLaunch& p) { ADA_DISPATCH_GROUP(launch_partial_g, p) }

hipError_t launch_combine(const CombineLaunch& p) { return launch_combine_impl(p); }

hipError_t launch_rope_kv_append(const void* q, void* q_out, const void* k_new, const void* v_new,
                                 const void* cos, const void* sin, void* k_cache, void* v_cache,
                                 const int32_t* pos, int batch, int n_head, int n_kv_head, int capacity,
                                 int dtype, hipStream_t stream) {
  const int q_rows = q != nullptr ? batch * n_head : 0;
  const int rows = q_rows + batch * n_kv_head;
  const int blocks = (rows * 16 + 255) / 256;
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3(blocks), dim3(256), 0, stream, static_cast<const uint16_t*>(q),
                       static_cast<uint16_t*>(q_out), static_cast<const uint16_t*>(k_new),
                       static_cast<const uint16_t*>(v_new), static_cast<const uint16_t*>(cos),
                       static_cast<const uint16_t*>(sin), static_cast<uint16_t*>(k_cache),
                       static_cast<uint16_t*>(v_cache), pos, n_head, n_kv_head, capacity, q_rows, rows);
  };
  if (dtype == 1) {
    go(rope_append_kernel<BF16>);
  } else {
    go(rope_append_kernel<F16>);
  }
  return hipGetLastError();
}

hipError_t launch_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                            const int32_t* pos, int batch, int n_kv_head, int capacity,
                            hipStream_t stream) {
  const int rows = batch * n_kv_head;
  const int total = rows * (kHeadDim * 2 / 16);
  const int blocks = (total + 255) / 256;
  hipLaunchKernelGGL(kv_append_kernel, dim3(blocks), dim3(256), 0, stream,
                     static_cast<const uint4*>(k_new), static_cast<const uint4*>(v_new),
                     static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache), pos, n_kv_head,
                     capacity, rows);
  return hipGetLastError();
}

}  // namespace ada
