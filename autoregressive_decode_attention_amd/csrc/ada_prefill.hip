// ada_prefill.hip -- gfx950 kernels of libada for prompt prefill: the T
// prompt rows appended to the preallocated cache, and causal attention of the
// T prompt tokens over the cache.
//
// Pages cited (by title and section):
//   [ACTIVE-PREFIX] fish-speech issue #1310, "Optimize native AR decoding by
//                   attending only to the active KV-cache prefix" (section 2:
//                   kv_len = T after the prompt prefill).
//   [FORWARD-STEP]  VoxCPM issue #395, "MiniCPM4 MiniCPMAttention.forward_step
//                   Attention Performance Fix" (section 5: the batch prefill
//                   path runs attention with is_causal=True).
//
// Token t of batch row b sits at position start[b] + t and attends cache
// slots 0 .. start[b] + t (start = 0: the square causal mask of a prompt).
// Unlike the one-token decode, this is a dense contraction: G*T query rows
// share every key and value row of their KV head, so the scores and the
// weighted sum of values run on the matrix cores.
//
// Attention kernel, per workgroup: one (batch row, KV head) and 64 * RB
// query rows, where row r of the head group is token r / G and query head
// g*G + r % G (the G heads of a token share its causal limit). Four
// wavefronts own RB blocks of 16 rows each. Key/value tiles of 64 slots go
// through LDS:
//   * Staging: direct-to-LDS loads (global_load_lds_dwordx4) carry each K
//     and V tile from memory into one of two LDS buffers with no staging
//     registers and no LDS store instructions; the next tile's loads are in
//     flight while this tile is computed, and one barrier per tile both
//     publishes the next tile and frees the current buffer. Such a load
//     writes a wave's 64 x 16 bytes contiguously in lane order, so rows
//     cannot be padded: row R keeps its 16-byte chunk c in slot c ^ swz(R)
//     instead, which makes the K operand reads and the transposing V reads
//     below bank-conflict-free (each lane loads the chunk that belongs in
//     its slot, so every 16 lanes still read one whole 256-byte row).
//   * S^T = K Q^T with v_mfma_f32_16x16x32 (16-bit inputs, fp32 sums): keys
//     on M, query rows on N, head dims on K. A lane then holds, for one query
//     row, 16 scores (4 keys in each of the tile's four 16-key blocks).
//   * Online softmax in base 2 per row in fp32 against a lazy reference: the
//     output is rescaled only when a row's maximum passes its reference by
//     more than 2^8, so the weights exp2(|scale| s - m) <= 256 need one FMA
//     and one exp each. A negative scale is applied as |scale| to the
//     negated query (an exact sign flip), which keeps the largest raw score
//     the largest scaled one. The weights stay fp32 in effect: each becomes
//     a pair of 16-bit values hi = rnd(p), lo = rnd(p - hi), two per
//     conversion, and the row sums add both (a dot with ones), so numerator
//     and denominator see the same values. Keys past a row's causal limit
//     are masked only on the tiles that reach it.
//   * O += P V with the same instruction, once for the hi and once for the
//     lo weights: P is the A operand straight from registers, its K index
//     running over the lane's 8 keys of a 32-key step (a fixed permutation
//     of the keys, the same one the V operand uses).
//     V stays row-major and is read with the transposing LDS read
//     (ds_read_b64_tr_b16): within each 16-lane group, lane s addresses key
//     row r + s / 4 at dims 4 * (s % 4) .. + 3 of a 16-dim block, and lane d
//     receives keys r .. r + 3 of dim d of that block (the layout was
//     measured with a probe on MI355X). Two such reads give a lane its 8
//     keys.
//   * Row statistics move from the score layout (row = lane % 16) to the
//     output layout (rows 4 * (lane / 16) + j) with ds_bpermute.
//   * LDS traffic bounded an earlier, register-staged version (on MI355X,
//     removing its LDS operand reads and tile stores made it 44 % faster,
//     removing either matrix product or the softmax 7-12 %). With RB = 2
//     each K and V operand read serves two row blocks, halving the LDS bytes
//     per matrix instruction, and the LDS now runs at about 40 % of its
//     bandwidth; RB = 1 is for launches too small to fill the device with
//     128-row workgroups (prefill_rows_per_workgroup decides).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "ada_internal.h"

namespace ada {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef __bf16 bh2 __attribute__((ext_vector_type(2)));
typedef short s4 __attribute__((ext_vector_type(4)));

struct PF16 {
  static __device__ __forceinline__ f4 mma(const uint4& a, const uint4& b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, a), __builtin_bit_cast(h8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t round(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
  }
  // a and b rounded to nearest even, a in the low half.
  static __device__ __forceinline__ uint32_t pack(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2{a, b}), h2));
  }
  // The two packed values, exactly, as fp32.
  static __device__ __forceinline__ void unpack(uint32_t w, float& a, float& b) {
    const h2 h = __builtin_bit_cast(h2, w);
    a = static_cast<float>(h.x);
    b = static_cast<float>(h.y);
  }
  // c plus both packed values (a dot with (1, 1): exact products, fp32 sum).
  static __device__ __forceinline__ float sum2(uint32_t w, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, w), __builtin_bit_cast(h2, 0x3C003C00u), c, false);
  }
  // Base-2 exponent added to every softmax weight (and so to the row sums,
  // which cancels): weights up to 2^15 still fit fp16, and the low parts of
  // the weight pairs stay in fp16's normal range down to weights of 2^-3.
  static constexpr float kWeightExp = 7.0f;
};

struct PBF16 {
  static __device__ __forceinline__ f4 mma(const uint4& a, const uint4& b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8, a), __builtin_bit_cast(b8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t round(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
  }
  static __device__ __forceinline__ uint32_t pack(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2{a, b}), bh2));
  }
  static __device__ __forceinline__ void unpack(uint32_t w, float& a, float& b) {
    a = __uint_as_float(w << 16);
    b = __uint_as_float(w & 0xffff0000u);
  }
  static __device__ __forceinline__ float sum2(uint32_t w, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bh2, w), __builtin_bit_cast(bh2, 0x3F803F80u), c, false);
  }
  static constexpr float kWeightExp = 0.0f;  // bf16 has fp32's exponent range
};

constexpr int D = kHeadDim;     // 128
constexpr int kKeys = 64;        // key/value slots per tile
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ float finite_ref(float m) { return m == kNegInf ? 0.0f : m; }

__device__ __forceinline__ float xor16_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Value of x held by lane `src` of the wavefront.
__device__ __forceinline__ float from_lane(float x, int src) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(x)));
}

__device__ __forceinline__ uint4 ld16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

// Number of cache slots token t of a row starting at `start` attends to.
__device__ __forceinline__ int visible(int start, int t, int capacity) {
  const long n = static_cast<long>(start) + t + 1;
  return n < 0 ? 0 : (n > capacity ? capacity : static_cast<int>(n));
}

// Slot swizzle of the LDS tiles: row R keeps its 16-byte chunk c in slot
// c ^ tile_swz(R). The low three bits are a bijection of R mod 8 that sends
// each aligned group of four rows to values never differing in bit 0 alone,
// and bit 3 separates the values whose low bits differ only there. Then a
// 16-byte K operand read of one chunk by 8 or 16 consecutive rows, and a
// transposing V read (4 rows x 2 adjacent chunks per 16 lanes), touch each
// bank at most once whether the LDS serves them as 32 or 64 four-byte banks
// (checked exhaustively on the host).
__device__ __forceinline__ int tile_swz(int row) {
  const int x = row & 7;
  const int sig = ((2 * x) & 7) | (x >> 2);
  return sig + 8 * ((sig & 1) ^ ((row >> 3) & 1));
}

// Scores of one 64-key tile for RB blocks of 16 query rows, S^T = K Q^T:
// s[rb][nb] holds, for the lane's query row (lane % 16 of block rb), keys
// 16 * nb + 4 * (lane / 16) .. + 3 of the tile. Each K operand read from LDS
// serves all RB blocks.
template <class E, int RB>
__device__ __forceinline__ void tile_scores(const uint4* sk, const uint4 (&qb)[RB][4], int lr, int a, f4 (&s)[RB][4]) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) s[rb][nb] = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int row = 16 * nb + lr;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const uint4 kop = sk[row * 16 + ((4 * ks + a) ^ tile_swz(row))];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) s[rb][nb] = E::mma(kop, qb[rb][ks], s[rb][nb]);
    }
  }
}

// Online softmax of one tile's scores (keys base .. base + 63). FULL: every
// key is within every row's causal limit, so nothing is masked. Moves the
// running reference m_run (rescaling o and l_run) when a row's maximum
// passes it by more than 2^8 and adds the tile's weights to l_run.
//
// The weights reach the P V product on the matrix cores, whose A operand is
// 16-bit, as a pair: hi = rnd16(p) in ph and lo = rnd16(p - hi) in pl (p - hi
// is exact in fp32), and the product is taken with both. hi + lo holds p to
// a relative 2^-16 (bf16) or 2^-22 (fp16), so the weighted sum sees the fp32
// softmax weights, not weights rounded to 16 bits (whose 2^-9 relative error
// in bf16 moves an output by up to 2^-9 times the spread of the value rows
// it averages). The row sums add the same pairs.
template <class E, int RB, bool FULL>
__device__ __forceinline__ void tile_softmax(const f4 (&s)[RB][4], int base, const int (&my_n)[RB], int a,
                                             float cscale, float (&m_run)[RB], float (&l_run)[RB], f4 (&o)[RB][8],
                                             uint4 (&ph)[RB][2], uint4 (&pl)[RB][2]) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    bool ok[4][4];
    float mx = kNegInf;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ok[nb][j] = FULL || base + 16 * nb + 4 * a + j < my_n[rb];
        mx = fmaxf(mx, ok[nb][j] ? s[rb][nb][j] : kNegInf);
      }
    }
    mx = xor32_max(xor16_max(mx));
    const float m_tile = mx == kNegInf ? kNegInf : mx * cscale;
    const bool grow = m_tile > m_run[rb] + 8.0f;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float m_new = grow ? m_tile : m_run[rb];
      const float alpha = __builtin_amdgcn_exp2f(m_run[rb] - finite_ref(m_new));
      m_run[rb] = m_new;
      l_run[rb] *= alpha;
      float al[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) al[j] = from_lane(alpha, 4 * a + j);
#pragma unroll
      for (int db = 0; db < 8; ++db) {
#pragma unroll
        for (int j = 0; j < 4; ++j) o[rb][db][j] *= al[j];
      }
    }
    const float nref = E::kWeightExp - finite_ref(m_run[rb]);
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
      uint32_t wh[4], wl[4];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int nb = 2 * ks2 + h;
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          float p0 = __builtin_amdgcn_exp2f(fmaf(s[rb][nb][2 * jj], cscale, nref));
          float p1 = __builtin_amdgcn_exp2f(fmaf(s[rb][nb][2 * jj + 1], cscale, nref));
          if constexpr (!FULL) {
            p0 = ok[nb][2 * jj] ? p0 : 0.0f;
            p1 = ok[nb][2 * jj + 1] ? p1 : 0.0f;
          }
          const uint32_t hi = E::pack(p0, p1);
          float h0, h1;
          E::unpack(hi, h0, h1);
          const uint32_t lo = E::pack(p0 - h0, p1 - h1);
          wh[2 * h + jj] = hi;
          wl[2 * h + jj] = lo;
          l_run[rb] = E::sum2(lo, E::sum2(hi, l_run[rb]));
        }
      }
      ph[rb][ks2] = make_uint4(wh[0], wh[1], wh[2], wh[3]);
      pl[rb][ks2] = make_uint4(wl[0], wl[1], wl[2], wl[3]);
    }
  }
}

// O += P V over one tile for RB row blocks, P given as the pair hi + lo. V
// stays row-major in LDS and is read with the transposing LDS read; each V
// operand serves both halves of all RB blocks.
template <class E, int RB>
__device__ __forceinline__ void tile_pv(const uint4* sv, const uint4 (&ph)[RB][2], const uint4 (&pl)[RB][2], int lr,
                                        int a, f4 (&o)[RB][8]) {
  const uint16_t* sv16 = reinterpret_cast<const uint16_t*>(sv);
#pragma unroll
  for (int ks2 = 0; ks2 < 2; ++ks2) {
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      // rows R and R + 16 (R = 32*ks2 + 4*a + lr / 4), dims 16*db + 4*(lr % 4) .. + 3
      const int rA = 32 * ks2 + 4 * a + (lr >> 2);
      const int rB = rA + 16;
      const int col = 16 * db + 4 * (lr & 3);
      const uint16_t* pA = sv16 + rA * D + 8 * ((col >> 3) ^ tile_swz(rA)) + (col & 7);
      const uint16_t* pB = sv16 + rB * D + 8 * ((col >> 3) ^ tile_swz(rB)) + (col & 7);
      const s4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)(pA));
      const s4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)(pB));
      const uint2 w0 = __builtin_bit_cast(uint2, v0);
      const uint2 w1 = __builtin_bit_cast(uint2, v1);
      const uint4 vop = make_uint4(w0.x, w0.y, w1.x, w1.y);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) o[rb][db] = E::mma(pl[rb][ks2], vop, E::mma(ph[rb][ks2], vop, o[rb][db]));
    }
  }
}

// Normalised rows of o to the output ([B, H_q, T, D], rounded to nearest
// even); rows past the head group's last are skipped.
template <class E, int G, int RB>
__device__ __forceinline__ void store_rows(const f4 (&o)[RB][8], const float (&l_run)[RB], uint16_t* out, int wave_row0,
                                           int rows, int b, int g, int n_head, int q_len, int lr, int a) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float l_row = xor32_sum(xor16_sum(l_run[rb]));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float lj = from_lane(l_row, 4 * a + j);
      const int row = wave_row0 + 16 * rb + 4 * a + j;
      if (row >= rows) continue;
      const int t = row / G;
      const int i = row % G;
      uint16_t* orow = out + ((static_cast<size_t>(b) * n_head + g * G + i) * q_len + t) * D;
      const float inv = lj > 0.0f ? 1.0f / lj : 0.0f;
#pragma unroll
      for (int db = 0; db < 8; ++db) orow[16 * db + lr] = static_cast<uint16_t>(E::round(o[rb][db][j] * inv));
    }
  }
}

template <class E, int G, int RB>
__global__ __launch_bounds__(256, 2) void prefill_kernel(const uint16_t* __restrict__ q,
                                                          const uint16_t* __restrict__ k_cache,
                                                          const uint16_t* __restrict__ v_cache,
                                                          const int32_t* __restrict__ start_arr,
                                                          uint16_t* __restrict__ out, int n_kv_head, int q_len,
                                                          int capacity, int units, int row_tiles, float scale_log2) {
  constexpr int kRows = 64 * RB;
  constexpr int kTileU4 = kKeys * D / 8;  // 16-byte chunks per tile (1024)
  __shared__ __align__(16) uint4 s_k0[kTileU4];
  __shared__ __align__(16) uint4 s_v0[kTileU4];
  __shared__ __align__(16) uint4 s_k1[kTileU4];
  __shared__ __align__(16) uint4 s_v1[kTileU4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int a = lane >> 4;
  const int lr = lane & 15;
  const int unit = blockIdx.x % units;
  const int rt = row_tiles - 1 - blockIdx.x / units;
  const int b = unit / n_kv_head;
  const int g = unit % n_kv_head;
  const int n_head = n_kv_head * G;
  const int rows = G * q_len;
  const int start = start_arr != nullptr ? start_arr[b] : 0;
  const int r0 = rt * kRows;
  const int t_last = min(q_len - 1, (min(r0 + kRows, rows) - 1) / G);
  const int n_max = visible(start, t_last, capacity);
  const int ntiles = (n_max + kKeys - 1) / kKeys;

  const size_t head_off = static_cast<size_t>(unit) * capacity * D;
  const uint16_t* kbase = k_cache + head_off;
  const uint16_t* vbase = v_cache + head_off;

  const int wave_row0 = r0 + wave * 16 * RB;
  const float cscale = fabsf(scale_log2);
  const uint32_t sign = scale_log2 < 0.0f ? 0x80008000u : 0u;
  int my_n[RB];
  uint4 qb[RB][4];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int my_row = wave_row0 + 16 * rb + lr;
    const int my_t = my_row / G;
    const bool row_ok = my_row < rows;
    my_n[rb] = row_ok ? visible(start, my_t, capacity) : 0;
    const int i = my_row % G;
    const uint16_t* qrow = q + ((static_cast<size_t>(b) * n_head + g * G + i) * q_len + (row_ok ? my_t : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      uint4 v = row_ok ? ld16(qrow + 32 * ks + 8 * a) : make_uint4(0, 0, 0, 0);
      qb[rb][ks] = make_uint4(v.x ^ sign, v.y ^ sign, v.z ^ sign, v.w ^ sign);
    }
  }
  const int wave_n_min = wave_row0 < rows ? visible(start, wave_row0 / G, capacity) : 0;

  f4 o[RB][8];
  float m_run[RB], l_run[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
    for (int db = 0; db < 8; ++db) o[rb][db] = f4{0.0f, 0.0f, 0.0f, 0.0f};
    m_run[rb] = kNegInf;
    l_run[rb] = 0.0f;
  }

  // Wave w loads 1 KB blocks 4w .. 4w + 3 of each tile: block k holds rows
  // 4k .. 4k + 3, lane l the row 4k + l / 16 chunk (l % 16) ^ swz(row).
  // Buffer loads over the (batch row, KV head) slab take 32-bit byte offsets
  // (the host keeps capacity * 256 bytes below 2^31), so a row costs three
  // integer instructions instead of 64-bit address arithmetic; the LDS
  // destination is wave-uniform (scalar).
  const __amdgpu_buffer_rsrc_t k_rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kbase), static_cast<short>(0), 0x7fffffff, 0x00020000);
  const __amdgpu_buffer_rsrc_t v_rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vbase), static_cast<short>(0), 0x7fffffff, 0x00020000);
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  auto issue_tile = [&](int tile, uint4* sk, uint4* sv) {
    const int base = tile * kKeys;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int row = 16 * wave + 4 * it + lane / 16;
      const int chunk = (lane % 16) ^ tile_swz(row);
      const uint32_t off = (static_cast<uint32_t>(min(base + row, n_max - 1)) << 8) | (chunk << 4);
      const int blk = 4 * wave_s + it;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(k_rsrc, (__attribute__((address_space(3))) void*)(sk + 64 * blk), 16,
                                               off, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(v_rsrc, (__attribute__((address_space(3))) void*)(sv + 64 * blk), 16,
                                               off, 0, 0, 0);
    }
  };

  // full_tile: every key of the tile is visible to every row of the
  // wavefront (no causal mask on this tile).
  auto compute = [&](int tile, const uint4* sk, const uint4* sv, auto full_tile) __attribute__((always_inline)) {
    f4 s[RB][4];
    uint4 ph[RB][2], pl[RB][2];
    tile_scores<E, RB>(sk, qb, lr, a, s);
    tile_softmax<E, RB, decltype(full_tile)::value>(s, tile * kKeys, my_n, a, cscale, m_run, l_run, o, ph, pl);
    tile_pv<E, RB>(sv, ph, pl, lr, a, o);
  };

  // Tiles wholly below the wavefront's smallest causal limit take the
  // unmasked body. Every lane of a wavefront takes the same side, so the
  // other side is skipped. (With the wave index in a scalar register the
  // test would be a scalar branch, but the register allocator then spills
  // the two-block kernel.)
  auto compute_tile = [&](int tile, const uint4* sk, const uint4* sv) __attribute__((always_inline)) {
    if ((tile + 1) * kKeys <= wave_n_min) {
      compute(tile, sk, sv, std::true_type{});
    } else {
      compute(tile, sk, sv, std::false_type{});
    }
  };

  if (ntiles > 0) issue_tile(0, s_k0, s_v0);
  __syncthreads();  // tile 0 has landed (the barrier waits for the loads)
  for (int tile = 0; tile < ntiles; tile += 2) {
    if (tile + 1 < ntiles) issue_tile(tile + 1, s_k1, s_v1);
    compute_tile(tile, s_k0, s_v0);
    __syncthreads();  // tile + 1 has landed; every wave is done with buffer 0
    if (tile + 1 < ntiles) {
      if (tile + 2 < ntiles) issue_tile(tile + 2, s_k0, s_v0);
      compute_tile(tile + 1, s_k1, s_v1);
      __syncthreads();
    }
  }

  store_rows<E, G, RB>(o, l_run, out, wave_row0, rows, b, g, n_head, q_len, lr, a);
}

// Prompt append: row t of every (batch row, KV head) to slot start[b] + t,
// as 16-byte chunks; slots outside [0, capacity) are skipped.
__global__ __launch_bounds__(256) void prefill_append_kernel(const uint4* __restrict__ k_new,
                                                             const uint4* __restrict__ v_new,
                                                             uint4* __restrict__ k_cache, uint4* __restrict__ v_cache,
                                                             const int32_t* __restrict__ start_arr, int n_kv_head,
                                                             int q_len, int capacity, long total) {
  constexpr int kChunks = D * 2 / 16;
  const long idx = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int c = static_cast<int>(idx % kChunks);
  const long row = idx / kChunks;  // (b * n_kv_head + h) * q_len + t
  const int t = static_cast<int>(row % q_len);
  const long unit = row / q_len;
  const int b = static_cast<int>(unit / n_kv_head);
  const long p = static_cast<long>(start_arr != nullptr ? start_arr[b] : 0) + t;
  if (p < 0 || p >= capacity) return;
  const size_t dst = (static_cast<size_t>(unit) * capacity + static_cast<size_t>(p)) * kChunks + c;
  k_cache[dst] = k_new[static_cast<size_t>(row) * kChunks + c];
  v_cache[dst] = v_new[static_cast<size_t>(row) * kChunks + c];
}

template <class E, int G, int RB>
hipError_t launch_prefill_rb(const PrefillLaunch& p) {
  const int rows = G * p.q_len;
  const int row_tiles = (rows + 64 * RB - 1) / (64 * RB);
  const int units = p.batch * p.n_kv_head;
  hipLaunchKernelGGL((prefill_kernel<E, G, RB>), dim3(row_tiles * units), dim3(256), 0, p.stream,
                     static_cast<const uint16_t*>(p.q), static_cast<const uint16_t*>(p.k_cache),
                     static_cast<const uint16_t*>(p.v_cache), p.start, static_cast<uint16_t*>(p.out), p.n_kv_head,
                     p.q_len, p.capacity, units, row_tiles, p.scale_log2);
  return hipGetLastError();
}

template <class E, int G>
hipError_t launch_prefill_g(const PrefillLaunch& p) {
  return p.rows_per_workgroup == 128 ? launch_prefill_rb<E, G, 2>(p) : launch_prefill_rb<E, G, 1>(p);
}

template <class E>
hipError_t launch_prefill_e(const PrefillLaunch& p) {
  switch (p.n_head / p.n_kv_head) {
    case 1: return launch_prefill_g<E, 1>(p);
    case 2: return launch_prefill_g<E, 2>(p);
    case 3: return launch_prefill_g<E, 3>(p);
    case 4: return launch_prefill_g<E, 4>(p);
    case 5: return launch_prefill_g<E, 5>(p);
    case 6: return launch_prefill_g<E, 6>(p);
    case 7: return launch_prefill_g<E, 7>(p);
    case 8: return launch_prefill_g<E, 8>(p);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// Two 16-row blocks per wavefront halve the LDS traffic per matrix
// instruction (each K and V operand read serves both blocks) but halve the
// workgroup count, so they pay only when the launch still has at least two
// workgroups per compute unit (measured on MI355X: 16 % faster than one
// block at a 3072-token 32/8 prompt, even at 2048 tokens, slower at 1024,
// where one workgroup per unit would remain).
int prefill_rows_per_workgroup(int batch, int n_head, int n_kv_head, int q_len, int num_cus) {
  if (batch <= 0 || n_head <= 0 || n_kv_head <= 0 || q_len <= 0 || num_cus <= 0 || n_head % n_kv_head != 0)
    return 64;
  const long rows = static_cast<long>(n_head / n_kv_head) * q_len;
  const long workgroups = (rows + 127) / 128 * batch * n_kv_head;
  return workgroups >= 2L * num_cus ? 128 : 64;
}

hipError_t launch_prefill(const PrefillLaunch& p) {
  return p.dtype == 1 ? launch_prefill_e<PBF16>(p) : launch_prefill_e<PF16>(p);
}

hipError_t launch_prefill_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                                 const int32_t* start, int batch, int n_kv_head, int q_len, int capacity,
                                 hipStream_t stream) {
  const long total = static_cast<long>(batch) * n_kv_head * q_len * (D * 2 / 16);
  const long blocks = (total + 255) / 256;
  hipLaunchKernelGGL(prefill_append_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                     static_cast<const uint4*>(k_new), static_cast<const uint4*>(v_new), static_cast<uint4*>(k_cache),
                     static_cast<uint4*>(v_cache), start, n_kv_head, q_len, capacity, total);
  return hipGetLastError();
}

}  // namespace ada
