// Device helpers shared by the libkv4 HIP kernels (gfx950, wave64).
//
// Randomized Hadamard rotation of the INT4 per-token-head KV cache:
// K_s = H.D.k with H block-diagonal H_b (b = largest power-of-two divisor of
// head_size), D a seeded +-1 diagonal -- vLLM PR #62881 "[Bugfix][Test]
// Rotate KV into RHT domain in the INT4 unified attn test", Details / Root
// cause, and runguoli.com "vLLM -- Attention Kernels & KV Cache
// Quantization", section "PR #56198".
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kv4.h"

namespace kv4 {

// Debug builds (-DKV4_DEBUG): each kernel records the inputs it clamps or
// skips as KV4_DEBUG_* bits of a device word of its translation unit (a
// vector atomic OR; never a trap), read and cleared through
// kv4_debug_flags(). Release builds compile the checks away.
#ifdef KV4_DEBUG
namespace {
__device__ unsigned int g_debug_flags;
}
#define KV4_DBG(cond, bit)                                  \
  do {                                                      \
    if (cond) atomicOr(&::kv4::g_debug_flags, (unsigned)(bit)); \
  } while (0)
// host accessor of this translation unit's word (defined once per file)
#define KV4_DEBUG_ACCESSOR(fn)                                                  \
  uint32_t fn(bool clear) {                                                     \
    unsigned v = 0;                                                             \
    if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(::kv4::g_debug_flags), sizeof(v)) != hipSuccess) v = 0;       \
    if (clear) {                                                                \
      const unsigned z = 0;                                                     \
      (void)hipMemcpyToSymbol(HIP_SYMBOL(::kv4::g_debug_flags), &z, sizeof(z)); \
    }                                                                           \
    return v;                                                                   \
  }
#else
#define KV4_DBG(cond, bit) \
  do {                     \
  } while (0)
#define KV4_DEBUG_ACCESSOR(fn) \
  uint32_t fn(bool) { return 0; }
#endif

constexpr int kWave = 64;
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// D: sign i is -1 iff bit 63 of the (i+1)-th SplitMix64 output from state
// `seed` (SplitMix64: Steele, Lea & Flood 2014). Counter-based: output k is a
// pure function of seed + k * gamma.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t splitmix64_at(uint64_t seed, uint64_t k) {
  uint64_t z = seed + k * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// 8-bit mask of the signs of elements 8*chunk .. 8*chunk+7 (bit e set = -1).
__device__ __forceinline__ uint32_t sign_bits8(uint64_t seed, int chunk) {
  uint32_t m = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e)
    m |= (uint32_t)(splitmix64_at(seed, (uint64_t)(8 * chunk + e) + 1) >> 63) << e;
  return m;
}

// XOR masks that flip the sign bits of 8 packed bf16 (4 dwords, element 2k in
// the low half of dword k).
__device__ __forceinline__ void sign_xor_bf16x8(uint32_t bits, uint32_t (&x)[4]) {
#pragma unroll
  for (int k = 0; k < 4; ++k)
    x[k] = (((bits >> (2 * k)) & 1u) << 15) | (((bits >> (2 * k + 1)) & 1u) << 31);
}

// Sign flip of a float by bit e of `bits` (exact).
__device__ __forceinline__ float apply_sign(float v, uint32_t bits, int e) {
  return __uint_as_float(__float_as_uint(v) ^ (((bits >> e) & 1u) << 31));
}

// ---------------------------------------------------------------------------
// bf16 <-> float32
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Round a finite float32 to the nearest bf16, ties to even; returns the bf16
// value as float32.
__device__ __forceinline__ float round_bf16(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return __uint_as_float(u & 0xFFFF0000u);
}
__device__ __forceinline__ uint32_t bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return bf16_bits(lo) | (bf16_bits(hi) << 16);
}

// ---------------------------------------------------------------------------
// Cross-lane exchange with lane ^ D inside a wave (D < 32): DPP quad
// permutations for 1 and 2, ds_swizzle (bitmask mode, xor within 32 lanes)
// for 4, 8, 16. All lanes of the wave must be active.
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ float xor_lane(float v) {
  int x = __float_as_int(v);
  if constexpr (D == 1) {
    x = __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true);   // quad_perm [1,0,3,2]
  } else if constexpr (D == 2) {
    x = __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true);   // quad_perm [2,3,0,1]
  } else if constexpr (D == 32) {
    x = __builtin_amdgcn_ds_bpermute((int)((__lane_id() ^ 32u) << 2), x);
  } else {
    static_assert(D == 4 || D == 8 || D == 16, "xor distance");
    x = __builtin_amdgcn_ds_swizzle(x, (D << 10) | 0x1F);
  }
  return __int_as_float(x);
}

// Runtime-distance variant (d is wave-uniform, a power of two < 64).
__device__ __forceinline__ float xor_lane_rt(float v, int d) {
  switch (d) {
    case 1: return xor_lane<1>(v);
    case 2: return xor_lane<2>(v);
    case 4: return xor_lane<4>(v);
    case 8: return xor_lane<8>(v);
    case 16: return xor_lane<16>(v);
    default: return xor_lane<32>(v);
  }
}

// ---------------------------------------------------------------------------
// Radix-2 Walsh-Hadamard butterflies, float32, Sylvester order. Each lane
// holds 8 consecutive elements (chunk j = elements 8j..8j+7); strides 1, 2, 4
// are inside the lane, stride 8*d pairs lane j with lane j ^ d. Every output is
// one float32 add (lower index: x_i + x_{i+h}) or subtract (upper index:
// x_i - x_{i+h}), strides in ascending order.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void fwht8_inlane(float (&v)[8]) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if ((i & h) == 0) {
        const float a = v[i], c = v[i + h];
        v[i] = a + c;
        v[i + h] = a - c;
      }
    }
  }
}

// One cross-lane stage at lane distance d for all 8 elements.
__device__ __forceinline__ void fwht8_xlane(float (&v)[8], int d, bool upper) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float p = xor_lane_rt(v[e], d);
    v[e] = upper ? (p - v[e]) : (v[e] + p);
  }
}

// Full H_b on chunk-per-lane data: lanes j of one vector are consecutive lanes
// of the wave starting at a multiple of the (power-of-two) group size;
// `jj` = this lane's chunk index inside the vector; b >= 8.
__device__ __forceinline__ void fwht_b(float (&v)[8], int b, int jj) {
  fwht8_inlane(v);
  for (int d = 1; 8 * d < b; d <<= 1) fwht8_xlane(v, d, (jj & d) != 0);
}

// Compile-time variants for at most LPMAX lanes per vector (no runtime
// dispatch on the lane distance).
template <int D>
__device__ __forceinline__ void fwht8_xlane_ct(float (&v)[8], bool upper) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float p = xor_lane<D>(v[e]);
    v[e] = upper ? (p - v[e]) : (v[e] + p);
  }
}
template <int LPMAX>
__device__ __forceinline__ void fwht_b_ct(float (&v)[8], int b, int jj) {
  fwht8_inlane(v);
  if constexpr (LPMAX > 1) { if (b > 8) fwht8_xlane_ct<1>(v, (jj & 1) != 0); }
  if constexpr (LPMAX > 2) { if (b > 16) fwht8_xlane_ct<2>(v, (jj & 2) != 0); }
  if constexpr (LPMAX > 4) { if (b > 32) fwht8_xlane_ct<4>(v, (jj & 4) != 0); }
  if constexpr (LPMAX > 8) { if (b > 64) fwht8_xlane_ct<8>(v, (jj & 8) != 0); }
  if constexpr (LPMAX > 16) { if (b > 128) fwht8_xlane_ct<16>(v, (jj & 16) != 0); }
}
template <int W>
__device__ __forceinline__ float group_sum_ct(float v) {
  if constexpr (W > 1) v += xor_lane<1>(v);
  if constexpr (W > 2) v += xor_lane<2>(v);
  if constexpr (W > 4) v += xor_lane<4>(v);
  if constexpr (W > 8) v += xor_lane<8>(v);
  if constexpr (W > 16) v += xor_lane<16>(v);
  if constexpr (W > 32) v += xor_lane<32>(v);
  return v;
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int64_t uniform64(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// floor(num / den) for 0 <= num < 2^53, den > 0: a correctly rounded double
// quotient is within one of the floor, and one integer step fixes it (far
// cheaper than a 64-bit integer division).
__device__ __forceinline__ int64_t floor_div_small(int64_t num, int64_t den) {
  int64_t q = (int64_t)((double)num / (double)den);
  if (q * den > num) --q;
  else if ((q + 1) * den <= num) ++q;
  return q;
}

// Largest i in [0, n - 1] with arr[i] <= key (0 if there is none), for a
// non-decreasing arr and a wave-uniform key; every lane of the wave takes
// part. Each round probes 64 evenly spaced entries at once, so n entries
// take ceil(log64 n) dependent loads instead of log2 n. The result is
// wave-uniform and always in [0, n - 1], whatever arr holds.
__device__ __forceinline__ int wave_search_le(const int32_t* arr, int n, int64_t key) {
  const int lane = (int)__lane_id();
  int lo = 0, len = n;
  while (len > 1) {
    const int step = (len + kWave - 1) / kWave;
    const int idx = lo + lane * step;
    const bool le = idx < lo + len && (int64_t)arr[idx] <= key;
    int cnt = __builtin_popcountll(__builtin_amdgcn_ballot_w64(le));
    cnt = cnt < 1 ? 1 : cnt;
    const int end = lo + len;
    lo += (cnt - 1) * step;
    len = step < end - lo ? step : end - lo;
  }
  return uniform(lo);
}

// Reductions over lanes l, l ^ 16 and l ^ 32 with the gfx950 permlane swaps
// (full-rate VALU, no LDS round trip). With both operands equal, the swap
// returns the value of lane l ^ 16 (resp. l ^ 32) in one of its two results.
__device__ __forceinline__ float max_x16_x32(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t v = __float_as_uint(x);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_x16_x32(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const uint32_t v = __float_as_uint(x);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// max-reduce over the `width` lanes (power of two) of an aligned lane group.
__device__ __forceinline__ float group_max(float v, int width) {
  for (int d = 1; d < width; d <<= 1) v = fmaxf(v, xor_lane_rt(v, d));
  return v;
}
__device__ __forceinline__ float group_sum(float v, int width) {
  for (int d = 1; d < width; d <<= 1) v += xor_lane_rt(v, d);
  return v;
}

// 2^x on the transcendental unit (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ int next_pow2(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

}  // namespace kv4
