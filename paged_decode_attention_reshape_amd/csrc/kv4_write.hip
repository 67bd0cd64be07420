// Write path (reshape_and_cache_int4) and the dequant helper of libkv4.
//
// The write path stores K_s = H.D.k per (token, kv head) -- vLLM PR #62881
// "[Bugfix][Test] Rotate KV into RHT domain in the INT4 unified attn test",
// Details / Root cause -- with H block-diagonal H_b (runguoli.com "vLLM --
// Attention Kernels & KV Cache Quantization", section "PR #56198"), rounded
// through bf16 (PR #62881, Fix), one float32 scale per (token, kv head) and
// two int4 codes per uint8 byte (vLLM PR #40835 "[Feature] Triton INT4
// per-token-head KV cache quantization", review thread).
//
// Mapping on gfx950: one vector = one (token, kind, kv head) head vector of
// head_size bf16. Each lane owns 8 consecutive elements (one 16-byte load,
// one 4-byte store of packed codes); a vector spans LP = next_pow2(hs/8)
// consecutive lanes, a wave handles 64/LP vectors, ordered so that one wave's
// loads cover consecutive heads of one token row and its stores land in one
// contiguous cache row. Butterflies with stride < 8 stay in registers; larger
// strides exchange across lanes with DPP / ds_swizzle. Lanes past hs/8 carry
// zeros and never store.
#include <type_traits>

#include "kv4_device.hpp"
#include "kv4_launch.hpp"

namespace kv4 {

typedef __bf16 bf16x2_rt __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// The IEEE float32 quotient fl(y / scale) that the quantizers round, without a
// division per element: with r = fl(1 / scale) (one correctly rounded
// division per vector), q0 = fl(y r), e = y - q0 scale in one fma, and q =
// fl(q0 + e r) in another (Markstein's correction). For scale in [2^-100,
// 2^100] and every pair (amax, y) the write path can meet -- amax and y bf16
// values with |y| <= amax, scale = fl(amax / qmax) -- the codes taken from q
// equal those taken from the IEEE quotient: checked exhaustively on the host
// for qmax 7 (rint), 127 (rint) and 448 (e4m3fn, the sign taken from y), where
// the quotient differs only for subnormal y, whose codes are 0 either way.
// Scales outside that range take the quotient from the division itself.
constexpr float kMarksteinLo = 0x1p-100f, kMarksteinHi = 0x1p100f;

__device__ __forceinline__ float quotient(float y, float scale, float r) {
  const float q0 = y * r;
  const float e = fmaf(-q0, scale, y);
  return fmaf(e, r, q0);
}

// rint_half_even(fl(y / scale)) for all 8 values of a lane (int8 rule).
__device__ __forceinline__ void rint_quotients(const float (&y)[8], float scale, float (&q)[8]) {
  if (scale >= kMarksteinLo && scale <= kMarksteinHi) {
    const float r = 1.0f / scale;
#pragma unroll
    for (int e = 0; e < 8; ++e) q[e] = __builtin_rintf(quotient(y[e], scale, r));
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) q[e] = __builtin_rintf(y[e] / scale);
  }
}

// Packed int4 codes (element e in bits 4e..4e+3) of the quotients sg * v[e] /
// scale, scale > 0, sg = +1 or -1 (the quotient of sg * v is sg times that of
// v exactly: every step rounds symmetrically). The sum q + 1.5 * 2^23 is
// 1.5 * 2^23 + rint_half_even(q) exactly (|q| < 2^22, unit spacing there), so
// for |q| <= 8 the low nibble of its bit pattern is the two's-complement code;
// |q| <= 7 up to rounding for scale = fl(amax / 7), so the clamp to [-8, 7]
// cannot act. Scales outside the Markstein range (subnormal ones can give
// |y / scale| > 7.5) take the division and the clamp.
__device__ __forceinline__ uint32_t int4_codes(const float (&v)[8], float scale, float sg) {
  constexpr float kRound = 12582912.0f;   // 1.5 * 2^23
  if (scale >= kMarksteinLo && scale <= kMarksteinHi) {
    const float r = 1.0f / scale;
    uint32_t u[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) u[e] = __float_as_uint(fmaf(quotient(v[e], scale, r), sg, kRound));
    // byte 0 of the even elements' patterns into one word and of the odd
    // ones into another (v_perm_b32: selector 0-3 picks a byte of the second
    // operand, 4-7 of the first, 12 a zero byte), then each byte's low
    // nibble from the even word and high nibble from the odd one
    const uint32_t ev = __builtin_amdgcn_perm(u[2], u[0], 0x0C0C0400u) | __builtin_amdgcn_perm(u[6], u[4], 0x04000C0Cu);
    const uint32_t od = __builtin_amdgcn_perm(u[3], u[1], 0x0C0C0400u) | __builtin_amdgcn_perm(u[7], u[5], 0x04000C0Cu);
    return (ev & 0x0F0F0F0Fu) | ((od << 4) & 0xF0F0F0F0u);
  }
  uint32_t packed = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float q = fminf(fmaxf(__builtin_rintf(v[e] / scale) * sg, -8.0f), 7.0f);
    packed |= ((uint32_t)(int)q & 0xFu) << (4 * e);
  }
  return packed;
}

// The radix-2 Walsh-Hadamard butterflies of the write path with the sign of
// each cross-lane stage carried instead of applied: at the stage pairing
// lane j with lane j ^ d, both lanes have taken the same upper / lower roles
// in every earlier cross-lane stage, so they hold their values with the same
// carried sign s; the lower lane computes own + partner (= s * (x_i +
// x_{i+h})) and the upper lane own - partner (= -s * (x_i - x_{i+h}), the
// exact negation of partner - own), one v_fmac with the partner as its DPP /
// swizzle source. Returns the lane's final carried sign (+1 / -1): the true
// values are sign * v, each element rounded exactly as in fwht_b_ct.
//
// Distances 1, 2 and 8 stay inside a DPP row of 16 lanes (quad_perm
// [1,0,3,2], quad_perm [2,3,0,1], row_ror:8), so the exchange is the fmac's
// own DPP source: eight v_fmac_f32_dpp in one block, after two wait states
// for the DPP read of a register a vector instruction just wrote (the
// compiler does not look inside the block). Each reads its partner's value
// of a register before any instruction of the block writes that register.
// Distances 4 and 16 go through ds_swizzle (the LDS pipe, off the vector ALU
// that bounds the kernel).
#define KV4_DPP_FMAC8(CTRL)                                                                            \
  asm volatile("s_nop 1\n\t"                                                                          \
               "v_fmac_f32_dpp %0, %0, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"       \
               "v_fmac_f32_dpp %1, %1, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"       \
               "v_fmac_f32_dpp %2, %2, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"       \
               "v_fmac_f32_dpp %3, %3, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"       \
               "v_fmac_f32_dpp %4, %4, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"       \
               "v_fmac_f32_dpp %5, %5, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"       \
               "v_fmac_f32_dpp %6, %6, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"       \
               "v_fmac_f32_dpp %7, %7, %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1"             \
               : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]),   \
                 "+v"(v[7])                                                                            \
               : "v"(sgn))
template <int D>
__device__ __forceinline__ void fwht8_xlane_lazy(float (&v)[8], float sgn) {
  if constexpr (D == 1) {
    KV4_DPP_FMAC8("quad_perm:[1,0,3,2]");
  } else if constexpr (D == 2) {
    KV4_DPP_FMAC8("quad_perm:[2,3,0,1]");
  } else if constexpr (D == 8) {
    KV4_DPP_FMAC8("row_ror:8");
  } else {
    float p[8];   // all 8 exchanges in flight before the first use
#pragma unroll
    for (int e = 0; e < 8; ++e) p[e] = xor_lane<D>(v[e]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = fmaf(p[e], sgn, v[e]);
  }
}
#undef KV4_DPP_FMAC8
// XS cross-lane stages (b = 8 * 2^XS), in ascending stride order after the
// in-lane ones; XS is fixed per kernel, so the stages carry no branch.
template <int XS>
__device__ __forceinline__ float fwht_b_lazy(float (&v)[8], int jj) {
  fwht8_inlane(v);
  float sg = 1.0f;
  auto stage = [&](auto dc) {
    constexpr int D = decltype(dc)::value;
    const float s = (jj & D) ? -1.0f : 1.0f;
    fwht8_xlane_lazy<D>(v, s);
    sg *= s;
  };
  if constexpr (XS > 0) stage(std::integral_constant<int, 1>());
  if constexpr (XS > 1) stage(std::integral_constant<int, 2>());
  if constexpr (XS > 2) stage(std::integral_constant<int, 4>());
  if constexpr (XS > 3) stage(std::integral_constant<int, 8>());
  if constexpr (XS > 4) stage(std::integral_constant<int, 16>());
  return sg;
}

// max over the LP lanes of an aligned lane group of non-negative finite
// floats, compared as their bit patterns (same order; no NaN quieting)
template <int LP>
__device__ __forceinline__ float group_max_nonneg(float v) {
  uint32_t u = __float_as_uint(v);
  if constexpr (LP > 1) u = max(u, __float_as_uint(xor_lane<1>(__uint_as_float(u))));
  if constexpr (LP > 2) u = max(u, __float_as_uint(xor_lane<2>(__uint_as_float(u))));
  if constexpr (LP > 4) u = max(u, __float_as_uint(xor_lane<4>(__uint_as_float(u))));
  if constexpr (LP > 8) u = max(u, __float_as_uint(xor_lane<8>(__uint_as_float(u))));
  if constexpr (LP > 16) u = max(u, __float_as_uint(xor_lane<16>(__uint_as_float(u))));
  return __uint_as_float(u);
}

// Per-token-head control modes (no rotation; the pages' int8_per_token_head
// and fp8_per_token_head, vLLM PR #40835 review thread): one code byte per
// element, scale = absmax / qmax.
//   int8: rint_half_even(x / scale) clamped to [-128, 127];
//   fp8:  x / scale rounded to the nearest OCP FP8 E4M3 (e4m3fn) value, ties to
//         the even mantissa, magnitudes >= 448 saturating to 448; the sign bit
//         follows the quotient's.
__device__ __forceinline__ uint32_t f32_to_e4m3(float q) {
  const uint32_t u = __float_as_uint(q);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  uint32_t code;
  if (a >= 0x43E00000u) {                 // >= 448
    code = 0x7Eu;
  } else if (a < 0x3C800000u) {           // < 2^-6: subnormal steps of 2^-9 (8 -> the first normal)
    code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  } else {                                // keep 3 mantissa bits, round half to even
    uint32_t bits = a >> 20;
    const uint32_t rem = a & 0xFFFFFu;
    bits += (rem > 0x80000u || (rem == 0x80000u && (bits & 1u))) ? 1u : 0u;
    code = bits - (120u << 3);            // float32 exponent bias 127 -> e4m3 bias 7
    code = code > 0x7Eu ? 0x7Eu : code;
  }
  return code | sign;
}

// int8 code byte of an already rounded quotient q.
__device__ __forceinline__ uint32_t int8_byte(float q) {
  q = fminf(fmaxf(q, -128.0f), 127.0f);
  return (uint32_t)(int)q & 0xFFu;
}

// Page of a slot (block size a power of two: a shift).
template <typename Args>
__device__ __forceinline__ int64_t slot_page(const Args& a, int64_t slot) {
  return a.bs_shift >= 0 ? (slot >> a.bs_shift) : slot / a.bs;
}

// scale = RN(amax / QMAX) without the division sequence: q0 = RN(amax * c),
// c = RN(1 / QMAX); r = amax - q0 * QMAX is exact in one fma; RN(q0 + r * c)
// is the correctly rounded quotient. Checked exhaustively on the host against
// IEEE float32 division: for QMAX 7 and 127 on every non-negative finite
// float32, for 448 on every non-negative finite bf16 value (amax is always one:
// the inputs are bf16 and the rotated values are rounded to bf16 first).
template <int QMAX>
__device__ __forceinline__ float div_by_qmax(float amax) {
  constexpr float c = 1.0f / (float)QMAX;
  const float q0 = amax * c;
  const float r = fmaf(-q0, (float)QMAX, amax);
  return fmaf(r, c, q0);
}

// At most 96 scalar registers: eight waves per SIMD (101 left it at seven).
//
// A wave takes one token per iteration: its K head vectors, then its V head
// vectors, in slices of VPW = 64 / LP heads of one kind (ceil(nkv / VPW)
// slices per kind), U slices loaded before any of them is computed. The
// token, its slot, page and row bases are wave-uniform (scalar registers and
// scalar ALU); a lane adds a 32-bit offset fixed before the loop (its head
// within the slice and its 8-element chunk). The input rows are read whatever
// the slot (a skipped token's row is still a valid row), so no load waits for
// the slot; lanes past the heads or chunks read a clamped address of the same
// row and drop the value, so the loads carry no branch and stay in flight
// together.
template <int LP, int QM, int U, int XS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_num_sgpr(96))) void write_kernel(WriteArgs a) {
  constexpr int VPW = kWave / LP;                      // heads per slice
  constexpr int CB = QM == 0 ? 4 : 8;                  // code bytes per lane (8 elements)
  const int lane = threadIdx.x & (kWave - 1);
  const int jj = lane & (LP - 1);                      // chunk index in the vector
  const int grp = lane / LP;
  const int nchunk = a.hs >> 3;
  const bool lane_on = jj < nchunk;

  uint32_t sx[4] = {0u, 0u, 0u, 0u};
  if constexpr (QM == 0) sign_xor_bf16x8(lane_on ? sign_bits8(a.seed, jj) : 0u, sx);

  const int nkv = a.nkv;
  const int spk = (nkv + VPW - 1) / VPW;               // slices per kind
  const int spt = 2 * spk;                             // slices per token
  // lane offset within a slice's input (bytes from the slice's first head),
  // clamped into the row; and within a slice's cache row
  const uint32_t in_off = (uint32_t)(grp * a.hs * 2 + 16 * min(jj, nchunk - 1));
  const int64_t c_off = (int64_t)grp * a.lay.head + CB * jj;
  const uint32_t in_last = (uint32_t)((nkv - 1) * a.hs * 2 + 16 * min(jj, nchunk - 1));   // last head's chunk
  const int64_t wave_id = (int64_t)blockIdx.x * (blockDim.x / kWave) + uniform((int)(threadIdx.x / kWave));
  const int64_t n_waves = (int64_t)gridDim.x * (blockDim.x / kWave);

  for (int64_t t = wave_id; t < a.num_tokens; t += n_waves) {
    const char* krow = reinterpret_cast<const char*>(a.key + t * a.key_stride);
    const char* vrow = reinterpret_cast<const char*>(a.value + t * a.value_stride);
    int64_t crow = 0, srow = 0;                // code row (bytes) and scale row (floats) of the slot
    bool ok = false;
    for (int u0 = 0; u0 < spt; u0 += U) {
      // the input rows first: they do not depend on the slot
      u32x4_t w[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int su = min(u0 + u, spt - 1);               // slice (wave-uniform)
        const int kind = su >= spk ? 1 : 0;
        const int h0 = (su - kind * spk) * VPW;            // its first head
        const uint32_t off = min((uint32_t)(h0 * a.hs * 2) + in_off, in_last);
        w[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>((kind ? vrow : krow) + off));
      }
      if (u0 == 0) {                           // then the slot, while they are in flight
        const int64_t slot = uniform64(a.slot_mapping[t]);
        ok = slot >= 0 && slot < a.num_slots;
        KV4_DBG(slot >= a.num_slots, KV4_DEBUG_SLOT);
        const int64_t pg = ok ? slot_page(a, slot) : 0;
        const int64_t tk = ok ? slot - pg * a.bs : 0;
        crow = pg * a.lay.blk + tk * a.lay.tok;
        srow = pg * a.lay.sblk + tk * a.lay.stok;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int su = u0 + u;
        const int kind = su >= spk ? 1 : 0;
        const int h0 = (su - kind * spk) * VPW;
        const int h = h0 + grp;
        const bool st = ok && su < spt && h < nkv && lane_on;
        // lanes past the head's chunks take part in the vector's absmax: zero
        // them (other lanes' values stay inside their own vector and are not
        // stored)
        const u32x4_t wz = (nchunk == LP || lane_on) ? w[u] : u32x4_t{0u, 0u, 0u, 0u};
        const uint32_t wd[4] = {wz.x ^ sx[0], wz.y ^ sx[1], wz.z ^ sx[2], wz.w ^ sx[3]};
        float v[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          v[2 * k] = bf16_lo(wd[k]);
          v[2 * k + 1] = bf16_hi(wd[k]);
        }
        // rotation (carried sign sg: the rotated values are sg * v) and one
        // round-to-nearest-even to bf16 (v_cvt_pk_bf16_f32); rounding, absmax
        // and the int4 rule are symmetric in the sign, so sg is applied to the
        // codes only
        float sg = 1.0f;
        if constexpr (QM == 0) {
          sg = fwht_b_lazy<XS>(v, jj);
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const uint32_t w2 = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{v[2 * k], v[2 * k + 1]},
                                                                                      bf16x2_rt));
            v[2 * k] = bf16_lo(w2);
            v[2 * k + 1] = bf16_hi(w2);
          }
        }
        float amax = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
        amax = group_max_nonneg<LP>(amax);
        // the slice's first head in the cache row, uniform; the lane's head and chunk on top
        uint8_t* cache = (kind ? a.value_cache : a.key_cache) + crow + (int64_t)h0 * a.lay.head;
        float* scl = (kind ? a.v_scale : a.k_scale) + srow + (int64_t)h0 * a.lay.shead;
        if constexpr (QM == 0) {
          const float scale = div_by_qmax<7>(amax);
          const uint32_t packed = scale > 0.0f ? int4_codes(v, scale, sg) : 0u;
          if (st) {
            *reinterpret_cast<uint32_t*>(cache + c_off) = packed;
            if (jj == 0) scl[grp * a.lay.shead] = scale;
          }
        } else {
          const float scale = div_by_qmax<QM == 1 ? 127 : 448>(amax);
          uint32_t lo = 0, hi = 0;
          if (scale > 0.0f) {
            if constexpr (QM == 1) {
              float q[8];
              rint_quotients(v, scale, q);
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                lo |= int8_byte(q[e]) << (8 * e);
                hi |= int8_byte(q[e + 4]) << (8 * e);
              }
            } else {
              // the quotient of |v| with v's sign bit: -0 keeps its sign
              float q[8];
              if (scale >= kMarksteinLo && scale <= kMarksteinHi) {
                const float r = 1.0f / scale;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                  q[e] = __uint_as_float(__float_as_uint(quotient(fabsf(v[e]), scale, r)) |
                                         (__float_as_uint(v[e]) & 0x80000000u));
              } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) q[e] = v[e] / scale;
              }
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                lo |= f32_to_e4m3(q[e]) << (8 * e);
                hi |= f32_to_e4m3(q[e + 4]) << (8 * e);
              }
            }
          }
          if (st) {
            *reinterpret_cast<uint2*>(cache + c_off) = make_uint2(lo, hi);
            if (jj == 0) scl[grp * a.lay.shead] = scale;
          }
        }
      }
    }
  }
}

template <int LP, int QM>
__global__ __launch_bounds__(256) void dequant_kernel(DequantArgs a) {
  constexpr int VPW = kWave / LP;
  const int lane = threadIdx.x & (kWave - 1);
  const int jj = lane & (LP - 1);
  const int grp = lane / LP;
  const int nchunk = a.hs >> 3;
  const bool lane_on = jj < nchunk;
  const uint32_t sbits = lane_on ? sign_bits8(a.seed, jj) : 0u;
  const float inv_b = 1.0f / (float)a.b;   // exact: b is a power of two
  const int64_t n_items = a.num_tokens * a.nkv;
  const int64_t wave_id = (int64_t)blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
  const int64_t n_waves = (int64_t)gridDim.x * (blockDim.x / kWave);

  for (int64_t base = wave_id * VPW; base < n_items; base += n_waves * VPW) {
    const int64_t item = base + grp;
    const bool in = item < n_items;
    int64_t t = 0, slot = -1;
    int h = 0;
    if (in) {
      t = item / a.nkv;
      h = (int)(item - t * a.nkv);
      slot = a.slot_mapping[t];
    }
    const bool ok = in && slot >= 0 && slot < a.num_slots;
    KV4_DBG(in && slot >= a.num_slots, KV4_DEBUG_SLOT);
    uint32_t codes = 0;
    uint2 bytes = make_uint2(0u, 0u);
    float sc = 0.0f;
    if (ok && lane_on) {
      const int64_t pg = slot_page(a, slot), tk = slot - pg * a.bs;
      const uint8_t* src = a.cache + a.lay.code_off(pg, tk, h);
      if constexpr (QM == 0) codes = *reinterpret_cast<const uint32_t*>(src + 4 * jj);
      else bytes = *reinterpret_cast<const uint2*>(src + 8 * jj);
      sc = a.scale[a.lay.scale_off(pg, tk, h)];
    }
    float v[8];
    if constexpr (QM == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = ((int)(codes << (28 - 4 * e))) >> 28;   // sign-extend nibble e
        v[e] = (float)c * sc;
      }
    } else if constexpr (QM == 1) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] = (float)(int)(int8_t)(bytes.x >> (8 * e)) * sc;
        v[e + 4] = (float)(int)(int8_t)(bytes.y >> (8 * e)) * sc;
      }
    } else {
      // v_cvt_pk_f32_fp8: two e4m3fn bytes (word half lo / hi) -> exact floats
      const f32x2_t p0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)bytes.x, false);
      const f32x2_t p1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)bytes.x, true);
      const f32x2_t p2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)bytes.y, false);
      const f32x2_t p3 = __builtin_amdgcn_cvt_pk_f32_fp8((int)bytes.y, true);
      v[0] = p0.x * sc; v[1] = p0.y * sc; v[2] = p1.x * sc; v[3] = p1.y * sc;
      v[4] = p2.x * sc; v[5] = p2.y * sc; v[6] = p3.x * sc; v[7] = p3.y * sc;
    }
    if (QM == 0 && a.inverse_rotate) {
      fwht_b(v, a.b, jj);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = apply_sign(v[e] * inv_b, sbits, e);
    }
    if (in && lane_on) {
      float4* dst = reinterpret_cast<float4*>(a.out + item * a.hs + 8 * jj);
      dst[0] = make_float4(v[0], v[1], v[2], v[3]);
      dst[1] = make_float4(v[4], v[5], v[6], v[7]);
    }
  }
}

static int lanes_per_vector(int hs) { return host_next_pow2(hs / 8); }

template <int QM, int LP, int U>
static void launch_write_xs(const WriteArgs& a, dim3 grid, dim3 block, hipStream_t stream) {
  // cross-lane butterfly stages: log2(b / 8) for int4, none for int8 / fp8
  int xs = 0;
  if (QM == 0)
    while ((8 << xs) < a.b) ++xs;
  switch (xs) {
    case 0: hipLaunchKernelGGL((write_kernel<LP, QM, U, 0>), grid, block, 0, stream, a); break;
    case 1: if constexpr (QM == 0 && LP >= 2) hipLaunchKernelGGL((write_kernel<LP, QM, U, 1>), grid, block, 0, stream, a); break;
    case 2: if constexpr (QM == 0 && LP >= 4) hipLaunchKernelGGL((write_kernel<LP, QM, U, 2>), grid, block, 0, stream, a); break;
    case 3: if constexpr (QM == 0 && LP >= 8) hipLaunchKernelGGL((write_kernel<LP, QM, U, 3>), grid, block, 0, stream, a); break;
    case 4: if constexpr (QM == 0 && LP >= 16) hipLaunchKernelGGL((write_kernel<LP, QM, U, 4>), grid, block, 0, stream, a); break;
    default: if constexpr (QM == 0 && LP >= 32) hipLaunchKernelGGL((write_kernel<LP, QM, U, 5>), grid, block, 0, stream, a); break;
  }
}

template <int QM, int U>
static void launch_write_qu(const WriteArgs& a, int LP, dim3 grid, dim3 block, hipStream_t stream) {
  switch (LP) {
    case 1: launch_write_xs<QM, 1, U>(a, grid, block, stream); break;
    case 2: launch_write_xs<QM, 2, U>(a, grid, block, stream); break;
    case 4: launch_write_xs<QM, 4, U>(a, grid, block, stream); break;
    case 8: launch_write_xs<QM, 8, U>(a, grid, block, stream); break;
    case 16: launch_write_xs<QM, 16, U>(a, grid, block, stream); break;
    default: launch_write_xs<QM, 32, U>(a, grid, block, stream); break;
  }
}

template <int QM>
static void launch_write_qm(const WriteArgs& a, int LP, dim3 grid, dim3 block, hipStream_t stream) {
  if (a.slices == 2) launch_write_qu<QM, 2>(a, LP, grid, block, stream);
  else launch_write_qu<QM, 4>(a, LP, grid, block, stream);
}

hipError_t launch_write(const WriteArgs& a0, hipStream_t stream) {
  const int LP = lanes_per_vector(a0.hs);
  WriteArgs a = a0;
  // U: slices in flight, 4, or 2 where a token has only 2 (one slice of K
  // heads, one of V heads)
  const int64_t spt = 2 * (((int64_t)a.nkv + (kWave / LP) - 1) / (kWave / LP));
  a.slices = spt <= 2 ? 2 : 4;
  const int64_t blocks = std::min<int64_t>((a.num_tokens + 3) / 4, 256 * 64);
  dim3 grid((unsigned)std::max<int64_t>(blocks, 1)), block(256);
  switch (a.qm) {
    case 0: launch_write_qm<0>(a, LP, grid, block, stream); break;
    case 1: launch_write_qm<1>(a, LP, grid, block, stream); break;
    case 2: launch_write_qm<2>(a, LP, grid, block, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int QM>
static void launch_dequant_qm(const DequantArgs& a, int LP, dim3 grid, dim3 block, hipStream_t stream) {
  switch (LP) {
    case 1: hipLaunchKernelGGL((dequant_kernel<1, QM>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((dequant_kernel<2, QM>), grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL((dequant_kernel<4, QM>), grid, block, 0, stream, a); break;
    case 8: hipLaunchKernelGGL((dequant_kernel<8, QM>), grid, block, 0, stream, a); break;
    case 16: hipLaunchKernelGGL((dequant_kernel<16, QM>), grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL((dequant_kernel<32, QM>), grid, block, 0, stream, a); break;
  }
}

hipError_t launch_dequant(const DequantArgs& a, hipStream_t stream) {
  const int LP = lanes_per_vector(a.hs);
  const int64_t items = a.num_tokens * a.nkv;
  const int64_t waves = (items + (kWave / LP) - 1) / (kWave / LP);
  const int64_t blocks = std::min<int64_t>((waves + 3) / 4, 256 * 64);
  dim3 grid((unsigned)std::max<int64_t>(blocks, 1)), block(256);
  switch (a.qm) {
    case 0: launch_dequant_qm<0>(a, LP, grid, block, stream); break;
    case 1: launch_dequant_qm<1>(a, LP, grid, block, stream); break;
    case 2: launch_dequant_qm<2>(a, LP, grid, block, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

KV4_DEBUG_ACCESSOR(debug_flags_write)

}  // namespace kv4
