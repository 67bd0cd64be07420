// Matrix-core operand helpers shared by the gfx950 attention kernels: MFMA
// wrappers, exact nibble -> bf16 / fp16 operand conversions, float pair
// packing, and the direct buffer -> LDS loads with their wait.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kv4_device.hpp"

namespace kv4 {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma_bf16(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Nibble pair -> bf16 pair: for the nibbles at bits 0-3 and 16-19 of x,
// (nibble ^ 8) | 0x4300, i.e. the bf16 of 128 + u with u = code + 8; every
// other bit comes from the constant. One v_bitop3 (out = m ? x ^ k : k).
__device__ __forceinline__ uint32_t nib2bf(uint32_t x) {
  return __builtin_amdgcn_bitop3_b32(x, 0x43084308u, 0x000F000Fu, 0x6C);
}

// 8 codes of one token (one 32-bit word) -> A operand of one k-step, in
// k-order of element offsets [0, 4, 1, 5, 2, 6, 3, 7].
__device__ __forceinline__ uint4 k_operand(uint32_t w) {
  return make_uint4(nib2bf(w), nib2bf(w >> 4), nib2bf(w >> 8), nib2bf(w >> 12));
}

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4_t mfma_f16(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// Nibble pair -> fp16 pair: for the nibbles at bits 4-7 and 20-23 of x,
// (nibble ^ 8) becomes mantissa bits 4-7 under the exponent of 64, i.e. the
// fp16 of 64 + u with u = code + 8. One v_bitop3 (out = m ? x ^ k : k).
__device__ __forceinline__ uint32_t nib2h(uint32_t x) {
  return __builtin_amdgcn_bitop3_b32(x, 0x54805480u, 0x00F000F0u, 0x6C);
}

// Two floats -> fp16 pair, round to nearest even (v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, f16x2_t));
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two floats as a bf16 pair hi (round to nearest even, v_cvt_pk_bf16_f32)
// plus the bf16 pair of the remainders lo: hi + lo carries ~16 significant
// bits, which keeps sharp softmax rows (large k_scale) accurate.
__device__ __forceinline__ void split_bf16x2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
  const float ha = __uint_as_float(hi << 16), hb = __uint_as_float(hi & 0xFFFF0000u);
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a - ha, b - hb}, bf16x2_t));
}

// bytes jb of two words -> [a.jb, 0, b.jb, 0]
__device__ __forceinline__ uint32_t pair_byte(uint32_t a, uint32_t b, int jb) {
  const uint32_t sel = (uint32_t)jb | (0x0Cu << 8) | ((uint32_t)(4 + jb) << 16) | (0x0Cu << 24);
  return __builtin_amdgcn_perm(b, a, sel);
}

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void dma(const void* g, void* l, int size) {
  switch (size) {
    case 1: __builtin_amdgcn_global_load_lds(g, (lds_void*)l, 1, 0, 0); break;
    case 2: __builtin_amdgcn_global_load_lds(g, (lds_void*)l, 2, 0, 0); break;
    case 4: __builtin_amdgcn_global_load_lds(g, (lds_void*)l, 4, 0, 0); break;
    case 12: __builtin_amdgcn_global_load_lds(g, (lds_void*)l, 12, 0, 0); break;
    default: __builtin_amdgcn_global_load_lds(g, (lds_void*)l, 16, 0, 0); break;
  }
}

// Buffer-resource variant: uniform base in SGPRs, 32-bit per-lane offset;
// reads past num_records return 0 (never fault).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
// AUX is the load's cache-policy field: 0 = default, 2 = non-temporal (nt).
template <int SIZE, int AUX = 0>
__device__ __forceinline__ void dma_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, void* l) {
  if constexpr (SIZE == 1) __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)l, 1, voff, 0, 0, AUX);
  else if constexpr (SIZE == 2) __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)l, 2, voff, 0, 0, AUX);
  else if constexpr (SIZE == 4) __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)l, 4, voff, 0, 0, AUX);
  else if constexpr (SIZE == 12) __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)l, 12, voff, 0, 0, AUX);
  else __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)l, 16, voff, 0, 0, AUX);
}

// s_waitcnt with only the vector-memory counter (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

}  // namespace kv4
