// Device helpers for the gfx950 kernels: vector types, bf16 packing, the
// register-level 16-entry level lookup and the MFMA wrappers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace qlora {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t perm_b32(uint32_t hi, uint32_t lo, uint32_t sel) {
  // pool bytes 0..3 = lo, 4..7 = hi
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// Two fp32 -> packed bf16 pair (round to nearest even), low half = a.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo_to_f32(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi_to_f32(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ f32x4_t mfma16x16x32(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// 32x32x16 bf16: A lane l holds row l%32, k = 8*(l/32) + 0..7; B lane l holds
// column l%32, same k; result register r of lane l is row 8*(r/4) + 4*(l/32)
// + r%4, column l%32.  On gfx950 it has twice the throughput per flop of the
// 16x16x32 form.
__device__ __forceinline__ f32x16_t mfma32x32x16(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// Four 4-bit codes, one per byte of v (values 0..15) -> the four fp32 levels.
// The table is symmetric (L[15-i] = -L[i]); magnitude index m = c-8 for
// c >= 8 and 7-c for c < 8, sign negative for c < 8.  Each byte plane of the
// 8 magnitudes fits the 8-byte pool of one v_perm, so a lookup of four codes
// is four perms plus a byte transpose.
__device__ __forceinline__ void lookup4(uint32_t v, const ExpandConsts &t, float out[4]) {
  uint32_t u = v ^ 0x08080808u;            // c>=8 -> c-8 ; c<8 -> c+8
  uint32_t b3 = u & 0x08080808u;           // 8 where c < 8
  uint32_t m7 = b3 - (b3 >> 3);            // 7 where c < 8
  uint32_t m = (u ^ m7) & 0x07070707u;     // magnitude index per byte
  uint32_t p0 = perm_b32(t.plane[0][1], t.plane[0][0], m);
  uint32_t p1 = perm_b32(t.plane[1][1], t.plane[1][0], m);
  uint32_t p2 = perm_b32(t.plane[2][1], t.plane[2][0], m);
  uint32_t p3 = perm_b32(t.plane[3][1], t.plane[3][0], m) | (b3 << 4);
  uint32_t a = perm_b32(p1, p0, 0x05010400u);
  uint32_t b = perm_b32(p1, p0, 0x07030602u);
  uint32_t c = perm_b32(p3, p2, 0x05010400u);
  uint32_t d = perm_b32(p3, p2, 0x07030602u);
  out[0] = __uint_as_float(perm_b32(c, a, 0x05040100u));
  out[1] = __uint_as_float(perm_b32(c, a, 0x07060302u));
  out[2] = __uint_as_float(perm_b32(d, b, 0x05040100u));
  out[3] = __uint_as_float(perm_b32(d, b, 0x07060302u));
}

__device__ __forceinline__ int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }

}  // namespace qlora
