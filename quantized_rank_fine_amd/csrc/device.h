// Device helpers for the gfx950 kernels: vector types, bf16 packing and the
// MFMA wrappers.
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

__device__ __forceinline__ int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }

// One Adam (AdamW) step of one element, fp32 (Kingma & Ba, Algorithm 1, with
// decoupled weight decay):
//   m <- b1 m + (1 - b1) g,   v <- b2 v + (1 - b2) g g,
//   theta <- theta - lr ( (m c1) / (sqrt(v c2) + eps) + wd theta ).
// Shared by the Adam kernel and the backward's fused update, so the two give
// the same bits.
__device__ __forceinline__ void adam1(const AdamParams &a, float &th, float g, float &m,
                                      float &v) {
  m = a.b1 * m + a.omb1 * g;
  v = a.b2 * v + a.omb2 * (g * g);
  const float den = sqrtf(v * a.c2) + a.eps;
  th = th - a.lr * ((m * a.c1) / den + a.wd * th);
}

// Element (m, j) of an [M x R] rank-r intermediate after its multiplier (a
// dropped element is 0 whatever v is).
__device__ __forceinline__ float rank_mul(const RankMul &k, int64_t m, int64_t j, int64_t R,
                                          float v) {
  return (k.keep && k.keep[m * R + j] == 0) ? 0.0f : k.c * v;
}

}  // namespace qlora
