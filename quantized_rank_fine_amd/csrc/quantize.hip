// qlora_quantize kernel: blockwise absmax, fp32 nearest-level encode,
// nibble packing and int8 double quantization of the block scales.
//
// "LLMs · QLoRA", code listing: absmax per block of 64 consecutive weights,
// code = argmin_i |w/absmax - L_i|.  "QLoRA (low-rank adapters on a
// quantized model)", "What QLoRA adds": the block scales are quantized again
// to 8 bits (here: symmetric int8, one fp32 scale per 256 block scales).
//
// One workgroup (4 wavefronts) per double-quantization group of 256 blocks
// (64 KiB of fp32).  Each lane owns 16 consecutive weights (one quarter of a
// block), so a wavefront covers 16 blocks = 4 KiB per step and the absmax of
// a block is a 4-lane reduction.  x = w / c_b is the IEEE fp32 quotient,
// obtained from the correctly rounded reciprocal y = 1/c_b (one division per
// lane and block) and two Markstein corrections q <- q + (w - q*c)*y, which
// return the correctly rounded quotient; the code is then a 4-step binary
// search over the 15 exact fp32 decision thresholds held in LDS.
#include "device.h"

namespace qlora {
namespace {

constexpr int kThreads = 256;
constexpr int kBlocksPerGroup = 256;

__device__ __forceinline__ uint32_t encode_one(float w, float y, float cs, float sc,
                                               const float *sT) {
  float x;
  if (y == 0.0f) {
    x = 0.0f;                                   // zero block
  } else {
    float ws = w * sc;                          // exact power-of-two scaling
    float q = ws * y;
    float r = fmaf(-q, cs, ws);
    q = fmaf(r, y, q);
    r = fmaf(-q, cs, ws);
    x = fmaf(r, y, q);
  }
  uint32_t k = (x >= sT[8]) ? 8u : 0u;
  k += (x >= sT[k + 4]) ? 4u : 0u;
  k += (x >= sT[k + 2]) ? 2u : 0u;
  k += (x >= sT[k + 1]) ? 1u : 0u;
  return k;
}

__global__ __launch_bounds__(kThreads) void quantize_kernel(
    const float *__restrict__ W0, uint8_t *__restrict__ codes, int8_t *__restrict__ qscale,
    float *__restrict__ gscale, int64_t nblocks, QuantConsts qc) {
  __shared__ float sT[16];
  __shared__ float sc_blk[kBlocksPerGroup];
  __shared__ float sred[kThreads / 64];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int64_t g = blockIdx.x;

  if (t < 16) sT[t] = qc.T[t];
  __syncthreads();

#pragma unroll 1
  for (int it = 0; it < 4; ++it) {
    const int bl = wave * 64 + it * 16 + (lane >> 2);     // block within group
    const int64_t b = g * kBlocksPerGroup + bl;
    const bool valid = b < nblocks;
    f32x4_t v[4];
    if (valid) {
      const f32x4_t *src = reinterpret_cast<const f32x4_t *>(W0 + b * 64 + (lane & 3) * 16);
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = __builtin_nontemporal_load(src + j);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      m = fmaxf(m, fabsf(v[j].x));
      m = fmaxf(m, fabsf(v[j].y));
      m = fmaxf(m, fabsf(v[j].z));
      m = fmaxf(m, fabsf(v[j].w));
    }
    m = fmaxf(m, __shfl_xor(m, 1));
    m = fmaxf(m, __shfl_xor(m, 2));

    // reciprocal of the (power-of-two rescaled) absmax; y = 0 marks c = 0
    float sc = 1.0f;
    if (m < 0x1p-100f) sc = 0x1p64f;
    if (m > 0x1p100f) sc = 0x1p-64f;
    const float cs = m * sc;
    const float y = (m == 0.0f) ? 0.0f : 1.0f / cs;

    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      lo |= encode_one(v[j].x, y, cs, sc, sT) << (16 * j + 0);
      lo |= encode_one(v[j].y, y, cs, sc, sT) << (16 * j + 4);
      lo |= encode_one(v[j].z, y, cs, sc, sT) << (16 * j + 8);
      lo |= encode_one(v[j].w, y, cs, sc, sT) << (16 * j + 12);
    }
#pragma unroll
    for (int j = 2; j < 4; ++j) {
      hi |= encode_one(v[j].x, y, cs, sc, sT) << (16 * (j - 2) + 0);
      hi |= encode_one(v[j].y, y, cs, sc, sT) << (16 * (j - 2) + 4);
      hi |= encode_one(v[j].z, y, cs, sc, sT) << (16 * (j - 2) + 8);
      hi |= encode_one(v[j].w, y, cs, sc, sT) << (16 * (j - 2) + 12);
    }
    if (valid) {
      u32x2_t packed = {lo, hi};
      *reinterpret_cast<u32x2_t *>(codes + b * 32 + (lane & 3) * 8) = packed;
    }
    if ((lane & 3) == 0) sc_blk[bl] = m;                 // 0 for padding blocks
  }
  __syncthreads();

  // double quantization of this group's 256 block scales
  const float c = sc_blk[t];
  float gm = c;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) gm = fmaxf(gm, __shfl_xor(gm, off));
  if (lane == 0) sred[wave] = gm;
  __syncthreads();
  gm = fmaxf(fmaxf(sred[0], sred[1]), fmaxf(sred[2], sred[3]));
  const float s2 = gm / 127.0f;
  const int64_t b = g * kBlocksPerGroup + t;
  if (b < nblocks) {
    int q = 0;
    if (s2 != 0.0f) {
      q = (int)rintf(c / s2);
      q = q > 127 ? 127 : (q < -127 ? -127 : q);
    }
    qscale[b] = (int8_t)q;
  }
  if (t == 0) gscale[g] = s2;
}

}  // namespace

hipError_t launch_quantize(const float *W0, uint8_t *codes, int8_t *qscale, float *gscale,
                           int64_t nblocks, hipStream_t s) {
  const int64_t groups = (nblocks + kBlocksPerGroup - 1) / kBlocksPerGroup;
  if (groups == 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)groups), dim3(kThreads), 0, s, W0, codes,
                     qscale, gscale, nblocks, tables().quant);
  return hipGetLastError();
}

}  // namespace qlora
