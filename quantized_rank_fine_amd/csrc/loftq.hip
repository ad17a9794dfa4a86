// Products with the quantization residual R = W0 - deq(Wq), for the
// LoftQ-style start of the adapters (a rank-r SVD of the residual).
//
// "QLoRA (low-rank adapters on a quantized model)", "What QLoRA adds" (the
// paragraph on running it): LoftQ-style methods start A and B from an SVD of
// W0 - Q(W0) instead of zero.  The truncated SVD is found by randomized
// subspace iteration, which touches R only through the products
//   Y = R . M   (M [out x k], Y [in x k])   and   Z = R^T . Q   (Q [in x k]),
// k <= 128 columns.  R is never stored: each tile of it is formed in fp32
// (W0 minus L[code] * (q_b * s2_g), the value the fused GEMMs round to bf16)
// and multiplied with fp32 multiply-adds.
#include "device.h"

namespace qlora {
namespace {

constexpr int kMaxK = 128;

struct ResidualArgs {
  const float *W0;
  const uint8_t *codes;
  const int8_t *q8;
  const float *s2;
  int64_t in, out;
  const float *M;     // rmul: [out x k]; rtmul: [in x k]
  int k;
  float *Y;           // rmul: [in x k]; rtmul: [out x k]
};

// 16 consecutive residual elements of row `row`, columns col .. col + 15
// (col % 16 == 0: one 64-block, one scale).
__device__ __forceinline__ void residual16(const ResidualArgs &a, const float *L, int64_t row,
                                           int64_t col, float (&v)[16]) {
  const int64_t flat = row * a.out + col;
  const int64_t blk = flat / 64;
  const float c = float(a.q8[blk]) * a.s2[blk >> 8];
  const u32x2_t cw = *reinterpret_cast<const u32x2_t *>(a.codes + flat / 2);
  const f32x4_t *w = reinterpret_cast<const f32x4_t *>(a.W0 + flat);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const f32x4_t x = w[q];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 4 * q + e;
      const uint32_t code = (cw[i >> 3] >> (4 * (i & 7))) & 15u;
      v[i] = x[e] - L[code] * c;
    }
  }
}

// Y = R . M: workgroup = 16 rows of R; the out axis in chunks of 64
// columns.  Thread t: row t / 16 of the 16, output columns t % 16 + 16 m.
__global__ __launch_bounds__(256) void rmul_kernel(ResidualArgs a, Levels16 lv) {
  __shared__ float sL[16];
  __shared__ __align__(16) float sR[16][64 + 4];
  __shared__ __align__(16) float sM[64][kMaxK + 4];
  const int t = threadIdx.x;
  const int64_t r0 = int64_t(blockIdx.x) * 16;
  if (t < 16) sL[t] = lv.L[t];
  float acc[kMaxK / 16];
#pragma unroll
  for (int m = 0; m < kMaxK / 16; ++m) acc[m] = 0.0f;
  const int i = t >> 4, jl = t & 15;
  for (int64_t n0 = 0; n0 < a.out; n0 += 64) {
    __syncthreads();
    // R tile [16 x 64]: thread t (< 64) forms 16 elements of row t / 4
    if (t < 64) {
      float v[16];
      residual16(a, sL, r0 + (t >> 2), n0 + 16 * (t & 3), v);
#pragma unroll
      for (int e = 0; e < 16; ++e) sR[t >> 2][16 * (t & 3) + e] = v[e];
    }
    // M tile [64 x k]
    for (int e = t; e < 64 * a.k; e += 256) {
      const int n = e / a.k, j = e - n * a.k;
      sM[n][j] = a.M[(n0 + n) * a.k + j];
    }
    __syncthreads();
    for (int n = 0; n < 64; ++n) {
      const float rv = sR[i][n];
#pragma unroll
      for (int m = 0; m < kMaxK / 16; ++m)
        if (16 * m + jl < a.k) acc[m] = __builtin_fmaf(rv, sM[n][16 * m + jl], acc[m]);
    }
  }
#pragma unroll
  for (int m = 0; m < kMaxK / 16; ++m)
    if (16 * m + jl < a.k) a.Y[(r0 + i) * a.k + 16 * m + jl] = acc[m];
}

// Z = R^T . Q: workgroup = 32 columns of R; the in axis in chunks of 64 rows.
// Thread t: column t % 32 of the 32, output ranks t / 32 + 8 m.
__global__ __launch_bounds__(256) void rtmul_kernel(ResidualArgs a, Levels16 lv) {
  __shared__ float sL[16];
  __shared__ __align__(16) float sR[64][32 + 1];
  __shared__ __align__(16) float sQ[64][kMaxK + 4];
  const int t = threadIdx.x;
  const int64_t c0 = int64_t(blockIdx.x) * 32;
  if (t < 16) sL[t] = lv.L[t];
  float acc[kMaxK / 8];
#pragma unroll
  for (int m = 0; m < kMaxK / 8; ++m) acc[m] = 0.0f;
  const int c = t & 31, jg = t >> 5;
  for (int64_t i0 = 0; i0 < a.in; i0 += 64) {
    __syncthreads();
    // R tile [64 x 32]: thread t (< 128) forms 16 elements of row t / 2
    if (t < 128) {
      float v[16];
      residual16(a, sL, i0 + (t >> 1), c0 + 16 * (t & 1), v);
#pragma unroll
      for (int e = 0; e < 16; ++e) sR[t >> 1][16 * (t & 1) + e] = v[e];
    }
    for (int e = t; e < 64 * a.k; e += 256) {
      const int ii = e / a.k, j = e - ii * a.k;
      sQ[ii][j] = a.M[(i0 + ii) * a.k + j];
    }
    __syncthreads();
    for (int ii = 0; ii < 64; ++ii) {
      const float rv = sR[ii][c];
#pragma unroll
      for (int m = 0; m < kMaxK / 8; ++m)
        if (jg + 8 * m < a.k) acc[m] = __builtin_fmaf(rv, sQ[ii][jg + 8 * m], acc[m]);
    }
  }
#pragma unroll
  for (int m = 0; m < kMaxK / 8; ++m)
    if (jg + 8 * m < a.k) a.Y[(c0 + c) * a.k + jg + 8 * m] = acc[m];
}

}  // namespace

hipError_t launch_residual_mul(const float *W0, const uint8_t *codes, const int8_t *q8,
                               const float *s2, int64_t in, int64_t out, const float *M, int k,
                               float *Y, bool transpose, int codebook, hipStream_t s) {
  if (k < 1 || k > kMaxK) return hipErrorInvalidValue;
  ResidualArgs a{W0, codes, q8, s2, in, out, M, k, Y};
  Levels16 lv;
  const Tables &tb = tables(codebook);
  for (int i = 0; i < 16; ++i) lv.L[i] = tb.L[i];
  if (!transpose)
    hipLaunchKernelGGL(rmul_kernel, dim3(unsigned(in / 16)), dim3(256), 0, s, a, lv);
  else
    hipLaunchKernelGGL(rtmul_kernel, dim3(unsigned(out / 32)), dim3(256), 0, s, a, lv);
  return hipGetLastError();
}

}  // namespace qlora
