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

// Y = R . M.  Workgroup = 16 rows of R; the out axis in chunks of 256
// columns (fewer for wide k, to keep the M tile small).  A thread forms 16
// consecutive residual elements of one row (row t / 16, columns 16 (t % 16)
// ..) and loads its share of the chunk's rows of M; the next chunk's loads are issued into registers before
// the current chunk is multiplied, so HBM streams while the FMAs run.
// Thread t accumulates row t / 16, output columns t % 16 + 16 m, m < KB.
template <int KB>
__global__ __launch_bounds__(256) void rmul_kernel(ResidualArgs a, Levels16 lv) {
  constexpr int CH = KB <= 2 ? 256 : (KB == 4 ? 128 : 64);   // columns of R per chunk
  constexpr int KP = 16 * KB;                   // output columns held (k <= KP)
  __shared__ float sL[16];
  __shared__ __align__(16) float sR[16][CH + 4];
  __shared__ __align__(16) float sM[CH][KP + 4];
  const int t = threadIdx.x;
  const int64_t r0 = int64_t(blockIdx.x) * 16;
  if (t < 16) sL[t] = lv.L[t];
  __syncthreads();
  const int i = t >> 4, jl = t & 15;
  float acc[KB];
#pragma unroll
  for (int m = 0; m < KB; ++m) acc[m] = 0.0f;
  // M rows of a chunk: thread t loads element (n, j) = (t / KP' ...) in a
  // strided loop (k may be below KP: columns j >= k are zero)
  constexpr int MPER = CH * KP / 256;           // M elements per thread per chunk
  float rv[16], mv[MPER];
  // (the last chunk may run past out, a multiple of 64: those columns of R
  // and rows of M are zero and nothing past out is read)
  auto load = [&](int64_t n0) {
    if (16 * jl < CH && n0 + 16 * jl < a.out) {
      residual16(a, sL, r0 + i, n0 + 16 * jl, rv);
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) rv[e] = 0.0f;
    }
#pragma unroll
    for (int u = 0; u < MPER; ++u) {
      const int e = t + 256 * u, n = e / KP, j = e - n * KP;
      mv[u] = (j < a.k && n0 + n < a.out) ? a.M[(n0 + n) * a.k + j] : 0.0f;
    }
  };
  load(0);
  for (int64_t n0 = 0; n0 < a.out; n0 += CH) {
    __syncthreads();                            // the previous chunk's reads are done
    if (16 * jl < CH) {
#pragma unroll
      for (int e = 0; e < 16; ++e) sR[i][16 * jl + e] = rv[e];
    }
#pragma unroll
    for (int u = 0; u < MPER; ++u) {
      const int e = t + 256 * u, n = e / KP, j = e - n * KP;
      sM[n][j] = mv[u];
    }
    __syncthreads();
    if (n0 + CH < a.out) load(n0 + CH);         // in flight during the FMAs
#pragma unroll 8
    for (int n = 0; n < CH; ++n) {
      const float r = sR[i][n];
#pragma unroll
      for (int m = 0; m < KB; ++m) acc[m] = __builtin_fmaf(r, sM[n][16 * m + jl], acc[m]);
    }
  }
#pragma unroll
  for (int m = 0; m < KB; ++m)
    if (16 * m + jl < a.k) a.Y[(r0 + i) * a.k + 16 * m + jl] = acc[m];
}

// Z = R^T . Q.  Workgroup = 32 columns of R; the in axis in chunks of 128
// rows.  Thread t forms 16 residual elements of row t / 2, columns
// 16 (t % 2) .. (a whole 128-B line of W0 per thread pair) and loads its
// share of the chunk's Q rows; the next chunk is loaded into registers while
// the current one is multiplied.  Thread t accumulates column t % 32,
// output ranks t / 32 + 8 m, m < KB.
template <int KB>
__global__ __launch_bounds__(256) void rtmul_kernel(ResidualArgs a, Levels16 lv) {
  constexpr int CH = KB <= 8 ? 128 : 64;        // rows of R per chunk
  constexpr int KP = 8 * KB;
  __shared__ float sL[16];
  __shared__ __align__(16) float sR[CH][32 + 1];
  __shared__ __align__(16) float sQ[CH][KP + 4];
  const int t = threadIdx.x;
  const int64_t c0 = int64_t(blockIdx.x) * 32;
  if (t < 16) sL[t] = lv.L[t];
  __syncthreads();
  const int c = t & 31, jg = t >> 5;
  float acc[KB];
#pragma unroll
  for (int m = 0; m < KB; ++m) acc[m] = 0.0f;
  constexpr int QPER = CH * KP / 256;
  float rv[16], qv[QPER];
  // (the last chunk may run past in, a multiple of 64: zero rows)
  auto load = [&](int64_t i0) {
    if ((t >> 1) < CH && i0 + (t >> 1) < a.in) {
      residual16(a, sL, i0 + (t >> 1), c0 + 16 * (t & 1), rv);
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) rv[e] = 0.0f;
    }
#pragma unroll
    for (int u = 0; u < QPER; ++u) {
      const int e = t + 256 * u, ii = e / KP, j = e - ii * KP;
      qv[u] = (j < a.k && i0 + ii < a.in) ? a.M[(i0 + ii) * a.k + j] : 0.0f;
    }
  };
  load(0);
  for (int64_t i0 = 0; i0 < a.in; i0 += CH) {
    __syncthreads();
    if ((t >> 1) < CH) {
#pragma unroll
      for (int e = 0; e < 16; ++e) sR[t >> 1][16 * (t & 1) + e] = rv[e];
    }
#pragma unroll
    for (int u = 0; u < QPER; ++u) {
      const int e = t + 256 * u, ii = e / KP, j = e - ii * KP;
      sQ[ii][j] = qv[u];
    }
    __syncthreads();
    if (i0 + CH < a.in) load(i0 + CH);
#pragma unroll 8
    for (int ii = 0; ii < CH; ++ii) {
      const float r = sR[ii][c];
#pragma unroll
      for (int m = 0; m < KB; ++m) acc[m] = __builtin_fmaf(r, sQ[ii][jg + 8 * m], acc[m]);
    }
  }
#pragma unroll
  for (int m = 0; m < KB; ++m)
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
  // in % 64 == 0 and out % 64 == 0 (checked by the caller): whole 16-row
  // and 32-column workgroups; the kernels zero what a last chunk has past
  // the end.
  if (!transpose) {
    const dim3 g(unsigned(in / 16));
    if (k <= 16) hipLaunchKernelGGL(rmul_kernel<1>, g, dim3(256), 0, s, a, lv);
    else if (k <= 32) hipLaunchKernelGGL(rmul_kernel<2>, g, dim3(256), 0, s, a, lv);
    else if (k <= 64) hipLaunchKernelGGL(rmul_kernel<4>, g, dim3(256), 0, s, a, lv);
    else hipLaunchKernelGGL(rmul_kernel<8>, g, dim3(256), 0, s, a, lv);
  } else {
    const dim3 g(unsigned(out / 32));
    if (k <= 16) hipLaunchKernelGGL(rtmul_kernel<2>, g, dim3(256), 0, s, a, lv);
    else if (k <= 32) hipLaunchKernelGGL(rtmul_kernel<4>, g, dim3(256), 0, s, a, lv);
    else if (k <= 64) hipLaunchKernelGGL(rtmul_kernel<8>, g, dim3(256), 0, s, a, lv);
    else hipLaunchKernelGGL(rtmul_kernel<16>, g, dim3(256), 0, s, a, lv);
  }
  return hipGetLastError();
}

}  // namespace qlora
