// Rank-r ("skinny") products of the adapted linear layer and their helpers.
//
// "QLoRA (low-rank adapters on a quantized model)", "How it works": A is
// (in x r) and B is (r x out); the adapter path costs r*(in+out) parameters
// and adds the rank-r products
//   XA = X.A (forward),  G = dY.B^T,  dA = X^T.G,  dB = XA^T.dY (backward),
// which are memory-bound passes over X or dY (r <= 256 << in, out).
//
// rowdot: C[M x R] = P[M x K] . Qt[R x K]^T, contraction along rows of P
//         (P = X or dY, read once, coalesced).
// coldot: C[K x R] = P[M x K]^T . Qt[R x M]^T, contraction over the token
//         axis (P = X or dY).  P tiles are staged row-major in LDS and read
//         transposed with ds_read_b64_tr_b16 (16 lanes x 4 rows -> 4 columns).
// Both split the contraction over workgroups and write fp32 partials that
// launch_reduce sums in a fixed order (deterministic, no atomics).
//
// All matrix-core work is v_mfma_f32_16x16x32_bf16: operands rounded to bf16,
// fp32 accumulation.
#include "device.h"

namespace qlora {
namespace {

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
typedef __attribute__((address_space(3))) char lds_char;

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// 8 consecutive elements of a row starting at `p` (bf16 or fp32) as bf16x8.
template <bool kBf16>
__device__ __forceinline__ u32x4_t load8_bf16(const void *p) {
  if constexpr (kBf16) {
    return *reinterpret_cast<const u32x4_t *>(p);
  } else {
    const float4 *q = reinterpret_cast<const float4 *>(p);
    float4 a = q[0], b = q[1];
    u32x4_t r;
    r[0] = pack_bf16x2(a.x, a.y);
    r[1] = pack_bf16x2(a.z, a.w);
    r[2] = pack_bf16x2(b.x, b.y);
    r[3] = pack_bf16x2(b.z, b.w);
    return r;
  }
}

// ------------------------------------------------------------ conversions

__global__ __launch_bounds__(256) void transpose_bf16_kernel(const void *__restrict__ src,
                                                             bool src_bf16, int64_t K, int64_t R,
                                                             uint16_t *__restrict__ dst,
                                                             int64_t ldd) {
  // dst[j][k] = src[k][j] for k < K, j < R; dst[j][k] = 0 for K <= k < ldd.
  __shared__ uint16_t tile[32][33];
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const int64_t j0 = int64_t(blockIdx.x) * 32, k0 = int64_t(blockIdx.y) * 32;
  for (int yy = ty; yy < 32; yy += 8) {
    const int64_t k = k0 + yy, j = j0 + tx;
    uint16_t v = 0;
    if (k < K && j < R) {
      v = src_bf16 ? static_cast<const uint16_t *>(src)[k * R + j]
                   : f32_to_bf16_bits(static_cast<const float *>(src)[k * R + j]);
    }
    tile[yy][tx] = v;
  }
  __syncthreads();
  for (int yy = ty; yy < 32; yy += 8) {
    const int64_t j = j0 + yy, k = k0 + tx;
    if (j < R && k < ldd) dst[j * ldd + k] = tile[tx][yy];
  }
}

__global__ __launch_bounds__(256) void pad_bf16_kernel(const void *__restrict__ src,
                                                       bool src_bf16, int64_t rows, int64_t cols,
                                                       uint16_t *__restrict__ dst, int64_t ldd) {
  const int64_t n = rows * ldd;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256) {
    const int64_t r = i / ldd, j = i - r * ldd;
    uint16_t v = 0;
    if (j < cols) {
      v = src_bf16 ? static_cast<const uint16_t *>(src)[r * cols + j]
                   : f32_to_bf16_bits(static_cast<const float *>(src)[r * cols + j]);
    }
    dst[i] = v;
  }
}

__global__ __launch_bounds__(256) void convert_bf16_kernel(const void *__restrict__ src,
                                                           bool src_bf16, int64_t n,
                                                           uint16_t *__restrict__ dst) {
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256) {
    dst[i] = src_bf16 ? static_cast<const uint16_t *>(src)[i]
                      : f32_to_bf16_bits(static_cast<const float *>(src)[i]);
  }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float *__restrict__ p, int64_t n) {
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256)
    p[i] = 0.0f;
}

// ------------------------------------------------------------------ rowdot
//
// Workgroup: 4 wavefronts x 16 rows = 64 rows of P, all R columns, one
// contiguous K range.  Qt is staged per 64-wide K slice in LDS (rows of 128 B,
// 16-B chunks XOR-swizzled by row) and shared by the 4 wavefronts; P rows go
// straight from global memory into the MFMA A operand.

constexpr int kRowdotRows = 64;
constexpr int kSliceK = 64;

template <bool kPbf16>
__global__ __launch_bounds__(256) void rowdot_kernel(const void *__restrict__ Pv,
                                                     const uint16_t *__restrict__ Qt, int64_t M,
                                                     int64_t K, int R, int64_t kchunk,
                                                     float *__restrict__ part) {
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t *sQ = reinterpret_cast<uint16_t *>(smem);   // [RP][64]
  const int RT = (R + 15) / 16;
  const int RP = RT * 16;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int i16 = lane & 15, h = lane >> 4;
  const int64_t m0 = int64_t(blockIdx.x) * kRowdotRows;
  const int ks = blockIdx.y;
  const int64_t kb = int64_t(ks) * kchunk;
  const int64_t ke = min64(K, kb + kchunk);
  const int64_t row = m0 + wave * 16 + i16;
  const bool row_ok = row < M;
  const size_t esz = kPbf16 ? 2 : 4;
  const char *prow = static_cast<const char *>(Pv) + (row_ok ? row : 0) * K * esz;

  f32x4_t acc[16];
#pragma unroll
  for (int s = 0; s < 16; ++s) acc[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int64_t k0 = kb; k0 < ke; k0 += kSliceK) {
    // A operands of this slice: substep u covers k0 + 32u + 8h .. +8
    u32x4_t a[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      a[u] = row_ok ? load8_bf16<kPbf16>(prow + (k0 + 32 * u + 8 * h) * esz)
                    : u32x4_t{0u, 0u, 0u, 0u};
    }
    __syncthreads();
    // stage Qt[0..RP)[k0..k0+64) : RP rows x 8 chunks of 16 B
    for (int c = t; c < RP * 8; c += 256) {
      const int j = c >> 3, ch = c & 7;
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (j < R) v = *reinterpret_cast<const u32x4_t *>(Qt + int64_t(j) * K + k0 + 8 * ch);
      *reinterpret_cast<u32x4_t *>(sQ + j * 64 + ((ch ^ (j & 7)) * 8)) = v;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        if (s < RT) {
          const int j = 16 * s + i16;
          const int ch = 4 * u + h;
          u32x4_t b = *reinterpret_cast<const u32x4_t *>(sQ + j * 64 + ((ch ^ (j & 7)) * 8));
          acc[s] = mfma16x16x32(a[u], b, acc[s]);
        }
      }
    }
  }
  // C layout: lane holds rows 4h..4h+3 of the wave's 16, column i16 of subtile s
  float *out = part + int64_t(ks) * M * R;
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    if (s < RT) {
      const int j = 16 * s + i16;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t m = m0 + wave * 16 + 4 * h + q;
        if (m < M && j < R) out[m * R + j] = acc[s][q];
      }
    }
  }
}

// ------------------------------------------------------------------ coldot
//
// Workgroup: 4 wavefronts x 16 columns of P = 64 columns, all R, one
// contiguous range of tokens.  Per 64-token slice the P tile (64 x 64 bf16)
// is stored row-major in LDS with a 160-byte row pitch (conflict-free for the
// transposed reads) and Qt (R x 64) with swizzled 16-B chunks.

constexpr int kColdotCols = 64;
constexpr int kPPitch = 80;   // bf16 elements per P row in LDS (160 bytes)

template <bool kPbf16>
__global__ __launch_bounds__(256) void coldot_kernel(const void *__restrict__ Pv,
                                                     const uint16_t *__restrict__ Qt,
                                                     int64_t ldq, int64_t M,
                                                     int64_t K, int R, int64_t mchunk,
                                                     float *__restrict__ part) {
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t *sP = reinterpret_cast<uint16_t *>(smem);               // [64][kPPitch]
  uint16_t *sQ = sP + 64 * kPPitch;                                // [RP][64]
  const int RT = (R + 15) / 16;
  const int RP = RT * 16;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int i16 = lane & 15, h = lane >> 4;
  const int64_t c0 = int64_t(blockIdx.x) * kColdotCols;
  const int ks = blockIdx.y;
  const int64_t mb = int64_t(ks) * mchunk;
  const int64_t me = min64(M, mb + mchunk);
  const size_t esz = kPbf16 ? 2 : 4;
  const char *P = static_cast<const char *>(Pv);

  f32x4_t acc[16];
#pragma unroll
  for (int s = 0; s < 16; ++s) acc[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int64_t mm = mb; mm < me; mm += 64) {
    // P tile rows mm..mm+63, columns c0..c0+63: 64 rows x 8 chunks of 16 B
    u32x4_t pv[2];
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int c = t + 256 * it;
      const int rr = c >> 3, ch = c & 7;
      const int64_t m = mm + rr, col = c0 + 8 * ch;
      pv[it] = (m < me && col < K) ? load8_bf16<kPbf16>(P + (m * K + col) * esz)
                                   : u32x4_t{0u, 0u, 0u, 0u};
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int c = t + 256 * it;
      const int rr = c >> 3, ch = c & 7;
      *reinterpret_cast<u32x4_t *>(sP + rr * kPPitch + 8 * ch) = pv[it];
    }
    for (int c = t; c < RP * 8; c += 256) {
      const int j = c >> 3, ch = c & 7;
      const int64_t m = mm + 8 * ch;
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (j < R) {
        if (m + 8 <= me) {
          v = *reinterpret_cast<const u32x4_t *>(Qt + int64_t(j) * ldq + m);
        } else {
          uint16_t e[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) e[q] = (m + q < me) ? Qt[int64_t(j) * ldq + m + q] : 0;
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = uint32_t(e[2 * q]) | (uint32_t(e[2 * q + 1]) << 16);
        }
      }
      *reinterpret_cast<u32x4_t *>(sQ + j * 64 + ((ch ^ (j & 7)) * 8)) = v;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      // A operand: column (16*wave + i16) of P, tokens 32u + 8h .. +8, via two
      // transposed reads of 4 rows x 4 columns per 16-lane group.
      u32x4_t a;
      {
        const int q = i16 & 3, tq = i16 >> 2;
        const int rr = 32 * u + 8 * h + tq;
        lds_char *base = (lds_char *)(sP);
        i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4 *)(base + (rr * kPPitch + 16 * wave + 4 * q) * 2));
        i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4 *)(base + ((rr + 4) * kPPitch + 16 * wave + 4 * q) * 2));
        u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
        a = u32x4_t{l2[0], l2[1], h2[0], h2[1]};
      }
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        if (s < RT) {
          const int j = 16 * s + i16;
          const int ch = 4 * u + h;
          u32x4_t b = *reinterpret_cast<const u32x4_t *>(sQ + j * 64 + ((ch ^ (j & 7)) * 8));
          acc[s] = mfma16x16x32(a, b, acc[s]);
        }
      }
    }
  }
  float *out = part + int64_t(ks) * K * R;
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    if (s < RT) {
      const int j = 16 * s + i16;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t col = c0 + 16 * wave + 4 * h + q;
        if (col < K && j < R) out[col * R + j] = acc[s][q];
      }
    }
  }
}

// ------------------------------------------------------------------ reduce

__global__ __launch_bounds__(256) void reduce_kernel(const float *__restrict__ part, int64_t ks,
                                                     int64_t rows, int64_t R,
                                                     float *__restrict__ out, bool transpose_out,
                                                     uint16_t *__restrict__ out_bf16,
                                                     int64_t ld_bf16,
                                                     uint16_t *__restrict__ outT_bf16,
                                                     int64_t ldT) {
  const int64_t n = rows * R;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256) {
    float s = 0.0f;
    for (int64_t k = 0; k < ks; ++k) s += part[k * n + i];
    const int64_t rr = i / R, j = i - rr * R;
    if (out) out[transpose_out ? j * rows + rr : i] = s;
    if (out_bf16) out_bf16[rr * ld_bf16 + j] = f32_to_bf16_bits(s);
    if (outT_bf16) outT_bf16[j * ldT + rr] = f32_to_bf16_bits(s);
  }
  if (out_bf16 && ld_bf16 > R) {   // zero padding columns R..ld_bf16-1
    const int64_t pad = ld_bf16 - R, np = rows * pad;
    for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < np;
         i += int64_t(gridDim.x) * 256) {
      const int64_t rr = i / pad, j = R + (i - rr * pad);
      out_bf16[rr * ld_bf16 + j] = 0;
    }
  }
}

unsigned grid_for(int64_t n) {
  int64_t g = (n + 255) / 256;
  if (g > 4096) g = 4096;
  if (g < 1) g = 1;
  return unsigned(g);
}

}  // namespace

hipError_t launch_transpose_to_bf16(const void *src, bool src_bf16, int64_t K, int64_t R,
                                    uint16_t *dst, int64_t ldd, hipStream_t s) {
  if (K == 0 || R == 0) return hipSuccess;
  dim3 grid(unsigned((R + 31) / 32), unsigned((ldd + 31) / 32));
  hipLaunchKernelGGL(transpose_bf16_kernel, grid, dim3(256), 0, s, src, src_bf16, K, R, dst, ldd);
  return hipGetLastError();
}

hipError_t launch_convert_to_bf16(const void *src, bool src_bf16, int64_t n, uint16_t *dst,
                                  hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(convert_bf16_kernel, dim3(grid_for(n)), dim3(256), 0, s, src, src_bf16, n,
                     dst);
  return hipGetLastError();
}

hipError_t launch_pad_to_bf16(const void *src, bool src_bf16, int64_t rows, int64_t cols,
                              uint16_t *dst, int64_t ldd, hipStream_t s) {
  if (rows == 0 || ldd == 0) return hipSuccess;
  hipLaunchKernelGGL(pad_bf16_kernel, dim3(grid_for(rows * ldd)), dim3(256), 0, s, src, src_bf16,
                     rows, cols, dst, ldd);
  return hipGetLastError();
}

hipError_t launch_fill_zero(float *p, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(grid_for(n)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

namespace {
int64_t rowdot_chunk(int64_t M, int64_t K) {
  const int64_t rt = (M + kRowdotRows - 1) / kRowdotRows;
  const int64_t slices = K / kSliceK;
  int64_t ks = (512 + rt - 1) / rt;
  if (ks < 1) ks = 1;
  if (ks > slices) ks = slices;
  const int64_t per = (slices + ks - 1) / ks;   // slices per split
  return per * kSliceK;
}
int64_t coldot_chunk(int64_t M, int64_t K) {
  const int64_t ct = (K + kColdotCols - 1) / kColdotCols;
  const int64_t mt = (M + 63) / 64;
  int64_t ks = (512 + ct - 1) / ct;
  if (ks < 1) ks = 1;
  if (ks > mt) ks = mt;
  const int64_t per = (mt + ks - 1) / ks;
  return per * 64;
}
}  // namespace

int64_t rowdot_splits(int64_t M, int64_t K, int64_t R) {
  (void)R;
  if (M == 0) return 0;
  const int64_t kc = rowdot_chunk(M, K);
  return (K + kc - 1) / kc;
}

int64_t coldot_splits(int64_t M, int64_t K, int64_t R) {
  (void)R;
  if (M == 0) return 0;
  const int64_t mc = coldot_chunk(M, K);
  return (M + mc - 1) / mc;
}

hipError_t launch_rowdot(const void *P, bool p_bf16, const uint16_t *Qt, int64_t M, int64_t K,
                         int64_t R, float *part, hipStream_t s) {
  if (M == 0 || R == 0) return hipSuccess;
  const int64_t kc = rowdot_chunk(M, K);
  const int64_t ks = (K + kc - 1) / kc;
  const int RP = int((R + 15) / 16 * 16);
  const size_t lds = size_t(RP) * 64 * 2;
  dim3 grid(unsigned((M + kRowdotRows - 1) / kRowdotRows), unsigned(ks));
  if (p_bf16)
    hipLaunchKernelGGL(rowdot_kernel<true>, grid, dim3(256), lds, s, P, Qt, M, K, int(R), kc,
                       part);
  else
    hipLaunchKernelGGL(rowdot_kernel<false>, grid, dim3(256), lds, s, P, Qt, M, K, int(R), kc,
                       part);
  return hipGetLastError();
}

hipError_t launch_coldot(const void *P, bool p_bf16, const uint16_t *Qt, int64_t ldq, int64_t M,
                         int64_t K, int64_t R, float *part, hipStream_t s) {
  if (M == 0 || R == 0) return hipSuccess;
  const int64_t mc = coldot_chunk(M, K);
  const int64_t ks = (M + mc - 1) / mc;
  const int RP = int((R + 15) / 16 * 16);
  const size_t lds = size_t(64) * kPPitch * 2 + size_t(RP) * 64 * 2;
  dim3 grid(unsigned((K + kColdotCols - 1) / kColdotCols), unsigned(ks));
  if (p_bf16)
    hipLaunchKernelGGL(coldot_kernel<true>, grid, dim3(256), lds, s, P, Qt, ldq, M, K, int(R),
                       mc, part);
  else
    hipLaunchKernelGGL(coldot_kernel<false>, grid, dim3(256), lds, s, P, Qt, ldq, M, K, int(R),
                       mc, part);
  return hipGetLastError();
}

hipError_t launch_reduce(const float *part, int64_t ks, int64_t rows, int64_t R, float *out,
                         bool transpose_out, uint16_t *out_bf16, int64_t ld_bf16,
                         uint16_t *outT_bf16, int64_t ldT, hipStream_t s) {
  if (rows == 0 || R == 0) return hipSuccess;
  hipLaunchKernelGGL(reduce_kernel, dim3(grid_for(rows * R)), dim3(256), 0, s, part, ks, rows, R,
                     out, transpose_out, out_bf16, ld_bf16, outT_bf16, ldT);
  return hipGetLastError();
}

}  // namespace qlora
