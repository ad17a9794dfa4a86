// Rank-r ("skinny") products of the adapted linear layer and their helpers.
//
// "QLoRA (low-rank adapters on a quantized model)", "How it works": A is
// (in x r) and B is (r x out); the adapter path costs r*(in+out) parameters
// and adds the rank-r products
//   XA = X.A (forward),  G = dY.B^T,  dA = X^T.G,  dB = XA^T.dY (backward),
// which are memory-bound passes over X or dY (r <= 256 << in, out).
//
// rowdot: C[M x R] = P[M x K] . Q, contraction along rows of P (P = X or dY,
//         read once, coalesced).  Q is given either as Qt [R x K] (B for G)
//         or as [K x R] (A for XA); a 64-wide K slice of it is staged in LDS
//         in the [R][64] form the MFMA B operand reads.
// coldot: C[K x R] = P[M x K]^T . Q[M x R], contraction over the token axis
//         (P = X or dY, Q = G or XA given row-major).  P tiles are staged
//         row-major in LDS and read transposed with ds_read_b64_tr_b16
//         (16 lanes x 4 rows -> 4 columns).
// Both split the contraction over workgroups and write fp32 partials that a
// reduce pass sums in a fixed order (deterministic, no atomics).
//
// Launches are merged where the data allow it: the forward runs one prep
// launch (XA partials + the GEMM's block scales) and one reduce; the backward
// runs one pass over dY (G partials, dB partials, block scales), one reduce
// of G and dB, one pass over X (dA partials) and one reduce of dA.  A merged
// launch gives each role a contiguous range of workgroup ids.
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

// One element (bf16 or fp32) as bf16 bits.
template <bool kBf16>
__device__ __forceinline__ uint32_t load1_bf16(const void *p, int64_t i) {
  if constexpr (kBf16)
    return static_cast<const uint16_t *>(p)[i];
  else
    return f32_to_bf16_bits(static_cast<const float *>(p)[i]);
}

// 8 elements p[i0 + q*stride], q = 0..7, as bf16x8 (elements with
// (q < nvalid) only; the rest are 0).
template <bool kBf16>
__device__ __forceinline__ u32x4_t gather8_bf16(const void *p, int64_t i0, int64_t stride,
                                               int nvalid) {
  uint32_t e[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) e[q] = (q < nvalid) ? load1_bf16<kBf16>(p, i0 + q * stride) : 0u;
  return u32x4_t{e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16)};
}

// ------------------------------------------------------------ conversions

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

// ------------------------------------------------------------ block scales
// cs[b][row] = q8[row * NB + b] * s2[(row * NB + b) >> 8]  (fp32 product), the
// per-block scales of a quantized [rows x 64 NB] weight laid out one row per
// 64-wide block column (the layout the fused GEMMs stream).  Role of a merged
// launch: workgroups wg = 0 .. nwg-1 of it.
struct ScalesArgs {
  const int8_t *q8;
  const float *s2;
  int64_t rows, NB;
  float *cs;
};

__device__ __forceinline__ void scales_role(const ScalesArgs &a, int64_t wg, int64_t nwg) {
  const int64_t n = a.rows * a.NB;
  for (int64_t i = wg * 256 + threadIdx.x; i < n; i += nwg * 256) {
    const int64_t b = i / a.rows, row = i - b * a.rows;
    const int64_t src = row * a.NB + b;
    a.cs[i] = float(a.q8[src]) * a.s2[src >> 8];
  }
}

// ------------------------------------------------------------------ rowdot
//
// Workgroup: 4 wavefronts x 16 rows = 64 rows of P, all R columns, one
// contiguous K range.  Q is staged per 64-wide K slice in LDS as [RP][64]
// (rows of 128 B, 16-B chunks XOR-swizzled by row) and shared by the 4
// wavefronts; P rows go straight from global memory into the MFMA A operand.

constexpr int kRowdotRows = 64;
constexpr int kSliceK = 64;

struct RowdotArgs {
  const void *P;      // [M x K]
  const void *Q;      // Qt [R x K] (kQt) or Q [K x R]
  int64_t M, K;
  int R;
  int64_t kchunk;     // K range per split (multiple of 64)
  int64_t mt;         // row tiles
  float *part;        // [ks][M][R]
};

template <bool kPbf16, bool kQt, bool kQbf16>
__device__ __forceinline__ void rowdot_role(const RowdotArgs &a, int64_t wg, unsigned char *smem) {
  uint16_t *sQ = reinterpret_cast<uint16_t *>(smem);   // [RP][64]
  const int R = a.R;
  const int RT = (R + 15) / 16;
  const int RP = RT * 16;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int i16 = lane & 15, h = lane >> 4;
  const int64_t m0 = (wg % a.mt) * kRowdotRows;
  const int ks = int(wg / a.mt);
  const int64_t kb = int64_t(ks) * a.kchunk;
  const int64_t ke = min64(a.K, kb + a.kchunk);
  const int64_t row = m0 + wave * 16 + i16;
  const bool row_ok = row < a.M;
  const size_t esz = kPbf16 ? 2 : 4;
  const char *prow = static_cast<const char *>(a.P) + (row_ok ? row : 0) * a.K * esz;

  f32x4_t acc[16];
#pragma unroll
  for (int s = 0; s < 16; ++s) acc[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int64_t k0 = kb; k0 < ke; k0 += kSliceK) {
    // A operands of this slice: substep u covers k0 + 32u + 8h .. +8
    u32x4_t av[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      av[u] = row_ok ? load8_bf16<kPbf16>(prow + (k0 + 32 * u + 8 * h) * esz)
                     : u32x4_t{0u, 0u, 0u, 0u};
    }
    __syncthreads();
    // stage Q for k0..k0+63 as [RP][64]: RP rows x 8 chunks of 8 k
    for (int c = t; c < RP * 8; c += 256) {
      const int j = c >> 3, ch = c & 7;
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (j < R) {
        const int64_t k = k0 + 8 * ch;
        if constexpr (kQt)
          v = load8_bf16<kQbf16>(static_cast<const char *>(a.Q) + (int64_t(j) * a.K + k) * (kQbf16 ? 2 : 4));
        else
          v = gather8_bf16<kQbf16>(a.Q, k * R + j, R, 8);
      }
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
          acc[s] = mfma16x16x32(av[u], b, acc[s]);
        }
      }
    }
  }
  // C layout: lane holds rows 4h..4h+3 of the wave's 16, column i16 of subtile s
  float *out = a.part + int64_t(ks) * a.M * R;
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    if (s < RT) {
      const int j = 16 * s + i16;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t m = m0 + wave * 16 + 4 * h + q;
        if (m < a.M && j < R) out[m * R + j] = acc[s][q];
      }
    }
  }
}

// ------------------------------------------------------------------ coldot
//
// Workgroup: 4 wavefronts x 16 columns of P = 64 columns, all R, one
// contiguous range of tokens.  Per 64-token slice the P tile (64 x 64 bf16)
// is stored row-major in LDS with a 160-byte row pitch (conflict-free for the
// transposed reads) and Q^T (R x 64) with swizzled 16-B chunks.

constexpr int kColdotCols = 64;
constexpr int kPPitch = 80;   // bf16 elements per P row in LDS (160 bytes)

struct ColdotArgs {
  const void *P;      // [M x K]
  const void *Q;      // [M x ldq], columns 0..R-1 used
  int64_t ldq;
  int64_t M, K;
  int R;
  int64_t mchunk;     // tokens per split (multiple of 64)
  int64_t ct;         // column tiles
  float *part;        // [ks][K][R]
};

template <bool kPbf16, bool kQbf16>
__device__ __forceinline__ void coldot_role(const ColdotArgs &a, int64_t wg, unsigned char *smem) {
  uint16_t *sP = reinterpret_cast<uint16_t *>(smem);               // [64][kPPitch]
  uint16_t *sQ = sP + 64 * kPPitch;                                // [RP][64]
  const int R = a.R;
  const int RT = (R + 15) / 16;
  const int RP = RT * 16;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int i16 = lane & 15, h = lane >> 4;
  const int64_t c0 = (wg % a.ct) * kColdotCols;
  const int ks = int(wg / a.ct);
  const int64_t mb = int64_t(ks) * a.mchunk;
  const int64_t me = min64(a.M, mb + a.mchunk);
  const int64_t K = a.K;
  const size_t esz = kPbf16 ? 2 : 4;
  const char *P = static_cast<const char *>(a.P);

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
    // Q^T for tokens mm..mm+63: RP rows x 8 chunks of 8 tokens
    for (int c = t; c < RP * 8; c += 256) {
      const int j = c >> 3, ch = c & 7;
      const int64_t m = mm + 8 * ch;
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (j < R && m < me) {
        const int64_t left = me - m;
        v = gather8_bf16<kQbf16>(a.Q, m * a.ldq + j, a.ldq, left < 8 ? int(left) : 8);
      }
      *reinterpret_cast<u32x4_t *>(sQ + j * 64 + ((ch ^ (j & 7)) * 8)) = v;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      // A operand: column (16*wave + i16) of P, tokens 32u + 8h .. +8, via two
      // transposed reads of 4 rows x 4 columns per 16-lane group.
      u32x4_t av;
      {
        const int q = i16 & 3, tq = i16 >> 2;
        const int rr = 32 * u + 8 * h + tq;
        lds_char *base = (lds_char *)(sP);
        i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4 *)(base + (rr * kPPitch + 16 * wave + 4 * q) * 2));
        i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4 *)(base + ((rr + 4) * kPPitch + 16 * wave + 4 * q) * 2));
        u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
        av = u32x4_t{l2[0], l2[1], h2[0], h2[1]};
      }
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        if (s < RT) {
          const int j = 16 * s + i16;
          const int ch = 4 * u + h;
          u32x4_t b = *reinterpret_cast<const u32x4_t *>(sQ + j * 64 + ((ch ^ (j & 7)) * 8));
          acc[s] = mfma16x16x32(av, b, acc[s]);
        }
      }
    }
  }
  float *out = a.part + int64_t(ks) * K * R;
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
// out[i] = sum over ks of part[k][i] in k order for a [rows x R] result.
// Outputs (each optional): out fp32 ([R x rows] if transpose_out), out_bf16
// [rows x ld_bf16] with zero padding columns R..ld_bf16-1.
struct ReduceArgs {
  const float *part;
  int64_t ks, rows, R;
  float *out;
  bool transpose_out;
  uint16_t *out_bf16;
  int64_t ld_bf16;
};

__device__ __forceinline__ void reduce_role(const ReduceArgs &a, int64_t wg, int64_t nwg) {
  const int64_t n = a.rows * a.R;
  for (int64_t i = wg * 256 + threadIdx.x; i < n; i += nwg * 256) {
    float s = 0.0f;
    for (int64_t k = 0; k < a.ks; ++k) s += a.part[k * n + i];
    const int64_t rr = i / a.R, j = i - rr * a.R;
    if (a.out) a.out[a.transpose_out ? j * a.rows + rr : i] = s;
    if (a.out_bf16) a.out_bf16[rr * a.ld_bf16 + j] = f32_to_bf16_bits(s);
  }
  if (a.out_bf16 && a.ld_bf16 > a.R) {   // zero padding columns R..ld_bf16-1
    const int64_t pad = a.ld_bf16 - a.R, np = a.rows * pad;
    for (int64_t i = wg * 256 + threadIdx.x; i < np; i += nwg * 256) {
      const int64_t rr = i / pad, j = a.R + (i - rr * pad);
      a.out_bf16[rr * a.ld_bf16 + j] = 0;
    }
  }
}

// ------------------------------------------------------------------ kernels

// XA partials (rowdot with Q = A [in x r]) on workgroups [0, n_row), block
// scales on [n_row, grid).  Either role may be empty.
template <bool kXbf16, bool kAbf16>
__global__ __launch_bounds__(256) void fwd_prep_kernel(RowdotArgs ra, int64_t n_row,
                                                       ScalesArgs sa) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int64_t wg = blockIdx.x;
  if (wg < n_row)
    rowdot_role<kXbf16, false, kAbf16>(ra, wg, smem);
  else
    scales_role(sa, wg - n_row, int64_t(gridDim.x) - n_row);
}

// One pass over dY: G partials (rowdot with Qt = B [r x out]) on [0, n_row),
// dB partials (coldot with Q = XA fp32 [M x r]) on [n_row, n_row + n_col),
// block scales on the rest.
template <bool kDYbf16, bool kBbf16>
__global__ __launch_bounds__(256) void bwd_dy_kernel(RowdotArgs ra, int64_t n_row, ColdotArgs ca,
                                                     int64_t n_col, ScalesArgs sa) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int64_t wg = blockIdx.x;
  if (wg < n_row)
    rowdot_role<kDYbf16, true, kBbf16>(ra, wg, smem);
  else if (wg < n_row + n_col)
    coldot_role<kDYbf16, false>(ca, wg - n_row, smem);
  else
    scales_role(sa, wg - n_row - n_col, int64_t(gridDim.x) - n_row - n_col);
}

// One pass over X: dA partials (coldot with Q = G16 bf16 [M x rp]).
template <bool kXbf16>
__global__ __launch_bounds__(256) void bwd_x_kernel(ColdotArgs ca) {
  extern __shared__ __align__(16) unsigned char smem[];
  coldot_role<kXbf16, true>(ca, blockIdx.x, smem);
}

// Two independent reductions in one launch: a on [0, n_a), b on the rest.
__global__ __launch_bounds__(256) void reduce2_kernel(ReduceArgs ra, int64_t n_a, ReduceArgs rb) {
  const int64_t wg = blockIdx.x;
  if (wg < n_a)
    reduce_role(ra, wg, n_a);
  else
    reduce_role(rb, wg - n_a, int64_t(gridDim.x) - n_a);
}

int64_t grid_for(int64_t n) {
  int64_t g = (n + 255) / 256;
  if (g > 2048) g = 2048;
  if (g < 1) g = 1;
  return g;
}

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

RowdotArgs rowdot_args(const void *P, const void *Q, int64_t M, int64_t K, int64_t R,
                       float *part, int64_t &nwg) {
  RowdotArgs a;
  a.P = P; a.Q = Q; a.M = M; a.K = K; a.R = int(R);
  a.kchunk = rowdot_chunk(M, K);
  a.mt = (M + kRowdotRows - 1) / kRowdotRows;
  a.part = part;
  nwg = (M == 0 || R == 0) ? 0 : a.mt * ((K + a.kchunk - 1) / a.kchunk);
  return a;
}

ColdotArgs coldot_args(const void *P, const void *Q, int64_t ldq, int64_t M, int64_t K, int64_t R,
                       float *part, int64_t &nwg) {
  ColdotArgs a;
  a.P = P; a.Q = Q; a.ldq = ldq; a.M = M; a.K = K; a.R = int(R);
  a.mchunk = coldot_chunk(M, K);
  a.ct = (K + kColdotCols - 1) / kColdotCols;
  a.part = part;
  nwg = (M == 0 || R == 0) ? 0 : a.ct * ((M + a.mchunk - 1) / a.mchunk);
  return a;
}

size_t rowdot_lds(int64_t R) { return size_t((R + 15) / 16 * 16) * 64 * 2; }
size_t coldot_lds(int64_t R) { return size_t(64) * kPPitch * 2 + rowdot_lds(R); }

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

hipError_t launch_convert_to_bf16(const void *src, bool src_bf16, int64_t n, uint16_t *dst,
                                  hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(convert_bf16_kernel, dim3(unsigned(grid_for(n))), dim3(256), 0, s, src,
                     src_bf16, n, dst);
  return hipGetLastError();
}

hipError_t launch_fill_zero(float *p, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(unsigned(grid_for(n))), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_fwd_prep(const void *X, bool x_bf16, const void *A, bool a_bf16, int64_t M,
                           int64_t in, int64_t r, float *xa_part, const int8_t *qscale,
                           const float *gscale, int64_t out, float *cs, hipStream_t s) {
  int64_t n_row = 0;
  const RowdotArgs ra = rowdot_args(X, A, M, in, r, xa_part, n_row);
  ScalesArgs sa{qscale, gscale, in, out / 64, cs};
  const int64_t n_sc = cs ? grid_for(in * (out / 64)) : 0;
  if (n_row + n_sc == 0) return hipSuccess;
  const size_t lds = n_row ? rowdot_lds(r) : 0;
  const dim3 grid = dim3(unsigned(n_row + n_sc));
#define QLORA_PREP(XB, AB) \
  hipLaunchKernelGGL((fwd_prep_kernel<XB, AB>), grid, dim3(256), lds, s, ra, n_row, sa)
  if (x_bf16) {
    if (a_bf16) QLORA_PREP(true, true); else QLORA_PREP(true, false);
  } else {
    if (a_bf16) QLORA_PREP(false, true); else QLORA_PREP(false, false);
  }
#undef QLORA_PREP
  return hipGetLastError();
}

hipError_t launch_bwd_dy(const void *dY, bool dy_bf16, const void *B, bool b_bf16,
                         const float *XA, int64_t M, int64_t out, int64_t r, float *g_part,
                         float *db_part, const int8_t *qscale, const float *gscale, int64_t in,
                         float *cs, hipStream_t s) {
  int64_t n_row = 0, n_col = 0;
  const RowdotArgs ra = rowdot_args(dY, B, M, out, r, g_part, n_row);
  const ColdotArgs ca = coldot_args(dY, XA, r, M, out, r, db_part, n_col);
  ScalesArgs sa{qscale, gscale, in, out / 64, cs};
  const int64_t n_sc = cs ? grid_for(in * (out / 64)) : 0;
  if (n_row + n_col + n_sc == 0) return hipSuccess;
  const size_t lds = (n_row + n_col) ? coldot_lds(r) : 0;
  const dim3 grid = dim3(unsigned(n_row + n_col + n_sc));
#define QLORA_DY(DB, BB) \
  hipLaunchKernelGGL((bwd_dy_kernel<DB, BB>), grid, dim3(256), lds, s, ra, n_row, ca, n_col, sa)
  if (dy_bf16) {
    if (b_bf16) QLORA_DY(true, true); else QLORA_DY(true, false);
  } else {
    if (b_bf16) QLORA_DY(false, true); else QLORA_DY(false, false);
  }
#undef QLORA_DY
  return hipGetLastError();
}

hipError_t launch_bwd_x(const void *X, bool x_bf16, const uint16_t *G16, int64_t ldg, int64_t M,
                        int64_t in, int64_t r, float *da_part, hipStream_t s) {
  int64_t n_col = 0;
  const ColdotArgs ca = coldot_args(X, G16, ldg, M, in, r, da_part, n_col);
  if (n_col == 0) return hipSuccess;
  const dim3 grid = dim3(unsigned(n_col));
  if (x_bf16)
    hipLaunchKernelGGL((bwd_x_kernel<true>), grid, dim3(256), coldot_lds(r), s, ca);
  else
    hipLaunchKernelGGL((bwd_x_kernel<false>), grid, dim3(256), coldot_lds(r), s, ca);
  return hipGetLastError();
}

hipError_t launch_reduce2(const float *part_a, int64_t ks_a, int64_t rows_a, int64_t R,
                          float *out_a, bool transpose_a, uint16_t *bf16_a, int64_t ld_a,
                          const float *part_b, int64_t ks_b, int64_t rows_b, float *out_b,
                          bool transpose_b, uint16_t *bf16_b, int64_t ld_b, hipStream_t s) {
  ReduceArgs ra{part_a, ks_a, rows_a, R, out_a, transpose_a, bf16_a, ld_a};
  ReduceArgs rb{part_b, ks_b, rows_b, R, out_b, transpose_b, bf16_b, ld_b};
  const int64_t n_a = part_a ? grid_for(rows_a * (ld_a > R ? ld_a : R)) : 0;
  const int64_t n_b = part_b ? grid_for(rows_b * (ld_b > R ? ld_b : R)) : 0;
  if (n_a + n_b == 0) return hipSuccess;
  hipLaunchKernelGGL(reduce2_kernel, dim3(unsigned(n_a + n_b)), dim3(256), 0, s, ra, n_a, rb);
  return hipGetLastError();
}

}  // namespace qlora
