// Fused dequantizing GEMMs of the adapted linear layer on bf16 matrix cores.
//
//   forward  y  = X . deq(Wq) + XA . B          (contraction over `in`)
//   backward dX = dY . deq(Wq)^T + G . A^T      (contraction over `out`)
//
// "QLoRA (low-rank adapters on a quantized model)", "What QLoRA adds": the
// frozen 4-bit weights are expanded to bf16 on the fly for each matmul and
// never updated; "How it works": W = Wq + A B with the rank-r term added as
// "one small extra matmul".  Here that extra matmul runs on the same
// accumulators after the main K loop.
//
// Tiling (both kernels): workgroup 256 threads = 4 wavefronts in 2 x 2, tile
// 256 (M) x 128 (N) x 64 (K); each wavefront owns 128 x 64 of the output as
// 8 x 4 tiles of v_mfma_f32_16x16x32_bf16.  X / dY tiles are staged in LDS
// (16-B chunks XOR-swizzled, double-buffered); the weight tile is staged as
// raw packed codes (1/4 of the bf16 bytes) and expanded in registers:
//   w = bf16(L[code] * (q_b * s2_g)), L looked up with v_perm byte planes.
// K slots are permuted inside each 64-wide K tile: lane group h of the MFMA
// owns k = 16h .. 16h+15 (8 per substep), for both operands.
//
// Forward: the code tile is (64 k-rows) x (128 n-cols) nibbles, n-contiguous;
// ds_read_b64_tr_b4 hands lane i of a 16-lane group column i of the 16 rows
// the group points at, i.e. 16 consecutive k of one column, in one read.
// Every wavefront's 64 columns form one 64-wide scale block, so its scales
// depend on k only (16 per lane per K tile).
// Backward dX: the code tile is (128 W-rows) x (64 W-cols); the contraction
// runs along a W row, so a plain 8-byte read gives 16 consecutive k, and the
// K tile is one scale block, so each W row has a single scale per tile.
#include "device.h"

namespace qlora {
namespace {

typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2_t lds_i32x2;
typedef __attribute__((address_space(3))) char lds_char;

constexpr int BM = 256, BN = 128, BK = 64;
constexpr int kThreads = 256;
constexpr int kFwdCodePitch = 72;   // bytes per k-row of the forward code tile
constexpr int kDxCodePitch = 40;    // bytes per W-row of the dX code tile

__device__ __forceinline__ uint16_t bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// 8 codes (nibble t = k slot t) times per-slot scales -> MFMA bf16 operand.
__device__ __forceinline__ u32x4_t expand8(uint32_t d, const float *s, const ExpandConsts &tb) {
  float le[4], lo[4];
  lookup4(d & 0x0F0F0F0Fu, tb, le);
  lookup4((d >> 4) & 0x0F0F0F0Fu, tb, lo);
  u32x4_t r;
  r[0] = pack_bf16x2(le[0] * s[0], lo[0] * s[1]);
  r[1] = pack_bf16x2(le[1] * s[2], lo[1] * s[3]);
  r[2] = pack_bf16x2(le[2] * s[4], lo[2] * s[5]);
  r[3] = pack_bf16x2(le[3] * s[6], lo[3] * s[7]);
  return r;
}

// Same with one scale for all 8 slots.
__device__ __forceinline__ u32x4_t expand8u(uint32_t d, float s, const ExpandConsts &tb) {
  float le[4], lo[4];
  lookup4(d & 0x0F0F0F0Fu, tb, le);
  lookup4((d >> 4) & 0x0F0F0F0Fu, tb, lo);
  u32x4_t r;
  r[0] = pack_bf16x2(le[0] * s, lo[0] * s);
  r[1] = pack_bf16x2(le[1] * s, lo[1] * s);
  r[2] = pack_bf16x2(le[2] * s, lo[2] * s);
  r[3] = pack_bf16x2(le[3] * s, lo[3] * s);
  return r;
}

template <bool kBf16>
__device__ __forceinline__ u32x4_t load8(const void *base, int64_t idx) {
  if constexpr (kBf16) {
    return *reinterpret_cast<const u32x4_t *>(static_cast<const uint16_t *>(base) + idx);
  } else {
    const float4 *q = reinterpret_cast<const float4 *>(static_cast<const float *>(base) + idx);
    float4 a = q[0], b = q[1];
    return u32x4_t{pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w), pack_bf16x2(b.x, b.y),
                   pack_bf16x2(b.z, b.w)};
  }
}

// Map the linear workgroup id to a (m-tile, n-tile): workgroups are dealt to
// the 8 XCDs round-robin, so tile index T = (id % 8) * (n / 8) + id / 8 gives
// each XCD a contiguous run of tiles sharing m-tiles (and their X rows in the
// XCD's L2).
__device__ __forceinline__ void tile_of(int nt_count, int &mt, int &nt) {
  const int n = gridDim.x, id = blockIdx.x;
  const int T = (n % 8 == 0) ? (id % 8) * (n / 8) + id / 8 : id;
  mt = T / nt_count;
  nt = T % nt_count;
}

// ---------------------------------------------------------------- A staging
// BM x BK tile of a row-major [M x K] activation into LDS, bf16, 16-B chunks
// at position (c ^ (row & 7)).  Thread t loads rows t/8 + 32j, chunk t%8.
template <bool kBf16>
__device__ __forceinline__ void load_a_tile(const void *Av, int64_t M, int64_t K, int64_t m0,
                                            int64_t k0, u32x4_t (&reg)[8]) {
  const int t = threadIdx.x;
  const int c = t & 7;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int row = (t >> 3) + 32 * j;
    const int64_t gm = m0 + row;
    reg[j] = (gm < M) ? load8<kBf16>(Av, gm * K + k0 + 8 * c) : u32x4_t{0u, 0u, 0u, 0u};
  }
}

__device__ __forceinline__ void store_a_tile(uint16_t *sA, const u32x4_t (&reg)[8]) {
  const int t = threadIdx.x;
  const int c = t & 7;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int row = (t >> 3) + 32 * j;
    *reinterpret_cast<u32x4_t *>(sA + row * BK + ((c ^ (row & 7)) * 8)) = reg[j];
  }
}

__device__ __forceinline__ u32x4_t read_a_frag(const uint16_t *sA, int row, int chunk) {
  return *reinterpret_cast<const u32x4_t *>(sA + row * BK + ((chunk ^ (row & 7)) * 8));
}

template <bool kBf16>
__device__ __forceinline__ void store_out(void *Yv, int64_t M, int64_t N, int64_t m, int64_t n,
                                          float v) {
  if (m < M && n < N) {
    if constexpr (kBf16)
      static_cast<uint16_t *>(Yv)[m * N + n] = bf16_bits(v);
    else
      static_cast<float *>(Yv)[m * N + n] = v;
  }
}

// ================================================================ forward
template <bool kXbf16>
__global__ __launch_bounds__(kThreads, 1) void fwd_gemm_kernel(
    const uint8_t *__restrict__ codes, const int8_t *__restrict__ q8,
    const float *__restrict__ s2, int64_t K, int64_t N, const void *__restrict__ X, int64_t M,
    const float *__restrict__ XA, const uint16_t *__restrict__ Bt, int r, int rp,
    void *__restrict__ Y, ExpandConsts tb, int nt_count) {
  __shared__ __align__(16) uint16_t sX[2][BM * BK];
  __shared__ __align__(16) uint8_t sC[2][BK * kFwdCodePitch];
  __shared__ __align__(16) float sS[2][2 * BK];

  int mt, nt;
  tile_of(nt_count, mt, nt);
  const int64_t m0 = int64_t(mt) * BM, n0 = int64_t(nt) * BN;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int i16 = lane & 15, h = lane >> 4;
  const int64_t N2 = N / 2, NB = N / 64;
  const int KT = int(K / BK);

  f32x4_t acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int s = 0; s < 4; ++s) acc[i][s] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // staging registers
  u32x4_t ra[8];
  u32x4_t rc;
  float rs = 0.f;
  const int c_row = t >> 2, c_piece = t & 3;          // code tile: 64 rows x 4 x 16 B
  const bool c_ok = n0 + 32 * (c_piece + 1) <= N;
  const int s_kk = t & 63, s_j = (t >> 6) & 1;        // scales: threads 0..127
  const bool s_ok = (t < 128) && (n0 / 64 + s_j < NB);

  auto load_tile = [&](int kt) {
    const int64_t k0 = int64_t(kt) * BK;
    load_a_tile<kXbf16>(X, M, K, m0, k0, ra);
    rc = c_ok ? *reinterpret_cast<const u32x4_t *>(codes + (k0 + c_row) * N2 + n0 / 2 +
                                                   16 * c_piece)
              : u32x4_t{0u, 0u, 0u, 0u};
    if (s_ok) {
      const int64_t b = (k0 + s_kk) * NB + n0 / 64 + s_j;
      rs = float(q8[b]) * s2[b >> 8];
    } else {
      rs = 0.f;
    }
  };
  auto store_tile = [&](int buf) {
    store_a_tile(sX[buf], ra);
    uint8_t *cdst = sC[buf] + c_row * kFwdCodePitch + 16 * c_piece;
    *reinterpret_cast<u32x2_t *>(cdst) = u32x2_t{rc[0], rc[1]};
    *reinterpret_cast<u32x2_t *>(cdst + 8) = u32x2_t{rc[2], rc[3]};
    if (t < 128) sS[buf][s_j * BK + s_kk] = rs;
  };

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) load_tile(kt + 1);

    // weight operands: 4 column groups of 16, 16 consecutive k each
    uint32_t nib[4][2];
    lds_char *cbase = (lds_char *)(sC[buf]);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      i32x2_t v = __builtin_amdgcn_ds_read_tr4_b64_v2i32((lds_i32x2 *)(
          cbase + (16 * h + i16) * kFwdCodePitch + 32 * wn + 8 * s));
      nib[s][0] = uint32_t(v[0]);
      nib[s][1] = uint32_t(v[1]);
    }
    float sc[16];
    {
      const float4 *sp = reinterpret_cast<const float4 *>(&sS[buf][wn * BK + 16 * h]);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float4 v = sp[q];
        sc[4 * q + 0] = v.x;
        sc[4 * q + 1] = v.y;
        sc[4 * q + 2] = v.z;
        sc[4 * q + 3] = v.w;
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      u32x4_t bop[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) bop[s] = expand8(nib[s][u], sc + 8 * u, tb);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const u32x4_t a = read_a_frag(sX[buf], 128 * wm + 16 * i + i16, 2 * h + u);
#pragma unroll
        for (int s = 0; s < 4; ++s) acc[i][s] = mfma16x16x32(a, bop[s], acc[i][s]);
      }
    }
    if (kt + 1 < KT) store_tile(buf ^ 1);
    __syncthreads();
  }

  // rank-r term: acc += bf16(XA) . bf16(B), B read transposed (Bt [N x rp])
  for (int r0 = 0; r0 < rp; r0 += 32) {
    u32x4_t bop[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int64_t n = n0 + 64 * wn + 16 * s + i16;
      bop[s] = (n < N) ? *reinterpret_cast<const u32x4_t *>(Bt + n * rp + r0 + 8 * h)
                       : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t m = m0 + 128 * wm + 16 * i + i16;
      float v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int j = r0 + 8 * h + q;
        v[q] = (m < M && j < r) ? XA[m * r + j] : 0.f;
      }
      const u32x4_t a = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                         pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
#pragma unroll
      for (int s = 0; s < 4; ++s) acc[i][s] = mfma16x16x32(a, bop[s], acc[i][s]);
    }
  }

#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        store_out<kXbf16>(Y, M, N, m0 + 128 * wm + 16 * i + 4 * h + q,
                          n0 + 64 * wn + 16 * s + i16, acc[i][s][q]);
}

// ================================================================ dX
template <bool kYbf16, bool kAbf16>
__global__ __launch_bounds__(kThreads, 1) void dx_gemm_kernel(
    const uint8_t *__restrict__ codes, const int8_t *__restrict__ q8,
    const float *__restrict__ s2, int64_t IN, int64_t OUT, const void *__restrict__ dY,
    int64_t M, const uint16_t *__restrict__ G16, int rp, const void *__restrict__ A, int r,
    void *__restrict__ dX, ExpandConsts tb, int nt_count) {
  __shared__ __align__(16) uint16_t sY[2][BM * BK];
  __shared__ __align__(16) uint8_t sC[2][BN * kDxCodePitch];
  __shared__ __align__(16) float sS[2][BN];

  int mt, nt;
  tile_of(nt_count, mt, nt);
  const int64_t m0 = int64_t(mt) * BM, i0 = int64_t(nt) * BN;   // i: W row = dX column
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int i16 = lane & 15, h = lane >> 4;
  const int64_t OUT2 = OUT / 2, OB = OUT / 64;
  const int KT = int(OUT / BK);

  f32x4_t acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int s = 0; s < 4; ++s) acc[i][s] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  u32x4_t ra[8];
  u32x4_t rc;
  float rs = 0.f;
  const int c_row = t >> 1, c_piece = t & 1;          // code tile: 128 rows x 2 x 16 B
  const bool c_ok = i0 + c_row < IN;
  const bool s_ok = (t < 128) && (i0 + t < IN);

  auto load_tile = [&](int kt) {
    const int64_t k0 = int64_t(kt) * BK;
    load_a_tile<kYbf16>(dY, M, OUT, m0, k0, ra);
    rc = c_ok ? *reinterpret_cast<const u32x4_t *>(codes + (i0 + c_row) * OUT2 + k0 / 2 +
                                                   16 * c_piece)
              : u32x4_t{0u, 0u, 0u, 0u};
    if (s_ok) {
      const int64_t b = (i0 + t) * OB + k0 / 64;
      rs = float(q8[b]) * s2[b >> 8];
    } else {
      rs = 0.f;
    }
  };
  auto store_tile = [&](int buf) {
    store_a_tile(sY[buf], ra);
    uint8_t *cdst = sC[buf] + c_row * kDxCodePitch + 16 * c_piece;
    *reinterpret_cast<u32x2_t *>(cdst) = u32x2_t{rc[0], rc[1]};
    *reinterpret_cast<u32x2_t *>(cdst + 8) = u32x2_t{rc[2], rc[3]};
    if (t < 128) sS[buf][t] = rs;
  };

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) load_tile(kt + 1);

    uint32_t nib[4][2];
    float sc[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int wr = 64 * wn + 16 * s + i16;
      const u32x2_t v = *reinterpret_cast<const u32x2_t *>(sC[buf] + wr * kDxCodePitch + 8 * h);
      nib[s][0] = v[0];
      nib[s][1] = v[1];
      sc[s] = sS[buf][wr];
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      u32x4_t bop[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) bop[s] = expand8u(nib[s][u], sc[s], tb);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const u32x4_t a = read_a_frag(sY[buf], 128 * wm + 16 * i + i16, 2 * h + u);
#pragma unroll
        for (int s = 0; s < 4; ++s) acc[i][s] = mfma16x16x32(a, bop[s], acc[i][s]);
      }
    }
    if (kt + 1 < KT) store_tile(buf ^ 1);
    __syncthreads();
  }

  // rank-r term: acc += G . A^T, G bf16 [M x rp] (zero padded), A [IN x r]
  for (int r0 = 0; r0 < rp; r0 += 32) {
    u32x4_t bop[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int64_t i = i0 + 64 * wn + 16 * s + i16;
      float v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int j = r0 + 8 * h + q;
        float x = 0.f;
        if (i < IN && j < r) {
          if constexpr (kAbf16)
            x = __uint_as_float(uint32_t(static_cast<const uint16_t *>(A)[i * r + j]) << 16);
          else
            x = static_cast<const float *>(A)[i * r + j];
        }
        v[q] = x;
      }
      bop[s] = u32x4_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                       pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t m = m0 + 128 * wm + 16 * i + i16;
      const u32x4_t a = (m < M) ? *reinterpret_cast<const u32x4_t *>(G16 + m * rp + r0 + 8 * h)
                                : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
      for (int s = 0; s < 4; ++s) acc[i][s] = mfma16x16x32(a, bop[s], acc[i][s]);
    }
  }

#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        store_out<kYbf16>(dX, M, IN, m0 + 128 * wm + 16 * i + 4 * h + q,
                          i0 + 64 * wn + 16 * s + i16, acc[i][s][q]);
}

}  // namespace

hipError_t launch_fwd_gemm(const uint8_t *codes, const int8_t *qscale, const float *gscale,
                           int64_t K, int64_t N, const void *X, bool x_bf16, int64_t M,
                           const float *XA, const uint16_t *Bt, int32_t r, void *Y,
                           hipStream_t s) {
  if (M == 0) return hipSuccess;
  const int mtc = int((M + BM - 1) / BM), ntc = int((N + BN - 1) / BN);
  const int rp = r > 0 ? int((r + 31) / 32 * 32) : 0;
  dim3 grid(unsigned(mtc * ntc));
  const ExpandConsts tb = tables().expand;
  if (x_bf16)
    hipLaunchKernelGGL(fwd_gemm_kernel<true>, grid, dim3(kThreads), 0, s, codes, qscale, gscale,
                       K, N, X, M, XA, Bt, int(r), rp, Y, tb, ntc);
  else
    hipLaunchKernelGGL(fwd_gemm_kernel<false>, grid, dim3(kThreads), 0, s, codes, qscale,
                       gscale, K, N, X, M, XA, Bt, int(r), rp, Y, tb, ntc);
  return hipGetLastError();
}

hipError_t launch_dx_gemm(const uint8_t *codes, const int8_t *qscale, const float *gscale,
                          int64_t in, int64_t out, const void *dY, bool dy_bf16, int64_t M,
                          const uint16_t *G16, const void *A, bool a_bf16, int32_t r, void *dX,
                          hipStream_t s) {
  if (M == 0) return hipSuccess;
  const int mtc = int((M + BM - 1) / BM), ntc = int((in + BN - 1) / BN);
  const int rp = r > 0 ? int((r + 31) / 32 * 32) : 0;
  dim3 grid(unsigned(mtc * ntc));
  const ExpandConsts tb = tables().expand;
#define QLORA_DX(YB, AB)                                                                       \
  hipLaunchKernelGGL((dx_gemm_kernel<YB, AB>), grid, dim3(kThreads), 0, s, codes, qscale,     \
                     gscale, in, out, dY, M, G16, rp, A, int(r), dX, tb, ntc)
  if (dy_bf16 && a_bf16)
    QLORA_DX(true, true);
  else if (dy_bf16)
    QLORA_DX(true, false);
  else if (a_bf16)
    QLORA_DX(false, true);
  else
    QLORA_DX(false, false);
#undef QLORA_DX
  return hipGetLastError();
}

}  // namespace qlora
