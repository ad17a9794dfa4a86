// Forward of the adapted linear for a few tokens (M <= 16, decode-shaped):
//   y = X . deq(Wq) + (X . A) . B
// "QLoRA (low-rank adapters on a quantized model)", "How it works" (forward
// with W = Wq + A B) and "What QLoRA adds" (4-bit weights expanded to bf16
// for each matmul).  With a handful of tokens the layer is bound by the HBM
// read of the packed codes (half a byte per weight), so the work is split
// over K as well as N to put every CU on the stream, and reduced in a second
// launch in a fixed order.
//
// Pass 1 (grid: 256-column slices x K chunks, 4 wavefronts): wavefront w owns
// the 64 columns n0 + 64 w .. +63, i.e. one block column, so the scale of a
// weight depends on its k row only and is applied to the activation instead:
//   y[m][n] = sum_k bf16(X[m][k] * c(k)) * bf16(L[code(k, n)])
// with c(k) = q_b * s2_g (fp32).  The codes of a wavefront (rows x 32 B) go
// to LDS and come back with ds_read_b64_tr_b4, which hands lane i of a
// 16-lane group column i of 16 consecutive k rows: the k run of one MFMA
// operand lane.  Codes expand to bf16 levels through two v_perm byte planes
// (sign-symmetric level set: 8 magnitudes).  v_mfma_f32_16x16x32_bf16 runs
// with the tokens as its 16 rows (rows >= M are zero).  Workgroups of slice 0
// also accumulate the chunk's X . A (unscaled X, A staged in LDS and read
// transposed).  Partials: P[chunk][m][n] and PXA[chunk][m][j], fp32.
// Pass 2: XA = sum over chunks of PXA (written out), y = sum of P + XA . B.
#include "device.h"

namespace qlora {
namespace {

typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i32x2_t lds_i32x2;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
typedef __attribute__((address_space(3))) char lds_char;

constexpr int kThreads = 256;
constexpr int kSliceN = 256;            // columns per workgroup (4 block columns)
constexpr int kSub = 128;               // k rows per LDS sub-chunk
constexpr int kCodePitch = 40;          // bytes per k row of a wavefront's code tile
constexpr int kXPitchS = kSub + 4;      // fp32 per X row in LDS
constexpr int kAPitch = kSmallMaxR + 8; // bf16 per A row in LDS
constexpr int32_t kBufFlags = 0x00020000;

struct SmallArgs {
  const uint8_t *codes;
  const int8_t *qscale;
  const float *gscale;
  int64_t K, N;          // in, out
  const void *X;         // [M x K]
  const void *A;         // [K x r]
  int64_t M, r;
  int64_t Kc;            // rows per K chunk (multiple of 64)
  float *P;              // [KS][M][N]
  float *PXA;            // [KS][M][r]
};

__device__ __forceinline__ float load_act(const void *p, int64_t i, bool bf16) {
  if (bf16) return __uint_as_float(uint32_t(static_cast<const uint16_t *>(p)[i]) << 16);
  return static_cast<const float *>(p)[i];
}

// 8 codes (nibble t of d = k row t of the lane's run) -> four bf16 pairs of
// levels, in the k order (0,2) (4,6) (1,3) (5,7); the activation operand is
// packed in the same order.
__device__ __forceinline__ u32x4_t expand_levels(uint32_t d, const ExpandConsts16 &T) {
  const uint32_t u = d ^ 0x88888888u;                 // c >= 8 -> c - 8; c < 8 -> c + 8
  const uint32_t neg = u & 0x88888888u;               // nibble bit 3: negative level
  const uint32_t m = (u ^ (neg - (neg >> 3))) & 0x77777777u;   // magnitude index 0..7
  const uint32_t ml = m & 0x07070707u, mh = (m >> 4) & 0x07070707u;
  const uint32_t LL = perm_b32(T.plane[0][1], T.plane[0][0], ml);   // low bytes, even rows
  const uint32_t HL = perm_b32(T.plane[1][1], T.plane[1][0], ml) | ((neg << 4) & 0x80808080u);
  const uint32_t LH = perm_b32(T.plane[0][1], T.plane[0][0], mh);   // odd rows
  const uint32_t HH = perm_b32(T.plane[1][1], T.plane[1][0], mh) | (neg & 0x80808080u);
  u32x4_t r;
  r[0] = perm_b32(HL, LL, 0x05010400u);   // rows 0, 2
  r[1] = perm_b32(HL, LL, 0x07030602u);   // rows 4, 6
  r[2] = perm_b32(HH, LH, 0x05010400u);   // rows 1, 3
  r[3] = perm_b32(HH, LH, 0x07030602u);   // rows 5, 7
  return r;
}

template <bool kX16, bool kA16>
__global__ __launch_bounds__(kThreads) void fwd_small_kernel(SmallArgs a, ExpandConsts16 t16) {
  __shared__ __attribute__((aligned(16))) float xs[16][kXPitchS];
  __shared__ __attribute__((aligned(16))) float cs[4][kSub];
  __shared__ __attribute__((aligned(16))) uint8_t ct[4][kSub * kCodePitch];
  __shared__ __attribute__((aligned(16))) uint16_t as[kSub][kAPitch];

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, g = lane >> 4, i = lane & 15;
  const int64_t n0 = int64_t(blockIdx.x) * kSliceN;
  const int c = blockIdx.y;
  const int64_t kbeg = int64_t(c) * a.Kc;
  const int64_t kend = min64(kbeg + a.Kc, a.K);
  const int64_t nblk = a.N / 64, blk = n0 / 64 + wave;   // this wavefront's block column
  const bool blk_ok = blk < nblk;
  const int64_t half_n = a.N / 2;
  const bool xa_tile = blockIdx.x == 0 && 16 * wave < a.r;   // X . A column tile `wave`

  f32x4_t acc[4], xacc;
#pragma unroll
  for (int q = 0; q < 4; ++q) acc[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  xacc = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // codes of this wavefront's block column, rows kbeg .. kend
  const int64_t cbase = kbeg * half_n + n0 / 2 + 32 * wave;
  const int64_t cbytes = (kend - kbeg) * half_n - (n0 / 2 + 32 * wave);
  const __amdgpu_buffer_rsrc_t rC = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(a.codes + cbase), (short)0, int32_t(cbytes > 0x7fffffff ? 0x7fffffff : cbytes),
      kBufFlags);

  for (int64_t kb = kbeg; kb < kend; kb += kSub) {
    const int rows = int(min64(kSub, kend - kb));        // multiple of 64
    // ---- issue the code loads: 2 lanes per row, 32 rows per instruction
    u32x4_t cv[kSub / 32];
#pragma unroll
    for (int it = 0; it < kSub / 32; ++it) {
      const int row = (lane >> 1) + 32 * it;
      const uint32_t off = uint32_t((kb - kbeg + row) * half_n) + 16u * uint32_t(lane & 1);
      cv[it] = row < rows ? __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rC, off, 0, 2))
                          : u32x4_t{0u, 0u, 0u, 0u};
    }
    // ---- activations [16][kSub] fp32 (rows >= M and k >= kend are zero)
    {
      const int m = t >> 4, k8 = (t & 15) * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int64_t k = kb + k8 + e;
        xs[m][k8 + e] = (m < a.M && k < kend) ? load_act(a.X, int64_t(m) * a.K + k, kX16) : 0.0f;
      }
    }
    // ---- block scales of this wavefront's block column
#pragma unroll
    for (int e = 0; e < kSub / 64; ++e) {
      const int kk = lane + 64 * e;
      const int64_t k = kb + kk;
      float s = 0.0f;
      if (blk_ok && kk < rows) {
        const int64_t b = k * nblk + blk;
        s = float(a.qscale[b]) * a.gscale[b >> 8];
      }
      cs[wave][kk] = s;
    }
    // ---- adapter A rows of this sub-chunk (slice 0 only), as bf16
    if (blockIdx.x == 0 && a.r > 0) {
      for (int e = t; e < kSub * a.r; e += kThreads) {
        const int kk = e / int(a.r), j = e % int(a.r);
        const int64_t k = kb + kk;
        const float v = (kk < rows) ? load_act(a.A, k * a.r + j, kA16) : 0.0f;
        as[kk][j] = __builtin_bit_cast(uint16_t, (__bf16)v);
      }
    }
    // ---- codes to this wavefront's LDS tile (read back only by this wavefront)
#pragma unroll
    for (int it = 0; it < kSub / 32; ++it) {
      const int row = (lane >> 1) + 32 * it;
      uint8_t *dst = &ct[wave][row * kCodePitch + 16 * (lane & 1)];
      *reinterpret_cast<u32x2_t *>(dst) = u32x2_t{cv[it][0], cv[it][1]};
      *reinterpret_cast<u32x2_t *>(dst + 8) = u32x2_t{cv[it][2], cv[it][3]};
    }
    __syncthreads();

    for (int rb = 0; rb < rows; rb += 64) {
      // activation operand: X[m = i][rb + 16 g + 0..15] times the row scales
      float xv[16], sv[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4_t x4 = *reinterpret_cast<const f32x4_t *>(&xs[i][rb + 16 * g + 4 * q]);
        const f32x4_t s4 = *reinterpret_cast<const f32x4_t *>(&cs[wave][rb + 16 * g + 4 * q]);
        xv[4 * q] = x4.x; xv[4 * q + 1] = x4.y; xv[4 * q + 2] = x4.z; xv[4 * q + 3] = x4.w;
        sv[4 * q] = s4.x; sv[4 * q + 1] = s4.y; sv[4 * q + 2] = s4.z; sv[4 * q + 3] = s4.w;
      }
      u32x4_t A1, A2;
      A1[0] = pack_bf16x2(xv[0] * sv[0], xv[2] * sv[2]);
      A1[1] = pack_bf16x2(xv[4] * sv[4], xv[6] * sv[6]);
      A1[2] = pack_bf16x2(xv[1] * sv[1], xv[3] * sv[3]);
      A1[3] = pack_bf16x2(xv[5] * sv[5], xv[7] * sv[7]);
      A2[0] = pack_bf16x2(xv[8] * sv[8], xv[10] * sv[10]);
      A2[1] = pack_bf16x2(xv[12] * sv[12], xv[14] * sv[14]);
      A2[2] = pack_bf16x2(xv[9] * sv[9], xv[11] * sv[11]);
      A2[3] = pack_bf16x2(xv[13] * sv[13], xv[15] * sv[15]);
      // weight operand: lane (g, i) <- column 16 q + i, rows rb + 16 g + 0..15
      const lds_char *crow = (const lds_char *)(&ct[wave][(rb + 16 * g + i) * kCodePitch]);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const i32x2_t d = __builtin_amdgcn_ds_read_tr4_b64_v2i32((lds_i32x2 *)(crow + 8 * q));
        acc[q] = mfma16x16x32(A1, expand_levels(uint32_t(d[0]), t16), acc[q]);
        acc[q] = mfma16x16x32(A2, expand_levels(uint32_t(d[1]), t16), acc[q]);
      }
      if (xa_tile) {
        // X . A for columns 16 wave .. +15, natural k order
        u32x4_t U1, U2, B1, B2;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          U1[p] = pack_bf16x2(xv[2 * p], xv[2 * p + 1]);
          U2[p] = pack_bf16x2(xv[8 + 2 * p], xv[9 + 2 * p]);
        }
        const int tq = i >> 2, qq = i & 3;
        const lds_char *ab = (const lds_char *)(&as[0][0]);
        const int col = 16 * wave + 4 * qq;
        const i16x4_t r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4 *)(ab + ((rb + 16 * g + tq) * kAPitch + col) * 2));
        const i16x4_t r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4 *)(ab + ((rb + 16 * g + 4 + tq) * kAPitch + col) * 2));
        const i16x4_t r2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4 *)(ab + ((rb + 16 * g + 8 + tq) * kAPitch + col) * 2));
        const i16x4_t r3 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4 *)(ab + ((rb + 16 * g + 12 + tq) * kAPitch + col) * 2));
        const u32x2_t w0 = __builtin_bit_cast(u32x2_t, r0), w1 = __builtin_bit_cast(u32x2_t, r1);
        const u32x2_t w2 = __builtin_bit_cast(u32x2_t, r2), w3 = __builtin_bit_cast(u32x2_t, r3);
        B1 = u32x4_t{w0[0], w0[1], w1[0], w1[1]};
        B2 = u32x4_t{w2[0], w2[1], w3[0], w3[1]};
        xacc = mfma16x16x32(U1, B1, xacc);
        xacc = mfma16x16x32(U2, B2, xacc);
      }
    }
    __syncthreads();   // LDS tiles are rewritten by the next sub-chunk
  }

  // ---- partials: lane (g, i) holds rows 4 g .. 4 g + 3 of column 16 q + i
  float *P = a.P + int64_t(c) * a.M * a.N;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t n = n0 + 64 * wave + 16 * q + i;
    if (!blk_ok || n >= a.N) continue;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = 4 * g + e;
      if (m < a.M) P[int64_t(m) * a.N + n] = acc[q][e];
    }
  }
  if (xa_tile) {
    float *PX = a.PXA + int64_t(c) * a.M * a.r;
    const int j = 16 * wave + i;
    if (j < a.r) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = 4 * g + e;
        if (m < a.M) PX[int64_t(m) * a.r + j] = xacc[e];
      }
    }
  }
}

// Pass 2: 64 columns per workgroup, thread (m-group, column).
template <bool kY16, bool kB16>
__global__ __launch_bounds__(kThreads) void fwd_small_reduce_kernel(
    const float *__restrict__ P, const float *__restrict__ PXA, int64_t KS, int64_t M, int64_t N,
    int64_t r, const void *B, float *XA, void *Y) {
  __shared__ float xa[16][kSmallMaxR];
  const int t = threadIdx.x;
  // XA = sum over chunks of PXA, fixed order
  for (int e = t; e < M * r; e += kThreads) {
    float s = 0.0f;
    for (int64_t k = 0; k < KS; ++k) s += PXA[k * M * r + e];
    xa[e / r][e % r] = s;
    if (blockIdx.x == 0) XA[e] = s;
  }
  __syncthreads();
  const int64_t n = int64_t(blockIdx.x) * 64 + (t & 63);
  if (n >= N) return;
  for (int m = t >> 6; m < M; m += 4) {
    float s = 0.0f;
    for (int64_t k = 0; k < KS; ++k) s += P[(k * M + m) * N + n];
    float u = 0.0f;
    for (int j = 0; j < r; ++j) u += xa[m][j] * load_act(B, int64_t(j) * N + n, kB16);
    const float y = s + u;
    if (kY16)
      static_cast<uint16_t *>(Y)[int64_t(m) * N + n] = __builtin_bit_cast(uint16_t, (__bf16)y);
    else
      static_cast<float *>(Y)[int64_t(m) * N + n] = y;
  }
}

}  // namespace

int64_t small_fwd_chunk_rows(int64_t M, int64_t K, int64_t N) {
  const int64_t slices = (N + kSliceN - 1) / kSliceN;
  const int64_t target = M <= 4 ? 512 : (M <= 8 ? 256 : 128);
  int64_t ks = (target + slices - 1) / slices;
  ks = ks < 1 ? 1 : (ks > K / 64 ? K / 64 : ks);
  return ((K + ks - 1) / ks + 63) / 64 * 64;
}

hipError_t launch_fwd_small_partial(const uint8_t *codes, const int8_t *qscale,
                                    const float *gscale, int64_t K, int64_t N, const void *X,
                                    bool x_bf16, int64_t M, const void *A, bool a_bf16, int64_t r,
                                    int64_t Kc, float *P, float *PXA, hipStream_t s) {
  const int64_t KS = (K + Kc - 1) / Kc;
  const int64_t slices = (N + kSliceN - 1) / kSliceN;
  SmallArgs a{codes, qscale, gscale, K, N, X, A, M, r, Kc, P, PXA};
  const ExpandConsts16 &t16 = tables().expand16;
  const dim3 grid = dim3(unsigned(slices), unsigned(KS));
  if (x_bf16) {
    if (a_bf16) hipLaunchKernelGGL((fwd_small_kernel<true, true>), grid, dim3(kThreads), 0, s, a, t16);
    else hipLaunchKernelGGL((fwd_small_kernel<true, false>), grid, dim3(kThreads), 0, s, a, t16);
  } else {
    if (a_bf16) hipLaunchKernelGGL((fwd_small_kernel<false, true>), grid, dim3(kThreads), 0, s, a, t16);
    else hipLaunchKernelGGL((fwd_small_kernel<false, false>), grid, dim3(kThreads), 0, s, a, t16);
  }
  return hipGetLastError();
}

hipError_t launch_fwd_small_reduce(const float *P, const float *PXA, int64_t KS, int64_t M,
                                   int64_t N, int64_t r, const void *B, bool b_bf16, float *XA,
                                   void *Y, bool y_bf16, hipStream_t s) {
  const dim3 grid = dim3(unsigned((N + 63) / 64));
  if (y_bf16) {
    if (b_bf16) hipLaunchKernelGGL((fwd_small_reduce_kernel<true, true>), grid, dim3(kThreads), 0, s, P, PXA, KS, M, N, r, B, XA, Y);
    else hipLaunchKernelGGL((fwd_small_reduce_kernel<true, false>), grid, dim3(kThreads), 0, s, P, PXA, KS, M, N, r, B, XA, Y);
  } else {
    if (b_bf16) hipLaunchKernelGGL((fwd_small_reduce_kernel<false, true>), grid, dim3(kThreads), 0, s, P, PXA, KS, M, N, r, B, XA, Y);
    else hipLaunchKernelGGL((fwd_small_reduce_kernel<false, false>), grid, dim3(kThreads), 0, s, P, PXA, KS, M, N, r, B, XA, Y);
  }
  return hipGetLastError();
}

}  // namespace qlora
