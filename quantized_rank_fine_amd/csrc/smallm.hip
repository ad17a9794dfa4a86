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
// with the tokens as its 16 rows (rows >= M are zero).  A chunk of K is
// walked in sub-chunks of 128 rows; the loads of the next sub-chunk are in
// flight while the current one is multiplied.  One extra column of
// workgroups accumulates each chunk's X . A (unscaled X, A staged in LDS and
// read transposed).  Partials: P[chunk][m][n] and PXA[chunk][m][j], fp32.
// Pass 2: XA = sum over chunks of PXA (written out), y = sum of P + XA . B.
//
// The lab's 16-entry format (one fp32 scale per 16 consecutive weights, no
// double quantization) takes the same route with one scale per (k row,
// 16-column MFMA tile q): the activation operand is scaled once per q.
#include "device.h"

namespace qlora {
namespace {

typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i32x2_t lds_i32x2;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
typedef __attribute__((address_space(3))) char lds_char;

constexpr int kThreads = 256;           // reduction pass
constexpr int kThreads1 = 512;          // partial pass: 8 wavefronts
constexpr int kSliceN = 256;            // columns per workgroup (4 block columns)
constexpr int kSub = 128;               // k rows per LDS sub-chunk
constexpr int kCodePitch = 40;          // bytes per k row of a wavefront's code tile
constexpr int kRegion = kSub * kCodePitch + 32;   // bytes per wavefront code tile (bank shift 8)
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

__device__ __forceinline__ int32_t clamp_records(int64_t bytes) {
  return bytes > 0x7fffffff ? 0x7fffffff : (bytes < 0 ? 0 : int32_t(bytes));
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

// One sub-chunk of loads in registers (prefetched while the previous
// sub-chunk is multiplied).
// Raw loads of one sub-chunk, kept unconverted so that prefetching them does
// not wait for them: converted when they are written to LDS.
template <bool kX16>
struct Stage {
  u32x4_t cv[kSub / 64];   // codes: 16-B chunk t & 7 of row (t >> 3) + 64 it
  u32x4_t xr;              // X[t >> 5][4 (t & 31) .. +3] (bf16: first 8 bytes)
  int qv;                  // int8 block scale of k row 64 (wave >> 2) + lane
  float s2;                // its group scale
  f32x4_t s16;             // 16-entry format: the row's 4 group scales of the block column
};

// X[16 x kSub] of rows kb.. to registers: thread t -> row t >> 5, k run
// 4 (t & 31) .. +3 (rows >= M read as zero through the descriptor range).
template <bool kX16>
__device__ __forceinline__ u32x4_t load_x4(__amdgpu_buffer_rsrc_t rX, int64_t K, int64_t kb) {
  const int t = threadIdx.x;
  constexpr int esx = kX16 ? 2 : 4;
  const uint32_t off = uint32_t((int64_t(t >> 5) * K + kb + 4 * (t & 31)) * esx);
  if constexpr (kX16) {
    const u32x2_t v = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rX, off, 0, 0));
    return u32x4_t{v[0], v[1], 0u, 0u};
  } else {
    return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rX, off, 0, 0));
  }
}

template <bool kX16>
__device__ __forceinline__ void store_x4(float (*xs)[kXPitchS], u32x4_t v, int64_t kb, int64_t kend) {
  const int t = threadIdx.x;
  f32x4_t f;
  if constexpr (kX16)
    f = f32x4_t{bf16_lo_to_f32(v[0]), bf16_hi_to_f32(v[0]), bf16_lo_to_f32(v[1]), bf16_hi_to_f32(v[1])};
  else
    f = __builtin_bit_cast(f32x4_t, v);
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
  *reinterpret_cast<f32x4_t *>(&xs[t >> 5][4 * (t & 31)]) = (kb + 4 * (t & 31) < kend) ? f : zero4;
}

// The X . A workgroups (slice index == number of code slices): X[16 x kSub]
// times A[kSub x r] for the chunk, wavefront w -> columns 16 w .. 16 w + 15.
template <bool kX16, bool kA16>
__device__ __forceinline__ void xa_worker(const SmallArgs &a, int64_t kbeg, int64_t kend, int by,
                                          float (*xs)[kXPitchS], uint16_t (*as)[kAPitch]) {
  const int t = threadIdx.x, lane = t & 63, g = lane >> 4, i = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  constexpr int esx = kX16 ? 2 : 4, esa = kA16 ? 2 : 4;
  const __amdgpu_buffer_rsrc_t rX = __builtin_amdgcn_make_buffer_rsrc(
      (void *)a.X, (short)0, clamp_records(a.M * a.K * esx), kBufFlags);   // rows >= M: zero
  const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(
      (void *)a.A, (short)0, clamp_records(a.K * a.r * esa), kBufFlags);
  const bool active = wave < 4 && 16 * wave < a.r;
  f32x4_t xacc = {0.f, 0.f, 0.f, 0.f};
  for (int64_t kb = kbeg; kb < kend; kb += kSub) {
    const int rows = int(min64(kSub, kend - kb));
    const u32x4_t xv = load_x4<kX16>(rX, a.K, kb);
    float av[kSub / 8];      // A rows (t >> 6) + 8 u, column lane
#pragma unroll
    for (int u = 0; u < kSub / 8; ++u) {
      const uint32_t off = uint32_t(((kb + (t >> 6) + 8 * u) * a.r + lane) * esa);
      if constexpr (kA16)
        av[u] = __uint_as_float(uint32_t(__builtin_amdgcn_raw_buffer_load_b16(rA, off, 0, 0)) << 16);
      else
        av[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rA, off, 0, 0));
    }
    store_x4<kX16>(xs, xv, kb, kend);
#pragma unroll
    for (int u = 0; u < kSub / 8; ++u) {
      const int kk = (t >> 6) + 8 * u;
      const float v = (lane < a.r && kk < rows) ? av[u] : 0.0f;
      as[kk][lane] = __builtin_bit_cast(uint16_t, (__bf16)v);
    }
    __syncthreads();
    if (active) {
      for (int rb = 0; rb < rows; rb += 64) {
        // natural k order: lane (g, i) <- X[i][rb + 16 g + 0..15]
        u32x4_t U1, U2;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const f32x4_t x0 = *reinterpret_cast<const f32x4_t *>(&xs[i][rb + 16 * g + 8 * q]);
          const f32x4_t x1 = *reinterpret_cast<const f32x4_t *>(&xs[i][rb + 16 * g + 8 * q + 4]);
          u32x4_t &U = q ? U2 : U1;
          U[0] = pack_bf16x2(x0.x, x0.y);
          U[1] = pack_bf16x2(x0.z, x0.w);
          U[2] = pack_bf16x2(x1.x, x1.y);
          U[3] = pack_bf16x2(x1.z, x1.w);
        }
        // A^T operand: two ds_read_b64_tr_b16 per 8 k rows (16 lanes x 4 rows
        // -> lane i gets column i of the 4 rows)
        const int tq = i >> 2, qq = i & 3;
        const lds_char *ab = (const lds_char *)(&as[0][0]);
        const int col = 16 * wave + 4 * qq;
        u32x2_t w[4];
#pragma unroll
        for (int h = 0; h < 4; ++h)
          w[h] = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                 (lds_i16x4 *)(ab + ((rb + 16 * g + 4 * h + tq) * kAPitch + col) * 2)));
        xacc = mfma16x16x32(U1, u32x4_t{w[0][0], w[0][1], w[1][0], w[1][1]}, xacc);
        xacc = mfma16x16x32(U2, u32x4_t{w[2][0], w[2][1], w[3][0], w[3][1]}, xacc);
      }
    }
    __syncthreads();
  }
  const int j = 16 * wave + i;
  if (active && j < a.r) {
    float *PX = a.PXA + int64_t(by) * a.M * a.r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = 4 * g + e;
      if (m < a.M) PX[int64_t(m) * a.r + j] = xacc[e];
    }
  }
}

// One workgroup of the partial pass: column slice bx (bx == slices: the X . A
// workgroup) of K chunk by.
template <bool kX16, bool kA16, bool kG16>
__device__ __forceinline__ void fwd_small_block(const SmallArgs &a, const ExpandConsts16 &t16,
                                                int bx, int by) {
  __shared__ __attribute__((aligned(16))) float xs[16][kXPitchS];
  // scales per block column and k row; 16-entry format: per 16-column tile too
  __shared__ __attribute__((aligned(16))) float cs[4][kG16 ? 4 : 1][kSub];
  // codes of the 4 block columns, or (X . A workgroups) the adapter rows;
  // after the K loop, the k-half partial sums
  __shared__ __attribute__((aligned(16))) uint8_t ct[4 * kRegion];
  static_assert(kSub * kAPitch * 2 <= 4 * kRegion, "A tile fits the code tiles");
  static_assert(4 * 16 * 64 * 4 <= 4 * kRegion, "k-half sums fit the code tiles");

  const int c = by;
  const int64_t kbeg = int64_t(c) * a.Kc;
  const int64_t kend = min64(kbeg + a.Kc, a.K);
  const int64_t slices = (a.N + kSliceN - 1) / kSliceN;
  if (bx == slices) {
    xa_worker<kX16, kA16>(a, kbeg, kend, by, xs, reinterpret_cast<uint16_t (*)[kAPitch]>(ct));
    return;
  }

  // wavefront w: block column bc = w & 3 (64 columns), k half kh = w >> 2
  // (rows 64 kh .. 64 kh + 63 of every sub-chunk)
  const int t = threadIdx.x, lane = t & 63, g = lane >> 4, i = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);   // uniform: buffer descriptors
  const int bc = wave & 3, kh = wave >> 2;
  const int64_t n0 = int64_t(bx) * kSliceN;
  const int64_t nblk = a.N / 64, blk = n0 / 64 + bc;
  const bool blk_ok = blk < nblk;
  const int64_t half_n = a.N / 2;
  constexpr int esx = kX16 ? 2 : 4;
  uint8_t *myct = ct + bc * kRegion;

  // Every global read goes through a buffer descriptor whose range ends at
  // the last valid byte: reads past it return zero, so no load is predicated.
  const int64_t cbase = kbeg * half_n + n0 / 2;
  const __amdgpu_buffer_rsrc_t rC = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(a.codes + cbase), (short)0, clamp_records((kend - kbeg) * half_n - n0 / 2),
      kBufFlags);
  const __amdgpu_buffer_rsrc_t rX = __builtin_amdgcn_make_buffer_rsrc(
      (void *)a.X, (short)0, clamp_records(a.M * a.K * esx), kBufFlags);   // rows >= M: zero
  const __amdgpu_buffer_rsrc_t rQ = __builtin_amdgcn_make_buffer_rsrc(
      (void *)a.qscale, (short)0, clamp_records(a.K * nblk), kBufFlags);
  const __amdgpu_buffer_rsrc_t rG = __builtin_amdgcn_make_buffer_rsrc(
      (void *)a.gscale, (short)0,
      clamp_records(kG16 ? a.K * nblk * 16 : (a.K * nblk + 255) / 256 * 4), kBufFlags);

  auto load_stage = [&](int64_t kb, Stage<kX16> &S) {
    // the workgroup's 128-B segment of 8 rows per load instruction (whole
    // lines); rows past the chunk read as zero
#pragma unroll
    for (int it = 0; it < kSub / 64; ++it) {
      const int row = (t >> 3) + 64 * it;
      const uint32_t off = uint32_t((kb - kbeg + row) * half_n) + 16u * uint32_t(t & 7);
      S.cv[it] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rC, off, 0, 2));
    }
    // The code loads go out first: scheduled after the scale loads, their
    // address arithmetic (a 64-bit multiply-add whose unused high half the
    // compiler may take from any register) could name the register of an
    // in-flight load and wait for it.
    __builtin_amdgcn_sched_barrier(0);
    S.xr = load_x4<kX16>(rX, a.K, kb);
    const uint32_t b = uint32_t((kb + 64 * kh + lane) * nblk + blk);
    if constexpr (kG16) {
      // scales [K][N/16]: groups 4 blk .. 4 blk + 3 of k row kb + 64 kh + lane
      S.s16 = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rG, b * 16u, 0, 0));
    } else {
      S.qv = int(__builtin_amdgcn_raw_buffer_load_b8(rQ, b, 0, 0));
      S.s2 = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rG, (b >> 8) * 4u, 0, 0));
    }
  };

  f32x4_t acc[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) acc[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  Stage<kX16> S;
  load_stage(kbeg, S);
  for (int64_t kb = kbeg; kb < kend; kb += kSub) {
    const int rows = int(min64(kSub, kend - kb));        // 64 or 128
    // ---- this sub-chunk to LDS
#pragma unroll
    for (int it = 0; it < kSub / 64; ++it) {
      const int row = (t >> 3) + 64 * it, ch = t & 7;   // chunk ch -> block column ch / 2
      uint8_t *dst = ct + (ch >> 1) * kRegion + row * kCodePitch + 16 * (ch & 1);
      *reinterpret_cast<u32x2_t *>(dst) = u32x2_t{S.cv[it][0], S.cv[it][1]};
      *reinterpret_cast<u32x2_t *>(dst + 8) = u32x2_t{S.cv[it][2], S.cv[it][3]};
    }
    store_x4<kX16>(xs, S.xr, kb, kend);
    if constexpr (kG16) {
      const bool in = blk_ok && 64 * kh + lane < rows;
#pragma unroll
      for (int q = 0; q < 4; ++q) cs[bc][q][64 * kh + lane] = in ? S.s16[q] : 0.0f;
    } else {
      cs[bc][0][64 * kh + lane] = (blk_ok && 64 * kh + lane < rows) ? float(int8_t(S.qv)) * S.s2 : 0.0f;
    }
    __syncthreads();
    // ---- the next sub-chunk's loads fly while this one is multiplied
    if (kb + kSub < kend) load_stage(kb + kSub, S);

    const int rb = 64 * kh;
    if (rb < rows) {
      // activation operand: X[m = i][rb + 16 g + 0..15] times the row scales
      // (of the block column, or of 16-column tile sq in the 16-entry format)
      float xv[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4_t x4 = *reinterpret_cast<const f32x4_t *>(&xs[i][rb + 16 * g + 4 * q]);
        xv[4 * q] = x4.x; xv[4 * q + 1] = x4.y; xv[4 * q + 2] = x4.z; xv[4 * q + 3] = x4.w;
      }
      auto scaled_x = [&](int sq, u32x4_t &A1, u32x4_t &A2) {
        float sv[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4_t s4 = *reinterpret_cast<const f32x4_t *>(&cs[bc][sq][rb + 16 * g + 4 * q]);
          sv[4 * q] = s4.x; sv[4 * q + 1] = s4.y; sv[4 * q + 2] = s4.z; sv[4 * q + 3] = s4.w;
        }
        A1[0] = pack_bf16x2(xv[0] * sv[0], xv[2] * sv[2]);
        A1[1] = pack_bf16x2(xv[4] * sv[4], xv[6] * sv[6]);
        A1[2] = pack_bf16x2(xv[1] * sv[1], xv[3] * sv[3]);
        A1[3] = pack_bf16x2(xv[5] * sv[5], xv[7] * sv[7]);
        A2[0] = pack_bf16x2(xv[8] * sv[8], xv[10] * sv[10]);
        A2[1] = pack_bf16x2(xv[12] * sv[12], xv[14] * sv[14]);
        A2[2] = pack_bf16x2(xv[9] * sv[9], xv[11] * sv[11]);
        A2[3] = pack_bf16x2(xv[13] * sv[13], xv[15] * sv[15]);
      };
      u32x4_t A1, A2;
      if constexpr (!kG16) scaled_x(0, A1, A2);
      // weight operand: lane (g, i) <- column 16 q + i, rows rb + 16 g + 0..15
      const lds_char *crow = (const lds_char *)(myct + (rb + 16 * g + i) * kCodePitch);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if constexpr (kG16) scaled_x(q, A1, A2);
        const i32x2_t d = __builtin_amdgcn_ds_read_tr4_b64_v2i32((lds_i32x2 *)(crow + 8 * q));
        acc[q] = mfma16x16x32(A1, expand_levels(uint32_t(d[0]), t16), acc[q]);
        acc[q] = mfma16x16x32(A2, expand_levels(uint32_t(d[1]), t16), acc[q]);
      }
    }
    __syncthreads();   // LDS tiles are rewritten by the next sub-chunk
  }

  // ---- k half 1 hands its sums to k half 0 (fixed order: half 0 + half 1)
  float *red = reinterpret_cast<float *>(ct) + bc * (16 * 64);
  if (kh == 1) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) red[(4 * q + e) * 64 + lane] = acc[q][e];
  }
  __syncthreads();
  if (kh == 1) return;
  // ---- partials: lane (g, i) holds rows 4 g .. 4 g + 3 of column 16 q + i
  float *P = a.P + int64_t(c) * a.M * a.N;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t n = n0 + 64 * bc + 16 * q + i;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float v = acc[q][e] + red[(4 * q + e) * 64 + lane];
      const int m = 4 * g + e;
      if (blk_ok && n < a.N && m < a.M) P[int64_t(m) * a.N + n] = v;
    }
  }
}

template <bool kX16, bool kA16, bool kG16>
__global__ __launch_bounds__(kThreads1) void fwd_small_kernel(SmallArgs a, ExpandConsts16 t16) {
  fwd_small_block<kX16, kA16, kG16>(a, t16, int(blockIdx.x), int(blockIdx.y));
}

// Several independent linears' partial passes in one launch: workgroups
// base[g] .. base[g + 1] - 1 are linear g's grid, row-major over (slice,
// chunk) with gx[g] slices per chunk.
struct SmallGroup {
  int n;
  SmallArgs a[kSmallMaxGroup];
  int base[kSmallMaxGroup + 1];
  int gx[kSmallMaxGroup];
};

template <bool kX16, bool kA16, bool kG16>
__global__ __launch_bounds__(kThreads1) void fwd_small_group_kernel(SmallGroup g,
                                                                    ExpandConsts16 t16) {
  const int bid = int(blockIdx.x);
  int l = 0;
#pragma unroll
  for (int j = 1; j < kSmallMaxGroup; ++j)
    if (j < g.n && bid >= g.base[j]) l = j;
  const int local = bid - g.base[l];
  fwd_small_block<kX16, kA16, kG16>(g.a[l], t16, local % g.gx[l], local / g.gx[l]);
}

// Pass 2: a workgroup covers `cols` = 256 / Mp columns of all M rows (Mp =
// M rounded up to a power of two); thread -> (row, column).  The partials of
// up to 32 chunks, 16 rows of B and the XA partials are all requested before
// any is used (range-checked buffer loads: zero past the end), so the pass
// waits for memory about once; sums run in chunk order.
struct SmallReduceArgs {
  const float *P, *PXA;
  int64_t KS, M, N, r;
  int cols;
  const void *B;
  float *XA;
  void *Y;
  RankMul mul;
};

template <bool kY16, bool kB16>
__device__ __forceinline__ void fwd_small_reduce_block(const SmallReduceArgs &ra, int bx) {
  const float *__restrict__ P = ra.P;
  const float *__restrict__ PXA = ra.PXA;
  const int64_t KS = ra.KS, M = ra.M, N = ra.N, r = ra.r;
  const int cols = ra.cols;
  const void *B = ra.B;
  float *XA = ra.XA;
  void *Y = ra.Y;
  const RankMul &mul = ra.mul;
  __shared__ float xa[16][kSmallMaxR];
  const int t = threadIdx.x;
  const int64_t ER = M * r;
  constexpr int esb = kB16 ? 2 : 4;
  const __amdgpu_buffer_rsrc_t rP = __builtin_amdgcn_make_buffer_rsrc(
      (void *)P, (short)0, clamp_records(KS * M * N * 4), kBufFlags);
  const __amdgpu_buffer_rsrc_t rPX = __builtin_amdgcn_make_buffer_rsrc(
      (void *)PXA, (short)0, clamp_records(KS * ER * 4), kBufFlags);
  const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc(
      (void *)B, (short)0, clamp_records(r * N * esb), kBufFlags);
  const int m = t / cols;
  const int64_t n = int64_t(bx) * cols + (t % cols);
  const bool ok = m < M && n < N;
  auto load_b = [&](int j) -> float {
    const uint32_t off = uint32_t((int64_t(j) * N + n) * esb);
    if constexpr (kB16)
      return __uint_as_float(uint32_t(__builtin_amdgcn_raw_buffer_load_b16(rB, off, 0, 0)) << 16);
    else
      return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rB, off, 0, 0));
  };
  // ---- requests: partials of chunks 0..31, rows 0..15 of B
  float pv[32], bv[16];
#pragma unroll
  for (int u = 0; u < 32; ++u)
    pv[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                          rP, uint32_t(((u * M + m) * N + n) * 4), 0, 0));
#pragma unroll
  for (int q = 0; q < 16; ++q) bv[q] = load_b(q);
  // ---- XA = sum over chunks of PXA
  for (int e = t; e < ER; e += kThreads) {
    float xv[32];
    float sx = 0.0f;
    for (int64_t c0 = 0; c0 < KS; c0 += 32) {
#pragma unroll
      for (int u = 0; u < 32; ++u)
        xv[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                              rPX, uint32_t(((c0 + u) * ER + e) * 4), 0, 0));
#pragma unroll
      for (int u = 0; u < 32; ++u) sx += xv[u];
    }
    xa[e / r][e % r] = rank_mul(mul, e / r, e % r, r, sx);
    if (bx == 0 && XA) XA[e] = sx;
  }
  __syncthreads();
  if (!ok) return;
  float sum = 0.0f;
#pragma unroll
  for (int u = 0; u < 32; ++u) sum += pv[u];
  for (int64_t c0 = 32; c0 < KS; c0 += 32) {
#pragma unroll
    for (int u = 0; u < 32; ++u)
      pv[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                            rP, uint32_t((((c0 + u) * M + m) * N + n) * 4), 0, 0));
#pragma unroll
    for (int u = 0; u < 32; ++u) sum += pv[u];
  }
  float ua = 0.0f;
#pragma unroll
  for (int q = 0; q < 16; ++q)
    if (q < r) ua += xa[m][q] * bv[q];
  for (int j0 = 16; j0 < r; j0 += 16) {
#pragma unroll
    for (int q = 0; q < 16; ++q) bv[q] = load_b(j0 + q);
#pragma unroll
    for (int q = 0; q < 16; ++q)
      if (j0 + q < r) ua += xa[m][j0 + q] * bv[q];
  }
  const float y = sum + ua;
  if (kY16)
    static_cast<uint16_t *>(Y)[int64_t(m) * N + n] = __builtin_bit_cast(uint16_t, (__bf16)y);
  else
    static_cast<float *>(Y)[int64_t(m) * N + n] = y;
}

template <bool kY16, bool kB16>
__global__ __launch_bounds__(kThreads) void fwd_small_reduce_kernel(SmallReduceArgs ra) {
  fwd_small_reduce_block<kY16, kB16>(ra, int(blockIdx.x));
}

struct SmallReduceGroup {
  int n;
  SmallReduceArgs a[kSmallMaxGroup];
  int base[kSmallMaxGroup + 1];
};

template <bool kY16, bool kB16>
__global__ __launch_bounds__(kThreads) void fwd_small_reduce_group_kernel(SmallReduceGroup g) {
  const int bid = int(blockIdx.x);
  int l = 0;
#pragma unroll
  for (int j = 1; j < kSmallMaxGroup; ++j)
    if (j < g.n && bid >= g.base[j]) l = j;
  fwd_small_reduce_block<kY16, kB16>(g.a[l], bid - g.base[l]);
}

}  // namespace

namespace {
int reduce_cols(int64_t M) {
  int mp = 1;
  while (mp < M) mp *= 2;
  return kThreads / mp;
}
}  // namespace

int64_t small_fwd_chunk_rows(int64_t M, int64_t K, int64_t N) {
  const int64_t slices = (N + kSliceN - 1) / kSliceN;
  const int64_t target = M <= 4 ? 512 : 256;
  int64_t ks = (target + slices - 1) / slices;
  ks = ks < 1 ? 1 : (ks > K / 64 ? K / 64 : ks);
  return ((K + ks - 1) / ks + 63) / 64 * 64;
}

hipError_t launch_fwd_small_partial(const uint8_t *codes, const int8_t *qscale,
                                    const float *gscale, int64_t K, int64_t N, const void *X,
                                    bool x_bf16, int64_t M, const void *A, bool a_bf16, int64_t r,
                                    int64_t Kc, float *P, float *PXA, int codebook, bool g16,
                                    hipStream_t s) {
  const int64_t KS = (K + Kc - 1) / Kc;
  const int64_t slices = (N + kSliceN - 1) / kSliceN;
  SmallArgs a{codes, qscale, gscale, K, N, X, A, M, r, Kc, P, PXA};
  if (!tables(codebook).symmetric) return hipErrorInvalidValue;
  const ExpandConsts16 &t16 = tables(codebook).expand16;
  // one extra column of workgroups computes the X . A partials
  const dim3 grid = dim3(unsigned(slices + (r > 0 ? 1 : 0)), unsigned(KS));
#define QLORA_SMALL(XB, AB, G) \
  hipLaunchKernelGGL((fwd_small_kernel<XB, AB, G>), grid, dim3(kThreads1), 0, s, a, t16)
  if (g16) {
    if (x_bf16) {
      if (a_bf16) QLORA_SMALL(true, true, true);
      else QLORA_SMALL(true, false, true);
    } else {
      if (a_bf16) QLORA_SMALL(false, true, true);
      else QLORA_SMALL(false, false, true);
    }
  } else {
    if (x_bf16) {
      if (a_bf16) QLORA_SMALL(true, true, false);
      else QLORA_SMALL(true, false, false);
    } else {
      if (a_bf16) QLORA_SMALL(false, true, false);
      else QLORA_SMALL(false, false, false);
    }
  }
#undef QLORA_SMALL
  return hipGetLastError();
}

hipError_t launch_fwd_small_reduce(const float *P, const float *PXA, int64_t KS, int64_t M,
                                   int64_t N, int64_t r, const void *B, bool b_bf16, float *XA,
                                   void *Y, bool y_bf16, hipStream_t s,
                         RankMul mul) {
  const int cols = reduce_cols(M);
  const dim3 grid = dim3(unsigned((N + cols - 1) / cols));
  const SmallReduceArgs ra{P, PXA, KS, M, N, r, cols, B, XA, Y, mul};
  if (y_bf16) {
    if (b_bf16) hipLaunchKernelGGL((fwd_small_reduce_kernel<true, true>), grid, dim3(kThreads), 0, s, ra);
    else hipLaunchKernelGGL((fwd_small_reduce_kernel<true, false>), grid, dim3(kThreads), 0, s, ra);
  } else {
    if (b_bf16) hipLaunchKernelGGL((fwd_small_reduce_kernel<false, true>), grid, dim3(kThreads), 0, s, ra);
    else hipLaunchKernelGGL((fwd_small_reduce_kernel<false, false>), grid, dim3(kThreads), 0, s, ra);
  }
  return hipGetLastError();
}

hipError_t launch_fwd_small_group(int n, const SmallLinear *lin, int64_t M, bool x_bf16,
                                  bool a_bf16, int64_t r, int codebook, bool g16,
                                  hipStream_t s) {
  if (n < 1 || n > kSmallMaxGroup) return hipErrorInvalidValue;
  if (!tables(codebook).symmetric) return hipErrorInvalidValue;
  const ExpandConsts16 &t16 = tables(codebook).expand16;
  SmallGroup g{};
  SmallReduceGroup rg{};
  g.n = rg.n = n;
  int64_t nb = 0, nr = 0;
  const int cols = reduce_cols(M);
  for (int l = 0; l < n; ++l) {
    const SmallLinear &L = lin[l];
    const int64_t KS = (L.K + L.Kc - 1) / L.Kc;
    const int64_t gx = (L.N + kSliceN - 1) / kSliceN + (r > 0 ? 1 : 0);
    g.a[l] = SmallArgs{L.codes, L.qscale, L.gscale, L.K, L.N, L.X, L.A, M, r, L.Kc, L.P, L.PXA};
    g.base[l] = int(nb);
    g.gx[l] = int(gx);
    nb += gx * KS;
    rg.a[l] = SmallReduceArgs{L.P, L.PXA, KS, M, L.N, r, cols, L.B, L.XA, L.Y, L.mul};
    rg.base[l] = int(nr);
    nr += (L.N + cols - 1) / cols;
  }
  g.base[n] = int(nb);
  rg.base[n] = int(nr);
#define QLORA_SMALLG(XB, AB, G) \
  hipLaunchKernelGGL((fwd_small_group_kernel<XB, AB, G>), dim3(unsigned(nb)), dim3(kThreads1), 0, \
                     s, g, t16)
  if (g16) {
    if (x_bf16) {
      if (a_bf16) QLORA_SMALLG(true, true, true);
      else QLORA_SMALLG(true, false, true);
    } else {
      if (a_bf16) QLORA_SMALLG(false, true, true);
      else QLORA_SMALLG(false, false, true);
    }
  } else {
    if (x_bf16) {
      if (a_bf16) QLORA_SMALLG(true, true, false);
      else QLORA_SMALLG(true, false, false);
    } else {
      if (a_bf16) QLORA_SMALLG(false, true, false);
      else QLORA_SMALLG(false, false, false);
    }
  }
#undef QLORA_SMALLG
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the reduction: y and B in the activation / adapter dtypes as the partial pass's X, A
  if (x_bf16) {
    if (a_bf16) hipLaunchKernelGGL((fwd_small_reduce_group_kernel<true, true>), dim3(unsigned(nr)), dim3(kThreads), 0, s, rg);
    else hipLaunchKernelGGL((fwd_small_reduce_group_kernel<true, false>), dim3(unsigned(nr)), dim3(kThreads), 0, s, rg);
  } else {
    if (a_bf16) hipLaunchKernelGGL((fwd_small_reduce_group_kernel<false, true>), dim3(unsigned(nr)), dim3(kThreads), 0, s, rg);
    else hipLaunchKernelGGL((fwd_small_reduce_group_kernel<false, false>), dim3(unsigned(nr)), dim3(kThreads), 0, s, rg);
  }
  return hipGetLastError();
}

}  // namespace qlora
