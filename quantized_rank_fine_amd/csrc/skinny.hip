// Rank-r ("skinny") products of the adapted linear layer and their helpers.
//
// "QLoRA (low-rank adapters on a quantized model)", "How it works": A is
// (in x r) and B is (r x out); the adapter path costs r*(in+out) parameters
// and adds the rank-r products
//   XA = X.A (forward),  G = dY.B^T,  dA = X^T.G,  dB = XA^T.dY (backward),
// which are memory-bound passes over X or dY (r <= 256 << in, out).
//
// rowfull: C[M x R] = P[M x K] . Q whole, R <= 32 and M >= 1024: a
//          workgroup owns a few rows of P and all of K (no partials).
// rowdot:  the same product split over K (any shape): a slice of P and of Q
//          is staged in LDS, Q in the form the MFMA B operand reads; fp32
//          partials.
// coldot:  C[K x R] = P[M x K]^T . Q[M x R], contraction over the token axis
//          (P = X or dY, Q = G or XA given row-major).  P tiles are staged
//          row-major in LDS and read transposed with ds_read_b64_tr_b16
//          (16 lanes x 4 rows -> 4 columns); fp32 partials over token chunks.
// Partials are summed by a reduce pass in a fixed order (deterministic, no
// atomics).
//
// Launches are merged where the data allow it, each role on a contiguous
// range of workgroup ids (the block-scale table for the GEMMs first).  At
// M >= 1024 and r <= 32 the forward runs one launch (XA whole + scales) and
// the backward one pass over dY (G whole, scales, and either dB partials or,
// when the dX GEMM forms dB, the bf16 XA^T it needs), one pass over X (dA
// partials) and one reduce of dA and dB; otherwise X.A and G come as split-K
// partials with a reduce after each pass.  The bf16 copies of XA and G carry
// the adapter options' multiplier (alpha/r, dropout; RankMul), and a reduce
// can apply an Adam step to the sums it forms (AdamTarget).
//
// All matrix-core work is v_mfma_f32_16x16x32_bf16: operands rounded to bf16,
// fp32 accumulation.
#include "device.h"

namespace qlora {
namespace {

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
constexpr int32_t kBufFlags = 0x00020000;   // raw buffer descriptor word 3
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

// 8 consecutive elements as loaded (bf16: one 16-B piece; fp32: two), and
// their conversion to the bf16x8 MFMA operand at the point of use.
template <bool kBf16>
struct Raw8 {
  u32x4_t v[kBf16 ? 1 : 2];
};

template <bool kBf16>
__device__ __forceinline__ Raw8<kBf16> buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  Raw8<kBf16> x;
  x.v[0] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
  if constexpr (!kBf16)
    x.v[1] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, 0));
  return x;
}

template <bool kBf16>
__device__ __forceinline__ u32x4_t as_bf16x8_op(const Raw8<kBf16> &x) {
  if constexpr (kBf16) {
    return x.v[0];
  } else {
    const f32x4_t a = __builtin_bit_cast(f32x4_t, x.v[0]), b = __builtin_bit_cast(f32x4_t, x.v[1]);
    return u32x4_t{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]),
                   pack_bf16x2(b[2], b[3])};
  }
}

// The same 8 elements from a flat address.
template <bool kBf16>
__device__ __forceinline__ Raw8<kBf16> raw_load8(const void *p) {
  Raw8<kBf16> x;
  const u32x4_t *q = static_cast<const u32x4_t *>(p);
  x.v[0] = q[0];
  if constexpr (!kBf16) x.v[1] = q[1];
  return x;
}

// Transposed read of a row-major bf16 LDS tile T (pitch PP elements): lane
// (i16 = lane & 15, h = (lane >> 4) & 3) receives column cb + i16, rows
// rb + 8h .. rb + 8h + 7 -- the k-run of one MFMA 16x16x32 operand lane --
// from two ds_read_b64_tr_b16 (each: 16 lanes x 4 rows -> 4 columns).
__device__ __forceinline__ u32x4_t lds_col8(const uint16_t *T, int PP, int rb, int cb) {
  const int lane = threadIdx.x & 63, i16 = lane & 15, h = (lane >> 4) & 3;
  const int q = i16 & 3, tq = i16 >> 2;
  const int rr = rb + 8 * h + tq;
  lds_char *base = (lds_char *)(T);
  i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4 *)(base + (rr * PP + cb + 4 * q) * 2));
  i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4 *)(base + ((rr + 4) * PP + cb + 4 * q) * 2));
  u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
  return u32x4_t{l2[0], l2[1], h2[0], h2[1]};
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
// 64-wide block column (the layout the fused GEMMs stream).  A thread owns one
// row and 16 consecutive blocks of it: one 16-B read of q8, the (at most two)
// second-level scales those 16 blocks use, 16 stores that are coalesced across
// the wavefront (consecutive rows).  Role of a merged launch: workgroups
// wg = 0 .. scales_workgroups(rows, NB) - 1, placed first in the grid so that
// their short dependent chain starts with the launch.
struct ScalesArgs {
  const int8_t *q8;
  const float *s2;
  int64_t rows, NB;
  float *cs;
};

constexpr int kScaleSpan = 16;   // blocks per thread

__host__ __device__ inline int64_t scales_workgroups(int64_t rows, int64_t NB) {
  return ((rows + 255) / 256) * ((NB + kScaleSpan - 1) / kScaleSpan);
}

__device__ __forceinline__ void scales_role(const ScalesArgs &a, int64_t wg) {
  const int64_t nspan = (a.NB + kScaleSpan - 1) / kScaleSpan;
  const int64_t row = (wg / nspan) * 256 + threadIdx.x;
  const int64_t b0 = (wg % nspan) * kScaleSpan;
  if (row >= a.rows) return;
  const int64_t f0 = row * a.NB + b0;                          // flat block index of b0
  const int nb = int(min64(kScaleSpan, a.NB - b0));            // blocks of this thread
  const float s2a = a.s2[f0 >> 8], s2b = a.s2[(f0 + nb - 1) >> 8];   // at most two groups
  int8_t v[kScaleSpan];
  if (a.NB % kScaleSpan == 0) {
    // every span is whole and 16-B aligned (q8 is)
    const u32x4_t w = *reinterpret_cast<const u32x4_t *>(a.q8 + f0);
#pragma unroll
    for (int e = 0; e < kScaleSpan; ++e) v[e] = int8_t(w[e >> 2] >> (8 * (e & 3)));
  } else {
    // byte loads, all issued (indices past the span repeat its last block)
#pragma unroll
    for (int e = 0; e < kScaleSpan; ++e) v[e] = a.q8[f0 + (e < nb ? e : nb - 1)];
  }
  float c[kScaleSpan];
#pragma unroll
  for (int e = 0; e < kScaleSpan; ++e)
    c[e] = float(v[e]) * (((f0 + e) >> 8) == (f0 >> 8) ? s2a : s2b);
#pragma unroll
  for (int e = 0; e < kScaleSpan; ++e)
    if (e < nb) a.cs[(b0 + e) * a.rows + row] = c[e];
}

// ------------------------------------------------------- XA^T for the dX GEMM
// xat[j][m] = bf16(mul(XA)[m][j]) for j < 16, m < ldm (ldm a multiple of 256), zero
// for j >= r or m >= M: the A operand of the dB products that the dX GEMM
// takes from the dY tiles in its LDS ring.  A thread owns 8 consecutive
// tokens of one rank index (one 16-B store).  Role of a merged launch.
struct XatArgs {
  const float *XA;    // [M x r]
  int64_t M;
  int r;
  uint16_t *xat;      // [16 x ldm]
  int64_t ldm;
  RankMul mul;        // applied before the rounding to bf16
};

__host__ __device__ inline int64_t xat_workgroups(int64_t ldm) { return ldm * 16 / 2048; }

__device__ __forceinline__ void xat_role(const XatArgs &a, int64_t wg) {
  const int64_t e0 = (wg * 256 + threadIdx.x) * 8;    // first element, row-major [16][ldm]
  const int j = int(e0 / a.ldm);
  const int64_t m0 = e0 % a.ldm;
  uint32_t h[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int64_t m = m0 + e;
    h[e] = (j < a.r && m < a.M)
               ? uint32_t(f32_to_bf16_bits(rank_mul(a.mul, m, j, a.r, a.XA[m * a.r + j])))
               : 0u;
  }
  *reinterpret_cast<u32x4_t *>(a.xat + e0) =
      u32x4_t{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
}

// ------------------------------------------------------------------ rowdot
//
// Workgroup: 4 wavefronts x 16 rows = 64 rows of P, all R columns, one
// contiguous K range walked in slices of kTK (256 for R <= 64, else 64).  Per
// slice, the P rows (64 x kTK) and Q go to LDS, Q as [RP][kTK] (16-B chunks
// XOR-swizzled by row) or [kTK][RP], shared by the 4 wavefronts, and the next
// slice's loads fly while the current one is multiplied.

constexpr int kRowdotRows = 64;

__host__ __device__ inline int rank_pad16(int R) { return (R + 15) / 16 * 16; }
__host__ __device__ inline bool skinny_wide(int R) { return rank_pad16(R) <= 64; }

struct RowdotArgs {
  const void *P;      // [M x K]
  const void *Q;      // Qt [R x K] (kQt) or Q [K x R]
  int64_t M, K;
  int R;
  int64_t kchunk;     // K range per split (multiple of the slice width)
  int64_t mt;         // row tiles
  float *part;        // [ks][M][R]
};

// Q modes: kQRows -- Qt [R x K], rows contiguous along k (B for G);
// kQFast -- Q [K x R] with R % 8 == 0, staged row-major [kTK][RP] with 16-B
// copies and read transposed; kQGeneric -- Q [K x R], any R, staged
// transposed element by element.
constexpr int kQRows = 0, kQFast = 1, kQGeneric = 2;

// One workgroup of rowdot with kRT 16-wide rank tiles (kGuard: at most kRT,
// the actual count R / 16 rounded up read at run time).  A slice's P rows
// (64 x kTK) and Q chunks are loaded with coalesced 16-B loads into
// registers, stored to LDS, and the next slice's loads are issued before the
// products of the current one, which read both operands from LDS.
// Out-of-range pieces load from an in-range address (row m0 or 0, column
// 0, k kb) and are stored as zero, so no load sits behind a branch.
template <int kTK>
__host__ __device__ constexpr int rowdot_ppitch() { return kTK + 8; }

template <bool kPbf16, int kQMode, bool kQbf16, int kTK, int kRT, bool kGuard>
__device__ __forceinline__ void rowdot_body(const RowdotArgs &a, int64_t wg, unsigned char *smem) {
  constexpr int kCPR = kTK / 8;              // 16-B chunks per staged row
  constexpr int kNS = kTK / 32;              // MFMA k substeps per slice
  constexpr int kMask = (kCPR < 16 ? kCPR : 16) - 1;
  constexpr int kNQ = (16 * kRT * kTK / 8 + 255) / 256;   // 16-B Q chunks per thread
  constexpr int kNP = kRowdotRows * kCPR / 256;            // 16-B P chunks per thread
  constexpr int kPP = rowdot_ppitch<kTK>();
  constexpr int pes = kPbf16 ? 2 : 4, qes = kQbf16 ? 2 : 4;
  uint16_t *sP = reinterpret_cast<uint16_t *>(smem);   // [64][kPP]
  uint16_t *sQ = sP + kRowdotRows * kPP;               // [RP][kTK], or [kTK][RP] (kQFast)
  const int R = a.R;
  const int RT = kGuard ? (R + 15) / 16 : kRT;
  const int RP = RT * 16;
  const int nq = RP * kTK / 8;               // 16-B Q chunks per slice
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int i16 = lane & 15, h = lane >> 4;
  const int64_t K = a.K;
  const int64_t m0 = (wg % a.mt) * kRowdotRows;
  const int ks = int(wg / a.mt);
  const int64_t kb = int64_t(ks) * a.kchunk;
  const int64_t ke = min64(K, kb + a.kchunk);
  const char *Pb = static_cast<const char *>(a.P);
  const char *qbase = static_cast<const char *>(a.Q);

  f32x4_t acc[kRT];
#pragma unroll
  for (int s = 0; s < kRT; ++s) acc[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // P chunk q of slice k0: 8 k of row m0 + rr
  auto p_chunk = [&](int64_t k0, int q, int64_t &off, int &dst) {
    const int cid = t + 256 * q, rr = cid / kCPR, ch = cid % kCPR;
    const int64_t m = m0 + rr, k = k0 + 8 * ch;
    const bool ok = m < a.M && k < ke;
    off = ok ? m * K + k : m0 * K + kb;
    dst = rr * kPP + 8 * ch;
    return ok;
  };
  // Q chunk cid of slice k0 (kQRows: 8 k of row j of Qt; kQFast: 8 columns
  // of row k of Q)
  auto q_chunk = [&](int64_t k0, int cid, int64_t &off, int &dst) {
    bool ok;
    if constexpr (kQMode == kQRows) {
      const int j = cid / kCPR, ch = cid % kCPR;
      const int64_t k = k0 + 8 * ch;
      ok = j < R && k < ke;
      off = ok ? int64_t(j) * K + k : kb;
      dst = j * kTK + ((ch ^ (j & kMask)) * 8);
    } else {
      const int C8 = RP / 8;
      const int kk = cid / C8, c = cid - kk * C8;
      const int64_t k = k0 + kk;
      ok = 8 * c < R && k < ke;
      off = ok ? k * R + 8 * c : kb * R;
      dst = kk * RP + 8 * c;
    }
    return ok;
  };
  Raw8<kPbf16> pv[kNP];
  Raw8<kQbf16> qv[kNQ];
  auto load_slice = [&](int64_t k0) {
    if constexpr (kQMode != kQGeneric) {
#pragma unroll
      for (int u = 0; u < kNQ; ++u) {
        if (kGuard && 256 * u >= nq) break;
        int64_t off;
        int dst;
        q_chunk(k0, t + 256 * u, off, dst);
        qv[u] = raw_load8<kQbf16>(qbase + off * qes);
      }
    }
#pragma unroll
    for (int q = 0; q < kNP; ++q) {
      int64_t off;
      int dst;
      p_chunk(k0, q, off, dst);
      pv[q] = raw_load8<kPbf16>(Pb + off * pes);
    }
  };

  load_slice(kb);
  for (int64_t k0 = kb; k0 < ke; k0 += kTK) {
    __syncthreads();                         // previous slice's readers are done
#pragma unroll
    for (int q = 0; q < kNP; ++q) {
      int64_t off;
      int dst;
      const bool ok = p_chunk(k0, q, off, dst);
      const u32x4_t v = as_bf16x8_op<kPbf16>(pv[q]);
      *reinterpret_cast<u32x4_t *>(sP + dst) = ok ? v : u32x4_t{0u, 0u, 0u, 0u};
    }
    if constexpr (kQMode != kQGeneric) {
      // columns R..RP-1 (kQFast) or rows R..RP-1 (kQRows) and k past ke are zero
#pragma unroll
      for (int u = 0; u < kNQ; ++u) {
        if (kGuard && 256 * u >= nq) break;
        int64_t off;
        int dst;
        const bool ok = q_chunk(k0, t + 256 * u, off, dst);
        const u32x4_t v = as_bf16x8_op<kQbf16>(qv[u]);
        if (!kGuard || t + 256 * u < nq)
          *reinterpret_cast<u32x4_t *>(sQ + dst) = ok ? v : u32x4_t{0u, 0u, 0u, 0u};
      }
    } else {
      // Q [K x R] row-major: coalesced element reads (16 in flight per
      // thread), transposed LDS writes
#pragma unroll 1
      for (int e0 = 0; e0 < kTK * RP; e0 += 256 * 16) {
        uint16_t v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int e = e0 + 256 * u + t;
          const int kk = e / RP, j = e - kk * RP;
          const int64_t k = k0 + kk;
          const bool ok = e < kTK * RP && j < R && k < ke;
          const uint16_t x = uint16_t(load1_bf16<kQbf16>(a.Q, ok ? k * R + j : int64_t(0)));
          v[u] = ok ? x : uint16_t(0);
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int e = e0 + 256 * u + t;
          const int kk = e / RP, j = e - kk * RP;
          if (e < kTK * RP) sQ[j * kTK + (((kk >> 3) ^ (j & kMask)) << 3) + (kk & 7)] = v[u];
        }
      }
    }
    __syncthreads();
    if (k0 + kTK < ke) load_slice(k0 + kTK);   // in flight during the products
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < kNS; ++s) {
      // A operand: row wave * 16 + i16, k 32 s + 8 h .. +8
      const u32x4_t av =
          *reinterpret_cast<const u32x4_t *>(sP + (wave * 16 + i16) * kPP + 32 * s + 8 * h);
#pragma unroll
      for (int st = 0; st < kRT; ++st) {
        if (!kGuard || st < RT) {
          u32x4_t b;
          if constexpr (kQMode == kQFast) {
            b = lds_col8(sQ, RP, 32 * s, 16 * st);
          } else {
            const int j = 16 * st + i16;
            const int c = 4 * s + h;
            b = *reinterpret_cast<const u32x4_t *>(sQ + j * kTK + ((c ^ (j & kMask)) * 8));
          }
          acc[st] = mfma16x16x32(av, b, acc[st]);
        }
      }
    }
  }
  // C layout: lane holds rows 4h..4h+3 of the wave's 16, column i16 of subtile st
  float *out = a.part + int64_t(ks) * a.M * R;
#pragma unroll
  for (int st = 0; st < kRT; ++st) {
    if (!kGuard || st < RT) {
      const int j = 16 * st + i16;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t m = m0 + wave * 16 + 4 * h + q;
        if (m < a.M && j < R) out[m * R + j] = acc[st][q];
      }
    }
  }
}

// R <= 64: 256-wide slices with the rank tile count fixed at compile time
// (one body per count); larger R: 64-wide slices, up to 16 tiles.
template <bool kPbf16, int kQMode, bool kQbf16, bool kWide>
__device__ __forceinline__ void rowdot_role(const RowdotArgs &a, int64_t wg, unsigned char *smem) {
  if constexpr (kWide) {
    switch ((a.R + 15) / 16) {
      case 1: rowdot_body<kPbf16, kQMode, kQbf16, 256, 1, false>(a, wg, smem); break;
      case 2: rowdot_body<kPbf16, kQMode, kQbf16, 256, 2, false>(a, wg, smem); break;
      case 3: rowdot_body<kPbf16, kQMode, kQbf16, 256, 3, false>(a, wg, smem); break;
      default: rowdot_body<kPbf16, kQMode, kQbf16, 256, 4, false>(a, wg, smem); break;
    }
  } else {
    rowdot_body<kPbf16, kQMode, kQbf16, 64, 16, true>(a, wg, smem);
  }
}

// ----------------------------------------------------------------- rowfull
//
// C[M x R] = P[M x K] . Q for R <= 32 at large M, without split-K partials:
// a workgroup owns kRows (8 or 16) rows of P and the whole K range, cut into
// four contiguous runs of 32-wide k steps, one per wavefront.  A wavefront
// keeps the loads of its next batch of kFullSteps steps in flight while it
// multiplies the current one: P rows go straight into the MFMA A operand
// (kept raw until use), Q either straight into the B operand (Qt [R x K],
// rows contiguous along k) or, for Q [K x R], through the wavefront's own LDS
// area (loaded as whole rows), read back transposed.  The four partial products are then summed in
// wavefront order through LDS and written as fp32 and/or zero-padded bf16.
// Rows past M, lanes past kRows and steps past a wavefront's run read zero
// through the range check of raw buffer loads (no branches around loads).

constexpr int kFullSteps = 8;                 // 32-wide k steps per batch
constexpr int kFullMinM = 1024;               // below this, split-K partials

struct RowfullArgs {
  const void *P;      // [M x K]
  const void *Q;      // Qt [R x K] (kQRows) or Q [K x R], R % 8 == 0 (kQFast)
  int64_t M, K;
  int R;
  int rows;           // rows per workgroup: 8 or 16
  float *out;         // fp32 [M x R], optional
  uint16_t *out16;    // bf16 [M x ld16], zero padding columns R..ld16-1, optional
  int64_t ld16;
  RankMul mul;        // applied to the bf16 copy only
};

__host__ __device__ inline int32_t clamp_records(int64_t bytes) {
  return bytes > 0x7fffffff ? 0x7fffffff : (bytes < 0 ? 0 : int32_t(bytes));
}

// Per-wavefront Q staging of one batch (kQFast only): [kFullSteps * 32][RP],
// read transposed.
template <int kQMode, int kRT>
__host__ __device__ constexpr size_t rowfull_stage_bytes() {
  return kQMode == kQFast ? size_t(kFullSteps) * 32 * (16 * kRT) * 2 : 0;
}

// Per-wavefront P staging of one batch: kRows rows x kFullSteps * 32 k, rows
// padded by 16 B.
constexpr int kFullPPitch = kFullSteps * 32 + 8;
template <int kRows>
__host__ __device__ constexpr size_t rowfull_pstage_bytes() {
  return size_t(kRows) * kFullPPitch * 2;
}

template <int kQMode, int kRT, int kRows>
__host__ __device__ constexpr size_t rowfull_lds_bytes() {
  return 4 * (rowfull_stage_bytes<kQMode, kRT>() + rowfull_pstage_bytes<kRows>()) +
         size_t(4) * kRT * 16 * 16 * 4;
}

template <bool kPbf16, int kQMode, bool kQbf16, int kRT, int kRows>
__device__ __forceinline__ void rowfull_role(const RowfullArgs &a, int64_t wg, unsigned char *smem) {
  constexpr int kRP = 16 * kRT;
  constexpr int pes = kPbf16 ? 2 : 4, qes = kQbf16 ? 2 : 4;
  constexpr int kCPR = kRP / 8;                                  // 16-B chunks per staged Q row
  // 16-B Q chunks per lane and batch: kQFast -- staging chunks; kQRows --
  // the B operands of every step and rank tile
  constexpr int kQN = kQMode == kQFast ? kFullSteps * 32 * kCPR / 64 : kFullSteps * kRT;
  constexpr size_t kStageBytes = rowfull_stage_bytes<kQMode, kRT>();   // per wavefront
  constexpr size_t kPStageBytes = rowfull_pstage_bytes<kRows>();      // per wavefront
  // 16-B P chunks per lane and batch: kRows rows x kFullSteps * 32 k
  constexpr int kNP = kRows * kFullSteps * 32 / 8 / 64;
  constexpr int kPCR = kFullSteps * 32 / 8;                      // 16-B chunks per P row and batch
  static_assert(kQMode == kQRows || kQMode == kQFast, "rowfull Q form");
  static_assert(kRows == 8 || kRows == 16, "rows per workgroup");
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int i16 = lane & 15, h = lane >> 4;
  const int64_t K = a.K;
  const int R = a.R;
  const int64_t m0 = wg * kRows;
  const int nrows = int(min64(kRows, a.M - m0));

  // P rows m0 .. m0 + nrows - 1; lanes past them address the first byte
  // past the range (every later k offset stays out of range too)
  const uint32_t p_rec = uint32_t(clamp_records(int64_t(nrows) * K * pes));
  const __amdgpu_buffer_rsrc_t rP = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(static_cast<const char *>(a.P) + m0 * K * pes), (short)0, int32_t(p_rec), kBufFlags);
  const uint32_t q_rec = uint32_t(clamp_records(int64_t(R) * K * qes));
  const __amdgpu_buffer_rsrc_t rQ = __builtin_amdgcn_make_buffer_rsrc((void *)a.Q, (short)0,
                                                                      int32_t(q_rec), kBufFlags);
  uint32_t qrow[kRT];                          // kQRows: row j = 16 st + i16 of Qt
#pragma unroll
  for (int st = 0; st < kRT; ++st) {
    const int j = 16 * st + i16;
    qrow[st] = j < R ? uint32_t(j * K * qes) : q_rec;
  }

  const int ns = int(K / 32);
  const int s0 = wave * ns / 4, s1 = (wave + 1) * ns / 4;
  const int nb = (s1 - s0 + kFullSteps - 1) / kFullSteps;
  uint16_t *sQ = reinterpret_cast<uint16_t *>(smem + wave * (kStageBytes + kPStageBytes));
  uint16_t *sPw = reinterpret_cast<uint16_t *>(smem + wave * (kStageBytes + kPStageBytes) + kStageBytes);

  Raw8<kPbf16> xb[2][kNP];
  Raw8<kQbf16> qb[2][kQN];
  auto load_batch = [&](int b, Raw8<kPbf16> (&xv)[kNP], Raw8<kQbf16> (&qv)[kQN]) {
    // P: whole 512-B row runs (32 lanes per row), rows past nrows and steps
    // past the run read zero
#pragma unroll
    for (int u = 0; u < kNP; ++u) {
      const int cid = lane + 64 * u, row = cid / kPCR, kc = cid % kPCR;
      const int st = s0 + kFullSteps * b + kc / 4;
      xv[u] = buf_load8<kPbf16>(
          rP, (row < nrows && st < s1) ? uint32_t((row * K + 32 * st + 8 * (kc % 4)) * pes) : p_rec);
    }
#pragma unroll
    for (int u = 0; u < kFullSteps; ++u) {
      const int st = s0 + kFullSteps * b + u;
      const bool in = st < s1;
      if constexpr (kQMode == kQRows) {
        // the B operand straight from the rows of Qt
#pragma unroll
        for (int r = 0; r < kRT; ++r)
          qv[u * kRT + r] = buf_load8<kQbf16>(rQ, in ? qrow[r] + uint32_t((32 * st + 8 * h) * qes) : q_rec);
      }
    }
    if constexpr (kQMode == kQFast) {
      // rows kb .. kb + 255 of Q [K x R], 16-B chunks in row order
      const int64_t kb = int64_t(32) * (s0 + kFullSteps * b), ke = int64_t(32) * s1;
#pragma unroll
      for (int u = 0; u < kQN; ++u) {
        const int cid = lane + 64 * u, kk = cid / kCPR, c = cid % kCPR;
        const int64_t k = kb + kk;
        qv[u] = buf_load8<kQbf16>(rQ, (k < ke && 8 * c < R) ? uint32_t((k * R + 8 * c) * qes) : q_rec);
      }
    }
  };

  f32x4_t acc[kRT];
#pragma unroll
  for (int r = 0; r < kRT; ++r) acc[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto compute_batch = [&](const Raw8<kPbf16> (&xv)[kNP], const Raw8<kQbf16> (&qv)[kQN]) {
    // P rows to this wavefront's area (LDS operations of one wavefront
    // complete in order, so the reads below see these writes, and the next
    // batch's writes follow this batch's reads)
#pragma unroll
    for (int u = 0; u < kNP; ++u) {
      const int cid = lane + 64 * u, row = cid / kPCR, kc = cid % kPCR;
      *reinterpret_cast<u32x4_t *>(sPw + row * kFullPPitch + 8 * kc) = as_bf16x8_op<kPbf16>(xv[u]);
    }
    if constexpr (kQMode == kQFast) {
      // stage Q rows [kFullSteps * 32][kRP] in this wavefront's area (LDS
      // operations of one wavefront complete in order, so the transposed
      // reads below see these writes and the next batch's writes follow them)
#pragma unroll
      for (int u = 0; u < kQN; ++u) {
        const int cid = lane + 64 * u, kk = cid / kCPR, c = cid % kCPR;
        *reinterpret_cast<u32x4_t *>(sQ + kk * kRP + 8 * c) = as_bf16x8_op<kQbf16>(qv[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < kFullSteps; ++u) {
      // A operand: row i16 (zero past kRows), k 32 u + 8 h .. +8
      const u32x4_t a8 =
          *reinterpret_cast<const u32x4_t *>(sPw + (i16 & (kRows - 1)) * kFullPPitch + 32 * u + 8 * h);
      const u32x4_t av = i16 < kRows ? a8 : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
      for (int r = 0; r < kRT; ++r) {
        u32x4_t bv;
        if constexpr (kQMode == kQFast)
          bv = lds_col8(sQ, kRP, 32 * u, 16 * r);
        else
          bv = as_bf16x8_op<kQbf16>(qv[u * kRT + r]);
        acc[r] = mfma16x16x32(av, bv, acc[r]);
      }
    }
  };

  // two register sets, alternating; the loads of batch b + 1 are issued
  // before batch b is multiplied (batches past nb read zero)
  load_batch(0, xb[0], qb[0]);
  for (int b = 0; b < nb; b += 2) {
    load_batch(b + 1, xb[1], qb[1]);
    __builtin_amdgcn_sched_barrier(0);     // keep the loads ahead of the products
    compute_batch(xb[0], qb[0]);
    if (b + 1 >= nb) break;
    load_batch(b + 2, xb[0], qb[0]);
    __builtin_amdgcn_sched_barrier(0);
    compute_batch(xb[1], qb[1]);
  }

  // fixed-order sum of the four wavefronts' products
  float *red = reinterpret_cast<float *>(smem + 4 * (kStageBytes + kPStageBytes));
#pragma unroll
  for (int r = 0; r < kRT; ++r)
#pragma unroll
    for (int e = 0; e < 4; ++e) red[((wave * kRT + r) * 16 + 4 * h + e) * 16 + i16] = acc[r][e];
  __syncthreads();
  const int L = a.out16 ? int(a.ld16) : R;
  for (int e = t; e < nrows * L; e += 256) {
    const int row = e / L, j = e - row * L;
    const int64_t m = m0 + row;
    if (j < R) {
      const int r = j >> 4, jj = j & 15;
      float v = red[((0 * kRT + r) * 16 + row) * 16 + jj];
      v += red[((1 * kRT + r) * 16 + row) * 16 + jj];
      v += red[((2 * kRT + r) * 16 + row) * 16 + jj];
      v += red[((3 * kRT + r) * 16 + row) * 16 + jj];
      if (a.out) a.out[m * R + j] = v;
      if (a.out16) a.out16[m * a.ld16 + j] = f32_to_bf16_bits(rank_mul(a.mul, m, j, R, v));
    } else {
      a.out16[m * a.ld16 + j] = 0;
    }
  }
}

// ------------------------------------------------------------------ coldot
//
// Workgroup: 4 wavefronts, kTN columns of P (128 for R <= 64, else 64; a
// wavefront owns kTN/4 of them as 16-wide MFMA tiles), all R, one contiguous
// token range walked in 64-token slices.  Per slice the P tile (64 x kTN
// bf16) is stored row-major in LDS with a row pitch that keeps the transposed
// reads conflict-free, and Q^T (R x 64) with swizzled 16-B chunks.

__host__ __device__ inline int coldot_tn(int R) { return skinny_wide(R) ? 128 : 64; }
__host__ __device__ inline int coldot_pitch(int TN) { return TN == 128 ? 144 : 80; }

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

// kQFastC: Q rows hold a multiple of 8 columns and are 16-B aligned (R % 8
// == 0 or a zero-padded bf16 Q), so Q[mm..mm+63][0..RP) is copied row-major
// with 16-B chunks and read transposed; otherwise Q^T is staged element by
// element.  kRT 16-wide rank tiles (kGuard: at most kRT, the actual count
// read at run time).  Out-of-range P and Q pieces load from an in-range
// address (token mb, column c0 or 0) and are stored to LDS as zero, so no
// load sits behind a branch.
template <bool kPbf16, bool kQbf16, int kTN, bool kQFastC, int kRT, bool kGuard>
__device__ __forceinline__ void coldot_body(const ColdotArgs &a, int64_t wg, unsigned char *smem) {
  constexpr int kPP = kTN == 128 ? 144 : 80;  // LDS row pitch of the P tile (elements)
  constexpr int kCPR = kTN / 8;               // 16-B chunks per P row
  constexpr int kNP = 64 * kCPR / 256;        // P chunks per thread: 8 or 2
  constexpr int kNCT = kTN / 64;              // 16-wide column tiles per wavefront
  constexpr int pes = kPbf16 ? 2 : 4, qes = kQbf16 ? 2 : 4;
  const int R = a.R;
  const int RT = kGuard ? (R + 15) / 16 : kRT;
  const int RP = RT * 16;
  uint16_t *sP = reinterpret_cast<uint16_t *>(smem);               // [64][kPP]
  uint16_t *sQ = sP + 64 * kPP;                        // [RP][64], or [64][RP] (kQFastC)
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int i16 = lane & 15, h = lane >> 4;
  const int64_t c0 = (wg % a.ct) * kTN;
  const int ks = int(wg / a.ct);
  const int64_t mb = int64_t(ks) * a.mchunk;
  const int64_t me = min64(a.M, mb + a.mchunk);
  const int64_t K = a.K;
  const char *P = static_cast<const char *>(a.P);
  const char *Qb = static_cast<const char *>(a.Q);

  f32x4_t acc[kNCT][kRT];
#pragma unroll
  for (int c4 = 0; c4 < kNCT; ++c4)
#pragma unroll
    for (int s = 0; s < kRT; ++s) acc[c4][s] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // P tile of tokens mm..mm+63 (and, kQFastC, the Q rows mm..mm+63 as 16-B
  // chunks) into registers; the next slice's loads are issued as soon as the
  // current slice is in LDS, so they are in flight during its products.
  constexpr int kNQ = kQFastC ? (64 * (16 * kRT) / 8 + 255) / 256 : 1;
  const int C8 = RP / 8;
  Raw8<kPbf16> pv[kNP];
  Raw8<kQbf16> qv[kNQ];
  auto p_ok = [&](int64_t mm, int q, int64_t &m, int64_t &col, int &rr, int &ch) {
    const int cid = t + 256 * q;
    rr = cid / kCPR;
    ch = cid % kCPR;
    m = mm + rr;
    col = c0 + 8 * ch;
    return m < me && col < K;
  };
  auto q_ok = [&](int64_t mm, int q, int64_t &m, int &mi, int &c) {
    const int cid = t + 256 * q;
    mi = cid / C8;
    c = cid - mi * C8;
    m = mm + mi;
    return cid < 64 * C8 && m < me && 8 * c < a.ldq;
  };
  auto load_slice = [&](int64_t mm) {
#pragma unroll
    for (int q = 0; q < kNP; ++q) {
      int64_t m, col;
      int rr, ch;
      const bool ok = p_ok(mm, q, m, col, rr, ch);
      pv[q] = raw_load8<kPbf16>(P + (ok ? m * K + col : mb * K + c0) * pes);
    }
    if constexpr (kQFastC) {
#pragma unroll
      for (int q = 0; q < kNQ; ++q) {
        if (kGuard && 256 * q >= 64 * C8) break;
        int64_t m;
        int mi, c;
        const bool ok = q_ok(mm, q, m, mi, c);
        qv[q] = raw_load8<kQbf16>(Qb + (ok ? m * a.ldq + 8 * c : mb * a.ldq) * qes);
      }
    }
  };
  if (mb < me) load_slice(mb);
  for (int64_t mm = mb; mm < me; mm += 64) {
    __syncthreads();                         // previous slice's readers are done
#pragma unroll
    for (int q = 0; q < kNP; ++q) {
      int64_t m, col;
      int rr, ch;
      const bool ok = p_ok(mm, q, m, col, rr, ch);
      const u32x4_t v = as_bf16x8_op<kPbf16>(pv[q]);
      *reinterpret_cast<u32x4_t *>(sP + rr * kPP + 8 * ch) = ok ? v : u32x4_t{0u, 0u, 0u, 0u};
    }
    if constexpr (kQFastC) {
      // Q rows mm..mm+63, columns 0..RP-1, as 16-B chunks into [64][RP]
#pragma unroll
      for (int q = 0; q < kNQ; ++q) {
        if (kGuard && 256 * q >= 64 * C8) break;
        int64_t m;
        int mi, c;
        const bool ok = q_ok(mm, q, m, mi, c);
        const u32x4_t v = as_bf16x8_op<kQbf16>(qv[q]);
        if (t + 256 * q < 64 * C8)
          *reinterpret_cast<u32x4_t *>(sQ + mi * RP + 8 * c) = ok ? v : u32x4_t{0u, 0u, 0u, 0u};
      }
    } else {
      // Q^T for tokens mm..mm+63: coalesced element reads of Q rows,
      // transposed LDS writes (16-B chunks of 8 tokens, swizzled by j)
#pragma unroll 1
      for (int e0 = 0; e0 < 64 * RP; e0 += 256 * 16) {
        uint16_t v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int e = e0 + 256 * u + t;
          const int mi = e / RP, j = e - mi * RP;
          const int64_t m = mm + mi;
          const bool ok = e < 64 * RP && j < R && m < me;
          const uint16_t x = uint16_t(load1_bf16<kQbf16>(a.Q, ok ? m * a.ldq + j : int64_t(0)));
          v[u] = ok ? x : uint16_t(0);
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int e = e0 + 256 * u + t;
          const int mi = e / RP, j = e - mi * RP;
          if (e < 64 * RP) sQ[j * 64 + (((mi >> 3) ^ (j & 7)) << 3) + (mi & 7)] = v[u];
        }
      }
    }
    __syncthreads();
    if (mm + 64 < me) load_slice(mm + 64);   // in flight during the products
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int c4 = 0; c4 < kNCT; ++c4) {
        // A operand: column cb + i16 of P, tokens 32u + 8h .. +8, via two
        // transposed reads of 4 rows x 4 columns per 16-lane group.
        const int cb = wave * (kTN / 4) + 16 * c4;
        u32x4_t av;
        {
          const int q = i16 & 3, tq = i16 >> 2;
          const int rr = 32 * u + 8 * h + tq;
          lds_char *base = (lds_char *)(sP);
          i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4 *)(base + (rr * kPP + cb + 4 * q) * 2));
          i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4 *)(base + ((rr + 4) * kPP + cb + 4 * q) * 2));
          u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
          av = u32x4_t{l2[0], l2[1], h2[0], h2[1]};
        }
#pragma unroll
        for (int st = 0; st < kRT; ++st) {
          if (!kGuard || st < RT) {
            u32x4_t b;
            if constexpr (kQFastC) {
              b = lds_col8(sQ, RP, 32 * u, 16 * st);
            } else {
              const int j = 16 * st + i16;
              const int ch = 4 * u + h;
              b = *reinterpret_cast<const u32x4_t *>(sQ + j * 64 + ((ch ^ (j & 7)) * 8));
            }
            acc[c4][st] = mfma16x16x32(av, b, acc[c4][st]);
          }
        }
      }
    }
  }
  float *out = a.part + int64_t(ks) * K * R;
#pragma unroll
  for (int c4 = 0; c4 < kNCT; ++c4) {
#pragma unroll
    for (int st = 0; st < kRT; ++st) {
      if (!kGuard || st < RT) {
        const int j = 16 * st + i16;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t col = c0 + wave * (kTN / 4) + 16 * c4 + 4 * h + q;
          if (col < K && j < R) out[col * R + j] = acc[c4][st][q];
        }
      }
    }
  }
}

// R <= 64: 128 columns per workgroup with the rank tile count fixed at
// compile time (one body per count); larger R: 64 columns, up to 16 tiles.
template <bool kPbf16, bool kQbf16, bool kWide, bool kQFastC>
__device__ __forceinline__ void coldot_role(const ColdotArgs &a, int64_t wg, unsigned char *smem) {
  if constexpr (kWide) {
    switch ((a.R + 15) / 16) {
      case 1: coldot_body<kPbf16, kQbf16, 128, kQFastC, 1, false>(a, wg, smem); break;
      case 2: coldot_body<kPbf16, kQbf16, 128, kQFastC, 2, false>(a, wg, smem); break;
      case 3: coldot_body<kPbf16, kQbf16, 128, kQFastC, 3, false>(a, wg, smem); break;
      default: coldot_body<kPbf16, kQbf16, 128, kQFastC, 4, false>(a, wg, smem); break;
    }
  } else {
    coldot_body<kPbf16, kQbf16, 64, kQFastC, 16, true>(a, wg, smem);
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
  RankMul mul;        // applied to the bf16 copy only
  AdamTarget adam;    // one Adam step from the sums, in the layout of out
};

// The Adam step of element i of the result (index in out's layout).
__device__ __forceinline__ void reduce_adam(const AdamTarget &t, int64_t i, float g) {
  float th = t.theta[i], m = t.m[i], v = t.v[i];
  adam1(t.p, th, g, m, v);
  t.theta[i] = th;
  t.m[i] = m;
  t.v[i] = v;
  if (t.theta16) t.theta16[i] = f32_to_bf16_bits(th);
}

// Vector form (R % 4 == 0): a thread owns 4 consecutive elements of one row
// and keeps up to kRedBatch 16-B partial loads in flight, so that a pass over
// ks partials costs ceil(ks / kRedBatch) load round trips.
constexpr int kRedBatch = 16;

__device__ __forceinline__ void reduce_role(const ReduceArgs &a, int64_t wg, int64_t nwg) {
  const int64_t n = a.rows * a.R;
  if (a.R % 4 == 0) {
    const int64_t n4 = n / 4;
    for (int64_t i4 = wg * 256 + threadIdx.x; i4 < n4; i4 += nwg * 256) {
      const f32x4_t *p = reinterpret_cast<const f32x4_t *>(a.part) + i4;
      f32x4_t s = {0.f, 0.f, 0.f, 0.f};
      for (int64_t k = 0; k < a.ks; k += kRedBatch) {
        f32x4_t v[kRedBatch];
#pragma unroll
        for (int u = 0; u < kRedBatch; ++u)
          v[u] = (k + u < a.ks) ? p[(k + u) * n4] : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < kRedBatch; ++u)
          if (k + u < a.ks) s += v[u];     // k order
      }
      const int64_t i = 4 * i4, rr = i / a.R, j = i - rr * a.R;
      if (a.out) {
        if (a.transpose_out) {
#pragma unroll
          for (int e = 0; e < 4; ++e) a.out[(j + e) * a.rows + rr] = s[e];
        } else {
          *reinterpret_cast<f32x4_t *>(a.out + i) = s;
        }
      }
      if (a.adam.theta) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          reduce_adam(a.adam, a.transpose_out ? (j + e) * a.rows + rr : i + e, s[e]);
      }
      if (a.out_bf16) {
        uint16_t *d = a.out_bf16 + rr * a.ld_bf16 + j;
        f32x4_t u;
#pragma unroll
        for (int e = 0; e < 4; ++e) u[e] = rank_mul(a.mul, rr, j + e, a.R, s[e]);
        const uint32_t lo = uint32_t(f32_to_bf16_bits(u[0])) | (uint32_t(f32_to_bf16_bits(u[1])) << 16);
        const uint32_t hi = uint32_t(f32_to_bf16_bits(u[2])) | (uint32_t(f32_to_bf16_bits(u[3])) << 16);
        *reinterpret_cast<u32x2_t *>(d) = u32x2_t{lo, hi};
      }
    }
  } else {
    for (int64_t i = wg * 256 + threadIdx.x; i < n; i += nwg * 256) {
      // partials are loaded 8 at a time (independent loads in flight) and
      // summed in k order
      float s = 0.0f;
      int64_t k = 0;
      for (; k + 8 <= a.ks; k += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = a.part[(k + u) * n + i];
#pragma unroll
        for (int u = 0; u < 8; ++u) s += v[u];
      }
      for (; k < a.ks; ++k) s += a.part[k * n + i];
      const int64_t rr = i / a.R, j = i - rr * a.R;
      if (a.out) a.out[a.transpose_out ? j * a.rows + rr : i] = s;
      if (a.adam.theta) reduce_adam(a.adam, a.transpose_out ? j * a.rows + rr : i, s);
      if (a.out_bf16) a.out_bf16[rr * a.ld_bf16 + j] = f32_to_bf16_bits(rank_mul(a.mul, rr, j, a.R, s));
    }
  }
  if (a.out_bf16 && a.ld_bf16 > a.R) {   // zero padding columns R..ld_bf16-1
    const int64_t pad = a.ld_bf16 - a.R, np = a.rows * pad;
    for (int64_t i = wg * 256 + threadIdx.x; i < np; i += nwg * 256) {
      const int64_t rr = i / pad, j = a.R + (i - rr * pad);
      a.out_bf16[rr * a.ld_bf16 + j] = 0;
    }
  }
}

// ------------------------------------------------------------ dA whole
//
// dA [K x R] = P[M x K]^T . Q[M x R] for R <= 16 without token partials (P =
// X, Q = G16 bf16 [M x ldq], zero beyond R): a workgroup owns 16 columns of P
// and every token.  The tokens go in 64-token slabs, slab s to wavefront
// s % 4; a wavefront stages a slab of P (64 x 16) and of Q (64 x 16) in its
// own LDS area, row-major as loaded, and reads both back transposed as the
// A and B operands of two v_mfma_f32_16x16x32_bf16.  It keeps the loads of
// its next kDaGroup slabs in flight while it multiplies the current ones.
// The four wavefronts' products are summed in wavefront order; every sum is
// therefore fixed by the shapes alone.  Optionally one Adam step of A from
// the sums (as in the reduce pass).
constexpr int kDaPitch = 24;                    // LDS row pitch of a staged slab (elements)

struct DaFullArgs {
  const void *P;
  const uint16_t *Q;
  int64_t ldq, M, K;
  int R;
  float *out;          // [K x R] fp32
  AdamTarget adam;
};

template <bool kPbf16>
__device__ __forceinline__ void da_full_role(const DaFullArgs &a, int64_t wg, unsigned char *smem) {
  constexpr int kG = kPbf16 ? 4 : 2;            // slabs per load group
  constexpr int kPL = kPbf16 ? 2 : 4;           // 16-B P loads per lane and slab
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int64_t c0 = wg * 16;
  const int64_t slabs = (a.M + 63) / 64;
  const int64_t mine = slabs > wave ? (slabs - wave + 3) / 4 : 0;   // slabs of this wavefront
  uint16_t *sP = reinterpret_cast<uint16_t *>(smem) + wave * (2 * 64 * kDaPitch);
  uint16_t *sQ = sP + 64 * kDaPitch;
  const size_t pes = kPbf16 ? 2 : 4;
  const char *P = static_cast<const char *>(a.P);

  // lane = token row of the slab: its 16 columns of P and its 16 of Q.  The
  // loads go through buffer descriptors that end at row M (rows past it,
  // including every row of a slab past this wavefront's last, read zero), so
  // none is conditional and the waits before each group's products leave
  // the next group's loads in flight.  (The host keeps every offset below
  // 2^31.)
  const __amdgpu_buffer_rsrc_t rP = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void *>(a.P), (short)0, clamp_records(a.M * a.K * int64_t(pes)), kBufFlags);
  const __amdgpu_buffer_rsrc_t rQ = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(a.Q), (short)0, clamp_records(a.M * a.ldq * 2), kBufFlags);
  u32x4_t pv[2][kG][kPL], qv[2][kG][2];
  auto load_group = [&](int64_t grp, u32x4_t (&pg)[kG][kPL], u32x4_t (&qg)[kG][2]) {
#pragma unroll
    for (int u = 0; u < kG; ++u) {
      const int64_t ls = grp * kG + u;                       // this wavefront's slab index
      // load c covers rows 32 (c / (kPL / 2)) .. +31 of the slab, two lanes
      // per row (lane & 1: the row's first or second 8 columns)
#pragma unroll
      for (int c = 0; c < kPL; ++c) {
        const int half = c / (kPL / 2), part = c % (kPL / 2);
        const int64_t m = (wave + 4 * ls) * 64 + 32 * half + (lane >> 1);   // >= M past the last slab
        const uint32_t po = uint32_t((m * a.K + c0) * int64_t(pes)) + 16u * uint32_t((lane & 1) * (kPL / 2) + part);
        pg[u][c] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rP, po, 0, 0));
      }
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int64_t m = (wave + 4 * ls) * 64 + 32 * c + (lane >> 1);
        const uint32_t qo = uint32_t(m * a.ldq * 2) + 16u * uint32_t(lane & 1);
        qg[u][c] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rQ, qo, 0, 0));
      }
    }
  };
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  auto compute_group = [&](const u32x4_t (&pg)[kG][kPL], const u32x4_t (&qg)[kG][2], int64_t grp) {
#pragma unroll
    for (int u = 0; u < kG; ++u) {
      if (grp * kG + u >= mine) break;
      // (LDS operations of one wavefront complete in order: these writes
      // follow the previous slab's reads and precede this slab's)
      // p16[h]: 8 columns (lane & 1) of row 32 h + (lane >> 1)
      u32x4_t p16[2];
      if constexpr (kPbf16) {
        p16[0] = pg[u][0];
        p16[1] = pg[u][1];
      } else {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          // fp32: loads 2c, 2c + 1 are the two 16-B halves of the lane's 32 B
          const f32x4_t x = __builtin_bit_cast(f32x4_t, pg[u][2 * c]);
          const f32x4_t y = __builtin_bit_cast(f32x4_t, pg[u][2 * c + 1]);
          p16[c] = u32x4_t{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                           pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
        }
      }
      const int rw = lane >> 1, cw = 8 * (lane & 1);
      *reinterpret_cast<u32x4_t *>(sP + rw * kDaPitch + cw) = p16[0];
      *reinterpret_cast<u32x4_t *>(sP + (32 + rw) * kDaPitch + cw) = p16[1];
      *reinterpret_cast<u32x4_t *>(sQ + rw * kDaPitch + cw) = qg[u][0];
      *reinterpret_cast<u32x4_t *>(sQ + (32 + rw) * kDaPitch + cw) = qg[u][1];
#pragma unroll
      for (int k = 0; k < 2; ++k)
        acc = mfma16x16x32(lds_col8(sP, kDaPitch, 32 * k, 0), lds_col8(sQ, kDaPitch, 32 * k, 0), acc);
    }
  };
  const int64_t groups = (mine + kG - 1) / kG;
  // The first two groups' loads go out before any product, outside the
  // loop (whose waits, merged over its back edge, would otherwise make the
  // first iteration wait for group 0 before issuing group 1); the scheduling
  // barriers keep each group's loads ahead of the previous group's products.
  if (groups > 0) load_group(0, pv[0], qv[0]);
  if (groups > 1) load_group(1, pv[1], qv[1]);
  __builtin_amdgcn_sched_barrier(0);
  if (groups > 0) compute_group(pv[0], qv[0], 0);
  for (int64_t grp = 1; grp < groups; grp += 2) {
    // pv[1] holds group grp
    if (grp + 1 < groups) load_group(grp + 1, pv[0], qv[0]);
    __builtin_amdgcn_sched_barrier(0);
    compute_group(pv[1], qv[1], grp);
    if (grp + 1 >= groups) break;
    if (grp + 2 < groups) load_group(grp + 2, pv[1], qv[1]);
    __builtin_amdgcn_sched_barrier(0);
    compute_group(pv[0], qv[0], grp + 1);
  }

  // C layout: lane holds rows 4 h .. 4 h + 3 (columns of P), column i16 (rank)
  float *red = reinterpret_cast<float *>(smem + 4 * 2 * 64 * kDaPitch * 2);   // [4][16][16]
  const int i16 = lane & 15, h = lane >> 4;
#pragma unroll
  for (int e = 0; e < 4; ++e) red[(wave * 16 + 4 * h + e) * 16 + i16] = acc[e];
  __syncthreads();
  const int row = t >> 4, j = t & 15;
  if (j < a.R && c0 + row < a.K) {
    const float v = ((red[row * 16 + j] + red[(16 + row) * 16 + j]) + red[(32 + row) * 16 + j]) +
                    red[(48 + row) * 16 + j];
    const int64_t i = (c0 + row) * a.R + j;
    if (a.out) a.out[i] = v;
    if (a.adam.theta) reduce_adam(a.adam, i, v);
  }
}

constexpr size_t kDaLdsBytes = size_t(4) * 2 * 64 * kDaPitch * 2 + size_t(4) * 16 * 16 * 4;

// ------------------------------------------------------------------ kernels

// Block scales on workgroups [0, n_sc), XA partials (rowdot with Q = A
// [in x r]) on [n_sc, grid).  Either role may be empty.
template <bool kXbf16, bool kAbf16, bool kWide, int kQMode>
__global__ __launch_bounds__(256) void fwd_prep_kernel(RowdotArgs ra, int64_t n_sc,
                                                       ScalesArgs sa) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int64_t wg = blockIdx.x;
  if (wg < n_sc)
    scales_role(sa, wg);
  else
    rowdot_role<kXbf16, kQMode, kAbf16, kWide>(ra, wg - n_sc, smem);
}

// Block scales on [0, n_sc), XA = X . A complete (rowfull with Q = A
// [in x r], r % 8 == 0) on the rest.
template <bool kXbf16, bool kAbf16, int kRT>
__global__ __launch_bounds__(256) void fwd_full_kernel(RowfullArgs ra, int64_t n_sc, ScalesArgs sa) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int64_t wg = blockIdx.x;
  if (wg < n_sc)
    scales_role(sa, wg);
  else if (ra.rows == 8)
    rowfull_role<kXbf16, kQFast, kAbf16, kRT, 8>(ra, wg - n_sc, smem);
  else
    rowfull_role<kXbf16, kQFast, kAbf16, kRT, 16>(ra, wg - n_sc, smem);
}

// One pass over dY with G complete: block scales on [0, n_sc), XA^T bf16 on
// [n_sc, n_sc + n_xat) (only when the dX GEMM takes dB over), G = dY . B^T
// (rowfull with Qt = B [r x out]) on the next n_row, and otherwise dB
// partials (coldot with Q = XA fp32 [M x r]) on the rest.
template <bool kDYbf16, bool kBbf16, int kRT, bool kQFastC>
__global__ __launch_bounds__(256) void dy_full_kernel(RowfullArgs ra, int64_t n_row, ColdotArgs ca,
                                                      int64_t n_sc, ScalesArgs sa, int64_t n_xat,
                                                      XatArgs xa) {
  extern __shared__ __align__(16) unsigned char smem[];
  int64_t wg = blockIdx.x;
  if (wg < n_sc) {
    scales_role(sa, wg);
    return;
  }
  wg -= n_sc;
  if (wg < n_xat) {
    xat_role(xa, wg);
    return;
  }
  wg -= n_xat;
  if (wg < n_row) {
    if (ra.rows == 8)
      rowfull_role<kDYbf16, kQRows, kBbf16, kRT, 8>(ra, wg, smem);
    else
      rowfull_role<kDYbf16, kQRows, kBbf16, kRT, 16>(ra, wg, smem);
  } else
    coldot_role<kDYbf16, false, true, kQFastC>(ca, wg - n_row, smem);
}

// One pass over dY: block scales on [0, n_sc), G partials (rowdot with
// Qt = B [r x out]) on [n_sc, n_sc + n_row), dB partials (coldot with Q = XA
// fp32 [M x r]) on the rest.
template <bool kDYbf16, bool kBbf16, bool kWide, bool kQFastC>
__global__ __launch_bounds__(256) void bwd_dy_kernel(RowdotArgs ra, int64_t n_row, ColdotArgs ca,
                                                     int64_t n_sc, ScalesArgs sa) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int64_t wg = blockIdx.x;
  if (wg < n_sc)
    scales_role(sa, wg);
  else if (wg < n_sc + n_row)
    rowdot_role<kDYbf16, kQRows, kBbf16, kWide>(ra, wg - n_sc, smem);
  else
    coldot_role<kDYbf16, false, kWide, kQFastC>(ca, wg - n_sc - n_row, smem);
}

// One pass over X: dA partials (coldot with Q = G16 bf16 [M x rp], zero-padded).
template <bool kXbf16, bool kWide>
__global__ __launch_bounds__(256) void bwd_x_kernel(ColdotArgs ca) {
  extern __shared__ __align__(16) unsigned char smem[];
  coldot_role<kXbf16, true, kWide, true>(ca, blockIdx.x, smem);
}

// After the dX GEMM: dA whole (da_full_role) on workgroups [0, n_da) and
// the reduction of dB's partials (reduce_role) on the rest.
template <bool kXbf16>
__global__ __launch_bounds__(256) void bwd_tail_kernel(DaFullArgs da, int64_t n_da, ReduceArgs rb) {
  __shared__ __align__(16) unsigned char smem[kDaLdsBytes];
  const int64_t wg = blockIdx.x;
  if (wg < n_da) {
    // Workgroups are dealt to the 8 XCDs round-robin: give each XCD a
    // contiguous run of column groups, so that the four groups sharing a
    // 128-B line of P read it through one L2.
    const int64_t c = n_da % 8 == 0 ? (wg % 8) * (n_da / 8) + wg / 8 : wg;
    da_full_role<kXbf16>(da, c, smem);
  } else {
    reduce_role(rb, wg - n_da, int64_t(gridDim.x) - n_da);
  }
}

// U = mul(XA), element by element.
__global__ __launch_bounds__(256) void rank_mul_kernel(const float *__restrict__ XA, int64_t M,
                                                       int64_t R, RankMul mul,
                                                       float *__restrict__ U) {
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < M * R; i += int64_t(gridDim.x) * 256)
    U[i] = rank_mul(mul, i / R, i % R, R, XA[i]);
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

int64_t rowdot_chunk(int64_t M, int64_t K, int64_t R) {
  const int64_t TK = skinny_wide(int(R)) ? 256 : 64;
  const int64_t rt = (M + kRowdotRows - 1) / kRowdotRows;
  const int64_t slices = (K + TK - 1) / TK;
  // about two workgroups per CU (512), but at least 4 slices per workgroup
  // while that keeps 256 or more: the next slice's loads fly during the
  // current products, so fewer, longer splits cost little and write fewer
  // partials
  int64_t ks = (512 + rt - 1) / rt;
  if (ks > slices / 4) ks = slices / 4;
  if (ks < (256 + rt - 1) / rt) ks = (256 + rt - 1) / rt;
  if (ks < 1) ks = 1;
  if (ks > slices) ks = slices;
  const int64_t per = (slices + ks - 1) / ks;   // slices per split
  return per * TK;
}

int64_t coldot_chunk(int64_t M, int64_t K, int64_t R) {
  const int64_t ct = (K + coldot_tn(int(R)) - 1) / coldot_tn(int(R));
  const int64_t mt = (M + 63) / 64;
  // splits of about 8 slices while that keeps the grid within two
  // workgroups per CU (512), and at least 256 workgroups
  int64_t ks = (mt + 7) / 8;
  if (ks > 512 / ct) ks = 512 / ct;
  if (ks < (256 + ct - 1) / ct) ks = (256 + ct - 1) / ct;
  if (ks < 1) ks = 1;
  if (ks > mt) ks = mt;
  const int64_t per = (mt + ks - 1) / ks;
  return per * 64;
}

RowdotArgs rowdot_args(const void *P, const void *Q, int64_t M, int64_t K, int64_t R,
                       float *part, int64_t &nwg) {
  RowdotArgs a;
  a.P = P; a.Q = Q; a.M = M; a.K = K; a.R = int(R);
  a.kchunk = rowdot_chunk(M, K, R);
  a.mt = (M + kRowdotRows - 1) / kRowdotRows;
  a.part = part;
  nwg = (M == 0 || R == 0) ? 0 : a.mt * ((K + a.kchunk - 1) / a.kchunk);
  return a;
}

ColdotArgs coldot_args(const void *P, const void *Q, int64_t ldq, int64_t M, int64_t K, int64_t R,
                       float *part, int64_t &nwg) {
  ColdotArgs a;
  a.P = P; a.Q = Q; a.ldq = ldq; a.M = M; a.K = K; a.R = int(R);
  a.mchunk = coldot_chunk(M, K, R);
  a.ct = (K + coldot_tn(int(R)) - 1) / coldot_tn(int(R));
  a.part = part;
  nwg = (M == 0 || R == 0) ? 0 : a.ct * ((M + a.mchunk - 1) / a.mchunk);
  return a;
}

size_t rowdot_lds(int64_t R) {
  const bool wide = skinny_wide(int(R));
  const size_t p = size_t(kRowdotRows) * (wide ? rowdot_ppitch<256>() : rowdot_ppitch<64>()) * 2;
  return p + size_t(rank_pad16(int(R))) * (wide ? 256 : 64) * 2;
}
size_t coldot_lds(int64_t R) {
  return size_t(64) * coldot_pitch(coldot_tn(int(R))) * 2 + size_t(rank_pad16(int(R))) * 64 * 2;
}

int rowfull_rows(int64_t M) { return M >= 4096 ? 16 : 8; }

// rowfull applies: enough rows for a full grid, R <= 32, and every buffer
// offset of a workgroup inside the 31-bit range of a raw buffer.
bool rowfull_fits(int64_t M, int64_t K, int64_t R) {
  return M >= kFullMinM && R > 0 && R <= 32 && int64_t(16) * K * 4 <= 0x7fffffff &&
         R * K * 4 <= 0x7fffffff;
}

RowfullArgs rowfull_args(const void *P, const void *Q, int64_t M, int64_t K, int64_t R, float *out,
                         uint16_t *out16, int64_t ld16, int64_t &nwg) {
  RowfullArgs a;
  a.P = P; a.Q = Q; a.M = M; a.K = K; a.R = int(R);
  a.rows = rowfull_rows(M);
  a.out = out; a.out16 = out16; a.ld16 = ld16;
  nwg = (M + a.rows - 1) / a.rows;
  return a;
}

}  // namespace

bool xa_complete(int64_t M, int64_t in, int64_t r) { return r % 8 == 0 && rowfull_fits(M, in, r); }
bool g_complete(int64_t M, int64_t out, int64_t r) { return rowfull_fits(M, out, r); }

int64_t rowdot_splits(int64_t M, int64_t K, int64_t R) {
  if (M == 0) return 0;
  const int64_t kc = rowdot_chunk(M, K, R);
  return (K + kc - 1) / kc;
}

int64_t coldot_splits(int64_t M, int64_t K, int64_t R) {
  if (M == 0) return 0;
  const int64_t mc = coldot_chunk(M, K, R);
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
                           int64_t in, int64_t r, float *xa_part, float *XA, uint16_t *XA16,
                           int64_t ld16, const int8_t *qscale, const float *gscale, int64_t out,
                           float *cs, hipStream_t s,
                         RankMul mul) {
  ScalesArgs sa{qscale, gscale, in, out / 64, cs};
  const int64_t n_sc = cs ? scales_workgroups(in, out / 64) : 0;
  if (r > 0 && xa_complete(M, in, r)) {
    int64_t n_full = 0;
    RowfullArgs fa = rowfull_args(X, A, M, in, r, XA, XA16, ld16, n_full);
    fa.mul = mul;
    const dim3 grid = dim3(unsigned(n_full + n_sc));
    const bool r8 = fa.rows == 8;
    const size_t lds1 = r8 ? rowfull_lds_bytes<kQFast, 1, 8>() : rowfull_lds_bytes<kQFast, 1, 16>();
    const size_t lds2 = r8 ? rowfull_lds_bytes<kQFast, 2, 8>() : rowfull_lds_bytes<kQFast, 2, 16>();
#define QLORA_FULL(XB, AB)                                                                      \
  do {                                                                                          \
    if (r <= 16)                                                                                \
      hipLaunchKernelGGL((fwd_full_kernel<XB, AB, 1>), grid, dim3(256), lds1, s, fa, n_sc, sa);  \
    else                                                                                        \
      hipLaunchKernelGGL((fwd_full_kernel<XB, AB, 2>), grid, dim3(256), lds2, s, fa, n_sc, sa);  \
  } while (0)
    if (x_bf16) {
      if (a_bf16) QLORA_FULL(true, true); else QLORA_FULL(true, false);
    } else {
      if (a_bf16) QLORA_FULL(false, true); else QLORA_FULL(false, false);
    }
#undef QLORA_FULL
    return hipGetLastError();
  }
  int64_t n_row = 0;
  const RowdotArgs ra = rowdot_args(X, A, M, in, r, xa_part, n_row);
  if (n_row + n_sc == 0) return hipSuccess;
  const size_t lds = n_row ? rowdot_lds(r) : 0;
  const dim3 grid = dim3(unsigned(n_row + n_sc));
#define QLORA_PREP2(XB, AB, W)                                                              \
  do {                                                                                      \
    if (r % 8 == 0)                                                                         \
      hipLaunchKernelGGL((fwd_prep_kernel<XB, AB, W, kQFast>), grid, dim3(256), lds, s, ra, n_sc, sa); \
    else                                                                                    \
      hipLaunchKernelGGL((fwd_prep_kernel<XB, AB, W, kQGeneric>), grid, dim3(256), lds, s, ra, n_sc, sa); \
  } while (0)
#define QLORA_PREP(XB, AB)                                                                  \
  do {                                                                                      \
    if (skinny_wide(int(r))) QLORA_PREP2(XB, AB, true); else QLORA_PREP2(XB, AB, false);    \
  } while (0)
  if (x_bf16) {
    if (a_bf16) QLORA_PREP(true, true); else QLORA_PREP(true, false);
  } else {
    if (a_bf16) QLORA_PREP(false, true); else QLORA_PREP(false, false);
  }
#undef QLORA_PREP2
#undef QLORA_PREP
  return hipGetLastError();
}

hipError_t launch_bwd_dy(const void *dY, bool dy_bf16, const void *B, bool b_bf16,
                         const float *XA, int64_t M, int64_t out, int64_t r, float *g_part,
                         uint16_t *G16, int64_t ldg, float *db_part, uint16_t *xat,
                         int64_t ldm, const int8_t *qscale, const float *gscale, int64_t in,
                         float *cs, hipStream_t s,
                         RankMul mul) {
  int64_t n_col = 0;
  const ColdotArgs ca = coldot_args(dY, XA, r, M, out, r, db_part, n_col);
  ScalesArgs sa{qscale, gscale, in, out / 64, cs};
  const int64_t n_sc = cs ? scales_workgroups(in, out / 64) : 0;
  if (xat && !(r > 0 && r <= 16 && g_complete(M, out, r) && ldm % 256 == 0 && ldm >= M))
    return hipErrorInvalidValue;
  if (r > 0 && g_complete(M, out, r)) {
    int64_t n_full = 0;
    RowfullArgs fa = rowfull_args(dY, B, M, out, r, nullptr, G16, ldg, n_full);
    fa.mul = mul;
    const XatArgs xa{XA, M, int(r), xat, ldm, mul};
    const int64_t n_xat = xat ? xat_workgroups(ldm) : 0;
    if (xat) n_col = 0;    // dB is formed by the dX GEMM
    const dim3 grid = dim3(unsigned(n_sc + n_xat + n_full + n_col));
    const size_t lds_full =
        fa.rows == 8 ? rowfull_lds_bytes<kQRows, 2, 8>() : rowfull_lds_bytes<kQRows, 2, 16>();
    const size_t lds = coldot_lds(r) > lds_full ? coldot_lds(r) : lds_full;
#define QLORA_DYF2(DB, BB, RT)                                                                  \
  do {                                                                                          \
    if (r % 8 == 0)                                                                             \
      hipLaunchKernelGGL((dy_full_kernel<DB, BB, RT, true>), grid, dim3(256), lds, s, fa, n_full, \
                         ca, n_sc, sa, n_xat, xa);                                              \
    else                                                                                        \
      hipLaunchKernelGGL((dy_full_kernel<DB, BB, RT, false>), grid, dim3(256), lds, s, fa,       \
                         n_full, ca, n_sc, sa, n_xat, xa);                                      \
  } while (0)
#define QLORA_DYF(DB, BB)                                                                       \
  do {                                                                                          \
    if (r <= 16) QLORA_DYF2(DB, BB, 1); else QLORA_DYF2(DB, BB, 2);                             \
  } while (0)
    if (dy_bf16) {
      if (b_bf16) QLORA_DYF(true, true); else QLORA_DYF(true, false);
    } else {
      if (b_bf16) QLORA_DYF(false, true); else QLORA_DYF(false, false);
    }
#undef QLORA_DYF2
#undef QLORA_DYF
    return hipGetLastError();
  }
  if (xat) return hipErrorInvalidValue;
  int64_t n_row = 0;
  const RowdotArgs ra = rowdot_args(dY, B, M, out, r, g_part, n_row);
  if (n_row + n_col + n_sc == 0) return hipSuccess;
  const size_t lds = (n_row + n_col) ? (coldot_lds(r) > rowdot_lds(r) ? coldot_lds(r) : rowdot_lds(r)) : 0;
  const dim3 grid = dim3(unsigned(n_row + n_col + n_sc));
#define QLORA_DY2(DB, BB, W)                                                                \
  do {                                                                                      \
    if (r % 8 == 0)                                                                         \
      hipLaunchKernelGGL((bwd_dy_kernel<DB, BB, W, true>), grid, dim3(256), lds, s, ra, n_row, ca, n_sc, sa); \
    else                                                                                    \
      hipLaunchKernelGGL((bwd_dy_kernel<DB, BB, W, false>), grid, dim3(256), lds, s, ra, n_row, ca, n_sc, sa); \
  } while (0)
#define QLORA_DY(DB, BB)                                                                    \
  do {                                                                                      \
    if (skinny_wide(int(r))) QLORA_DY2(DB, BB, true); else QLORA_DY2(DB, BB, false);        \
  } while (0)
  if (dy_bf16) {
    if (b_bf16) QLORA_DY(true, true); else QLORA_DY(true, false);
  } else {
    if (b_bf16) QLORA_DY(false, true); else QLORA_DY(false, false);
  }
#undef QLORA_DY2
#undef QLORA_DY
  return hipGetLastError();
}

hipError_t launch_bwd_x(const void *X, bool x_bf16, const uint16_t *G16, int64_t ldg, int64_t M,
                        int64_t in, int64_t r, float *da_part, hipStream_t s) {
  int64_t n_col = 0;
  const ColdotArgs ca = coldot_args(X, G16, ldg, M, in, r, da_part, n_col);
  if (n_col == 0) return hipSuccess;
  const dim3 grid = dim3(unsigned(n_col));
  const bool wide = skinny_wide(int(r));
  if (x_bf16) {
    if (wide) hipLaunchKernelGGL((bwd_x_kernel<true, true>), grid, dim3(256), coldot_lds(r), s, ca);
    else hipLaunchKernelGGL((bwd_x_kernel<true, false>), grid, dim3(256), coldot_lds(r), s, ca);
  } else {
    if (wide) hipLaunchKernelGGL((bwd_x_kernel<false, true>), grid, dim3(256), coldot_lds(r), s, ca);
    else hipLaunchKernelGGL((bwd_x_kernel<false, false>), grid, dim3(256), coldot_lds(r), s, ca);
  }
  return hipGetLastError();
}

hipError_t launch_rank_mul(const float *XA, int64_t M, int64_t R, RankMul mul, float *U,
                           hipStream_t s) {
  if (M * R == 0) return hipSuccess;
  hipLaunchKernelGGL(rank_mul_kernel, dim3(unsigned(grid_for(M * R))), dim3(256), 0, s, XA, M, R,
                     mul, U);
  return hipGetLastError();
}

hipError_t launch_reduce2(const float *part_a, int64_t ks_a, int64_t rows_a, int64_t R,
                          float *out_a, bool transpose_a, uint16_t *bf16_a, int64_t ld_a,
                          const float *part_b, int64_t ks_b, int64_t rows_b, float *out_b,
                          bool transpose_b, uint16_t *bf16_b, int64_t ld_b, hipStream_t s,
                         RankMul mul,
                          const AdamTarget &adam_a, const AdamTarget &adam_b) {
  ReduceArgs ra{part_a, ks_a, rows_a, R, out_a, transpose_a, bf16_a, ld_a, mul, adam_a};
  ReduceArgs rb{part_b, ks_b, rows_b, R, out_b, transpose_b, bf16_b, ld_b, RankMul(), adam_b};
  // one thread per 4 elements (vector form), else per element
  const int64_t per = R % 4 == 0 ? 4 : 1;
  const int64_t n_a = part_a ? grid_for(rows_a * (ld_a > R ? ld_a : R) / per) : 0;
  const int64_t n_b = part_b ? grid_for(rows_b * (ld_b > R ? ld_b : R) / per) : 0;
  if (n_a + n_b == 0) return hipSuccess;
  hipLaunchKernelGGL(reduce2_kernel, dim3(unsigned(n_a + n_b)), dim3(256), 0, s, ra, n_a, rb);
  return hipGetLastError();
}

bool da_whole(int64_t M, int64_t in, int64_t r, bool x_bf16) {
  // every offset of the whole-dA loads below 2^31 (a slab past the last can
  // reach 4 * 64 rows past M)
  const int64_t rows = M + 4 * 64 * 2;
  return r > 0 && r <= 16 && rows * in * (x_bf16 ? 2 : 4) <= 0x7fffffff && rows * 64 * 2 <= 0x7fffffff;
}

hipError_t launch_bwd_tail(const void *X, bool x_bf16, const uint16_t *G16, int64_t ldg,
                           int64_t M, int64_t in, int64_t r, float *dA, const AdamTarget &adam_a,
                           const float *part_b, int64_t ks_b, int64_t out, float *dB,
                           const AdamTarget &adam_b, hipStream_t s) {
  if (!da_whole(M, in, r, x_bf16) || in % 16 != 0 || ldg < 16 || ldg % 8 != 0 || ldg > 64)
    return hipErrorInvalidValue;
  DaFullArgs da{X, G16, ldg, M, in, int(r), dA, adam_a};
  const int64_t n_da = in / 16;
  ReduceArgs rb{part_b, ks_b, out, r, dB, true, nullptr, 0, RankMul(), adam_b};
  const int64_t n_b = part_b ? grid_for(out * r / (r % 4 == 0 ? 4 : 1)) : 0;
  const dim3 grid = dim3(unsigned(n_da + n_b));
  if (x_bf16)
    hipLaunchKernelGGL((bwd_tail_kernel<true>), grid, dim3(256), 0, s, da, n_da, rb);
  else
    hipLaunchKernelGGL((bwd_tail_kernel<false>), grid, dim3(256), 0, s, da, n_da, rb);
  return hipGetLastError();
}

}  // namespace qlora
