// Products with the quantization residual R = W0 - deq(Wq), for the
// LoftQ-style start of the adapters (a rank-r SVD of the residual).
//
// "QLoRA (low-rank adapters on a quantized model)", "What QLoRA adds" (the
// paragraph on running it): LoftQ-style methods start A and B from an SVD of
// W0 - Q(W0) instead of zero.  The truncated SVD is found by randomized
// subspace iteration, which touches R only through the products
//   Y = R . M   (M [out x k], Y [in x k])   and   Z = R^T . Q   (Q [in x k]),
// k <= 128 columns.  R is never stored: each tile of it is formed in fp32
// (W0 minus L[code] * (q_b * s2_g), or L[code] * c_g in the 16-entry format:
// the value the fused GEMMs round to bf16)
// and multiplied with fp32 multiply-adds.  The thin panels between the
// products are orthonormalised here as well (Cholesky QR applied twice: the
// k x k Gram matrix and the panel update run on the GPU in fp64 arithmetic),
// and the final factors are formed from them.
#include <type_traits>

#include "device.h"

namespace qlora {
namespace {

constexpr int kMaxK = 128;
constexpr int64_t kMaxSlices = 16;   // slices of a residual product's summed axis
constexpr int64_t kGramSlabs = 64;   // workgroups (partial sums) of a Gram matrix

struct ResidualArgs {
  const float *W0;
  const uint8_t *codes;
  const int8_t *q8;
  const float *s2;    // 64-weight blocks: one fp32 scale per 256 blocks; g16: one per 16 weights
  int64_t in, out;
  const float *M;     // rmul: [out x k]; rtmul: [in x k]
  int k;
  float *Y;           // rmul: [in x k]; rtmul: [out x k]; one such block per slice
  int64_t span;       // length of a slice of the summed axis (a multiple of the chunk)
};

// The dequantization scale of flat weight f, as loaded (int8 q_b and the
// fp32 s2_g for 64-weight blocks; the group's fp32 absmax for the 16-entry
// format, with q = 1), and its value q * s -- the product the fused GEMMs
// form.  The kernels load it with the rest of a chunk and form the value
// only when the chunk is used, so that no wait follows the loads.
struct RawScale {
  int q;
  float s;
};

template <bool kG16>
__device__ __forceinline__ RawScale load_scale(const ResidualArgs &a, int64_t f) {
  if constexpr (kG16) return RawScale{1, a.s2[f / 16]};
  const int64_t blk = f / 64;
  return RawScale{int(a.q8[blk]), a.s2[blk >> 8]};
}

__device__ __forceinline__ float scale_value(RawScale r) { return float(r.q) * r.s; }

// The level table into LDS from one lane: the kernel argument's values come
// through scalar registers, so that staging them waits on no vector load.
__device__ __forceinline__ void stage_levels(float *sL, const Levels16 &lv, int t) {
  if (t == 0) {
#pragma unroll
    for (int i = 0; i < 16; ++i) sL[i] = lv.L[i];
  }
}

// Y = R . M on the fp32 matrix cores (v_mfma_f32_32x32x2_f32, products and
// sums in fp32).  Workgroup = 4 wavefronts = 128 rows of R and one slice of
// the out axis (blockIdx.y; its partial product goes to block blockIdx.y of
// Y), walked in chunks of 64 columns.  Lane l of a wavefront forms the 32
// residual elements of row l % 32, columns c0 + 32 (l / 32) .. + 31 (one
// 128-B line of W0, one 64-block), and feeds them as the A operand, one per
// step s: the two k slots of a step are columns c0 + s and c0 + 32 + s.  The
// B operand (the matching rows of M, staged in LDS per chunk and shared by
// the four wavefronts) gives output columns 32 t + l % 32 of tile t < KT.
// The next chunk's loads are in flight while the current one is multiplied.
template <int KT, bool kG16>
__global__ __launch_bounds__(256) void rmul_mfma_kernel(ResidualArgs a, Levels16 lv) {
  constexpr int KP = 32 * KT;
  __shared__ float sL[16];
  __shared__ __align__(16) float sM[64][KP + 1];   // (+1: the two half-waves' rows on other banks)
  const int t = threadIdx.x, l = t & 63, w = t >> 6, h = l >> 5;
  const int64_t row = int64_t(blockIdx.x) * 128 + 32 * w + (l & 31);
  const bool live = row < a.in;                 // in % 64 == 0: whole wavefronts
  const int64_t nb = int64_t(blockIdx.y) * a.span, ne = min64(a.out, nb + a.span);
  // the chunk's M rows: thread t stages (row e / KP, column e % KP) for
  // e = t + 256 u (columns >= k are zero)
  constexpr int MPER = 64 * KP / 256;
  float mv[MPER];
  uint32_t mok = 0;                             // bit u: mv[u] is a row of M (else it stages 0)
  f32x4_t wv[8];
  u32x4_t cv;
  RawScale cs{0, 0.0f}, cs2{0, 0.0f};
  // Every load is unconditional, so that no wait follows it: a row past
  // `in` reads row 0 (its wavefront writes nothing) and a staging slot
  // past k or out reads M[0] and is masked when it is stored.
  auto load = [&](int64_t c0) {
    const int64_t flat = live ? row * a.out + c0 + 32 * h : 0;
    const f32x4_t *src = reinterpret_cast<const f32x4_t *>(a.W0 + flat);
#pragma unroll
    for (int q = 0; q < 8; ++q) wv[q] = src[q];
    cv = *reinterpret_cast<const u32x4_t *>(a.codes + flat / 2);
    cs = load_scale<kG16>(a, flat);
    cs2 = kG16 ? load_scale<kG16>(a, flat + 16) : cs;   // elements 16..31 (another group)
    mok = 0;
#pragma unroll
    for (int u = 0; u < MPER; ++u) {
      const int e = t + 256 * u, n = e / KP, j = e - n * KP;
      const bool ok = j < a.k && c0 + n < a.out;
      mv[u] = a.M[ok ? (c0 + n) * a.k + j : 0];
      mok |= uint32_t(ok) << u;
    }
  };
  f32x16_t acc[KT];
#pragma unroll
  for (int q = 0; q < KT; ++q)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[q][e] = 0.0f;
  load(nb);
  stage_levels(sL, lv, t);                      // (visible at the loop's first barrier)
  for (int64_t c0 = nb; c0 < ne; c0 += 64) {
    __syncthreads();                            // the previous chunk's reads are done
#pragma unroll
    for (int u = 0; u < MPER; ++u) {
      const int e = t + 256 * u, n = e / KP, j = e - n * KP;
      sM[n][j] = (mok >> u) & 1u ? mv[u] : 0.0f;
    }
    float rv[32];
    const float c1 = scale_value(cs), c2 = scale_value(cs2);
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const uint32_t code = (cv[e >> 3] >> (4 * (e & 7))) & 15u;
      rv[e] = wv[e >> 2][e & 3] - sL[code] * (e < 16 ? c1 : c2);
    }
    __syncthreads();
    if (c0 + 64 < ne) load(c0 + 64);            // in flight during the products
#pragma unroll
    for (int st = 0; st < 32; ++st)
#pragma unroll
      for (int q = 0; q < KT; ++q)
        acc[q] = __builtin_amdgcn_mfma_f32_32x32x2f32(rv[st], sM[32 * h + st][32 * q + (l & 31)],
                                                      acc[q], 0, 0, 0);
  }
  if (!live) return;
  // register e of lane l: row 8 (e / 4) + 4 (l / 32) + e % 4 of the
  // wavefront's 32, column 32 q + l % 32
  float *Y = a.Y + int64_t(blockIdx.y) * a.in * a.k;
  const int64_t rb = int64_t(blockIdx.x) * 128 + 32 * w;
#pragma unroll
  for (int q = 0; q < KT; ++q) {
    const int j = 32 * q + (l & 31);
    if (j >= a.k) continue;
#pragma unroll
    for (int e = 0; e < 16; ++e)
      Y[(rb + 8 * (e >> 2) + 4 * h + (e & 3)) * a.k + j] = acc[q][e];
  }
}

// Z = R^T . Q on the fp32 matrix cores.  Output rows are columns of R:
// tile p < NQ of a wavefront holds the columns c0 + NQ m + p, m < 32, so a
// lane loads NQ consecutive elements of a row of R at once; output columns
// are 32 t + l % 32 for tiles t < KT.  Step s multiplies rows i0 + 2 s and
// i0 + 2 s + 1 (lane l takes row i0 + 2 s + l / 32 as its k slot); the B
// operand (the matching rows of Q) is the same for all NQ tiles.
// Workgroup = 4 wavefronts on the same 32 NQ columns, each over a quarter of
// the workgroup's slice of the in axis (blockIdx.y); their sums are added
// in wavefront order through LDS, and the slice's partial product goes to
// block blockIdx.y of Z.  Rows are walked 16 at a time, the next 16 loaded
// while the current ones are multiplied.
template <int KT, int NQ, bool kG16>
__global__ __launch_bounds__(256) void rtmul_mfma_kernel(ResidualArgs a, Levels16 lv) {
  __shared__ float sL[16];
  __shared__ float sRed[3][KT * NQ * 16][64];
  const int t = threadIdx.x, l = t & 63, w = t >> 6, h = l >> 5, m = l & 31;
  const int64_t c = int64_t(blockIdx.x) * 32 * NQ + NQ * m;   // first of the lane's columns
  const bool live = c < a.out;                                // out % 64 == 0
  const int64_t sb = int64_t(blockIdx.y) * a.span, se = min64(a.in, sb + a.span);
  const int64_t q4 = (se - sb + 3) / 4;                        // this wavefront's quarter
  const int64_t ib = min64(se, sb + w * q4), ie = min64(se, ib + q4);
  f32x16_t acc[NQ][KT];
#pragma unroll
  for (int p = 0; p < NQ; ++p)
#pragma unroll
    for (int q = 0; q < KT; ++q)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[p][q][e] = 0.0f;
  float wv[8][NQ], bq[8][KT];
  RawScale cs[8];
  uint32_t cd[8];
  uint32_t rok = 0, bok = 0;   // bit st: step st's row is in the slice; bit st KT + q: its M entry is
  // Every load is unconditional, so that no wait follows it: a row past the
  // quarter or a column past out reads element 0 and is masked at use.
  auto load = [&](int64_t i0) {
    rok = 0;
    bok = 0;
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const int64_t i = i0 + 2 * st + h;
      const bool ok = live && i < ie;
      const int64_t flat = ok ? i * a.out + c : 0;
      if constexpr (NQ == 4) {
        const f32x4_t v = *reinterpret_cast<const f32x4_t *>(a.W0 + flat);
#pragma unroll
        for (int p = 0; p < 4; ++p) wv[st][p] = v[p];
        cd[st] = *reinterpret_cast<const uint16_t *>(a.codes + flat / 2);
      } else if constexpr (NQ == 2) {
        const float2 v = *reinterpret_cast<const float2 *>(a.W0 + flat);
        wv[st][0] = v.x;
        wv[st][1] = v.y;
        cd[st] = a.codes[flat / 2];
      } else {
        wv[st][0] = a.W0[flat];
        cd[st] = uint32_t(a.codes[flat / 2]) >> (4 * (flat & 1));
      }
      cs[st] = load_scale<kG16>(a, flat);     // the lane's NQ columns lie in one group
      rok |= uint32_t(ok) << st;
#pragma unroll
      for (int q = 0; q < KT; ++q) {
        const int j = 32 * q + m;
        const bool okb = i < ie && j < a.k;
        bq[st][q] = a.M[okb ? i * a.k + j : 0];
        bok |= uint32_t(okb) << (st * KT + q);
      }
    }
  };
  load(ib);                                     // (an empty quarter: all masked)
  stage_levels(sL, lv, t);
  __syncthreads();
  for (int64_t i0 = ib; i0 < ie; i0 += 16) {
    float rv[8][NQ], bv[8][KT];
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const bool okr = (rok >> st) & 1u;
#pragma unroll
      for (int p = 0; p < NQ; ++p)
        rv[st][p] = okr ? wv[st][p] - sL[(cd[st] >> (4 * p)) & 15u] * scale_value(cs[st]) : 0.0f;
#pragma unroll
      for (int q = 0; q < KT; ++q) bv[st][q] = (bok >> (st * KT + q)) & 1u ? bq[st][q] : 0.0f;
    }
    if (i0 + 16 < ie) load(i0 + 16);            // in flight during the products
#pragma unroll
    for (int st = 0; st < 8; ++st)
#pragma unroll
      for (int p = 0; p < NQ; ++p)
#pragma unroll
        for (int q = 0; q < KT; ++q)
          acc[p][q] = __builtin_amdgcn_mfma_f32_32x32x2f32(rv[st][p], bv[st][q], acc[p][q], 0, 0, 0);
  }
  // the four quarters, added in wavefront order
  if (w > 0) {
#pragma unroll
    for (int p = 0; p < NQ; ++p)
#pragma unroll
      for (int q = 0; q < KT; ++q)
#pragma unroll
        for (int e = 0; e < 16; ++e) sRed[w - 1][(p * KT + q) * 16 + e][l] = acc[p][q][e];
  }
  __syncthreads();
  if (w > 0) return;
  // register e of lane l: output row 8 (e / 4) + 4 (l / 32) + e % 4 of the
  // tile, i.e. column c0 + NQ (that row) + p of R (past out in a last,
  // half-filled workgroup: not written)
  float *Z = a.Y + int64_t(blockIdx.y) * a.out * a.k;
  const int64_t c0 = int64_t(blockIdx.x) * 32 * NQ;
#pragma unroll
  for (int p = 0; p < NQ; ++p)
#pragma unroll
    for (int q = 0; q < KT; ++q) {
      const int j = 32 * q + m;
      if (j >= a.k) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t col = c0 + NQ * (8 * (e >> 2) + 4 * h + (e & 3)) + p;
        if (col >= a.out) continue;
        const int slot = (p * KT + q) * 16 + e;
        const float v = ((acc[p][q][e] + sRed[0][slot][l]) + sRed[1][slot][l]) + sRed[2][slot][l];
        Z[col * a.k + j] = v;
      }
    }
}

// Y[e] = sum over s of P[s n + e], s in order (the slices' partial products).
__global__ __launch_bounds__(256) void slice_sum_kernel(const f32x4_t *P, int64_t n4, int S,
                                                        f32x4_t *Y) {
  const int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (e >= n4) return;
  f32x4_t p[kMaxSlices];
#pragma unroll
  for (int sl = 0; sl < kMaxSlices; ++sl)
    if (sl < S) p[sl] = P[sl * n4 + e];       // all loads first, then the sum in order
  f32x4_t v = p[0];
#pragma unroll
  for (int sl = 1; sl < kMaxSlices; ++sl)
    if (sl < S) v += p[sl];
  Y[e] = v;
}

// ---- panel kernels of the orthonormalisation (CholeskyQR2) and the final
// factors: fp32 panels [rows x k], fp64 arithmetic --------------------------

// G [ka x kb] (fp64) = X^T . Y for X [rows x ka], Y [rows x kb] fp32, in
// two passes.  Pass 1: workgroup w takes the 32-row slabs w, w + W, ... of
// both panels through LDS; thread t owns the entries e = t + 256 u of G
// (row-major) and sums their products over its slabs in fp64, in row order;
// the W partial matrices go to P.  Pass 2 adds them in workgroup order, so the
// result does not depend on timing.
template <int NE>
__global__ __launch_bounds__(256) void panel_gram_kernel(const float *X, int ka, const float *Y,
                                                         int kb, int64_t rows, double *P) {
  __shared__ float sX[32][kMaxK + 1], sY[32][kMaxK + 1];
  const int t = threadIdx.x, n = ka * kb;
  double acc[NE];
#pragma unroll
  for (int u = 0; u < NE; ++u) acc[u] = 0.0;
  for (int64_t r0 = int64_t(blockIdx.x) * 32; r0 < rows; r0 += int64_t(gridDim.x) * 32) {
    __syncthreads();                              // the previous slab's reads are done
    for (int e = t; e < 32 * ka; e += 256) {
      const int i = e / ka, a = e - i * ka;
      sX[i][a] = r0 + i < rows ? X[(r0 + i) * ka + a] : 0.0f;
    }
    for (int e = t; e < 32 * kb; e += 256) {
      const int i = e / kb, b = e - i * kb;
      sY[i][b] = r0 + i < rows ? Y[(r0 + i) * kb + b] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < NE; ++u) {
      const int e = t + 256 * u;
      if (e < n) {
        const int a = e / kb, b = e - a * kb;
        double v = acc[u];
#pragma unroll 8
        for (int i = 0; i < 32; ++i) v = __builtin_fma(double(sX[i][a]), double(sY[i][b]), v);
        acc[u] = v;
      }
    }
  }
#pragma unroll
  for (int u = 0; u < NE; ++u) {
    const int e = t + 256 * u;
    if (e < n) P[int64_t(blockIdx.x) * n + e] = acc[u];
  }
}

__global__ __launch_bounds__(256) void gram_sum_kernel(const double *P, int W, int n, double *G) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= n) return;
  double v = 0.0;
  for (int w0 = 0; w0 < W; w0 += 16) {
    double p[16];
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (w0 + u < W) p[u] = P[int64_t(w0 + u) * n + e];   // loads first, then the sum in order
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (w0 + u < W) v = (w0 + u == 0) ? p[u] : v + p[u];
  }
  G[e] = v;
}

// Out = X . T for X [rows x k] fp32 and T [k x m] fp64 (m <= 128), products
// summed in fp64 and rounded once to fp32 (and then, for bf16 output, from
// that fp32 value to bf16, nearest even).  Out is [rows x m], or [m x rows]
// when `transposed`.  Workgroup = 32 rows x 32 columns of Out, both operand
// tiles staged in LDS; thread t computes column t % 32 of rows t / 32 + 8 j.
__global__ __launch_bounds__(256) void panel_apply_kernel(const float *X, int k, const double *T,
                                                          int m, int64_t rows, void *Out,
                                                          bool transposed, bool bf16) {
  __shared__ float sX[32][129];
  __shared__ double sT[128][33];
  const int t = threadIdx.x;
  const int64_t i0 = int64_t(blockIdx.x) * 32;
  const int c0 = 32 * blockIdx.y;
  for (int e = t; e < 32 * k; e += 256) {
    const int i = e / k, a = e - i * k;
    sX[i][a] = i0 + i < rows ? X[(i0 + i) * k + a] : 0.0f;
  }
  for (int e = t; e < k * 32; e += 256) {
    const int a = e >> 5, c = e & 31;
    sT[a][c] = c0 + c < m ? T[a * m + c0 + c] : 0.0;
  }
  __syncthreads();
  const int c = t & 31;
  if (c0 + c >= m) return;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = (t >> 5) + 8 * j;
    if (i0 + i >= rows) break;
    double acc = 0.0;
    for (int a = 0; a < k; ++a) acc = __builtin_fma(double(sX[i][a]), sT[a][c], acc);
    const float v = float(acc);
    const int64_t o = transposed ? int64_t(c0 + c) * rows + i0 + i : (i0 + i) * m + c0 + c;
    if (bf16)
      static_cast<__bf16 *>(Out)[o] = (__bf16)v;
    else
      static_cast<float *>(Out)[o] = v;
  }
}

// ---- k x k steps of the orthonormalisation and of the final SVD, one
// workgroup each, in fp64, so that the call never waits for the host.

// T = C^-1 for the upper-triangular Cholesky factor C of the k x k Gram
// matrix G = C^T C (Cholesky QR, Fukaya et al.).  A column whose remaining
// squared length falls to 1e-12 of its own (or to nothing) depends on the
// columns before it: its row of C and its column of T are zero, so it leaves
// the panel as a zero column, as it would from Gram-Schmidt.  One wavefront:
// G is factored in place in LDS (right-looking: row j of C is finished at
// step j and the trailing upper triangle updated, so entry (j, l) receives
// the subtractions of rows 0 .. j-1 in that order); then lane t forms
// columns t, t + 64 of T by back substitution, each column stored in the
// free lower triangle (T[i][j], i < j, at row j, column i; the diagonal
// apart), so the lanes need no barrier between rows.
constexpr int kCholThreads = 64;

// The k x k row-major src (global fp64) into LDS with row pitch P, by nt
// threads, 16 loads per thread in flight before any is stored.
__device__ __forceinline__ void load_small(double *dst, const double *src, int k, int P, int t,
                                           int nt) {
  const int n = k * k;
  for (int base = 0; base < n; base += 16 * nt) {
    double v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int e = base + u * nt + t;
      v[u] = src[e < n ? e : 0];
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int e = base + u * nt + t;
      if (e < n) dst[(e / k) * P + e % k] = v[u];
    }
  }
}

constexpr int kSmallLds = kMaxK * (kMaxK + 1);

__global__ __launch_bounds__(kCholThreads) void chol_inv_kernel(const double *G, int k, double *T) {
  __shared__ double sA[kMaxK * (kMaxK + 8)];
  __shared__ double sDiag[kMaxK], sTd[kMaxK];
  __shared__ int sLive[kMaxK];
  const int t = threadIdx.x, P = (k + 7) | 1;       // odd pitch, >= 7 zero columns past k
  for (int e = t; e < k * P; e += kCholThreads) sA[e] = 0.0;
  __syncthreads();
  load_small(sA, G, k, P, t, kCholThreads);
  __syncthreads();
  for (int j = t; j < k; j += kCholThreads) sDiag[j] = sA[j * P + j];
  __syncthreads();
  for (int j = 0; j < k; ++j) {
    const double d = sA[j * P + j], own = sDiag[j];
    const bool live = own > 1e-300 && d > 1e-12 * own;
    double inv = 0.0;
    if (live) {                                      // 1 / sqrt(d): rsq and one Newton step
      inv = __builtin_amdgcn_rsq(d);
      inv = inv * __builtin_fma(-0.5 * d * inv, inv, 1.5);
    }
    const double cjj = d * inv;
    __syncthreads();                                 // every lane has read d
    for (int l = j + t; l < k; l += kCholThreads)
      sA[j * P + l] = live ? (l == j ? cjj : sA[j * P + l] * inv) : 0.0;
    if (t == 0) {
      sLive[j] = live;
      sTd[j] = inv;                                  // T[j][j] = 1 / C[j][j]
    }
    __syncthreads();                                 // row j of C is final
    // trailing update, one row l per lane: A[l][m] -= C[j][l] C[j][m], m >= l
    // (8 columns at a time; the zero columns past k absorb the overshoot)
    for (int l = j + 1 + t; l < k; l += kCholThreads) {
      const double cl = sA[j * P + l];
      for (int m0 = l; m0 < k; m0 += 8) {
        double cm[8], am[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          cm[u] = sA[j * P + m0 + u];
          am[u] = sA[l * P + m0 + u];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) sA[l * P + m0 + u] = __builtin_fma(-cl, cm[u], am[u]);
      }
    }
    __syncthreads();
  }
  for (int j = t; j < k; j += kCholThreads) {
    const double tjj = sTd[j];
    for (int i = j - 1; i >= 0; --i) {
      double v = 0.0;
      if (sLive[i]) {
        double acc = sA[i * P + j] * tjj;            // p = j
#pragma unroll 8
        for (int p = j - 1; p > i; --p) acc = __builtin_fma(sA[i * P + p], sA[j * P + p], acc);
        v = -acc * sTd[i];
      }
      sA[j * P + i] = v;                             // T[i][j]
    }
  }
  __syncthreads();
  for (int e = t; e < k * k; e += kCholThreads) {
    const int i = e / k, j = e - i * k;
    T[e] = i < j ? sA[j * P + i] : (i == j ? sTd[j] : 0.0);
  }
}

// v summed over the four lanes of its quad (DPP quad permutations).
__device__ __forceinline__ double quad_sum(double v) {
  auto perm = [](double x, auto ctrl) {
    constexpr int c = decltype(ctrl)::value;
    const int lo = __builtin_amdgcn_mov_dpp(__double2loint(x), c, 0xF, 0xF, true);
    const int hi = __builtin_amdgcn_mov_dpp(__double2hiint(x), c, 0xF, 0xF, true);
    return __hiloint2double(hi, lo);
  };
  v += perm(v, std::integral_constant<int, 0xB1>{});   // lanes ^ 1
  v += perm(v, std::integral_constant<int, 0x4E>{});   // lanes ^ 2
  return v;
}

// The rank-r factors of the k x k matrix Rz^T (Rz = Qz^T Z, row-major):
// one-sided Jacobi SVD (Hestenes) of G = Rz^T -- column pairs are rotated
// until every pair is orthogonal, so that G V = U S with orthonormal V and
// the rotated columns g_j = u_j s_j -- and then P = [Pa | Pb'] [k x r each]
// for the r largest singular values in descending order (ties: lower index
// first): Pa = U_r S_r^(1/2), column j of Pb' = g_j / s_j^(3/2).  V is not
// formed: Qz V_r S_r^(1/2) = Qz Rz U_r S_r^(-1/2) = Z Pb', so B^T = Z Pb'
// (Z = Qz Rz, Qz an orthonormal basis of Z's columns).  A sweep visits every pair once in the round-robin order (k/2
// disjoint pairs per step, one quad of lanes each); sweeps repeat until one
// rotates nothing (|g_p . g_q| <= 1e-10 |g_p| |g_q|: singular vectors far
// beyond the fp32 accuracy of the factors), at most 80.  The
// workgroup has 4 lanes per pair (one wavefront up to k = 32); a lane keeps
// its rows of the pair's two columns in registers for the step.
constexpr int kSvdMaxThreads = 4 * (kMaxK / 2);

template <int RPL>   // rows of G per lane: k <= 4 RPL
__global__ __launch_bounds__(kSvdMaxThreads) void small_svd_kernel(const double *Rz, int k, int r,
                                                                   double *P) {
  // column j of G at sG[j LP ..] (row j of Rz), rows k .. 4 RPL - 1 and the
  // round robin's padding column k (odd k) zero, so that every access of a
  // step is unconditional: zero rows and columns stay zero under rotation
  __shared__ double sG[kSmallLds];
  __shared__ double sS[kMaxK];
  __shared__ int sOrd[kMaxK];
  __shared__ int sRot;
  constexpr int LP = 4 * RPL + 1;
  const int t = threadIdx.x, nt = blockDim.x, g = t >> 2, li = t & 3;
  const int kp = (k + 1) & ~1;                       // players of the round robin
  for (int e = t; e < kp * LP; e += nt) sG[e] = 0.0;
  __syncthreads();
  load_small(sG, Rz, k, LP, t, nt);
  const int n1 = kp - 1;
  // round-robin positions: pair g holds the players at positions g and
  // kp - 1 - g; position 0 keeps player 0, position m >= 1 holds player
  // (m - 1 + step) mod (kp - 1) + 1
  auto player = [&](int m, int step) {
    if (m == 0) return 0;
    int v = m - 1 + step;
    if (v >= n1) v -= n1;
    return v + 1;
  };
  for (int sweep = 0; sweep < 80; ++sweep) {
    if (t == 0) sRot = 0;
    __syncthreads();
    for (int step = 0; step < n1; ++step) {
      if (g < kp / 2) {
        double *gp = sG + player(g, step) * LP + li, *gq = sG + player(kp - 1 - g, step) * LP + li;
        double x[RPL], y[RPL];
#pragma unroll
        for (int u = 0; u < RPL; ++u) {
          x[u] = gp[4 * u];
          y[u] = gq[4 * u];
        }
        double a = 0.0, b = 0.0, c = 0.0;
#pragma unroll
        for (int u = 0; u < RPL; ++u) {
          a = __builtin_fma(x[u], x[u], a);
          b = __builtin_fma(y[u], y[u], b);
          c = __builtin_fma(x[u], y[u], c);
        }
        a = quad_sum(a);
        b = quad_sum(b);
        c = quad_sum(c);
        if (c != 0.0 && c * c > 1e-20 * (a * b)) {
          // tan of the rotation angle, t = sign(z) / (|z| + sqrt(1 + z^2)) for
          // z = (b - a) / 2c (1 / 2z for |z| > 1e15: the same to fp64 rounding,
          // and z^2 never overflows); cos and sin from t with one Newton step on rsq, so the
          // rotation is orthogonal to fp64 rounding.  (An fp32 tangent took
          // as many sweeps and was 4 % slower.)
          const double zeta = (b - a) / (2.0 * c);
          const double tt = fabs(zeta) > 1e15
                                ? 0.5 / zeta
                                : (zeta >= 0.0 ? 1.0 : -1.0) / (fabs(zeta) + sqrt(__builtin_fma(zeta, zeta, 1.0)));
          const double w = __builtin_fma(tt, tt, 1.0);
          double cs = __builtin_amdgcn_rsq(w);
          cs = cs * __builtin_fma(-0.5 * w * cs, cs, 1.5);          // one Newton step
          const double sn = cs * tt;
#pragma unroll
          for (int u = 0; u < RPL; ++u) {
            gp[4 * u] = cs * x[u] - sn * y[u];
            gq[4 * u] = sn * x[u] + cs * y[u];
          }
          if (li == 0) sRot = 1;
        }
      }
      __syncthreads();
    }
    const int rot = sRot;
    __syncthreads();                                 // every thread has read the flag
    if (!rot) break;
  }
  for (int j = t; j < kMaxK; j += nt) sOrd[j] = 0;   // (no gaps even if S holds NaN)
  for (int j = t; j < k; j += nt) {
    double n2 = 0.0;
    for (int i = 0; i < k; ++i) n2 = __builtin_fma(sG[j * LP + i], sG[j * LP + i], n2);
    sS[j] = sqrt(n2);
  }
  __syncthreads();
  for (int j = t; j < k; j += nt) {
    int rank = 0;
    for (int i = 0; i < k; ++i) rank += (sS[i] > sS[j]) || (sS[i] == sS[j] && i < j);
    sOrd[rank] = j;
  }
  __syncthreads();
  double *Pa = P, *Pb = P + k * r;
  for (int e = t; e < k * r; e += nt) {
    const int a = e / r, cc = e - a * r, j = sOrd[cc];
    const double sj = sS[j];
    double pa = 0.0, pb = 0.0;
    if (sj > 0.0) {
      const double sq = sqrt(sj), gj = sG[j * LP + a];
      pa = gj / sq;
      pb = gj / (sj * sq);
    }
    Pa[e] = pa;
    Pb[e] = pb;
  }
}

}  // namespace

namespace {

// Slices of the summed axis (each a whole number of chunks of `ch`) so that a
// product of `base` wavefronts launches about 2048, two per SIMD, so that one
// wavefront's loads are in flight while the other multiplies (1024: one per
// SIMD took 34 and 41 us for the two products at 4096^2, 2048: 28 and 33 us;
// 4096 gained nothing more).
int64_t slice_span(int64_t base, int64_t len, int64_t ch) {
  const int64_t chunks = (len + ch - 1) / ch;
  int64_t S = (2048 + base - 1) / base;
  if (S > chunks) S = chunks;
  if (S > kMaxSlices) S = kMaxSlices;
  if (S < 1) S = 1;
  return (chunks + S - 1) / S * ch;
}

}  // namespace

size_t residual_mul_partial_bytes(int64_t in, int64_t out, int k) {
  const int64_t rows = in > out ? in : out;
  return size_t(kMaxSlices) * size_t(rows) * size_t(k) * 4;
}

hipError_t launch_residual_mul(const float *W0, const uint8_t *codes, const int8_t *q8,
                               const float *s2, bool g16, int64_t in, int64_t out, const float *M,
                               int k, float *Y, bool transpose, int codebook, float *partial,
                               hipStream_t s) {
  if (k < 1 || k > kMaxK) return hipErrorInvalidValue;
  Levels16 lv;
  const Tables &tb = tables(codebook);
  for (int i = 0; i < 16; ++i) lv.L[i] = tb.L[i];
  // in % 64 == 0 and out % 64 == 0 (checked by the caller): whole 16-row
  // and 32-column workgroups; the kernels zero what a last chunk has past
  // the end.  The summed axis is cut into slices whose partial products
  // are added in slice order.
  const int kt = k <= 32 ? 1 : (k <= 64 ? 2 : 4);   // 32-column output tiles
  int64_t span, nrows, base, len;
  if (!transpose) {
    base = (in + 127) / 128, len = out, nrows = in;
    span = slice_span(4 * base, len, 64);
  } else {
    const int nq = 4 / kt;                         // columns of R per lane
    base = (out + 32 * nq - 1) / (32 * nq), len = in, nrows = out;
    span = slice_span(4 * base, len, 64);
  }
  const int64_t S = (len + span - 1) / span;
  ResidualArgs a{W0, codes, q8, s2, in, out, M, k, S > 1 ? partial : Y, span};
  const dim3 g = dim3(unsigned(base), unsigned(S));
#define QLORA_RES(G)                                                                             \
  do {                                                                                           \
    if (!transpose) {                                                                            \
      if (kt == 1) hipLaunchKernelGGL((rmul_mfma_kernel<1, G>), g, dim3(256), 0, s, a, lv);      \
      else if (kt == 2) hipLaunchKernelGGL((rmul_mfma_kernel<2, G>), g, dim3(256), 0, s, a, lv); \
      else hipLaunchKernelGGL((rmul_mfma_kernel<4, G>), g, dim3(256), 0, s, a, lv);              \
    } else {                                                                                     \
      if (kt == 1) hipLaunchKernelGGL((rtmul_mfma_kernel<1, 4, G>), g, dim3(256), 0, s, a, lv);  \
      else if (kt == 2) hipLaunchKernelGGL((rtmul_mfma_kernel<2, 2, G>), g, dim3(256), 0, s, a, lv); \
      else hipLaunchKernelGGL((rtmul_mfma_kernel<4, 1, G>), g, dim3(256), 0, s, a, lv);          \
    }                                                                                            \
  } while (0)
  if (g16) QLORA_RES(true); else QLORA_RES(false);
#undef QLORA_RES
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || S == 1) return e;
  const int64_t n4 = nrows * k / 4;                // nrows % 64 == 0
  hipLaunchKernelGGL(slice_sum_kernel, dim3(unsigned((n4 + 255) / 256)), dim3(256), 0, s,
                     reinterpret_cast<const f32x4_t *>(partial), n4, int(S),
                     reinterpret_cast<f32x4_t *>(Y));
  return hipGetLastError();
}

size_t panel_gram_partial_bytes(int k) { return size_t(kGramSlabs) * size_t(k) * size_t(k) * 8; }

hipError_t launch_panel_gram(const float *X, int ka, const float *Y, int kb, int64_t rows,
                             double *G, double *partial, hipStream_t s) {
  if (ka < 1 || kb < 1 || ka > kMaxK || kb > kMaxK || rows < 1) return hipErrorInvalidValue;
  const int n = ka * kb;
  int64_t W = (rows + 31) / 32;
  if (W > kGramSlabs) W = kGramSlabs;
  const dim3 g = dim3(unsigned(W));
  if (n <= 256) hipLaunchKernelGGL(panel_gram_kernel<1>, g, dim3(256), 0, s, X, ka, Y, kb, rows, partial);
  else if (n <= 1024) hipLaunchKernelGGL(panel_gram_kernel<4>, g, dim3(256), 0, s, X, ka, Y, kb, rows, partial);
  else if (n <= 4096) hipLaunchKernelGGL(panel_gram_kernel<16>, g, dim3(256), 0, s, X, ka, Y, kb, rows, partial);
  else hipLaunchKernelGGL(panel_gram_kernel<64>, g, dim3(256), 0, s, X, ka, Y, kb, rows, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gram_sum_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s, partial,
                     int(W), n, G);
  return hipGetLastError();
}

hipError_t launch_panel_apply(const float *X, int k, const double *T, int m, int64_t rows,
                              void *Out, bool transposed, bool bf16, hipStream_t s) {
  if (k < 1 || m < 1 || k > kMaxK || m > kMaxK || rows < 1) return hipErrorInvalidValue;
  const dim3 g(unsigned((rows + 31) / 32), unsigned((m + 31) / 32));
  hipLaunchKernelGGL(panel_apply_kernel, g, dim3(256), 0, s, X, k, T, m, rows, Out, transposed,
                     bf16);
  return hipGetLastError();
}

hipError_t launch_chol_inv(const double *G, int k, double *T, hipStream_t s) {
  if (k < 1 || k > kMaxK) return hipErrorInvalidValue;
  hipLaunchKernelGGL(chol_inv_kernel, dim3(1), dim3(kCholThreads), 0, s, G, k, T);
  return hipGetLastError();
}

hipError_t launch_small_svd(const double *Rz, int k, int r, double *P, hipStream_t s) {
  if (k < 1 || k > kMaxK || r < 1 || r > k) return hipErrorInvalidValue;
  const int pairs = (k + 1) / 2;
  const unsigned threads = unsigned((4 * pairs + 63) / 64 * 64);   // whole wavefronts
  if (k <= 32)
    hipLaunchKernelGGL(small_svd_kernel<8>, dim3(1), dim3(threads), 0, s, Rz, k, r, P);
  else if (k <= 64)
    hipLaunchKernelGGL(small_svd_kernel<16>, dim3(1), dim3(threads), 0, s, Rz, k, r, P);
  else
    hipLaunchKernelGGL(small_svd_kernel<32>, dim3(1), dim3(threads), 0, s, Rz, k, r, P);
  return hipGetLastError();
}

}  // namespace qlora
