// Internal declarations shared by the host boundary and the kernel files.
#pragma once

#include <cstddef>
#include <cstdint>

#include <hip/hip_runtime_api.h>

namespace qlora {

// Multiplier of a rank-r intermediate (XA in the forward, G = dY B^T in the
// backward) on its way into the next product: the alpha / r factor and the
// dropout on A x ("LoRA & QLoRA", sections Scaling Factor alpha and Dropout).
// Element (m, j) of an [M x R] intermediate becomes c * v where keep is null
// or keep[m * R + j] != 0, and 0 elsewhere; c = 1 with no mask leaves v as is.
struct RankMul {
  const uint8_t *keep = nullptr;
  float c = 1.0f;
};

// One Adam (AdamW) step's constants, fp32 (the bias corrections and 1 - beta
// formed in double on the host, rounded once).
struct AdamParams {
  float lr, b1, omb1, b2, omb2, eps, wd, c1, c2;
};
AdamParams make_adam_params(int64_t step, float lr, float beta1, float beta2, float eps,
                            float weight_decay);

// An adapter matrix updated in place by one Adam step from a gradient that
// a reduction has just formed (theta == nullptr: none).  Same layout as the
// gradient the reduction writes.
struct AdamTarget {
  float *theta = nullptr;
  float *m = nullptr, *v = nullptr;
  uint16_t *theta16 = nullptr;    // optional bf16 copy of the updated theta
  AdamParams p{};
};

// Encoder thresholds, passed by value as a kernel argument.
// Encoder bucket table: x = w/absmax in [-1, 1] is bucketed by the top 7
// bits of the fp32 pattern of u = x + 3 past its exponent (u in [2, 4]):
// bucket i covers x in [-1 + i/32, -1 + (i+1)/32), bucket 64 is x = 1.  Every
// bucket holds at most one threshold, so code = base + (x >= T) with the
// bucket's entry (entries 65..127 are never addressed by finite x).
constexpr int kBuckets = 128;
struct BucketEntry {
  float T;              // the threshold inside the bucket, +inf if none
  uint32_t base;        // number of thresholds below the bucket
};
struct QuantConsts {
  BucketEntry bucket[kBuckets];
  int ok;               // 1 if the bucket scheme is exact for these thresholds
};

// The 8 level magnitudes |L|_m = L[8+m] (m = 0..7) as fp32; the fused GEMMs
// build their per-scale tables from them.
struct ExpandConsts {
  float mag[8];
};
struct ExpandConsts16 {
  uint32_t plane[2][2];  // bytes 2 and 3 of the bf16-rounded magnitudes
};

struct Tables {
  float L[16];
  float T[16];
  int symmetric;        // 1 if L[15 - i] == -L[i] for every i (the expansions need it)
  QuantConsts quant;
  ExpandConsts expand;
  ExpandConsts16 expand16;
};

// Codebooks (values of qlora_nf4.codebook): the level set of the 4-bit codes.
constexpr int kCodebookNF4 = 0;
constexpr int kCodebookUniform4 = 1;
constexpr int kCodebookInt4 = 2;      // symmetric integers -7..7 (/7)
constexpr int kCodebookInt3 = 3;      // -3..3 (/3)
constexpr int kCodebookTernary = 4;   // -1, 0, 1
constexpr int kCodebooks = 5;

// The tables of one codebook (built once, on first use).
const Tables &tables(int codebook);

// ---------------------------------------------------------------- launchers
// Every launcher enqueues on `s` and returns hipGetLastError() of the launch.

// g16: the 16-entry format (one fp32 absmax per 16 weights into gscale, no
// double quantization, qscale unused); nblocks counts 64-weight blocks.
hipError_t launch_quantize(const float *W0, uint8_t *codes, int8_t *qscale,
                           float *gscale, int64_t nblocks, int codebook, bool g16,
                           hipStream_t s);

// dst[n] (bf16) = src[n] (f32 or bf16)
hipError_t launch_convert_to_bf16(const void *src, bool src_bf16, int64_t n,
                                  uint16_t *dst, hipStream_t s);

// Number of split-K partials the rank-r passes write (host-only planning).
//   rowdot: C[M x R] = P[M x K] . Q, split over K;
//   coldot: C[K x R] = P[M x K]^T . Q[M x R], split over the tokens M.
int64_t rowdot_splits(int64_t M, int64_t K, int64_t R);
int64_t coldot_splits(int64_t M, int64_t K, int64_t R);

// Forward prep, one launch: the block scales cs[b][row] = q8[row][b] *
// s2[group] of the [in x out] weight (if cs != nullptr) and X . A (X [M x in],
// A [in x r], each f32 or bf16) -- complete into XA (fp32 [M x r]) and XA16
// (bf16 [M x ld16], zero-padded), each optional, when xa_complete(M, in, r),
// else as split-K partials xa_part[ks][M][r] for launch_reduce2.
bool xa_complete(int64_t M, int64_t in, int64_t r);
hipError_t launch_fwd_prep(const void *X, bool x_bf16, const void *A, bool a_bf16,
                           int64_t M, int64_t in, int64_t r, float *xa_part, float *XA,
                           uint16_t *XA16, int64_t ld16, const int8_t *qscale,
                           const float *gscale, int64_t out, float *cs, hipStream_t s,
                          RankMul mul = RankMul());

// Backward pass over dY, one launch: G = dY . B^T (B [r x out]) -- complete
// into G16 (bf16 [M x ldg], zero-padded) when g_complete(M, out, r), else as
// partials g_part[ks][M][r]; db_part[ks][out][r] = partial dY^T . XA (XA fp32
// [M x r]); and, if cs != nullptr, the block scales as in launch_fwd_prep.
// With xat != nullptr (only when r <= 16 and g_complete; ldm a multiple of
// 256, >= M) the dB partials are left to launch_dx_gemm and the launch
// instead writes xat [16 x ldm] = XA^T in bf16, zero-padded.
bool g_complete(int64_t M, int64_t out, int64_t r);
hipError_t launch_bwd_dy(const void *dY, bool dy_bf16, const void *B, bool b_bf16,
                         const float *XA, int64_t M, int64_t out, int64_t r,
                         float *g_part, uint16_t *G16, int64_t ldg, float *db_part,
                         uint16_t *xat, int64_t ldm, const int8_t *qscale,
                         const float *gscale, int64_t in, float *cs, hipStream_t s,
                          RankMul mul = RankMul());

// Backward pass over X: da_part[ks][in][r] = partial X^T . G with G given as
// G16 bf16 [M x ldg].
hipError_t launch_bwd_x(const void *X, bool x_bf16, const uint16_t *G16, int64_t ldg,
                        int64_t M, int64_t in, int64_t r, float *da_part,
                        hipStream_t s);

// Two fixed-order split sums in one launch.  For each of a, b (skipped when
// its part is nullptr): out[i] = sum_k part[k][i] over a [rows x R] result;
// outputs (each optional) fp32 ([R x rows] if transpose) and bf16
// [rows x ld] with zero padding columns R..ld-1.
// U = mul(XA) in fp32 ([M x R]), the dB operand of the dY pass when XA
// carries a multiplier.
hipError_t launch_rank_mul(const float *XA, int64_t M, int64_t R, RankMul mul, float *U,
                           hipStream_t s);

// dA = X^T . G whole, for 0 < r <= 16 (da_whole): G16 bf16 [M x ldg] (ldg a
// multiple of 8, 16 <= ldg <= 64, zero beyond r), dA fp32 [in x r] (in % 16 == 0),
// optionally with one Adam step of A (adam_a.theta != nullptr); in the same
// launch, if part_b != nullptr, dB[r x out] = the sum of ks_b partials
// part_b[ks][out][r] (optionally with Adam, adam_b) as launch_reduce2 forms it.
// The sums depend on the shapes only, not on which other outputs a call asks for.
bool da_whole(int64_t M, int64_t in, int64_t r, bool x_bf16);
hipError_t launch_bwd_tail(const void *X, bool x_bf16, const uint16_t *G16, int64_t ldg,
                           int64_t M, int64_t in, int64_t r, float *dA, const AdamTarget &adam_a,
                           const float *part_b, int64_t ks_b, int64_t out, float *dB,
                           const AdamTarget &adam_b, hipStream_t s);

hipError_t launch_reduce2(const float *part_a, int64_t ks_a, int64_t rows_a, int64_t R,
                          float *out_a, bool transpose_a, uint16_t *bf16_a, int64_t ld_a,
                          const float *part_b, int64_t ks_b, int64_t rows_b, float *out_b,
                          bool transpose_b, uint16_t *bf16_b, int64_t ld_b, hipStream_t s,
                          RankMul mul = RankMul(),
                          const AdamTarget &adam_a = AdamTarget(),
                          const AdamTarget &adam_b = AdamTarget());

// y = X16 . deq(Wq) + XA16 . B (K = in, N = out).  X16 [M x K] bf16; XA16
// [M x ldp] bf16 with zero padding columns r..ldp-1; B [r x N] (f32 or bf16)
// as given by the caller; cs from the prep pass (rows = K), or with g16 the
// weight's own fp32 scales [K][N/16].
hipError_t launch_fwd_gemm(const uint8_t *codes, const float *cs, int64_t K,
                           int64_t N, const uint16_t *X16, int64_t M,
                           const uint16_t *XA16, int32_t ldp, const void *B,
                           bool b_bf16, int32_t r, void *Y, bool y_bf16, int codebook,
                           bool g16, hipStream_t s);

// dX = dY16 . deq(Wq)^T + G16 . A^T.  dY16 [M x out] bf16; G16 [M x ldp] bf16
// zero-padded; A [in x r] (f32 or bf16) as given; cs as in the forward.
// With db_part != nullptr (r <= 16, r % 4 == 0, dx_fold_fits; xat from
// launch_bwd_dy) also db_part[ceil(M / 256)][out][r] = XA^T . dY over each
// 256-token block.
bool dx_fold_fits(int64_t M, int64_t in, int64_t out);
hipError_t launch_dx_gemm(const uint8_t *codes, const float *cs, int64_t in,
                          int64_t out, const uint16_t *dY16, int64_t M,
                          const uint16_t *G16, int32_t ldp, const void *A,
                          bool a_bf16, int32_t r, void *dX, bool dx_bf16, int codebook,
                          bool g16, const uint16_t *xat, int64_t ldm, float *db_part,
                          hipStream_t s);

// Small-M forward (M <= kSmallMaxM tokens, r <= kSmallMaxR), two launches:
// partials over K chunks of small_fwd_chunk_rows(M, K, N) rows,
//   P[ks][M][N] = X . deq(Wq) over the chunk, PXA[ks][M][r] = X . A over the
//   chunk (ks = number of chunks);
// then XA = sum_ks PXA (fp32 [M x r], optional when r == 0) and
//   Y = sum_ks P + XA . B (act dtype), both sums in a fixed order.
constexpr int kSmallMaxM = 16;
constexpr int kSmallMaxR = 64;
int64_t small_fwd_chunk_rows(int64_t M, int64_t K, int64_t N);
hipError_t launch_fwd_small_partial(const uint8_t *codes, const int8_t *qscale,
                                    const float *gscale, int64_t K, int64_t N, const void *X,
                                    bool x_bf16, int64_t M, const void *A, bool a_bf16, int64_t r,
                                    int64_t Kc, float *P, float *PXA, int codebook, bool g16,
                                    hipStream_t s);
hipError_t launch_fwd_small_reduce(const float *P, const float *PXA, int64_t KS, int64_t M,
                                   int64_t N, int64_t r, const void *B, bool b_bf16, float *XA,
                                   void *Y, bool y_bf16, hipStream_t s,
                          RankMul mul = RankMul());

// Up to kSmallMaxGroup independent few-token linears (same M, r and dtypes)
// in the same two launches: each workgroup of the partial pass (and of the
// reduction) is one of one linear's, so every linear's result is that of its
// own launch pair.
constexpr int kSmallMaxGroup = 4;
struct SmallLinear {
  const uint8_t *codes;
  const int8_t *qscale;
  const float *gscale;
  int64_t K, N;                 // in, out
  const void *X, *A, *B;
  int64_t Kc;                   // small_fwd_chunk_rows(M, K, N)
  float *P, *PXA;               // this linear's partials (workspace)
  float *XA;
  void *Y;
  RankMul mul;
};
hipError_t launch_fwd_small_group(int n, const SmallLinear *lin, int64_t M, bool x_bf16,
                                  bool a_bf16, int64_t r, int codebook, bool g16,
                                  hipStream_t s);

// W = deq(Wq) + A . B (W [in x out] fp32 or bf16; A [in x r], B [r x out]
// in the adapter dtype), per element in fp32, one rounding at the end.
hipError_t launch_merge(const uint8_t *codes, const int8_t *q8, const float *s2, int64_t in,
                        int64_t out, const void *A, const void *B, bool a_bf16, int32_t r,
                        void *W, bool w_bf16, int codebook, bool g16, hipStream_t s);

// One Adam (AdamW) step over n fp32 elements in place (bias corrections for
// step t >= 1); theta16, if not null, receives the updated theta as bf16.
hipError_t launch_adam(float *theta, const float *g, float *m, float *v, int64_t n, int64_t step,
                       float lr, float beta1, float beta2, float eps, float weight_decay,
                       uint16_t *theta16, hipStream_t s);

// The 16 fp32 levels of a codebook, passed by value to a kernel.
struct Levels16 {
  float L[16];
};

// Products with the quantization residual R = W0 - deq(Wq) (formed on the
// fly in fp32; g16: the 16-entry format, s2 = the fp32 scale per 16
// weights): transpose = false: Y [in x k] = R . M (M [out x k]);
// transpose = true: Y [out x k] = R^T . M (M [in x k]); 1 <= k <= 128.
// `partial` holds the slices' partial products:
// residual_mul_partial_bytes(in, out, k) bytes.
size_t residual_mul_partial_bytes(int64_t in, int64_t out, int k);
hipError_t launch_residual_mul(const float *W0, const uint8_t *codes, const int8_t *q8,
                               const float *s2, bool g16, int64_t in, int64_t out, const float *M,
                               int k, float *Y, bool transpose, int codebook, float *partial,
                               hipStream_t s);

// Thin-panel products for the orthonormalisation and the final factors, fp64
// arithmetic on fp32 panels (ka, kb, k, m <= 128):
// G [ka x kb] (fp64) = X^T . Y for X [rows x ka], Y [rows x kb] (`partial`:
// panel_gram_partial_bytes(max(ka, kb)) bytes);
// Out = X . T for X [rows x k] and T [k x m] fp64, rounded to fp32 (then to
// bf16 when `bf16`), Out [rows x m] or, `transposed`, [m x rows].
size_t panel_gram_partial_bytes(int k);
hipError_t launch_panel_gram(const float *X, int ka, const float *Y, int kb, int64_t rows,
                             double *G, double *partial, hipStream_t s);
hipError_t launch_panel_apply(const float *X, int k, const double *T, int m, int64_t rows,
                              void *Out, bool transposed, bool bf16, hipStream_t s);
// k x k steps on the GPU (one workgroup, fp64): T [k x k] = C^-1 for the
// Cholesky factor of the Gram matrix G (dependent columns leave as zero
// columns); P = [Pa | Pb'] ([k x r] each) from the SVD Rz^T = U S V^T, Rz
// [k x k] row-major: Pa = U_r S_r^(1/2), Pb' = U_r S_r^(-1/2) (so that
// Z Pb' = Qz V_r S_r^(1/2) when Rz = Qz^T Z).  k <= 128, r <= k.
hipError_t launch_chol_inv(const double *G, int k, double *T, hipStream_t s);
hipError_t launch_small_svd(const double *Rz, int k, int r, double *P, hipStream_t s);

inline int64_t rank_pad32(int64_t r) { return (r + 31) / 32 * 32; }
inline int64_t pad8(int64_t m) { return (m + 7) / 8 * 8; }

hipError_t launch_fill_zero(float *p, int64_t n, hipStream_t s);

// Size of the device-resident scratch array of the forward that allocates
// nothing, and the device address of the current device's copy (looked up
// once per device).
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
hipError_t noalloc_scratch(void **ptr);

}  // namespace qlora
