// Internal declarations shared by the host boundary and the kernel files.
#pragma once

#include <cstddef>
#include <cstdint>

#include <hip/hip_runtime_api.h>

namespace qlora {

// Encoder thresholds, passed by value as a kernel argument.
struct QuantConsts {
  float T[16];          // T[1..15]: code = #{j : x >= T[j]}; T[0] unused
};

// Byte planes of the 8 level magnitudes |L|_m = L[8+m], m = 0..7.
// plane[p][0] holds byte p of |L|_0..|L|_3, plane[p][1] of |L|_4..|L|_7.
struct ExpandConsts {
  uint32_t plane[4][2];
};
struct ExpandConsts16 {
  uint32_t plane[2][2];  // bytes 2 and 3 of the bf16-rounded magnitudes
};

struct Tables {
  float L[16];
  float T[16];
  QuantConsts quant;
  ExpandConsts expand;
  ExpandConsts16 expand16;
};

const Tables &tables();

// ---------------------------------------------------------------- launchers
// Every launcher enqueues on `s` and returns hipGetLastError() of the launch.

hipError_t launch_quantize(const float *W0, uint8_t *codes, int8_t *qscale,
                           float *gscale, int64_t nblocks, hipStream_t s);

// dst[j][k] = src[k][j] as bf16 for src [K x R] (f32 or bf16); dst rows have
// length ldd >= K and are zero-padded in [K, ldd).
hipError_t launch_transpose_to_bf16(const void *src, bool src_bf16, int64_t K,
                                    int64_t R, uint16_t *dst, int64_t ldd,
                                    hipStream_t s);
// dst[n] (bf16) = src[n] (f32 or bf16)
hipError_t launch_convert_to_bf16(const void *src, bool src_bf16, int64_t n,
                                  uint16_t *dst, hipStream_t s);

// part[ks][M][R] = sum over k in split ks of P[m][k] * Qt[j][k]
//   P: [M x K] (f32 or bf16), Qt: [R x K] bf16.  rowdot_splits gives the
//   number of splits (host-only planning).
int64_t rowdot_splits(int64_t M, int64_t K, int64_t R);
hipError_t launch_rowdot(const void *P, bool p_bf16, const uint16_t *Qt,
                         int64_t M, int64_t K, int64_t R, float *part,
                         hipStream_t s);

// part[ks][K][R] = sum over m in split ks of P[m][k] * Qt[j][m]
//   P: [M x K] (f32 or bf16), Qt: [R x ldq] bf16 (the transposed skinny
//   factor, ldq % 8 == 0)
int64_t coldot_splits(int64_t M, int64_t K, int64_t R);
hipError_t launch_coldot(const void *P, bool p_bf16, const uint16_t *Qt,
                         int64_t ldq, int64_t M, int64_t K, int64_t R,
                         float *part, hipStream_t s);

// out[i] = sum_ks part[ks][i] in ks order (fp32) for a [rows x R] result,
// with optional extra outputs: out (fp32; [R x rows] if transpose_out),
// out_bf16 ([rows x ld_bf16], zero-padded columns) and outT_bf16
// ([R x ldT]).
hipError_t launch_reduce(const float *part, int64_t ks, int64_t rows, int64_t R,
                         float *out, bool transpose_out, uint16_t *out_bf16,
                         int64_t ld_bf16, uint16_t *outT_bf16, int64_t ldT,
                         hipStream_t s);

// cs[b][row] = q8[row][b] * s2[group] (fp32) for a quantized [rows x cols]
// weight: the block scales, one row per 64-wide block column.
hipError_t launch_scales(const int8_t *qscale, const float *gscale, int64_t rows,
                         int64_t cols, float *cs, hipStream_t s);

// dst[i][j] = src[i][j] as bf16 for j < cols, 0 for cols <= j < ldd.
hipError_t launch_pad_to_bf16(const void *src, bool src_bf16, int64_t rows,
                              int64_t cols, uint16_t *dst, int64_t ldd,
                              hipStream_t s);

// y = X16 . deq(Wq) + XA16 . Bt^T (K = in, N = out).  X16 [M x K] bf16;
// XA16 [M x rp], Bt [N x rp] bf16 zero-padded (rp = round_up(r, 32), 0 for
// no adapter); cs from launch_scales(rows = K, cols = N).
hipError_t launch_fwd_gemm(const uint8_t *codes, const float *cs, int64_t K,
                           int64_t N, const uint16_t *X16, int64_t M,
                           const uint16_t *XA16, const uint16_t *Bt, int32_t rp,
                           void *Y, bool y_bf16, bool exact, hipStream_t s);

// dX = dY16 . deq(Wq)^T + G16 . A16^T.  dY16 [M x out] bf16; G16 [M x rp],
// A16 [in x rp] bf16 zero-padded; cs from launch_scales(rows = in, cols = out).
hipError_t launch_dx_gemm(const uint8_t *codes, const float *cs, int64_t in,
                          int64_t out, const uint16_t *dY16, int64_t M,
                          const uint16_t *G16, const uint16_t *A16, int32_t rp,
                          void *dX, bool dx_bf16, bool exact, hipStream_t s);

inline int64_t rank_pad32(int64_t r) { return (r + 31) / 32 * 32; }
inline int64_t pad8(int64_t m) { return (m + 7) / 8 * 8; }

hipError_t launch_fill_zero(float *p, int64_t n, hipStream_t s);

}  // namespace qlora
