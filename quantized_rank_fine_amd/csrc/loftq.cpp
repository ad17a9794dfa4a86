// LoftQ-style start of the adapters: A, B from a rank-r truncated SVD of the
// quantization residual R = W0 - deq(Wq).
//
// "QLoRA (low-rank adapters on a quantized model)", "What QLoRA adds" (the
// paragraph on running it): LoftQ-style methods start A and B from an SVD of
// W0 - Q(W0) instead of zero, so training starts closer to the original
// model.  The SVD is found by randomized subspace iteration (Halko,
// Martinsson & Tropp, "Finding structure with randomness": a range finder
// from the caller's random test matrix, power iterations with
// re-orthonormalisation, then the SVD of the small projected matrix):
//   Q = orth(R . Omega);  repeat: Q = orth(R . orth(R^T . Q));
//   Z = R^T . Q  (so R ~ Q Z^T);  Z = Qz Rz;  Rz^T = U~ S W~^T;
//   R ~ (Q U~) S (Qz W~)^T;  A = (Q U~)_r sqrt(S_r),  B = sqrt(S_r) (Qz W~)_r^T.
// The two large products run on the GPU (residual formed on the fly, fp32);
// the k x k and (rows x k) orthonormalisations and the small SVD (one-sided
// Jacobi rotations) run on the host in double.  The call is synchronous.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#include "internal.h"
#include "qlora.h"

namespace qlora {
namespace {

using Mat = std::vector<double>;   // row-major

// Orthonormal columns of X (rows x k) by modified Gram-Schmidt, applied
// twice; a column that vanishes becomes zero.
// (The columns are copied out contiguously first, so every pass streams.)
void orthonormalize(Mat &X, int64_t rows, int k) {
  Mat C(X.size());
  for (int64_t i = 0; i < rows; ++i)
    for (int j = 0; j < k; ++j) C[j * rows + i] = X[i * k + j];
  for (int pass = 0; pass < 2; ++pass) {
    for (int j = 0; j < k; ++j) {
      double *cj = C.data() + j * rows;
      for (int p = 0; p < j; ++p) {
        const double *cp = C.data() + p * rows;
        double d = 0.0;
        for (int64_t i = 0; i < rows; ++i) d += cp[i] * cj[i];
        for (int64_t i = 0; i < rows; ++i) cj[i] -= d * cp[i];
      }
      double n2 = 0.0;
      for (int64_t i = 0; i < rows; ++i) n2 += cj[i] * cj[i];
      const double inv = n2 > 1e-300 ? 1.0 / std::sqrt(n2) : 0.0;
      for (int64_t i = 0; i < rows; ++i) cj[i] *= inv;
    }
  }
  for (int64_t i = 0; i < rows; ++i)
    for (int j = 0; j < k; ++j) X[i * k + j] = C[j * rows + i];
}

// C (k x k) = Q^T X for Q, X (rows x k).
Mat gram(const Mat &Q, const Mat &X, int64_t rows, int k) {
  Mat C(size_t(k) * k, 0.0);
  for (int64_t i = 0; i < rows; ++i)
    for (int a = 0; a < k; ++a) {
      const double q = Q[i * k + a];
      for (int b = 0; b < k; ++b) C[a * k + b] += q * X[i * k + b];
    }
  return C;
}

// One-sided Jacobi SVD of a square k x k matrix G: rotate column pairs until
// all are orthogonal; then G V = U S with V the accumulated rotations, S the
// column norms.  G is overwritten by U S.
void jacobi_svd(Mat &G, Mat &V, std::vector<double> &S, int k) {
  V.assign(size_t(k) * k, 0.0);
  for (int i = 0; i < k; ++i) V[i * k + i] = 1.0;
  for (int sweep = 0; sweep < 80; ++sweep) {
    bool rotated = false;
    for (int p = 0; p < k - 1; ++p)
      for (int q = p + 1; q < k; ++q) {
        double a = 0.0, b = 0.0, g = 0.0;
        for (int i = 0; i < k; ++i) {
          a += G[i * k + p] * G[i * k + p];
          b += G[i * k + q] * G[i * k + q];
          g += G[i * k + p] * G[i * k + q];
        }
        if (std::fabs(g) <= 1e-15 * std::sqrt(a * b) || g == 0.0) continue;
        rotated = true;
        const double zeta = (b - a) / (2.0 * g);
        const double t = (zeta >= 0 ? 1.0 : -1.0) / (std::fabs(zeta) + std::sqrt(1.0 + zeta * zeta));
        const double c = 1.0 / std::sqrt(1.0 + t * t), s = c * t;
        for (int i = 0; i < k; ++i) {
          const double gp = G[i * k + p], gq = G[i * k + q];
          G[i * k + p] = c * gp - s * gq;
          G[i * k + q] = s * gp + c * gq;
          const double vp = V[i * k + p], vq = V[i * k + q];
          V[i * k + p] = c * vp - s * vq;
          V[i * k + q] = s * vp + c * vq;
        }
      }
    if (!rotated) break;
  }
  S.assign(k, 0.0);
  for (int j = 0; j < k; ++j) {
    double n2 = 0.0;
    for (int i = 0; i < k; ++i) n2 += G[i * k + j] * G[i * k + j];
    S[j] = std::sqrt(n2);
  }
}

struct Residual {
  const float *W0;
  const qlora_nf4 *wq;
  float *dM, *dY;      // device [max(in, out) x k] each
  int k;
  hipStream_t s;
};

// Y = R . M (transpose = false; M rows = out, Y rows = in) or R^T . M.
hipError_t residual_product(const Residual &r, const Mat &M, Mat &Y, bool transpose) {
  const int64_t in = r.wq->in, out = r.wq->out;
  const int64_t mrows = transpose ? in : out, yrows = transpose ? out : in;
  std::vector<float> mf(M.begin(), M.end());
  hipError_t e = hipMemcpyAsync(r.dM, mf.data(), sizeof(float) * mf.size(),
                                hipMemcpyHostToDevice, r.s);
  if (e != hipSuccess) return e;
  e = launch_residual_mul(r.W0, r.wq->codes, r.wq->qscale, r.wq->gscale, in, out, r.dM, r.k,
                          r.dY, transpose, r.wq->codebook, r.s);
  if (e != hipSuccess) return e;
  std::vector<float> yf(size_t(yrows) * r.k);
  e = hipMemcpyAsync(yf.data(), r.dY, sizeof(float) * yf.size(), hipMemcpyDeviceToHost, r.s);
  if (e != hipSuccess) return e;
  e = hipStreamSynchronize(r.s);
  (void)mrows;
  Y.assign(yf.begin(), yf.end());
  return e;
}

}  // namespace
}  // namespace qlora

using namespace qlora;

extern "C" size_t qlora_loftq_workspace_bytes(int64_t in, int64_t out, int32_t k) {
  if (in <= 0 || out <= 0 || k < 1 || k > 128) return 0;
  const size_t rows = size_t(in > out ? in : out);
  return 2 * ((rows * size_t(k) * 4 + 255) / 256 * 256);
}

extern "C" qlora_status qlora_loftq_init(const float *W0, const qlora_nf4 *wq, const float *omega,
                                         int32_t k, int32_t r, int32_t iters, void *A, void *B,
                                         qlora_dtype adt, void *ws, size_t ws_bytes,
                                         hipStream_t stream) {
  if (!wq || !W0 || !omega || !A || !B || !ws) return QLORA_ERR_NULL;
  if (wq->in <= 0 || wq->out <= 0 || wq->in % 64 || wq->out % 64) return QLORA_ERR_SHAPE;
  if (wq->codebook < 0 || wq->codebook >= kCodebooks) return QLORA_ERR_DTYPE;
  if (wq->block != 0 && wq->block != QLORA_BLOCK) return QLORA_ERR_DTYPE;   // 64-weight format only
  if (!wq->codes || !wq->qscale || !wq->gscale) return QLORA_ERR_NULL;
  if (adt != QLORA_F32 && adt != QLORA_BF16) return QLORA_ERR_DTYPE;
  if (k < 1 || k > 128 || r < 1 || r > k || k > wq->in || k > wq->out || iters < 0 || iters > 16)
    return QLORA_ERR_SHAPE;
  const uintptr_t al = reinterpret_cast<uintptr_t>(W0) | reinterpret_cast<uintptr_t>(omega) |
                       reinterpret_cast<uintptr_t>(A) | reinterpret_cast<uintptr_t>(B) |
                       reinterpret_cast<uintptr_t>(ws) |
                       reinterpret_cast<uintptr_t>(wq->codes) |
                       reinterpret_cast<uintptr_t>(wq->qscale) |
                       reinterpret_cast<uintptr_t>(wq->gscale);
  if (al & 15u) return QLORA_ERR_ALIGN;
  if (ws_bytes < qlora_loftq_workspace_bytes(wq->in, wq->out, k)) return QLORA_ERR_WORKSPACE;
  const int64_t in = wq->in, out = wq->out;
  const size_t half = qlora_loftq_workspace_bytes(in, out, k) / 2;
  Residual res{W0, wq, static_cast<float *>(ws),
               reinterpret_cast<float *>(static_cast<char *>(ws) + half), k, stream};

  // range finder from the caller's test matrix
  std::vector<float> om(size_t(out) * k);
  if (hipMemcpyAsync(om.data(), omega, sizeof(float) * om.size(), hipMemcpyDeviceToHost, stream) !=
          hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return QLORA_ERR_DEVICE;
  Mat M(om.begin(), om.end()), Y, Z;
  if (residual_product(res, M, Y, false) != hipSuccess) return QLORA_ERR_DEVICE;
  orthonormalize(Y, in, k);
  for (int it = 0; it < iters; ++it) {
    if (residual_product(res, Y, Z, true) != hipSuccess) return QLORA_ERR_DEVICE;
    orthonormalize(Z, out, k);
    if (residual_product(res, Z, Y, false) != hipSuccess) return QLORA_ERR_DEVICE;
    orthonormalize(Y, in, k);
  }
  // R ~ Y Z^T with Z = R^T Y
  if (residual_product(res, Y, Z, true) != hipSuccess) return QLORA_ERR_DEVICE;
  Mat Qz = Z;
  orthonormalize(Qz, out, k);
  const Mat Rz = gram(Qz, Z, out, k);                  // Z = Qz Rz
  Mat G(size_t(k) * k);                                 // G = Rz^T
  for (int a = 0; a < k; ++a)
    for (int b = 0; b < k; ++b) G[a * k + b] = Rz[b * k + a];
  Mat W;
  std::vector<double> S;
  jacobi_svd(G, W, S, k);                               // G W = U~ S
  std::vector<int> ord(k);
  for (int j = 0; j < k; ++j) ord[j] = j;
  std::stable_sort(ord.begin(), ord.end(), [&](int x, int y) { return S[x] > S[y]; });

  // A = (Y U~)_r sqrt(S_r), B = sqrt(S_r) (Qz W~)_r^T
  std::vector<float> af(size_t(in) * r), bf(size_t(r) * out);
  for (int c = 0; c < r; ++c) {
    const int j = ord[c];
    const double sj = S[j], sq = std::sqrt(sj);
    for (int64_t i = 0; i < in; ++i) {
      double u = 0.0;
      if (sj > 0)
        for (int a = 0; a < k; ++a) u += Y[i * k + a] * G[a * k + j] / sj;
      af[i * r + c] = float(u * sq);
    }
    for (int64_t n = 0; n < out; ++n) {
      double v = 0.0;
      for (int a = 0; a < k; ++a) v += Qz[n * k + a] * W[a * k + j];
      bf[size_t(c) * out + n] = float(v * sq);
    }
  }
  hipError_t e = hipSuccess;
  if (adt == QLORA_F32) {
    e = hipMemcpyAsync(A, af.data(), sizeof(float) * af.size(), hipMemcpyHostToDevice, stream);
    if (e == hipSuccess)
      e = hipMemcpyAsync(B, bf.data(), sizeof(float) * bf.size(), hipMemcpyHostToDevice, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
  } else {
    auto to16 = [](float f) {
      uint32_t u;
      std::memcpy(&u, &f, 4);
      u += 0x7fffu + ((u >> 16) & 1u);
      return uint16_t(u >> 16);
    };
    std::vector<uint16_t> a16(af.size()), b16(bf.size());
    for (size_t i = 0; i < af.size(); ++i) a16[i] = to16(af[i]);
    for (size_t i = 0; i < bf.size(); ++i) b16[i] = to16(bf[i]);
    e = hipMemcpyAsync(A, a16.data(), 2 * a16.size(), hipMemcpyHostToDevice, stream);
    if (e == hipSuccess)
      e = hipMemcpyAsync(B, b16.data(), 2 * b16.size(), hipMemcpyHostToDevice, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
  }
  return e == hipSuccess ? QLORA_OK : QLORA_ERR_DEVICE;
}
