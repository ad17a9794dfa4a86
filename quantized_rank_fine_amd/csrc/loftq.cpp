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
//   Y = orth(R . Omega);  repeat: Z = orth(R^T . Y), Y = orth(R . Z);
//   Z = R^T . Y  (so R ~ Y Z^T);  Qz = orth(Z), Rz = Qz^T Z;  Rz^T = U~ S W~^T;
//   R ~ (Y U~) S (Qz W~)^T;  A = (Y U~)_r sqrt(S_r),  B = sqrt(S_r) (Qz W~)_r^T.
// orth is Cholesky QR applied twice (Fukaya, Nakatsukasa, Yanagisawa &
// Yamamoto, "CholeskyQR2: a simple and communication-avoiding algorithm for
// computing a tall-skinny QR factorization"): G = X^T X, G = C^T C with C
// upper triangular, X <- X C^-1; the second pass restores the orthogonality
// the first loses to rounding.  The panels stay on the GPU in fp32; the GPU
// forms the residual products, the Gram matrices and every panel update (in
// fp64 arithmetic).  The host does O(k^3) work only: the k x k Cholesky
// factor and its inverse, and the k x k SVD (one-sided Jacobi rotations), in
// double.  The call is synchronous.
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

// T = C^-1 for the upper-triangular Cholesky factor C of the k x k Gram
// matrix G (G = C^T C).  A column whose remaining squared length falls to
// 1e-12 of its own (or to nothing) depends on the columns before it: its row
// of C and its column of T are zero, so it leaves the panel as a zero
// column, as it would from Gram-Schmidt.
void cholesky_inverse(const Mat &G, int k, Mat &T) {
  Mat C(size_t(k) * k, 0.0);
  std::vector<char> live(k, 0);
  for (int j = 0; j < k; ++j) {
    double d = G[j * k + j];
    for (int p = 0; p < j; ++p) d -= C[p * k + j] * C[p * k + j];
    const double own = G[j * k + j];
    if (!(own > 1e-300) || !(d > 1e-12 * own)) continue;
    live[j] = 1;
    const double cjj = std::sqrt(d);
    C[j * k + j] = cjj;
    for (int l = j + 1; l < k; ++l) {
      double v = G[j * k + l];
      for (int p = 0; p < j; ++p) v -= C[p * k + j] * C[p * k + l];
      C[j * k + l] = v / cjj;
    }
  }
  // back substitution, one column of T at a time: C T = I on the live set
  T.assign(size_t(k) * k, 0.0);
  for (int j = 0; j < k; ++j) {
    if (!live[j]) continue;
    T[j * k + j] = 1.0 / C[j * k + j];
    for (int i = j - 1; i >= 0; --i) {
      if (!live[i]) continue;
      double v = 0.0;
      for (int p = i + 1; p <= j; ++p) v += C[i * k + p] * T[p * k + j];
      T[i * k + j] = -v / C[i * k + i];
    }
  }
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

// Device panels and the small host buffers of one call.
struct Ctx {
  const float *W0;
  const qlora_nf4 *wq;
  double *dG, *dT;     // device [k x k] Gram matrix, [2 k x k] transforms
  float *rpart;        // device partial products of the residual products
  double *gpart;       // device partial Gram matrices
  Mat hG, hT;
  hipStream_t s;
};

// Y = R . M (M [out x k] -> Y [in x k]) or, transposed, R^T . M.
hipError_t residual_product(const Ctx &c, const float *M, int k, float *Y, bool transpose) {
  return launch_residual_mul(c.W0, c.wq->codes, c.wq->qscale, c.wq->gscale,
                             c.wq->block == QLORA_LAB_GROUP, c.wq->in, c.wq->out, M, k, Y,
                             transpose, c.wq->codebook, c.rpart, c.s);
}

// H [ka x kb] on the host = X^T . Y (device panels [rows x ka], [rows x kb]).
hipError_t gram_to_host(Ctx &c, const float *X, int ka, const float *Y, int kb, int64_t rows,
                        Mat &H) {
  hipError_t e = launch_panel_gram(X, ka, Y, kb, rows, c.dG, c.gpart, c.s);
  if (e != hipSuccess) return e;
  H.assign(size_t(ka) * kb, 0.0);
  e = hipMemcpyAsync(H.data(), c.dG, sizeof(double) * H.size(), hipMemcpyDeviceToHost, c.s);
  if (e != hipSuccess) return e;
  return hipStreamSynchronize(c.s);
}

// Orthonormal columns of the device panel X [rows x k] (Cholesky QR, twice);
// Xt is a panel of the same size used in between.  The result is in X.
hipError_t orthonormalize(Ctx &c, float *X, float *Xt, int64_t rows, int k) {
  float *src = X, *dst = Xt;
  for (int pass = 0; pass < 2; ++pass) {
    hipError_t e = gram_to_host(c, src, k, src, k, rows, c.hG);
    if (e != hipSuccess) return e;
    cholesky_inverse(c.hG, k, c.hT);
    // (the host buffer is rewritten only after the next synchronisation,
    // which follows this copy on the stream)
    e = hipMemcpyAsync(c.dT, c.hT.data(), sizeof(double) * c.hT.size(), hipMemcpyHostToDevice,
                       c.s);
    if (e != hipSuccess) return e;
    e = launch_panel_apply(src, k, c.dT, k, rows, dst, false, false, c.s);
    if (e != hipSuccess) return e;
    std::swap(src, dst);
  }
  return hipSuccess;
}

size_t panel_bytes(int64_t rows, int k) { return (size_t(rows) * size_t(k) * 4 + 255) / 256 * 256; }
size_t small_bytes(int k) { return (size_t(k) * size_t(k) * 8 + 255) / 256 * 256; }
size_t align256(size_t b) { return (b + 255) / 256 * 256; }

}  // namespace
}  // namespace qlora

using namespace qlora;

extern "C" size_t qlora_loftq_workspace_bytes(int64_t in, int64_t out, int32_t k) {
  if (in <= 0 || out <= 0 || k < 1 || k > 128) return 0;
  // Y, Y' [in x k]; Z, Qz, Z' [out x k] fp32; G [k x k], T [2 k x k] fp64;
  // the partial sums of the residual products and of the Gram matrices
  return 2 * panel_bytes(in, k) + 3 * panel_bytes(out, k) + 3 * small_bytes(k) +
         align256(residual_mul_partial_bytes(in, out, k)) + align256(panel_gram_partial_bytes(k));
}

extern "C" qlora_status qlora_loftq_init(const float *W0, const qlora_nf4 *wq, const float *omega,
                                         int32_t k, int32_t r, int32_t iters, void *A, void *B,
                                         qlora_dtype adt, void *ws, size_t ws_bytes,
                                         hipStream_t stream) {
  if (!wq || !W0 || !omega || !A || !B || !ws) return QLORA_ERR_NULL;
  if (wq->in <= 0 || wq->out <= 0 || wq->in % 64 || wq->out % 64) return QLORA_ERR_SHAPE;
  if (wq->codebook < 0 || wq->codebook >= kCodebooks) return QLORA_ERR_DTYPE;
  if (wq->block != 0 && wq->block != QLORA_BLOCK && wq->block != QLORA_LAB_GROUP)
    return QLORA_ERR_DTYPE;
  const bool g16 = wq->block == QLORA_LAB_GROUP;
  if (!wq->codes || !wq->gscale || (!g16 && !wq->qscale)) return QLORA_ERR_NULL;
  if (adt != QLORA_F32 && adt != QLORA_BF16) return QLORA_ERR_DTYPE;
  if (k < 1 || k > 128 || r < 1 || r > k || k > wq->in || k > wq->out || iters < 0 || iters > 16)
    return QLORA_ERR_SHAPE;
  const uintptr_t al = reinterpret_cast<uintptr_t>(W0) | reinterpret_cast<uintptr_t>(omega) |
                       reinterpret_cast<uintptr_t>(A) | reinterpret_cast<uintptr_t>(B) |
                       reinterpret_cast<uintptr_t>(ws) |
                       reinterpret_cast<uintptr_t>(wq->codes) |
                       (g16 ? 0 : reinterpret_cast<uintptr_t>(wq->qscale)) |
                       reinterpret_cast<uintptr_t>(wq->gscale);
  if (al & 15u) return QLORA_ERR_ALIGN;
  if (ws_bytes < qlora_loftq_workspace_bytes(wq->in, wq->out, k)) return QLORA_ERR_WORKSPACE;
  const int64_t in = wq->in, out = wq->out;
  char *p = static_cast<char *>(ws);
  auto take = [&](size_t bytes) {
    char *q = p;
    p += bytes;
    return q;
  };
  float *Y = reinterpret_cast<float *>(take(panel_bytes(in, k)));
  float *Yt = reinterpret_cast<float *>(take(panel_bytes(in, k)));
  float *Z = reinterpret_cast<float *>(take(panel_bytes(out, k)));
  float *Qz = reinterpret_cast<float *>(take(panel_bytes(out, k)));
  float *Zt = reinterpret_cast<float *>(take(panel_bytes(out, k)));
  double *dG = reinterpret_cast<double *>(take(small_bytes(k)));
  double *dT = reinterpret_cast<double *>(take(2 * small_bytes(k)));
  float *rpart = reinterpret_cast<float *>(take(align256(residual_mul_partial_bytes(in, out, k))));
  double *gpart = reinterpret_cast<double *>(take(align256(panel_gram_partial_bytes(k))));
  Ctx c{W0, wq, dG, dT, rpart, gpart, {}, {}, stream};
  auto run = [&]() -> hipError_t {
    hipError_t e;
#define QLORA_TRY(x)              \
  if ((e = (x)) != hipSuccess) return e
    // range finder from the caller's test matrix, then the power iterations
    QLORA_TRY(residual_product(c, omega, k, Y, false));
    QLORA_TRY(orthonormalize(c, Y, Yt, in, k));
    for (int it = 0; it < iters; ++it) {
      QLORA_TRY(residual_product(c, Y, k, Z, true));
      QLORA_TRY(orthonormalize(c, Z, Zt, out, k));
      QLORA_TRY(residual_product(c, Z, k, Y, false));
      QLORA_TRY(orthonormalize(c, Y, Yt, in, k));
    }
    // R ~ Y Z^T with Z = R^T Y;  Z = Qz Rz
    QLORA_TRY(residual_product(c, Y, k, Z, true));
    QLORA_TRY(hipMemcpyAsync(Qz, Z, sizeof(float) * size_t(out) * k, hipMemcpyDeviceToDevice,
                             stream));
    QLORA_TRY(orthonormalize(c, Qz, Zt, out, k));
    Mat Rz;
    QLORA_TRY(gram_to_host(c, Qz, k, Z, k, out, Rz));
    Mat G(size_t(k) * k);                                 // G = Rz^T
    for (int a = 0; a < k; ++a)
      for (int b = 0; b < k; ++b) G[a * k + b] = Rz[b * k + a];
    Mat W;
    std::vector<double> S;
    jacobi_svd(G, W, S, k);                               // G W = U~ S
    std::vector<int> ord(k);
    for (int j = 0; j < k; ++j) ord[j] = j;
    std::stable_sort(ord.begin(), ord.end(), [&](int x, int y) { return S[x] > S[y]; });
    // A = Y Pa, B^T = Qz Pb with Pa = (U~)_r sqrt(S_r), Pb = (W~)_r sqrt(S_r)
    Mat P(size_t(2) * k * r, 0.0);
    double *Pa = P.data(), *Pb = P.data() + size_t(k) * r;
    for (int cc = 0; cc < r; ++cc) {
      const int j = ord[cc];
      const double sj = S[j], sq = std::sqrt(sj);
      for (int a = 0; a < k; ++a) {
        Pa[a * r + cc] = sj > 0 ? G[a * k + j] / sq : 0.0;
        Pb[a * r + cc] = W[a * k + j] * sq;
      }
    }
    QLORA_TRY(hipMemcpyAsync(c.dT, P.data(), sizeof(double) * P.size(), hipMemcpyHostToDevice,
                             stream));
    const bool b16 = adt == QLORA_BF16;
    QLORA_TRY(launch_panel_apply(Y, k, c.dT, r, in, A, false, b16, stream));
    QLORA_TRY(launch_panel_apply(Qz, k, c.dT + size_t(k) * r, r, out, B, true, b16, stream));
    return hipStreamSynchronize(stream);   // (P is read by the copy above)
#undef QLORA_TRY
  };
  return run() == hipSuccess ? QLORA_OK : QLORA_ERR_DEVICE;
}
