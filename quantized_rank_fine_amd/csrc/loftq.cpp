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
// the first loses to rounding.  Every step runs on the GPU, in order on the
// caller's stream: the residual products, the Gram matrices and the panel
// updates (fp64 arithmetic on fp32 panels), and the k x k steps (each
// Cholesky factor's inverse, and the final SVD by one-sided Jacobi
// rotations) in fp64 by one workgroup each.  The call only enqueues work:
// it never waits for the device, so it can be captured in a graph.
#include <cstdint>
#include <utility>

#include "internal.h"
#include "qlora.h"

namespace qlora {
namespace {

// The device buffers of one call.
struct Ctx {
  const float *W0;
  const qlora_nf4 *wq;
  double *dG, *dT;     // [k x k] Gram matrix; [k x k] transform or the [2 k x r] factors
  float *rpart;        // partial products of the residual products
  double *gpart;       // partial Gram matrices
  hipStream_t s;
};

// Y = R . M (M [out x k] -> Y [in x k]) or, transposed, R^T . M.
hipError_t residual_product(const Ctx &c, const float *M, int k, float *Y, bool transpose) {
  return launch_residual_mul(c.W0, c.wq->codes, c.wq->qscale, c.wq->gscale,
                             c.wq->block == QLORA_LAB_GROUP, c.wq->in, c.wq->out, M, k, Y,
                             transpose, c.wq->codebook, c.rpart, c.s);
}

// Orthonormal columns of the device panel X [rows x k] (Cholesky QR, twice);
// Xt is a panel of the same size used in between.  The result is in X.
hipError_t orthonormalize(Ctx &c, float *X, float *Xt, int64_t rows, int k) {
  float *src = X, *dst = Xt;
  for (int pass = 0; pass < 2; ++pass) {
    hipError_t e = launch_panel_gram(src, k, src, k, rows, c.dG, c.gpart, c.s);
    if (e != hipSuccess) return e;
    e = launch_chol_inv(c.dG, k, c.dT, c.s);
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
  Ctx c{W0, wq, dG, dT, rpart, gpart, stream};
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
    // R ~ Y Z^T with Z = R^T Y;  Z = Qz Rz, Rz = Qz^T Z;  from the SVD of
    // Rz^T = U~ S W~^T:  A = Y U~_r S_r^(1/2),
    // B^T = Qz W~_r S_r^(1/2) = Z U~_r S_r^(-1/2)  (Qz W~ = Qz Rz U~ S^-1)
    QLORA_TRY(residual_product(c, Y, k, Z, true));
    QLORA_TRY(hipMemcpyAsync(Qz, Z, sizeof(float) * size_t(out) * k, hipMemcpyDeviceToDevice,
                             stream));
    QLORA_TRY(orthonormalize(c, Qz, Zt, out, k));
    QLORA_TRY(launch_panel_gram(Qz, k, Z, k, out, c.dG, c.gpart, stream));
    QLORA_TRY(launch_small_svd(c.dG, k, r, c.dT, stream));
    const bool b16 = adt == QLORA_BF16;
    QLORA_TRY(launch_panel_apply(Y, k, c.dT, r, in, A, false, b16, stream));
    QLORA_TRY(launch_panel_apply(Z, k, c.dT + size_t(k) * r, r, out, B, true, b16, stream));
    return hipSuccess;
#undef QLORA_TRY
  };
  return run() == hipSuccess ? QLORA_OK : QLORA_ERR_DEVICE;
}
