// One Adam (AdamW) step of an adapter matrix, in place.
//
// "QLoRA (low-rank adapters on a quantized model)", "The code, line by line":
// the optimizer holds only A and B.  The pages do not print the update; this
// is the published Adam step (Kingma & Ba, Algorithm 1) with decoupled
// weight decay (AdamW), per element in fp32:
//   m <- b1 m + (1 - b1) g,   v <- b2 v + (1 - b2) g g,
//   theta <- theta - lr ( (m c1) / (sqrt(v c2) + eps) + wd theta ),
// with the bias corrections c1 = 1 / (1 - b1^t), c2 = 1 / (1 - b2^t) formed
// in double on the host.  Optionally the updated theta is also written as
// bf16 (the copy the bf16 forward reads).  HBM-bound: 16 B read and 12 B
// (+ 2) written per element, 16-B accesses, a grid-stride loop.
#include <cmath>

#include "device.h"

namespace qlora {
namespace {

struct AdamArgs {
  float *theta;
  const float *g;
  float *m, *v;
  int64_t n;
  AdamParams p;
  uint16_t *theta16;
};

__global__ __launch_bounds__(256) void adam_kernel(AdamArgs a) {
  const int64_t n4 = a.n / 4;
  const int64_t stride = int64_t(gridDim.x) * 256;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n4; i += stride) {
    f32x4_t th = reinterpret_cast<const f32x4_t *>(a.theta)[i];
    const f32x4_t g = reinterpret_cast<const f32x4_t *>(a.g)[i];
    f32x4_t m = reinterpret_cast<const f32x4_t *>(a.m)[i];
    f32x4_t v = reinterpret_cast<const f32x4_t *>(a.v)[i];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float t = th[e], mm = m[e], vv = v[e];
      adam1(a.p, t, g[e], mm, vv);
      th[e] = t; m[e] = mm; v[e] = vv;
    }
    reinterpret_cast<f32x4_t *>(a.theta)[i] = th;
    reinterpret_cast<f32x4_t *>(a.m)[i] = m;
    reinterpret_cast<f32x4_t *>(a.v)[i] = v;
    if (a.theta16)
      reinterpret_cast<u32x2_t *>(a.theta16)[i] = u32x2_t{pack_bf16x2(th[0], th[1]),
                                                          pack_bf16x2(th[2], th[3])};
  }
  // the last n % 4 elements
  const int64_t i = 4 * n4 + int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (blockIdx.x == 0 && i < a.n) {
    float t = a.theta[i], mm = a.m[i], vv = a.v[i];
    adam1(a.p, t, a.g[i], mm, vv);
    a.theta[i] = t; a.m[i] = mm; a.v[i] = vv;
    if (a.theta16) a.theta16[i] = __builtin_bit_cast(uint16_t, (__bf16)t);
  }
}

}  // namespace

AdamParams make_adam_params(int64_t step, float lr, float beta1, float beta2, float eps,
                            float weight_decay) {
  AdamParams a;
  a.lr = lr; a.b1 = beta1; a.b2 = beta2; a.eps = eps; a.wd = weight_decay;
  a.omb1 = float(1.0 - double(beta1));
  a.omb2 = float(1.0 - double(beta2));
  a.c1 = float(1.0 / (1.0 - std::pow(double(beta1), double(step))));
  a.c2 = float(1.0 / (1.0 - std::pow(double(beta2), double(step))));
  return a;
}

hipError_t launch_adam(float *theta, const float *g, float *m, float *v, int64_t n, int64_t step,
                       float lr, float beta1, float beta2, float eps, float weight_decay,
                       uint16_t *theta16, hipStream_t s) {
  if (n == 0) return hipSuccess;
  AdamArgs a;
  a.theta = theta; a.g = g; a.m = m; a.v = v; a.n = n; a.theta16 = theta16;
  a.p = make_adam_params(step, lr, beta1, beta2, eps, weight_decay);
  int64_t blocks = (n / 4 + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 2048) blocks = 2048;
  hipLaunchKernelGGL(adam_kernel, dim3(unsigned(blocks)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace qlora
