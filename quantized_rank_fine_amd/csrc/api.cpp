// C-ABI boundary of libqlora: argument validation, workspace planning,
// kernel sequencing on the caller's stream and optional kernel timing.
//
// The three calls follow "QLoRA (low-rank adapters on a quantized model)",
// "How it works": quantize once (Wq = Q(W0)), forward through W = Wq + A B,
// backward giving dA = dW B^T and dB = A^T dW (here in factored form,
// dA = X^T (dY B^T) and dB = (X A)^T dY, so dW is never formed).

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <vector>

#include "internal.h"
#include "qlora.h"

using namespace qlora;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool dtype_ok(qlora_dtype d) { return d == QLORA_F32 || d == QLORA_BF16; }

// Shapes every kernel can address.  The kernels reach memory through 32-bit
// offsets from a per-workgroup (or per-array) base, and a buffer descriptor
// spans at most 2^31 - 1 bytes.  With in, out <= 2^19 and in*out < 2^32
// weights the packed codes stay below 2^31 bytes, the block-scale tables
// below 2^28, and any 256 activation rows below 2^29 bytes; with at most
// 2^24 tokens the per-call token-major arrays (bf16 XA^T copies, few-token
// partials) stay inside the same range.  Larger shapes are rejected with
// QLORA_ERR_SHAPE rather than addressed wrongly.
constexpr int64_t kMaxDim = int64_t(1) << 19;
constexpr int64_t kMaxWeights = (int64_t(1) << 32) - 4096;
constexpr int64_t kMaxTokens = int64_t(1) << 24;

bool shape_ok(int64_t in, int64_t out) {
  return in > 0 && out > 0 && in % 64 == 0 && out % 64 == 0 && in <= kMaxDim &&
         out <= kMaxDim && in * out <= kMaxWeights;
}

bool tokens_ok(int64_t M) { return M >= 0 && M <= kMaxTokens; }

// ---------------------------------------------------------------- timing
// Optional instrumentation (off by default): the mask is read atomically on
// every launch, and the recorded event pairs are guarded by a mutex, so
// calls on several threads may run while timing is switched on or off.
struct TimingState {
  std::atomic<int> mask{0};
  std::mutex mu;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> pending[QLORA_KERNEL_COUNT];
  double total_ms[QLORA_KERNEL_COUNT] = {};
  int64_t launches[QLORA_KERNEL_COUNT] = {};
};
TimingState g_timing;

template <class F>
hipError_t timed(int kind, hipStream_t s, F &&launch) {
  if (!(g_timing.mask.load(std::memory_order_relaxed) & (1 << kind))) return launch();
  hipEvent_t a = nullptr, b = nullptr;
  if (hipEventCreate(&a) != hipSuccess) return launch();
  if (hipEventCreate(&b) != hipSuccess) {
    (void)hipEventDestroy(a);
    return launch();
  }
  (void)hipEventRecord(a, s);
  hipError_t e = launch();
  (void)hipEventRecord(b, s);
  std::lock_guard<std::mutex> lock(g_timing.mu);
  g_timing.pending[kind].emplace_back(a, b);
  return e;
}

qlora_status dev(hipError_t e) { return e == hipSuccess ? QLORA_OK : QLORA_ERR_DEVICE; }

// ---------------------------------------------------------------- plans
// Workspace layouts.  Every region starts on a 256-byte boundary.

struct Layout {
  size_t o = 0;
  size_t take(size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes);
    return at;
  }
};

struct FwdPlan {
  bool small = false;          // few-token path: split-K partials + fixed-order reduction
  int64_t ks = 0, rp = 0, kc = 0;
  size_t off_x16 = 0, off_cs = 0, off_part = 0, off_xa16 = 0, off_p = 0, off_pxa = 0, total = 0;
};

FwdPlan plan_fwd(int64_t M, int64_t in, int64_t out, int32_t r, bool act_bf16) {
  FwdPlan p;
  if (M == 0) return p;
  Layout L;
  if (M <= kSmallMaxM && r <= kSmallMaxR) {
    p.small = true;
    p.kc = small_fwd_chunk_rows(M, in, out);
    p.ks = (in + p.kc - 1) / p.kc;
    p.off_p = L.take(size_t(p.ks) * M * out * 4);
    if (r > 0) p.off_pxa = L.take(size_t(p.ks) * M * r * 4);
    p.total = L.o;
    return p;
  }
  p.off_x16 = act_bf16 ? 0 : L.take(size_t(M) * in * 2);
  p.off_cs = L.take(size_t(in) * (out / 64) * 4);
  if (r > 0) {
    p.rp = rank_pad32(r);
    p.ks = xa_complete(M, in, r) ? 0 : rowdot_splits(M, in, r);
    if (p.ks) p.off_part = L.take(size_t(p.ks) * M * r * 4);
    p.off_xa16 = L.take(size_t(M) * p.rp * 2);
  }
  p.total = L.o;
  return p;
}

// dB folded into the dX GEMM (bf16 activations, r <= 16 and a multiple of 4,
// G formed whole, at most a few dY tiles per GEMM workgroup): its partials
// are per 256-token block, and the dY pass writes XA^T in bf16.
bool db_in_dx(int64_t M, int64_t in, int64_t out, int32_t r, bool act_bf16) {
  return act_bf16 && r > 0 && r <= 16 && r % 4 == 0 && g_complete(M, out, r) &&
         dx_fold_fits(M, in, out) && (M + 255) / 256 * out * r * 4 <= 0x7fffffff;
}

struct BwdPlan {
  int64_t ks_g = 0, ks_x = 0, ks_b = 0, ks_a = 0, rp = 0;
  int64_t ks_bx = 0, ldm = 0;   // dB folded into the dX GEMM: partials, XA^T row length
  size_t off_dy16 = 0, off_cs = 0, off_gpart = 0, off_g16 = 0;
  size_t off_xapart = 0, off_xa = 0, off_u = 0, off_dbpart = 0, off_dapart = 0, off_xat = 0;
  size_t total = 0;
};

BwdPlan plan_bwd(int64_t M, int64_t in, int64_t out, int32_t r, bool act_bf16) {
  BwdPlan p;
  if (M == 0) return p;
  Layout L;
  p.off_dy16 = act_bf16 ? 0 : L.take(size_t(M) * out * 2);
  p.off_cs = L.take(size_t(in) * (out / 64) * 4);
  if (r > 0) {
    p.rp = rank_pad32(r);
    p.ks_g = g_complete(M, out, r) ? 0 : rowdot_splits(M, out, r);
    p.ks_x = xa_complete(M, in, r) ? 0 : rowdot_splits(M, in, r);
    p.ks_b = coldot_splits(M, out, r);
    p.ks_a = coldot_splits(M, in, r);
    if (p.ks_g) p.off_gpart = L.take(size_t(p.ks_g) * M * r * 4);
    p.off_g16 = L.take(size_t(M) * p.rp * 2);
    if (p.ks_x) p.off_xapart = L.take(size_t(p.ks_x) * M * r * 4);
    p.off_xa = L.take(size_t(M) * r * 4);
    p.off_u = L.take(size_t(M) * r * 4);
    if (db_in_dx(M, in, out, r, act_bf16)) {
      p.ks_bx = (M + 255) / 256;
      p.ldm = p.ks_bx * 256;
      p.off_xat = L.take(size_t(16) * p.ldm * 2);
    }
    p.off_dbpart = L.take(size_t(std::max(p.ks_b, p.ks_bx)) * out * r * 4);
    p.off_dapart = L.take(size_t(p.ks_a) * in * r * 4);
  }
  p.total = L.o;
  return p;
}

template <class T>
T *at(void *ws, size_t off) {
  return reinterpret_cast<T *>(static_cast<char *>(ws) + off);
}

// The 16-entry scale format (one fp32 absmax per 16 weights, no double
// quantization); block 0 or 64 is the double-quantized 64-weight format.
bool g16(const qlora_nf4 *wq) { return wq->block == QLORA_LAB_GROUP; }

qlora_status check_nf4(const qlora_nf4 *wq) {
  if (!wq) return QLORA_ERR_NULL;
  if (!shape_ok(wq->in, wq->out)) return QLORA_ERR_SHAPE;
  if (wq->codebook < 0 || wq->codebook >= kCodebooks) return QLORA_ERR_DTYPE;
  if (wq->block != 0 && wq->block != QLORA_BLOCK && wq->block != QLORA_LAB_GROUP)
    return QLORA_ERR_DTYPE;
  if (!wq->codes || !wq->gscale || (!g16(wq) && !wq->qscale)) return QLORA_ERR_NULL;
  if (!aligned16(wq->codes) || !aligned16(wq->gscale) || (!g16(wq) && !aligned16(wq->qscale)))
    return QLORA_ERR_ALIGN;
  return QLORA_OK;
}

// The multiplier of the rank-r intermediates from the caller's options:
// c = alpha/r / (1 - p) (double, rounded to fp32 once) on kept elements.
bool lora_mul(const qlora_lora *lora, RankMul &mul) {
  mul = RankMul();
  if (!lora) return true;
  const double sc = lora->scale, pd = lora->dropout_p;
  if (!std::isfinite(sc) || !std::isfinite(pd) || pd < 0.0 || pd >= 1.0) return false;
  if (!lora->keep && pd != 0.0) return false;
  mul.keep = lora->keep;
  mul.c = float(sc / (1.0 - pd));
  return std::isfinite(mul.c);
}

// The backward, with optional Adam steps of A and B fused into the final
// reductions (ta/tb.theta != nullptr; dA/dB may then be null).  Every read of
// A and B comes before those reductions, so the updated adapters may alias
// the ones the call reads.
qlora_status linear_bwd(const qlora_nf4 *wq, const void *X, const void *dY, int64_t M,
                        qlora_dtype act, const void *A, const void *B, int32_t r,
                        qlora_dtype adt, const RankMul &mul, const float *XA, void *dX,
                        float *dA, float *dB, const AdamTarget &ta, const AdamTarget &tb,
                        void *ws, size_t ws_bytes, hipStream_t stream) {
  const bool adam = ta.theta != nullptr;
  qlora_status st = check_nf4(wq);
  if (st != QLORA_OK) return st;
  if (!tokens_ok(M) || r < 0 || r > QLORA_MAX_RANK) return QLORA_ERR_SHAPE;
  if (!dtype_ok(act) || !dtype_ok(adt)) return QLORA_ERR_DTYPE;
  const int64_t in = wq->in, out = wq->out;
  if (r > 0) {
    if (!A || !B || (!adam && (!dA || !dB))) return QLORA_ERR_NULL;
    if (!aligned16(A) || !aligned16(B) || (dA && !aligned16(dA)) || (dB && !aligned16(dB)))
      return QLORA_ERR_ALIGN;
    if (XA && !aligned16(XA)) return QLORA_ERR_ALIGN;
  }
  const bool xb = act == QLORA_BF16, ab = adt == QLORA_BF16;
  hipError_t e = hipSuccess;
#define QLORA_RUN(KIND, CALL)                              \
  do {                                                     \
    e = timed(KIND, stream, [&] { return CALL; });         \
    if (e != hipSuccess) return QLORA_ERR_DEVICE;          \
  } while (0)
  if (M == 0) {
    if (adam) return QLORA_ERR_SHAPE;
    if (r > 0) {
      QLORA_RUN(QLORA_KERNEL_REDUCE, launch_fill_zero(dA, in * r, stream));
      QLORA_RUN(QLORA_KERNEL_REDUCE, launch_fill_zero(dB, int64_t(r) * out, stream));
    }
    return QLORA_OK;
  }
  if (!dY || !ws) return QLORA_ERR_NULL;
  if (r > 0 && !X) return QLORA_ERR_NULL;
  if (!aligned16(dY) || !aligned16(ws)) return QLORA_ERR_ALIGN;
  if (X && !aligned16(X)) return QLORA_ERR_ALIGN;
  if (dX && !aligned16(dX)) return QLORA_ERR_ALIGN;
  const BwdPlan p = plan_bwd(M, in, out, r, xb);
  if (ws_bytes < p.total) return QLORA_ERR_WORKSPACE;

  const uint16_t *dY16 = static_cast<const uint16_t *>(dY);
  if (!xb && dX) {
    uint16_t *d16 = at<uint16_t>(ws, p.off_dy16);
    QLORA_RUN(QLORA_KERNEL_REDUCE, launch_convert_to_bf16(dY, false, M * out, d16, stream));
    dY16 = d16;
  }
  float *cs = dX ? at<float>(ws, p.off_cs) : nullptr;
  uint16_t *G16 = nullptr;
  if (r > 0 && !XA) {
    // recompute XA = X . A into the workspace
    float *xpart = p.ks_x > 0 ? at<float>(ws, p.off_xapart) : nullptr;
    float *xaw = at<float>(ws, p.off_xa);
    QLORA_RUN(QLORA_KERNEL_XA, launch_fwd_prep(X, xb, A, ab, M, in, r, xpart, xaw, nullptr, 0,
                                               nullptr, nullptr, out, nullptr, stream));
    if (p.ks_x > 0) {
      QLORA_RUN(QLORA_KERNEL_REDUCE, launch_reduce2(xpart, p.ks_x, M, r, xaw, false, nullptr, 0,
                                                    nullptr, 0, 0, nullptr, false, nullptr, 0,
                                                    stream));
    }
    XA = xaw;
  }
  // one pass over dY: G = dY . B^T (complete, or partials), dB = XA^T . dY
  // partials (or, when the dX GEMM forms them, XA^T in bf16), block scales
  float *gpart = p.ks_g > 0 ? at<float>(ws, p.off_gpart) : nullptr;
  float *dbpart = r > 0 ? at<float>(ws, p.off_dbpart) : nullptr;
  if (r > 0) G16 = at<uint16_t>(ws, p.off_g16);
  const bool fold = dX && p.ks_bx > 0;
  uint16_t *xat = fold ? at<uint16_t>(ws, p.off_xat) : nullptr;
  // the dY pass's dB operand: XA after its multiplier (the dX GEMM's XA^T
  // copy applies it itself)
  const float *XAd = XA;
  if (r > 0 && !fold && (mul.keep || mul.c != 1.0f)) {
    float *U = at<float>(ws, p.off_u);
    QLORA_RUN(QLORA_KERNEL_REDUCE, launch_rank_mul(XA, M, r, mul, U, stream));
    XAd = U;
  }
  QLORA_RUN(QLORA_KERNEL_DY_PASS, launch_bwd_dy(dY, xb, B, ab, XAd, M, out, r, gpart, G16, p.rp,
                                                dbpart, xat, p.ldm, wq->qscale, wq->gscale, in,
                                                g16(wq) ? nullptr : cs, stream, mul));
  auto dx_gemm = [&](const uint16_t *xt, float *dbp) {
    return launch_dx_gemm(wq->codes, g16(wq) ? wq->gscale : cs, in, out, dY16, M, G16,
                          int32_t(p.rp), A, ab, r, dX, xb, wq->codebook, g16(wq), xt, p.ldm,
                          dbp, stream);
  };
  if (r == 0) {
    if (dX) QLORA_RUN(QLORA_KERNEL_DX_GEMM, dx_gemm(nullptr, nullptr));
    return QLORA_OK;
  }
  float *dapart = at<float>(ws, p.off_dapart);
  // r <= 16: dA is formed whole after the dX GEMM (the last reader of A), in
  // one launch with the reduction of dB's partials where those are pending;
  // the bits of dA then do not depend on whether dX is asked for.
  const bool whole = da_whole(M, in, r, xb);
  auto tail = [&](const float *dbp, int64_t ks) {
    return launch_bwd_tail(X, xb, G16, p.rp, M, in, r, dA, ta, dbp, ks, out, dB, tb, stream);
  };
  if (fold) {
    // dX and the dB partials in the GEMM; then dA and dB
    QLORA_RUN(QLORA_KERNEL_DX_GEMM, dx_gemm(xat, dbpart));
    QLORA_RUN(QLORA_KERNEL_DA_PASS, tail(dbpart, p.ks_bx));
    return QLORA_OK;
  }
  if (p.ks_g > 0) {
    // G (bf16, zero-padded) and dB (stored [r x out]) in one launch; B is
    // not read after the dY pass
    QLORA_RUN(QLORA_KERNEL_REDUCE,
              launch_reduce2(gpart, p.ks_g, M, r, nullptr, false, G16, p.rp, dbpart, p.ks_b, out,
                             dB, true, nullptr, 0, stream, mul, AdamTarget(), tb));
    if (whole) {
      if (dX) QLORA_RUN(QLORA_KERNEL_DX_GEMM, dx_gemm(nullptr, nullptr));
      QLORA_RUN(QLORA_KERNEL_DA_PASS, tail(nullptr, 0));
      return QLORA_OK;
    }
    // dA = X^T . G; dX (the last reader of A); dA
    QLORA_RUN(QLORA_KERNEL_DA_PASS, launch_bwd_x(X, xb, G16, p.rp, M, in, r, dapart, stream));
    if (dX) QLORA_RUN(QLORA_KERNEL_DX_GEMM, dx_gemm(nullptr, nullptr));
    QLORA_RUN(QLORA_KERNEL_REDUCE, launch_reduce2(dapart, p.ks_a, in, r, dA, false, nullptr, 0,
                                                  nullptr, 0, 0, nullptr, false, nullptr, 0,
                                                  stream, RankMul(), ta));
  } else if (whole) {
    // G is complete: dX, then dA and dB (stored [r x out]) in one launch
    if (dX) QLORA_RUN(QLORA_KERNEL_DX_GEMM, dx_gemm(nullptr, nullptr));
    QLORA_RUN(QLORA_KERNEL_DA_PASS, tail(dbpart, p.ks_b));
  } else {
    // G is complete: dA = X^T . G, dX, then dA and dB (stored [r x out]) in
    // one launch
    QLORA_RUN(QLORA_KERNEL_DA_PASS, launch_bwd_x(X, xb, G16, p.rp, M, in, r, dapart, stream));
    if (dX) QLORA_RUN(QLORA_KERNEL_DX_GEMM, dx_gemm(nullptr, nullptr));
    QLORA_RUN(QLORA_KERNEL_REDUCE,
              launch_reduce2(dapart, p.ks_a, in, r, dA, false, nullptr, 0, dbpart, p.ks_b, out,
                             dB, true, nullptr, 0, stream, RankMul(), ta, tb));
  }
  return QLORA_OK;
#undef QLORA_RUN
}

bool adam_hparams_ok(const qlora_adam_hparams *h) {
  return h && h->step >= 1 && std::isfinite(h->lr) && std::isfinite(h->eps) &&
         std::isfinite(h->weight_decay) && h->beta1 >= 0.0f && h->beta1 < 1.0f &&
         h->beta2 >= 0.0f && h->beta2 < 1.0f && h->eps >= 0.0f && h->weight_decay >= 0.0f;
}

qlora_status adam_target(const qlora_adam_state *s, const qlora_adam_hparams *h,
                         AdamTarget &t) {
  if (!s || !s->theta || !s->m || !s->v) return QLORA_ERR_NULL;
  if (!aligned16(s->theta) || !aligned16(s->m) || !aligned16(s->v) ||
      (s->theta_bf16 && !aligned16(s->theta_bf16)))
    return QLORA_ERR_ALIGN;
  t.theta = s->theta;
  t.m = s->m;
  t.v = s->v;
  t.theta16 = s->theta_bf16;
  t.p = make_adam_params(h->step, h->lr, h->beta1, h->beta2, h->eps, h->weight_decay);
  return QLORA_OK;
}

}  // namespace

extern "C" {

const char *qlora_status_string(qlora_status s) {
  switch (s) {
    case QLORA_OK: return "ok";
    case QLORA_ERR_NULL: return "null pointer";
    case QLORA_ERR_SHAPE: return "invalid shape";
    case QLORA_ERR_ALIGN: return "pointer not 16-byte aligned";
    case QLORA_ERR_DTYPE: return "invalid dtype";
    case QLORA_ERR_WORKSPACE: return "workspace too small";
    case QLORA_ERR_DEVICE: return "HIP runtime error";
    case QLORA_ERR_VALUE: return "invalid value";
  }
  return "unknown status";
}

size_t qlora_fwd_workspace_bytes(int64_t M, int64_t in, int64_t out, int32_t r,
                                 qlora_dtype act) {
  if (!tokens_ok(M) || r < 0 || r > QLORA_MAX_RANK || !shape_ok(in, out) || !dtype_ok(act)) return 0;
  return plan_fwd(M, in, out, r, act == QLORA_BF16).total;
}

size_t qlora_bwd_workspace_bytes(int64_t M, int64_t in, int64_t out, int32_t r,
                                 qlora_dtype act) {
  if (!tokens_ok(M) || r < 0 || r > QLORA_MAX_RANK || !shape_ok(in, out) || !dtype_ok(act)) return 0;
  return plan_bwd(M, in, out, r, act == QLORA_BF16).total;
}

qlora_status qlora_quantize(const float *W0, const qlora_nf4 *wq, hipStream_t stream) {
  qlora_status st = check_nf4(wq);
  if (st != QLORA_OK) return st;
  if (!W0) return QLORA_ERR_NULL;
  if (!aligned16(W0)) return QLORA_ERR_ALIGN;
  const int64_t nblocks = wq->in * wq->out / 64;
  return dev(timed(QLORA_KERNEL_QUANTIZE, stream, [&] {
    return launch_quantize(W0, wq->codes, wq->qscale, wq->gscale, nblocks, wq->codebook, g16(wq),
                           stream);
  }));
}

qlora_status qlora_linear_fwd(const qlora_nf4 *wq, const void *X, int64_t M, qlora_dtype act,
                              const void *A, const void *B, int32_t r, qlora_dtype adt,
                              void *Y, float *XA, void *ws, size_t ws_bytes,
                              hipStream_t stream) {
  return qlora_linear_fwd_lora(wq, X, M, act, A, B, r, adt, nullptr, Y, XA, ws, ws_bytes, stream);
}

qlora_status qlora_linear_bwd(const qlora_nf4 *wq, const void *X, const void *dY, int64_t M,
                              qlora_dtype act, const void *A, const void *B, int32_t r,
                              qlora_dtype adt, const float *XA, void *dX, float *dA, float *dB,
                              void *ws, size_t ws_bytes, hipStream_t stream) {
  return qlora_linear_bwd_lora(wq, X, dY, M, act, A, B, r, adt, nullptr, XA, dX, dA, dB, ws,
                               ws_bytes, stream);
}

qlora_status qlora_linear_fwd_lora(const qlora_nf4 *wq, const void *X, int64_t M,
                                   qlora_dtype act, const void *A, const void *B, int32_t r,
                                   qlora_dtype adt, const qlora_lora *lora, void *Y, float *XA,
                                   void *ws, size_t ws_bytes, hipStream_t stream) {
  RankMul mul;
  if (!lora_mul(lora, mul)) return QLORA_ERR_VALUE;
  qlora_status st = check_nf4(wq);
  if (st != QLORA_OK) return st;
  if (!tokens_ok(M) || r < 0 || r > QLORA_MAX_RANK) return QLORA_ERR_SHAPE;
  if (!dtype_ok(act) || !dtype_ok(adt)) return QLORA_ERR_DTYPE;
  if (M == 0) return QLORA_OK;
  if (!X || !Y || !ws) return QLORA_ERR_NULL;
  if (!aligned16(X) || !aligned16(Y) || !aligned16(ws)) return QLORA_ERR_ALIGN;
  if (r > 0) {
    if (!A || !B) return QLORA_ERR_NULL;
    if (!aligned16(A) || !aligned16(B) || (XA && !aligned16(XA))) return QLORA_ERR_ALIGN;
  }
  const bool xb = act == QLORA_BF16, ab = adt == QLORA_BF16;
  const int64_t in = wq->in, out = wq->out;
  const FwdPlan p = plan_fwd(M, in, out, r, xb);
  if (ws_bytes < p.total) return QLORA_ERR_WORKSPACE;
  hipError_t e = hipSuccess;
#define QLORA_RUN(KIND, CALL)                              \
  do {                                                     \
    e = timed(KIND, stream, [&] { return CALL; });         \
    if (e != hipSuccess) return QLORA_ERR_DEVICE;          \
  } while (0)
  if (p.small) {
    float *P = at<float>(ws, p.off_p);
    float *PXA = r > 0 ? at<float>(ws, p.off_pxa) : nullptr;
    QLORA_RUN(QLORA_KERNEL_FWD_SMALLM,
              launch_fwd_small_partial(wq->codes, wq->qscale, wq->gscale, in, out, X, xb, M, A,
                                       ab, r, p.kc, P, PXA, wq->codebook, g16(wq), stream));
    QLORA_RUN(QLORA_KERNEL_REDUCE, launch_fwd_small_reduce(P, PXA, p.ks, M, out, r, B, ab, XA,
                                                           Y, xb, stream, mul));
    return QLORA_OK;
  }
  const uint16_t *X16 = static_cast<const uint16_t *>(X);
  if (!xb) {
    uint16_t *x16 = at<uint16_t>(ws, p.off_x16);
    QLORA_RUN(QLORA_KERNEL_REDUCE, launch_convert_to_bf16(X, false, M * in, x16, stream));
    X16 = x16;
  }
  // one launch: X . A (complete, or split-K partials) and the GEMM's block scales
  float *cs = at<float>(ws, p.off_cs);
  float *part = p.ks > 0 ? at<float>(ws, p.off_part) : nullptr;
  uint16_t *XA16 = r > 0 ? at<uint16_t>(ws, p.off_xa16) : nullptr;
  QLORA_RUN(QLORA_KERNEL_XA, launch_fwd_prep(X, xb, A, ab, M, in, r, part, XA, XA16, p.rp,
                                             wq->qscale, wq->gscale, out,
                                             g16(wq) ? nullptr : cs, stream, mul));
  if (p.ks > 0) {
    QLORA_RUN(QLORA_KERNEL_REDUCE, launch_reduce2(part, p.ks, M, r, XA, false, XA16, p.rp,
                                                  nullptr, 0, 0, nullptr, false, nullptr, 0,
                                                  stream, mul));
  }
  QLORA_RUN(QLORA_KERNEL_FWD_GEMM,
            launch_fwd_gemm(wq->codes, g16(wq) ? wq->gscale : cs, in, out, X16, M, XA16,
                            int32_t(p.rp), B, ab, r, Y, xb, wq->codebook, g16(wq), stream));
  return QLORA_OK;
#undef QLORA_RUN
}

qlora_status qlora_linear_fwd_noalloc(const qlora_nf4 *wq, const void *X, int64_t M,
                                     qlora_dtype act, const void *A, const void *B, int32_t r,
                                     qlora_dtype adt, void *Y, float *XA, hipStream_t stream) {
  // The size check comes before the scratch lookup, so an oversized call
  // touches nothing on the device.
  qlora_status st = check_nf4(wq);
  if (st != QLORA_OK) return st;
  if (!tokens_ok(M) || r < 0 || r > QLORA_MAX_RANK) return QLORA_ERR_SHAPE;
  if (!dtype_ok(act) || !dtype_ok(adt)) return QLORA_ERR_DTYPE;
  if (M == 0) return QLORA_OK;
  if (plan_fwd(M, wq->in, wq->out, r, act == QLORA_BF16).total > kNoAllocScratchBytes)
    return QLORA_ERR_WORKSPACE;
  void *ws = nullptr;
  if (noalloc_scratch(&ws) != hipSuccess) return QLORA_ERR_DEVICE;
  return qlora_linear_fwd_lora(wq, X, M, act, A, B, r, adt, nullptr, Y, XA, ws,
                               kNoAllocScratchBytes, stream);
}

size_t qlora_fwd_group_workspace_bytes(int32_t n, int64_t M, const int64_t *in,
                                       const int64_t *out, int32_t r, qlora_dtype act) {
  if (n < 1 || n > kSmallMaxGroup || !in || !out || M < 1 || M > kSmallMaxM || r < 0 ||
      r > kSmallMaxR || !dtype_ok(act))
    return 0;
  size_t total = 0;
  for (int l = 0; l < n; ++l) {
    if (!shape_ok(in[l], out[l])) return 0;
    total += align_up(plan_fwd(M, in[l], out[l], r, act == QLORA_BF16).total);
  }
  return total;
}

qlora_status qlora_linear_fwd_group(int32_t n, const qlora_nf4 *const *wq, const void *const *X,
                                    int64_t M, qlora_dtype act, const void *const *A,
                                    const void *const *B, int32_t r, qlora_dtype adt,
                                    void *const *Y, float *const *XA, void *ws, size_t ws_bytes,
                                    hipStream_t stream) {
  if (n < 1 || n > kSmallMaxGroup) return QLORA_ERR_SHAPE;
  if (!wq || !X || !Y || (r > 0 && (!A || !B))) return QLORA_ERR_NULL;
  if (M < 1 || M > kSmallMaxM || r < 0 || r > kSmallMaxR) return QLORA_ERR_SHAPE;
  if (!dtype_ok(act) || !dtype_ok(adt)) return QLORA_ERR_DTYPE;
  SmallLinear lin[kSmallMaxGroup];
  size_t off = 0;
  for (int l = 0; l < n; ++l) {
    qlora_status st = check_nf4(wq[l]);
    if (st != QLORA_OK) return st;
    if (wq[l]->codebook != wq[0]->codebook || g16(wq[l]) != g16(wq[0])) return QLORA_ERR_DTYPE;
    if (!X[l] || !Y[l]) return QLORA_ERR_NULL;
    if (!aligned16(X[l]) || !aligned16(Y[l])) return QLORA_ERR_ALIGN;
    if (r > 0) {
      if (!A[l] || !B[l]) return QLORA_ERR_NULL;
      if (!aligned16(A[l]) || !aligned16(B[l]) || (XA && XA[l] && !aligned16(XA[l])))
        return QLORA_ERR_ALIGN;
    }
    const int64_t in = wq[l]->in, out = wq[l]->out;
    const FwdPlan p = plan_fwd(M, in, out, r, act == QLORA_BF16);
    SmallLinear &L = lin[l];
    L.codes = wq[l]->codes;
    L.qscale = wq[l]->qscale;
    L.gscale = wq[l]->gscale;
    L.K = in;
    L.N = out;
    L.X = X[l];
    L.A = r > 0 ? A[l] : nullptr;
    L.B = r > 0 ? B[l] : nullptr;
    L.Kc = p.kc;
    L.P = reinterpret_cast<float *>(static_cast<char *>(ws) + off + p.off_p);
    L.PXA = r > 0 ? reinterpret_cast<float *>(static_cast<char *>(ws) + off + p.off_pxa) : nullptr;
    L.XA = r > 0 && XA ? XA[l] : nullptr;
    L.Y = Y[l];
    off += align_up(p.total);
  }
  if (!ws) return QLORA_ERR_NULL;
  if (!aligned16(ws)) return QLORA_ERR_ALIGN;
  if (ws_bytes < off) return QLORA_ERR_WORKSPACE;
  return dev(timed(QLORA_KERNEL_FWD_SMALLM, stream, [&] {
    return launch_fwd_small_group(n, lin, M, act == QLORA_BF16, adt == QLORA_BF16, r,
                                  wq[0]->codebook, g16(wq[0]), stream);
  }));
}

qlora_status qlora_linear_bwd_lora(const qlora_nf4 *wq, const void *X, const void *dY,
                                   int64_t M, qlora_dtype act, const void *A, const void *B,
                                   int32_t r, qlora_dtype adt, const qlora_lora *lora,
                                   const float *XA, void *dX, float *dA, float *dB, void *ws,
                                   size_t ws_bytes, hipStream_t stream) {
  RankMul mul;
  if (!lora_mul(lora, mul)) return QLORA_ERR_VALUE;
  return linear_bwd(wq, X, dY, M, act, A, B, r, adt, mul, XA, dX, dA, dB, AdamTarget(),
                    AdamTarget(), ws, ws_bytes, stream);
}

qlora_status qlora_linear_bwd_adam(const qlora_nf4 *wq, const void *X, const void *dY,
                                   int64_t M, qlora_dtype act, const void *A, const void *B,
                                   int32_t r, qlora_dtype adt, const qlora_lora *lora,
                                   const float *XA, void *dX, const qlora_adam_state *state_A,
                                   const qlora_adam_state *state_B,
                                   const qlora_adam_hparams *hparams, float *dA, float *dB,
                                   void *ws, size_t ws_bytes, hipStream_t stream) {
  RankMul mul;
  if (!lora_mul(lora, mul) || !adam_hparams_ok(hparams)) return QLORA_ERR_VALUE;
  if (M < 1) return QLORA_ERR_SHAPE;
  AdamTarget ta, tb;
  if (r > 0) {
    qlora_status st = adam_target(state_A, hparams, ta);
    if (st == QLORA_OK) st = adam_target(state_B, hparams, tb);
    if (st != QLORA_OK) return st;
  }
  return linear_bwd(wq, X, dY, M, act, A, B, r, adt, mul, XA, dX, dA, dB, ta, tb, ws, ws_bytes,
                    stream);
}

qlora_status qlora_merge(const qlora_nf4 *wq, const void *A, const void *B, int32_t r,
                         qlora_dtype adt, void *W, qlora_dtype wdt, hipStream_t stream) {
  qlora_status st = check_nf4(wq);
  if (st != QLORA_OK) return st;
  if (r < 0 || r > QLORA_MAX_RANK) return QLORA_ERR_SHAPE;
  if (!dtype_ok(adt) || !dtype_ok(wdt)) return QLORA_ERR_DTYPE;
  if (!W) return QLORA_ERR_NULL;
  if (!aligned16(W)) return QLORA_ERR_ALIGN;
  if (r > 0) {
    if (!A || !B) return QLORA_ERR_NULL;
    if (!aligned16(A) || !aligned16(B)) return QLORA_ERR_ALIGN;
  }
  return dev(launch_merge(wq->codes, wq->qscale, wq->gscale, wq->in, wq->out, A, B,
                          adt == QLORA_BF16, r, W, wdt == QLORA_BF16, wq->codebook, g16(wq),
                          stream));
}

qlora_status qlora_adam_step(float *theta, const float *grad, float *m, float *v, int64_t n,
                             int64_t step, float lr, float beta1, float beta2, float eps,
                             float weight_decay, uint16_t *theta_bf16, hipStream_t stream) {
  if (n < 0 || step < 1) return QLORA_ERR_SHAPE;
  const bool ok = std::isfinite(lr) && std::isfinite(eps) && std::isfinite(weight_decay) &&
                  beta1 >= 0.0f && beta1 < 1.0f && beta2 >= 0.0f && beta2 < 1.0f &&
                  eps >= 0.0f && weight_decay >= 0.0f;
  if (!ok) return QLORA_ERR_VALUE;
  if (n == 0) return QLORA_OK;
  if (!theta || !grad || !m || !v) return QLORA_ERR_NULL;
  if (!aligned16(theta) || !aligned16(grad) || !aligned16(m) || !aligned16(v) ||
      (theta_bf16 && !aligned16(theta_bf16)))
    return QLORA_ERR_ALIGN;
  return dev(launch_adam(theta, grad, m, v, n, step, lr, beta1, beta2, eps, weight_decay,
                         theta_bf16, stream));
}

int qlora_timing_enable(int kind_mask) {
  g_timing.mask.store(kind_mask & ((1 << QLORA_KERNEL_COUNT) - 1), std::memory_order_relaxed);
  return 0;
}

int qlora_timing_read(int kind, double *total_ms, int64_t *launches) {
  if (kind < 0 || kind >= QLORA_KERNEL_COUNT) return -1;
  std::lock_guard<std::mutex> lock(g_timing.mu);
  for (auto &pr : g_timing.pending[kind]) {
    float ms = 0.0f;
    if (hipEventSynchronize(pr.second) != hipSuccess) return -2;
    if (hipEventElapsedTime(&ms, pr.first, pr.second) != hipSuccess) return -2;
    g_timing.total_ms[kind] += ms;
    g_timing.launches[kind] += 1;
    (void)hipEventDestroy(pr.first);
    (void)hipEventDestroy(pr.second);
  }
  g_timing.pending[kind].clear();
  if (total_ms) *total_ms = g_timing.total_ms[kind];
  if (launches) *launches = g_timing.launches[kind];
  return 0;
}

void qlora_timing_reset(void) {
  std::lock_guard<std::mutex> lock(g_timing.mu);
  for (int k = 0; k < QLORA_KERNEL_COUNT; ++k) {
    for (auto &pr : g_timing.pending[k]) {
      (void)hipEventSynchronize(pr.second);
      (void)hipEventDestroy(pr.first);
      (void)hipEventDestroy(pr.second);
    }
    g_timing.pending[k].clear();
    g_timing.total_ms[k] = 0.0;
    g_timing.launches[k] = 0;
  }
}

const char *qlora_kernel_name(int kind) {
  static const char *names[QLORA_KERNEL_COUNT] = {
      "quantize", "xa_rowdot", "fwd_gemm", "dy_pass", "dx_gemm", "da_pass", "reduce", "fwd_smallm"};
  if (kind < 0 || kind >= QLORA_KERNEL_COUNT) return "unknown";
  return names[kind];
}

}  // extern "C"
