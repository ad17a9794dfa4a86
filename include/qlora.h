/*
 * qlora.h -- C ABI of libqlora, the MI355X (gfx950) QLoRA adapted linear layer.
 *
 * Three calls carry the hot path:
 *   qlora_quantize    W0 (fp32, frozen)  -> Wq = (4-bit codes, int8 block
 *                                            scales, fp32 group scales)
 *   qlora_linear_fwd  y  = X.deq(Wq) + (X.A).B
 *   qlora_linear_bwd  dX = dY.deq(Wq)^T + (dY.B^T).A^T,
 *                     dA = X^T.(dY.B^T),  dB = (X.A)^T.dY
 *
 * Sources (page titles; sections):
 *   "QLoRA (low-rank adapters on a quantized model)", "How it works": the
 *     weight is stored (in, out); quantize once, Wq = Q(W0), and freeze it;
 *     A is (in x r), B is (r x out); W = Wq + A B; update only A and B with
 *     dA = dW B^T, dB = A^T dW.  "What QLoRA adds": blocks of 64 weights with
 *     an absmax scale each, 16 normal-quantile levels, block scales quantized
 *     again to 8 bits, weights expanded to bf16 for every matmul and never
 *     updated.
 *   "LLMs · QLoRA", NormalFloat paragraph and code listing: level table
 *     (normal quantiles at 16 evenly spaced probabilities in [0.02, 0.98],
 *     divided by the largest magnitude), absmax per block of 64, nearest
 *     level by argmin of |w/absmax - level|.
 *   "LoRA & QLoRA", "Mathematical Formulation": h = W0 x + B(A x), the same
 *     layer in column form.
 *
 * Conventions for every call:
 *   - All tensor pointers are DEVICE pointers on the current HIP device,
 *     16-byte aligned, owned by the caller, and must not overlap one another.
 *     Matrices are row-major and dense (no strides).
 *   - Arguments are validated on the host before anything is enqueued.  On
 *     any error nothing is enqueued and no output byte is written.
 *     QLORA_OK means the work was enqueued on `stream` (stream-ordered; the
 *     caller synchronizes).  A launch failure reported by the runtime maps to
 *     QLORA_ERR_DEVICE; device faults surface at the caller's next sync.
 *   - Outputs are overwritten, never accumulated.  Wq, X, A, B, dY and XA
 *     (in the backward) are only read.
 *   - The library keeps no state between calls except the constant tables
 *     it derives once from the level definition (and, only while switched
 *     on, the kernel-timing records at the end of this header), and
 *     allocates no device memory: scratch space is the caller's `ws`
 *     buffer.  Calls are reentrant; calls on different streams may run
 *     concurrently.
 *   - Shapes: in and out are multiples of 64, at most 2^19 each, with
 *     in*out < 2^32 weights; at most 2^24 tokens per call.  The kernels
 *     address memory with 32-bit offsets; larger shapes give QLORA_ERR_SHAPE.
 *   - Same inputs give the same output bits (no order-dependent atomics).
 *   - Finite inputs are assumed; NaN/Inf inputs give unspecified outputs.
 */
#ifndef QLORA_H
#define QLORA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QLORA_OK = 0,
  QLORA_ERR_NULL = 1,      /* a required pointer is NULL                    */
  QLORA_ERR_SHAPE = 2,     /* in/out not positive multiples of 64 or past
                              the limits above, M < 0 or M > 2^24, r
                              outside [0, QLORA_MAX_RANK]                   */
  QLORA_ERR_ALIGN = 3,     /* a pointer is not 16-byte aligned              */
  QLORA_ERR_DTYPE = 4,     /* unknown qlora_dtype or qlora_codebook         */
  QLORA_ERR_WORKSPACE = 5, /* ws too small (see qlora_bwd_workspace_bytes)  */
  QLORA_ERR_DEVICE = 6,    /* the HIP runtime reported an error             */
  QLORA_ERR_VALUE = 7      /* a hyperparameter out of its range             */
} qlora_status;

typedef enum { QLORA_F32 = 0, QLORA_BF16 = 1 } qlora_dtype;

/*
 * Level set of the 4-bit codes ("LLMs · QLoRA", NormalFloat paragraph and its
 * listing, which builds both and compares them):
 *   QLORA_CB_NF4       normal quantiles at 16 evenly spaced probabilities in
 *                      [0.02, 0.98], scaled so the largest magnitude is 1;
 *   QLORA_CB_UNIFORM4  16 evenly spaced values from -1 to 1.
 * and the symmetric integer grids of "QLoRA (low-rank adapters on a
 * quantized model)" ("The code, line by line", "What the simulations show":
 * symmetric uniform integers; "2-bit" is ternary), on the same 64-weight
 * absmax blocks and double-quantized scales:
 *   QLORA_CB_INT4      k / 7, k = -7..7      (4-bit)
 *   QLORA_CB_INT3      k / 3, k = -3..3      (3-bit)
 *   QLORA_CB_TERNARY   -1, 0, 1              (2-bit)
 * stored as 4-bit codes in sign-magnitude order (code 8 + m = +m/h, code
 * 7 - m = -m/h; zero twice, magnitudes above 1 never chosen).
 * Each level is computed in double and rounded to fp32 once
 * (qlora_codebook_levels returns the table).  A weight quantized with one
 * codebook must be used with the same codebook.
 */
typedef enum {
  QLORA_CB_NF4 = 0,
  QLORA_CB_UNIFORM4 = 1,
  QLORA_CB_INT4 = 2,
  QLORA_CB_INT3 = 3,
  QLORA_CB_TERNARY = 4
} qlora_codebook;

#define QLORA_BLOCK 64      /* weights per absmax block                      */
#define QLORA_GROUP 256     /* block scales per double-quantization group    */
#define QLORA_MAX_RANK 256  /* largest adapter rank r accepted               */

/*
 * Frozen quantized weight.  For W0 of shape (in, out), n = in*out, flattened
 * row-major:
 *   codes  [n/2]  uint8   byte j holds the 4-bit code of element 2j in its
 *                         low nibble and of element 2j+1 in its high nibble;
 *                         code i selects level L_i of the 16-entry table.
 *   codebook              a qlora_codebook value: the level table L (zero,
 *                         as in a zero-initialised struct, is NF4).
 *   block                 the scale format:
 *     0 or QLORA_BLOCK (64): absmax blocks of 64 weights, scales quantized
 *       again ("What QLoRA adds"):
 *         qscale [n/64] int8   block b (elements 64b..64b+63) scale q_b in
 *                              [0, 127];
 *         gscale [ceil(n/64/256)] fp32  group g (blocks 256g..256g+255)
 *                              scale s2_g;
 *       w_hat = L[code] * (q_b * s2_g).
 *     QLORA_LAB_GROUP (16): the lab's quantizer ("QLoRA (low-rank adapters
 *       on a quantized model)", "The code, line by line" and its
 *       Simplifications: one scale per 16 consecutive entries of the
 *       flattened (in, out) matrix, no double quantization):
 *         gscale [n/16] fp32   group g (elements 16g..16g+15) absmax c_g;
 *         qscale unused (may be NULL);
 *       w_hat = L[code] * c_g.  With QLORA_CB_INT4 / INT3 / TERNARY this is
 *       the lab's symmetric integer grid; any codebook may be used.
 * Requires in % 64 == 0 and out % 64 == 0, so blocks never straddle rows.
 * qlora_loftq_init takes either format.
 */
#define QLORA_LAB_GROUP 16
typedef struct {
  int64_t in;
  int64_t out;
  uint8_t *codes;
  int8_t *qscale;
  float *gscale;
  int32_t codebook;
  int32_t block;
} qlora_nf4;

/* Number of bytes of each part of a qlora_nf4 of shape (in, out) in the
 * 64-weight format (the 16-entry format: codes as here, in*out/16 fp32
 * scales in gscale, no qscale). */
static inline size_t qlora_codes_bytes(int64_t in, int64_t out) {
  return (size_t)(in * out / 2);
}
static inline size_t qlora_qscale_bytes(int64_t in, int64_t out) {
  return (size_t)(in * out / QLORA_BLOCK);
}
static inline size_t qlora_gscale_count(int64_t in, int64_t out) {
  return (size_t)((in * out / QLORA_BLOCK + QLORA_GROUP - 1) / QLORA_GROUP);
}

/*
 * qlora_quantize: Wq = Q(W0).
 *   W0  [in, out] fp32, device.  wq: host struct whose in/out give the shape
 *   and whose three device buffers are overwritten.
 * Encoding ("LLMs · QLoRA" listing): c_b = max |w| over the block (exact);
 * x = w / c_b rounded to fp32 (IEEE, round to nearest even); code = the
 * index i minimising fp32(|x - L_i|), the lower index on a tie; a block with
 * c_b = 0 encodes as x = 0 (code 7).  Double quantization ("What QLoRA
 * adds"): s2_g = fp32(max_b c_b) / 127, q_b = round_half_even(c_b / s2_g) in
 * fp32; an all-zero group has s2_g = 0 and q_b = 0.  Codes use the exact c_b.
 * With wq->block == 16: c_g = max |w| over each 16 consecutive weights, the
 * same encoding with c_g in place of c_b, and c_g stored in gscale (no
 * double quantization).
 */
qlora_status qlora_quantize(const float *W0, const qlora_nf4 *wq, hipStream_t stream);

/*
 * qlora_linear_fwd: y = X.deq(Wq) + XA.B with XA = X.A
 *   ("How it works" step 2; "Mathematical Formulation" forward pass).
 *   X   [M, in]  act dtype         Y  [M, out] act dtype (output)
 *   A   [in, r]  adt dtype         B  [r, out] adt dtype
 *   XA  [M, r]   fp32 (output, optional: the saved activation the backward
 *                reads; NULL skips it, and the backward then recomputes it).
 * The base weight is expanded to bf16 in registers, w = bf16(L[code] *
 * (q_b * s2_g)) computed in fp32; X (and XA, B) enter the bf16 matrix cores
 * rounded to bf16; accumulation is fp32.  ws must hold
 * qlora_fwd_workspace_bytes(M, in, out, r, act) bytes of device memory.
 * r = 0 gives a plain NF4 linear (A, B may be NULL).  M = 0 is a no-op
 * (ws may be NULL).
 */
qlora_status qlora_linear_fwd(const qlora_nf4 *wq, const void *X, int64_t M,
                              qlora_dtype act, const void *A, const void *B,
                              int32_t r, qlora_dtype adt, void *Y, float *XA,
                              void *ws, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes qlora_linear_fwd needs for this shape and activation dtype
 * (host-only); 0 when M == 0 or the arguments are invalid. */
size_t qlora_fwd_workspace_bytes(int64_t M, int64_t in, int64_t out, int32_t r,
                                 qlora_dtype act);

/*
 * qlora_linear_fwd_noalloc: qlora_linear_fwd without a workspace argument,
 * for callers that cannot allocate device memory at the call: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, kernels and output bits as qlora_linear_fwd.  Its scratch
 * is a device-resident array of QLORA_NOALLOC_SCRATCH_BYTES inside the
 * library, one per GPU, held until the process ends; the call allocates
 * nothing.  A shape whose qlora_fwd_workspace_bytes exceeds that size is
 * refused with QLORA_ERR_WORKSPACE before anything touches the device.
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (two streams, two threads) race and must be serialized by the caller.
 */
#define QLORA_NOALLOC_SCRATCH_BYTES (32u << 20)
qlora_status qlora_linear_fwd_noalloc(const qlora_nf4 *wq, const void *X, int64_t M,
                                      qlora_dtype act, const void *A, const void *B,
                                      int32_t r, qlora_dtype adt, void *Y, float *XA,
                                      hipStream_t stream);

/*
 * qlora_linear_bwd: with G = dY.B^T,
 *   dX = dY.deq(Wq)^T + G.A^T   (act dtype, [M, in]; NULL skips dX)
 *   dA = X^T.G                  (fp32, [in, r])
 *   dB = XA^T.dY                (fp32, [r, out])
 * ("How it works" steps 3-4: dA = dW B^T and dB = A^T dW with dW = X^T dY,
 * evaluated in factored form so dW is never formed; the base weight gets no
 * gradient.)  XA is the forward's saved X.A (fp32 [M, r]); NULL recomputes it
 * into the workspace.  ws must hold qlora_bwd_workspace_bytes(M, in, out, r,
 * act) bytes of device memory.  r = 0 computes dX only (A, B, dA, dB, XA may
 * be NULL).  M = 0 writes zeros to dA and dB (ws may be NULL).
 * With bf16 activations, M >= 1024, r <= 16 and r % 4 == 0, dB is formed
 * inside the dX GEMM from a bf16 copy of XA (one partial per 256 tokens);
 * without dX (dX == NULL) it comes from the pass over dY with XA in fp32, so
 * the two calls may differ in the last bits of dB (both within the stated
 * accuracy).  Same arguments always give the same bits.
 */
qlora_status qlora_linear_bwd(const qlora_nf4 *wq, const void *X, const void *dY,
                              int64_t M, qlora_dtype act, const void *A,
                              const void *B, int32_t r, qlora_dtype adt,
                              const float *XA, void *dX, float *dA, float *dB,
                              void *ws, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes qlora_linear_bwd needs for this shape and activation dtype
 * (host-only); 0 when M == 0 or the arguments are invalid. */
size_t qlora_bwd_workspace_bytes(int64_t M, int64_t in, int64_t out, int32_t r,
                                 qlora_dtype act);

/*
 * Adapter options ("LoRA & QLoRA", sections Scaling Factor alpha and
 * Dropout): the rank-r path becomes alpha/r . B(dropout(A x)), in row form
 *   U = c * (keep o XA),  c = scale / (1 - dropout_p),
 *   y = X.deq(Wq) + U.B,
 * with keep the caller's dropout draw (the library draws no random numbers).
 *   scale      alpha / r; any finite value (1 = no scaling).
 *   dropout_p  the dropout probability, 0 <= p < 1; kept elements are scaled
 *              by 1 / (1 - p) (inverted dropout).
 *   keep       [M, r] uint8 row-major, device, nonzero = kept; NULL = no
 *              dropout (then dropout_p must be 0).  The same mask must be
 *              passed to the forward and the backward of one step.
 * c is computed in double and rounded to fp32 once.  The backward follows
 * the chain rule: G' = c * (keep o dY.B^T) takes G's place in dX and dA, and
 * dB = U^T.dY.  XA (the saved activation) is always the plain X.A.  Invalid
 * options give QLORA_ERR_VALUE.
 */
typedef struct {
  float scale;
  float dropout_p;
  const uint8_t *keep;
} qlora_lora;

/* qlora_linear_fwd with adapter options (lora == NULL: qlora_linear_fwd). */
qlora_status qlora_linear_fwd_lora(const qlora_nf4 *wq, const void *X, int64_t M,
                                   qlora_dtype act, const void *A, const void *B,
                                   int32_t r, qlora_dtype adt, const qlora_lora *lora,
                                   void *Y, float *XA, void *ws, size_t ws_bytes,
                                   hipStream_t stream);

/* qlora_linear_bwd with adapter options (lora == NULL: qlora_linear_bwd). */
qlora_status qlora_linear_bwd_lora(const qlora_nf4 *wq, const void *X, const void *dY,
                                   int64_t M, qlora_dtype act, const void *A,
                                   const void *B, int32_t r, qlora_dtype adt,
                                   const qlora_lora *lora, const float *XA, void *dX,
                                   float *dA, float *dB, void *ws, size_t ws_bytes,
                                   hipStream_t stream);

/*
 * The backward with one Adam (AdamW) step of A and B fused into its final
 * reduction launch (the adapter update of "The code, line by line": the
 * optimizer holds only A and B), the same arithmetic as qlora_adam_step:
 * given the same gradients, the same bits.
 *   state_A / state_B: the fp32 master copy theta ([in, r] / [r, out]), the
 *     moments m, v (same layout, zero before step 1) and an optional bf16
 *     copy of the updated theta.  theta may be the A (B) the call reads when
 *     adt = QLORA_F32, and theta_bf16 the one it reads when adt = QLORA_BF16:
 *     every read of A and B comes before the update.
 *   hparams: step >= 1, 0 <= beta < 1, eps >= 0, weight_decay >= 0, finite
 *     lr (else QLORA_ERR_VALUE).
 *   dA, dB: NULL, or also receive the gradients.
 * Otherwise as qlora_linear_bwd_lora (lora may be NULL); M must be >= 1.
 */
typedef struct {
  float *theta;
  float *m;
  float *v;
  uint16_t *theta_bf16;
} qlora_adam_state;

typedef struct {
  int64_t step;
  float lr;
  float beta1;
  float beta2;
  float eps;
  float weight_decay;
} qlora_adam_hparams;

qlora_status qlora_linear_bwd_adam(const qlora_nf4 *wq, const void *X, const void *dY,
                                   int64_t M, qlora_dtype act, const void *A,
                                   const void *B, int32_t r, qlora_dtype adt,
                                   const qlora_lora *lora, const float *XA, void *dX,
                                   const qlora_adam_state *state_A,
                                   const qlora_adam_state *state_B,
                                   const qlora_adam_hparams *hparams, float *dA,
                                   float *dB, void *ws, size_t ws_bytes,
                                   hipStream_t stream);

/*
 * qlora_linear_fwd_group: the forward of up to 4 independent linears in one
 * pair of launches, for decode (the q, k, v projections of a step share
 * their input; gate and up too).  Only the few-token path: 1 <= M <= 16 and
 * r <= 64, the same M, r, act, adt and codebook for all n; linear l has its
 * own wq[l], X[l] [M, in_l], A[l], B[l], Y[l] [M, out_l] and XA[l] (as in
 * qlora_linear_fwd; X[l] may be shared; XA itself or any XA[l] may be NULL).  Each workgroup belongs to one
 * linear, so every output is bit-identical to qlora_linear_fwd of that
 * linear alone.  ws: qlora_fwd_group_workspace_bytes(n, M, in, out, r, act)
 * bytes (in, out: host arrays of the n shapes).  Other shapes or n outside
 * 1..4: QLORA_ERR_SHAPE; codebooks that differ: QLORA_ERR_DTYPE.
 */
qlora_status qlora_linear_fwd_group(int32_t n, const qlora_nf4 *const *wq,
                                    const void *const *X, int64_t M, qlora_dtype act,
                                    const void *const *A, const void *const *B, int32_t r,
                                    qlora_dtype adt, void *const *Y, float *const *XA,
                                    void *ws, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes of qlora_linear_fwd_group (host-only); 0 if invalid. */
size_t qlora_fwd_group_workspace_bytes(int32_t n, int64_t M, const int64_t *in,
                                       const int64_t *out, int32_t r, qlora_dtype act);

/*
 * qlora_merge: the merged dense weight W = deq(Wq) + A.B
 *   ("How it works" step 5: fold the trained adapters into the base weight;
 *   "What the simulations show": the result is a dense float matrix, off the
 *   quantization grid).
 *   A [in, r], B [r, out] in adt; W [in, out] in wdt (output, caller-owned).
 * Per element in fp32: L[code] * (q_b * s2_g), plus the rank-r sum, rounded
 * once to wdt.  With r % 8 == 0 the sum runs on the matrix cores (fp32
 * additions in the hardware's order; bf16 adapters give exact products);
 * otherwise it is accumulated in rank order with fp32 fused multiply-adds.
 * r = 0 writes deq(Wq) (A, B may be NULL).  To store the merged weight
 * in 4 bits again, merge with wdt = QLORA_F32 and pass W to qlora_quantize
 * ("When it breaks": corrections smaller than a quantization step are lost).
 */
qlora_status qlora_merge(const qlora_nf4 *wq, const void *A, const void *B, int32_t r,
                         qlora_dtype adt, void *W, qlora_dtype wdt, hipStream_t stream);

/*
 * qlora_adam_step: one Adam step of an adapter matrix (A or B), in place.
 * ("The code, line by line": the optimizer is handed only A and B.)  The
 * pages do not print the update; this is the published Adam algorithm
 * (Kingma & Ba) with decoupled weight decay (AdamW), per element in fp32:
 *   m <- beta1*m + (1-beta1)*g;  v <- beta2*v + (1-beta2)*g*g;
 *   theta <- theta - lr*((m*c1) / (sqrt(v*c2) + eps) + weight_decay*theta),
 *   c1 = 1/(1 - beta1^step), c2 = 1/(1 - beta2^step) (double on the host,
 *   rounded to fp32).  weight_decay = 0 is plain Adam.
 *   theta, grad, m, v: n fp32 elements each (device, 16-B aligned; the
 *   moments start at zero before step 1).  theta_bf16 (nullable): also
 *   receives the updated theta in bf16, for a bf16 forward.
 * n = 0 is a no-op.  step >= 1, 0 <= beta < 1, eps >= 0, weight_decay >= 0
 * and finite lr, else QLORA_ERR_VALUE (n < 0 or step < 1: QLORA_ERR_SHAPE).
 */
qlora_status qlora_adam_step(float *theta, const float *grad, float *m, float *v, int64_t n,
                             int64_t step, float lr, float beta1, float beta2, float eps,
                             float weight_decay, uint16_t *theta_bf16, hipStream_t stream);

/*
 * qlora_loftq_init: adapters started from the quantization residual instead
 * of B = 0 ("What QLoRA adds", the paragraph on running it: LoftQ-style
 * methods start A and B from an SVD of W0 - Q(W0)).
 *   W0 [in, out] fp32 (the weight wq was quantized from), omega [out, k]
 *   fp32: the caller's random test matrix (e.g. standard normal), k >= r
 *   columns (r plus some oversampling, k <= 128 and k <= in, out).
 *   Output A [in, r], B [r, out] in adt: the rank-r truncated SVD
 *   U_r S_r V_r^T of R = W0 - deq(Wq), split as A = U_r sqrt(S_r),
 *   B = sqrt(S_r) V_r^T, found by randomized subspace iteration with
 *   `iters` power iterations (0..16; 2 is usual).  R is formed on the fly in
 *   fp32 by the GPU products R.M and R^T.M.  The thin panels (fp32) are
 *   orthonormalised by Cholesky QR applied twice (Gram matrices and panel
 *   updates in fp64 arithmetic); the k x k steps (each Cholesky factor's
 *   inverse, the final SVD by one-sided Jacobi rotations) run in fp64 on the
 *   GPU as well.  ws: qlora_loftq_workspace_bytes(in, out, k) bytes of device
 *   memory.  Asynchronous like the other calls: the work is enqueued on
 *   `stream` and the call never waits for the device, so it can be captured
 *   in a graph; W0, omega, wq's arrays, A, B and ws must stay valid (and A,
 *   B, ws untouched by other work) until the stream has run it.
 */
qlora_status qlora_loftq_init(const float *W0, const qlora_nf4 *wq, const float *omega,
                              int32_t k, int32_t r, int32_t iters, void *A, void *B,
                              qlora_dtype adt, void *ws, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes qlora_loftq_init needs (host-only); 0 for invalid
 * arguments. */
size_t qlora_loftq_workspace_bytes(int64_t in, int64_t out, int32_t k);

/* Human-readable name of a status code (host-only, static string). */
const char *qlora_status_string(qlora_status s);

/* The library's own fp32 level table L[0..15], ascending, derived from the
 * level definition ("LLMs · QLoRA") in double precision (host-only). */
void qlora_levels(float out[16]);

/* Decision thresholds of the encoder (host-only): code = #{j in 1..15 :
 * x >= T[j]} reproduces the fp32 argmin rule exactly; out[j-1] = T[j]. */
void qlora_thresholds(float out[15]);

/* The same two tables for any codebook (host-only); return 0, or -1 for an
 * unknown codebook or a NULL out (nothing written). */
int qlora_codebook_levels(int codebook, float out[16]);
int qlora_codebook_thresholds(int codebook, float out[15]);

/*
 * Kernel-level event timing (instrumentation; off by default).
 * qlora_timing_enable(mask): bit k of mask selects kernel kind k; every
 * launch of a selected kind is bracketed by a pair of HIP events recorded on
 * the call's stream (mask 0 turns timing off).  qlora_timing_read
 * synchronizes those events and returns the summed duration (ms) and the
 * number of launches of one kind since the last reset.  The mask is read
 * atomically and the records are guarded by a lock, so these calls may run
 * on any thread while other threads launch; the records are process-wide.
 */
typedef enum {
  QLORA_KERNEL_QUANTIZE = 0,
  QLORA_KERNEL_XA = 1,          /* XA = X.A (forward; backward recompute) */
  QLORA_KERNEL_FWD_GEMM = 2,    /* fused y = X.deq(Wq) + XA.B             */
  QLORA_KERNEL_DY_PASS = 3,     /* G = dY.B^T and dB partials             */
  QLORA_KERNEL_DX_GEMM = 4,     /* fused dX = dY.deq(Wq)^T + G.A^T        */
  QLORA_KERNEL_DA_PASS = 5,     /* dA = X^T.G (partials, or whole with dB) */
  QLORA_KERNEL_REDUCE = 6,      /* deterministic reduction of partials    */
  QLORA_KERNEL_FWD_SMALLM = 7,  /* small-M forward                        */
  QLORA_KERNEL_COUNT = 8
} qlora_kernel_kind;

int qlora_timing_enable(int kind_mask);
int qlora_timing_read(int kind, double *total_ms, int64_t *launches);
void qlora_timing_reset(void);
const char *qlora_kernel_name(int kind);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_H */
