"""Adapted linear layer, forward and backward, in float64 (oracle).

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.

Notation follows "QLoRA (low-rank adapters on a quantized model)", section
"How it works": the weight is stored (in, out); A is (in x r), B is (r x out);
the layer's weight is W = Wq + A B; the dense weight gradient gives
dA = dW B^T and dB = A^T dW.  In row form the layer is y = X W, so with
dY = dL/dy:

  forward   XA = X A,          y  = X Wq + XA B
  backward  G  = dY B^T,       dX = dY Wq^T + G A^T,
            dA = X^T G,        dB = XA^T dY

The factored dA, dB equal dW B^T and A^T dW with dW = X^T dY (matrix
products are associative); ``backward_via_dense_dw`` computes them the way
the chain rule is written, for tiny shapes.  "LoRA & QLoRA",
"Mathematical Formulation", gives the same layer in column form,
h = W0 x + B (A x).  ``forward_lora`` / ``backward_lora`` add the alpha/r
factor and the dropout on A x of that page's Scaling Factor alpha and Dropout
sections (the mask is an input); there is no bias.

Every operand is widened to float64 first; the caller passes exactly the
values the GPU receives (bf16 inputs already rounded), so the only error left
in a comparison is the GPU's.
"""

import numpy as np


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def forward(X, W_hat, A=None, B=None):
    """Returns (XA, y).  ``W_hat`` is the dequantized (in, out) weight.

    With rank 0 (A or B is None) XA is an (M, 0) array and y = X W_hat.
    """
    X = _f64(X)
    y = X @ _f64(W_hat)
    if A is None or B is None or _f64(A).shape[1] == 0:
        return np.zeros((X.shape[0], 0)), y
    XA = X @ _f64(A)
    return XA, y + XA @ _f64(B)


def backward(X, dY, W_hat, A=None, B=None, XA=None):
    """Returns dict with G, dX, dA, dB (factored; dW never formed)."""
    X = _f64(X)
    dY = _f64(dY)
    dX = dY @ _f64(W_hat).T
    if A is None or B is None or _f64(A).shape[1] == 0:
        r = 0
        return {"G": np.zeros((X.shape[0], r)), "dX": dX,
                "dA": np.zeros((X.shape[1], r)), "dB": np.zeros((r, dY.shape[1]))}
    A = _f64(A)
    B = _f64(B)
    if XA is None:
        XA = X @ A
    G = dY @ B.T
    dX = dX + G @ A.T
    dA = X.T @ G
    dB = _f64(XA).T @ dY
    return {"G": G, "dX": dX, "dA": dA, "dB": dB}


def lora_factor(scale, dropout_p):
    """c = scale / (1 - p) computed in double and rounded to fp32 once (the
    multiplier the library applies to kept elements)."""
    return float(np.float32(float(scale) / (1.0 - float(dropout_p))))


def forward_lora(X, W_hat, A, B, scale, dropout_p=0.0, keep=None):
    """Returns (XA, U, y) with the alpha/r factor and dropout on X A.

    "LoRA & QLoRA", sections Scaling Factor alpha and Dropout: the adapter
    path is scaled by alpha/r and dropout is applied to A x, the rank-r
    intermediate.  In row form, with the caller's keep mask K (nonzero =
    kept) and inverted dropout (kept elements scaled by 1/(1 - p)):
      U = c * (K o XA),  c = scale / (1 - p),   y = X W_hat + U B.
    ``keep`` None means no dropout (every element kept).  XA is the plain
    X A (what the layer saves for the backward).
    """
    X = _f64(X)
    XA = X @ _f64(A)
    c = lora_factor(scale, dropout_p)
    K = np.ones_like(XA) if keep is None else (np.asarray(keep) != 0).astype(np.float64)
    U = c * (K * XA)
    return XA, U, X @ _f64(W_hat) + U @ _f64(B)


def backward_lora(X, dY, W_hat, A, B, scale, dropout_p=0.0, keep=None):
    """Gradients of ``forward_lora`` by the chain rule:
      G = dY B^T,  G' = c * (K o G)   (dL/dXA),
      dX = dY W_hat^T + G' A^T,  dA = X^T G',  dB = U^T dY.
    """
    X, dY, A, B = _f64(X), _f64(dY), _f64(A), _f64(B)
    XA = X @ A
    c = lora_factor(scale, dropout_p)
    K = np.ones_like(XA) if keep is None else (np.asarray(keep) != 0).astype(np.float64)
    U = c * (K * XA)
    G = dY @ B.T
    Gp = c * (K * G)
    return {"G": Gp, "dX": dY @ _f64(W_hat).T + Gp @ A.T, "dA": X.T @ Gp, "dB": U.T @ dY}


def backward_via_dense_dw(X, dY, W_hat, A, B):
    """Chain rule through the merged weight W = W_hat + A B, as written:
    dW = X^T dY, dA = dW B^T, dB = A^T dW, dX = dY W^T.  Tiny shapes only."""
    X, dY, A, B = _f64(X), _f64(dY), _f64(A), _f64(B)
    W = _f64(W_hat) + A @ B
    dW = X.T @ dY
    return {"dW": dW, "dX": dY @ W.T, "dA": dW @ B.T, "dB": A.T @ dW}


def merge(W_hat, A=None, B=None):
    """The merged dense weight W = W_hat + A B (float64, shape (in, out)).

    "QLoRA (low-rank adapters on a quantized model)", "How it works", step 5:
    after training the adapters may be folded into the base weight, which
    is then a dense float matrix, off the quantization grid ("What the
    simulations show"); re-quantizing it (``nf4.quantize``) gives the
    4-bit storage back at some loss ("When it breaks").  Rank 0 (A or B is
    None) returns W_hat.
    """
    W = _f64(W_hat).copy()
    if A is None or B is None or _f64(A).shape[1] == 0:
        return W
    return W + _f64(A) @ _f64(B)


def residual(W0, W_hat):
    """R = W0 - deq(Q(W0)) in float64: what the quantizer lost."""
    return _f64(W0) - _f64(W_hat)


def loftq_init(W0, W_hat, r):
    """Adapters that start from the residual instead of zero.

    "QLoRA (low-rank adapters on a quantized model)", "What QLoRA adds" (the
    paragraph on running it and its relatives): LoftQ-style methods start A
    and B from an SVD of W0 - Q(W0), so training begins closer to the
    original model.  Reading taken: the best rank-r approximation of the
    residual (truncated SVD, numpy's LAPACK routine as the step), split
    evenly, A = U_r sqrt(S_r), B = sqrt(S_r) V_r^T.  Returns (A, B) float64.
    """
    R = residual(W0, W_hat)
    U, S, Vt = np.linalg.svd(R, full_matrices=False)
    s = np.sqrt(S[:r])
    return U[:, :r] * s, s[:, None] * Vt[:r]
