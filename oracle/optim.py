"""Adam update of the adapter matrices, in float64 (oracle).

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.

"QLoRA (low-rank adapters on a quantized model)", "The code, line by line":
the optimizer is handed only A and B (Adam over the adapter matrices), so
nothing else changes; "LoRA & QLoRA" builds the same step with AdamW.  The
pages print neither the update nor its constants, so this follows the
published algorithm (Kingma & Ba, "Adam: A Method for Stochastic
Optimization", Algorithm 1), with decoupled weight decay as in AdamW
(Loshchilov & Hutter, "Decoupled Weight Decay Regularization"): at step t,

  m <- beta1 m + (1 - beta1) g
  v <- beta2 v + (1 - beta2) g^2
  theta <- theta - lr ( (m / (1 - beta1^t)) / (sqrt(v / (1 - beta2^t)) + eps)
                        + weight_decay * theta )

``weight_decay = 0`` is plain Adam.
"""

import numpy as np


def adam_step(theta, g, m, v, t, lr, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0):
    """One step; returns new (theta, m, v) as float64 arrays (inputs unchanged)."""
    theta = np.asarray(theta, np.float64)
    g = np.asarray(g, np.float64)
    m = beta1 * np.asarray(m, np.float64) + (1.0 - beta1) * g
    v = beta2 * np.asarray(v, np.float64) + (1.0 - beta2) * g * g
    m_hat = m / (1.0 - beta1 ** t)
    v_hat = v / (1.0 - beta2 ** t)
    theta = theta - lr * (m_hat / (np.sqrt(v_hat) + eps) + weight_decay * theta)
    return theta, m, v
