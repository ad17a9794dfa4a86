"""Level tables and parameter counts (oracle; test infrastructure only).

Sources:
* "LLMs · QLoRA" (blog.sahaj.si), the NormalFloat paragraph and the code
  listing under it: NF4-style levels are normal quantiles at 16 evenly spaced
  probabilities from 0.02 to 0.98, normalised to [-1, 1] by the largest
  magnitude; the comparison grid is 16 evenly spaced values in [-1, 1].
* "QLoRA (low-rank adapters on a quantized model)", section "How it works":
  an adapter pair costs r*(in+out) parameters per layer.

Reading taken (the listing calls its own table "an approximation"): the
quantiles are evaluated in double precision and the normalised table is
rounded to fp32 once.  The listing's float32 pipeline moves some levels by a
few ulp and makes the table slightly asymmetric; on the listing's own sample
both tables give the same codes.
"""

from statistics import NormalDist

import numpy as np

N_LEVELS = 16
P_LO = 0.02
P_HI = 0.98


def _probabilities():
    """16 evenly spaced probabilities in [0.02, 0.98] (double)."""
    n = N_LEVELS - 1
    return [(P_LO * (n - i) + P_HI * i) / n for i in range(N_LEVELS)]


def nf4_levels():
    """NF4-style level table, 16 fp32 values, ascending.

    q_i = Phi^-1(p_i) in double (Wichura's AS241 via ``statistics``), then
    L_i = fp32(q_i / max_j |q_j|).
    """
    nd = NormalDist()
    q = [nd.inv_cdf(p) for p in _probabilities()]
    qmax = max(abs(v) for v in q)
    return np.array([v / qmax for v in q], dtype=np.float64).astype(np.float32)


def uniform4_levels():
    """Uniform 4-bit grid: 16 evenly spaced values in [-1, 1], fp32."""
    n = N_LEVELS - 1
    return np.array([-1.0 + 2.0 * i / n for i in range(N_LEVELS)],
                    dtype=np.float64).astype(np.float32)


def int_levels(h):
    """Symmetric integer grid k / h (|k| <= h) as a 16-entry level table, fp32.

    "QLoRA (low-rank adapters on a quantized model)", "The code, line by
    line" and "What the simulations show": the lab quantizes to symmetric
    uniform integers, "2-bit" being ternary {-s, 0, s}.  h = 7, 3, 1 for 4,
    3 and 2 bits.  Entry 8 + m is +m/h and entry 7 - m is -m/h (m = 0..7):
    zero appears twice (-0.0, +0.0) and magnitudes m > h lie beyond 1, where
    x = w / absmax never reaches them; each entry is m/h in double rounded
    to fp32 once.
    """
    mag = np.array([m / h for m in range(8)], dtype=np.float64).astype(np.float32)
    return np.concatenate([-mag[::-1], mag]).astype(np.float32)


def adapter_params(n_in, n_out, rank):
    """Trainable parameters of one adapter pair A (in x r), B (r x out)."""
    return rank * (n_in + n_out)
