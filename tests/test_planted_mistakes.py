"""The oracle's pins have teeth: each test plants one plausible mistake in a
copy of an oracle function (on the CPU, never in the HIP path) and shows
that the corresponding pin rejects it."""

import numpy as np
import pytest

import oracle
from oracle import nf4 as onf4

import test_oracle_pins as pins


def _encode_ties_high(w_flat, c, levels=None):
    """Mistake: ties resolved to the higher index."""
    L = oracle.nf4_levels() if levels is None else np.asarray(levels, np.float32)
    w = np.asarray(w_flat, np.float32).reshape(-1, 64)
    cc = np.asarray(c, np.float32).reshape(-1, 1)
    safe = np.where(cc == 0, np.float32(1), cc)
    x = np.where(cc == 0, np.float32(0), (w / safe).astype(np.float32))
    d = np.abs(x[..., None] - L)
    return (15 - np.argmin(d[..., ::-1], axis=-1)).astype(np.uint8).reshape(-1)


def _encode_no_fp32(w_flat, c, levels=None):
    """Mistake: nearest level chosen in float64 and against the midpoint only
    (drops the fp32 tie behaviour around x = 0)."""
    L = (oracle.nf4_levels() if levels is None else np.asarray(levels, np.float32)).astype(np.float64)
    w = np.asarray(w_flat, np.float64).reshape(-1, 64)
    cc = np.asarray(c, np.float64).reshape(-1, 1)
    x = np.where(cc == 0, 0.0, w / np.where(cc == 0, 1.0, cc))
    mids = 0.5 * (L[1:] + L[:-1])
    return np.searchsorted(mids, x.reshape(-1), side="left").astype(np.uint8)


def _unnormalised_levels():
    """Mistake: quantiles not divided by the largest magnitude."""
    from statistics import NormalDist
    p = [(0.02 * (15 - i) + 0.98 * i) / 15 for i in range(16)]
    return np.array([NormalDist().inv_cdf(v) for v in p], np.float32)


def _dq_wrong_qmax(c):
    """Mistake: scales quantized against 255 instead of the symmetric 127."""
    c = np.asarray(c, np.float32)
    ng = (c.size + 255) // 256
    q8 = np.zeros(c.size, np.int8)
    s2 = np.zeros(ng, np.float32)
    for g in range(ng):
        cg = c[g * 256:(g + 1) * 256]
        s = np.float32(cg.max()) / np.float32(255)
        s2[g] = s
        if s:
            q8[g * 256:(g + 1) * 256] = np.clip(np.rint(cg / s), -127, 127).astype(np.int8)
    return q8, s2


def _dequant_transposed(packed, q8, s2, n_in, n_out):
    """Mistake: the flat code order read back as (out, in)."""
    W = oracle.dequantize(packed, q8, s2, n_in, n_out)
    return W.reshape(-1).reshape(n_out, n_in).T


def _forward_no_adapter(X, W, A=None, B=None):
    XA, y = oracle.forward(X, W, A, B)
    return XA, np.asarray(X, np.float64) @ np.asarray(W, np.float64)


def _backward_wrong_sign(X, dY, W, A=None, B=None, XA=None):
    g = oracle.backward(X, dY, W, A, B, XA)
    g["dX"] = g["dX"] - 2 * g["G"] @ np.asarray(A, np.float64).T
    return g


def _backward_dB_from_A(X, dY, W, A=None, B=None, XA=None):
    """Mistake: dB = A^T dY-shaped product built from the wrong operand."""
    g = oracle.backward(X, dY, W, A, B, XA)
    Xf = np.asarray(X, np.float64)
    g["dB"] = (Xf @ np.asarray(A, np.float64)[:, ::-1]).T @ np.asarray(dY, np.float64)
    return g


def _quantize_against_dq_scale(w0, levels=None):
    """Mistake: the codes taken against the double-quantized scale
    q_b * s2_g instead of the block's exact absmax."""
    w = np.ascontiguousarray(w0, np.float32).reshape(-1)
    c = onf4.block_absmax(w)
    q8, s2 = onf4.double_quantize(c)
    c_hat = (q8.astype(np.float32) * np.repeat(s2, 256)[:q8.size]).astype(np.float32)
    codes = onf4.encode(w, c_hat, levels)
    return {"codes": codes, "packed": onf4.pack_codes(codes), "absmax": c, "q8": q8, "s2": s2}


def _groups_of_64(w0, levels, group=16):
    """Mistake: one scale per 64 entries (the NF4 block) instead of 16."""
    q = onf4.quantize_groups(w0, levels, group=64)
    return {**q, "scales": np.repeat(q["scales"], 4)}


def _groups_down_columns(w0, levels, group=16):
    """Mistake: groups of 16 consecutive rows of a column, not of the
    flattened (in, out) matrix."""
    w = np.ascontiguousarray(w0, np.float32)
    q = onf4.quantize_groups(w.T.copy(), levels, group)
    codes = q["codes"].reshape(w.shape[1], w.shape[0]).T.reshape(-1)
    scales = np.repeat(q["scales"].reshape(w.shape[1], w.shape[0] // group), group, axis=1)
    scales = scales.T.reshape(-1)[::group]
    return {"codes": codes, "packed": onf4.pack_codes(codes), "scales": scales}


def test_wrong_group_size_is_caught():
    with pytest.raises(AssertionError):
        pins.check_group_quantizer(_groups_of_64)


def test_groups_down_columns_are_caught():
    with pytest.raises(AssertionError):
        pins.check_group_quantizer(_groups_down_columns)


def test_codes_against_dq_scale_are_caught():
    with pytest.raises(AssertionError):
        pins.check_quantize_scale_rule(_quantize_against_dq_scale)


def test_ties_high_is_caught():
    with pytest.raises(AssertionError):
        pins.check_encode_rules(_encode_ties_high)


def test_float64_midpoint_rule_is_caught():
    with pytest.raises(AssertionError):
        pins.check_encode_rules(_encode_no_fp32)


def test_unnormalised_levels_are_caught():
    with pytest.raises(AssertionError):
        pins.check_level_table(_unnormalised_levels())
    with pytest.raises(AssertionError):
        pins.check_p2_example(oracle.encode, _unnormalised_levels(), oracle.uniform4_levels())


def test_wrong_dq_range_is_caught():
    with pytest.raises(AssertionError):
        pins.check_double_quant(_dq_wrong_qmax)


def test_transposed_dequant_is_caught():
    with pytest.raises(AssertionError):
        pins.check_dequant_layout(_dequant_transposed)


def test_dropped_adapter_term_is_caught():
    with pytest.raises(AssertionError):
        pins.check_forward(_forward_no_adapter)


def test_wrong_sign_in_dX_is_caught():
    with pytest.raises(AssertionError):
        pins.check_backward_fd(oracle.forward, _backward_wrong_sign)


def test_wrong_operand_in_dB_is_caught():
    with pytest.raises(AssertionError):
        pins.check_backward_fd(oracle.forward, _backward_dB_from_A)


def _merge_wrong_sign(W, A=None, B=None):
    """Mistake: the adapter product subtracted from the base weight."""
    W = np.asarray(W, np.float64)
    if A is None or B is None:
        return W.copy()
    return W - np.asarray(A, np.float64) @ np.asarray(B, np.float64)


def test_wrong_sign_in_merge_is_caught():
    with pytest.raises(AssertionError):
        pins.check_merge(_merge_wrong_sign)


def _adam_no_bias_correction(theta, g, m, v, t, lr, beta1=0.9, beta2=0.999, eps=1e-8,
                             weight_decay=0.0):
    """Mistake: the moments used without bias correction."""
    theta, g = np.asarray(theta, np.float64), np.asarray(g, np.float64)
    m = beta1 * np.asarray(m, np.float64) + (1 - beta1) * g
    v = beta2 * np.asarray(v, np.float64) + (1 - beta2) * g * g
    return theta - lr * (m / (np.sqrt(v) + eps) + weight_decay * theta), m, v


def test_adam_without_bias_correction_is_caught():
    with pytest.raises(AssertionError):
        pins.check_adam(_adam_no_bias_correction)


def _loftq_smallest(W0, W_hat, r):
    """Mistake: the r smallest singular directions taken."""
    R = np.asarray(W0, np.float64) - np.asarray(W_hat, np.float64)
    U, S, Vt = np.linalg.svd(R, full_matrices=False)
    s = np.sqrt(S[-r:])
    return U[:, -r:] * s, s[:, None] * Vt[-r:]


def test_loftq_smallest_directions_are_caught():
    with pytest.raises(AssertionError):
        pins.check_loftq(_loftq_smallest)


def _backward_lora_unmasked_G(X, dY, W, A, B, scale, dropout_p=0.0, keep=None):
    """Mistake: the dropout mask is left out of the gradient of X A."""
    g = oracle.backward_lora(X, dY, W, A, B, scale, dropout_p, None)
    ref = oracle.backward_lora(X, dY, W, A, B, scale, dropout_p, keep)
    return {**g, "dB": ref["dB"]}


def test_unmasked_lora_gradient_is_caught():
    with pytest.raises(AssertionError):
        pins.check_lora(oracle.forward_lora, _backward_lora_unmasked_G)


def _forward_lora_no_rescale(X, W, A, B, scale, dropout_p=0.0, keep=None):
    """Mistake: kept elements are not scaled by 1 / (1 - p)."""
    return oracle.forward_lora(X, W, A, B, scale * (1.0 - dropout_p), dropout_p, keep)


def test_dropout_without_rescale_is_caught():
    with pytest.raises(AssertionError):
        pins.check_lora(_forward_lora_no_rescale, oracle.backward_lora)
