"""GPU parity of the adapter options (alpha/r factor and dropout on X.A,
"LoRA & QLoRA", sections Scaling Factor alpha and Dropout) against the
float64 oracle, through every path that carries a rank-r intermediate: the
whole-K rank passes with dB inside the dX GEMM, dB in the dY pass (r > 16,
fp32 activations), the split-K passes, and the few-token forward.  Plus the
identities the options must keep: no scaling and no mask is the plain call
bit for bit, and a mask of zeros leaves the base layer alone."""

import numpy as np
import pytest

import oracle
from quantized_rank_fine_amd import qlora as q

from gpu_harness import TOL, Layer, out_to_f64, rel_err, say, torch_dev

pytestmark = pytest.mark.gpu


def _mask(M, r, p, seed):
    return (np.random.default_rng(seed).random((M, r)) >= p).astype(np.uint8)


def _dev(a):
    torch, dev = torch_dev()
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


@pytest.mark.parametrize("M,n_in,n_out,r,act,adt", [
    (1030, 320, 448, 16, "bf16", "bf16"),   # whole-K rank passes, dB in the dX GEMM
    (1300, 384, 320, 12, "bf16", "f32"),    # dB in the dX GEMM, ragged token block
    (1100, 1088, 320, 24, "bf16", "f32"),   # r > 16: dB in the dY pass, from mul(XA)
    (1100, 384, 320, 16, "f32", "bf16"),    # fp32 activations: dB in the dY pass
    (300, 640, 704, 16, "bf16", "bf16"),    # split-K rank passes
    (130, 320, 448, 5, "f32", "f32"),       # split-K, r % 8 != 0, element paths
    (5, 576, 448, 16, "bf16", "bf16"),      # few-token forward
])
@pytest.mark.parametrize("scale,p", [(2.0, 0.25), (0.5, 0.0)])
def test_lora_parity(M, n_in, n_out, r, act, adt, scale, p):
    say(f"[lora] M={M} in={n_in} out={n_out} r={r} act={act} adt={adt} scale={scale} p={p}")
    L = Layer(31, M, n_in, n_out, r, act=act, adt=adt)
    K = _mask(M, r, p, 7) if p > 0 else None
    opts = (scale, p, _dev(K) if K is not None else None)
    Y, XA = L.fwd(lora=opts)
    dX, dA, dB = L.bwd(XA=XA, lora=opts)
    W = L.w_hat()
    X, dY = L.X.values.astype(np.float64), L.dY.values.astype(np.float64)
    A, B = L.A.values, L.B.values
    XAr, _, y = oracle.forward_lora(X, W, A, B, scale, p, K)
    g = oracle.backward_lora(X, dY, W, A, B, scale, p, K)
    errs = {"y": rel_err(out_to_f64(Y, act), y), "XA": rel_err(XA.cpu().numpy(), XAr),
            "dX": rel_err(out_to_f64(dX, act), g["dX"]),
            "dA": rel_err(dA.cpu().numpy(), g["dA"]), "dB": rel_err(dB.cpu().numpy(), g["dB"])}
    say(f"    errors {errs}")
    for k, v in errs.items():
        assert v <= TOL, f"{k}: {v}"
    # XA recomputed in the backward gives the same bits
    dX2, dA2, dB2 = L.bwd(XA=None, lora=opts)
    assert np.array_equal(dA.cpu().numpy(), dA2.cpu().numpy())
    assert np.array_equal(dB.cpu().numpy(), dB2.cpu().numpy())
    assert np.array_equal(out_to_f64(dX, act), out_to_f64(dX2, act))


@pytest.mark.parametrize("M,n_in,n_out,r", [(1030, 320, 448, 16), (300, 640, 704, 16),
                                             (5, 576, 448, 16), (1100, 1088, 320, 24)])
def test_lora_identity_options_are_the_plain_call(M, n_in, n_out, r):
    """scale 1 and no mask multiply by exactly 1: every output bit is that of
    qlora_linear_fwd / qlora_linear_bwd."""
    L = Layer(32, M, n_in, n_out, r)
    Y0, XA0 = L.fwd()
    dX0, dA0, dB0 = L.bwd(XA=XA0)
    Y1, XA1 = L.fwd(lora=(1.0, 0.0, None))
    dX1, dA1, dB1 = L.bwd(XA=XA1, lora=(1.0, 0.0, None))
    for a, b in ((Y0, Y1), (XA0, XA1), (dX0, dX1), (dA0, dA1), (dB0, dB1)):
        assert np.array_equal(a.float().cpu().numpy(), b.float().cpu().numpy())


@pytest.mark.parametrize("M,n_in,n_out", [(1030, 320, 448), (300, 640, 704), (5, 576, 448)])
def test_lora_all_dropped_leaves_the_base(M, n_in, n_out):
    """Every element of X.A dropped: y is the rank-0 output bit for bit, dA and
    dB are zero, dX is the rank-0 dX."""
    L = Layer(33, M, n_in, n_out, 16)
    L0 = Layer(33, M, n_in, n_out, 0)
    opts = (2.0, 0.5, _dev(np.zeros((M, 16), np.uint8)))
    Y, XA = L.fwd(lora=opts)
    dX, dA, dB = L.bwd(XA=XA, lora=opts)
    Y0, _ = L0.fwd()
    dX0, _, _ = L0.bwd()
    assert np.array_equal(out_to_f64(Y, "bf16"), out_to_f64(Y0, "bf16"))
    assert np.array_equal(out_to_f64(dX, "bf16"), out_to_f64(dX0, "bf16"))
    assert not dA.cpu().numpy().any() and not dB.cpu().numpy().any()
