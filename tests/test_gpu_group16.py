"""The lab's 16-entry format (symmetric integer levels, one fp32 absmax per
16 consecutive entries of the flattened (in, out) matrix, no double
quantization; "QLoRA (low-rank adapters on a quantized model)", "The code,
line by line") on the GPU: quantize bit-exact against the oracle's group
quantizer (codes and scales), and the forward and backward through every
path (few tokens, fused GEMMs with whole-K and split-K rank passes, dB in
the dX GEMM, grouped few-token calls) and the merge, against the float64
oracle on the oracle's own quantization of W0."""

import numpy as np
import pytest

import oracle
from quantized_rank_fine_amd import qlora as q
from quantized_rank_fine_amd import synth

from gpu_harness import (TOL, Layer, bf16_to_f64, levels_of, out_to_f64, quantize_gpu, rel_err,
                         say, torch_dev)

pytestmark = pytest.mark.gpu

GRIDS = [q.CB_INT4, q.CB_INT3, q.CB_TERNARY]


def _check_quantize(w0, codebook, tag):
    say(f"[g16 quantize] {tag} shape={w0.shape} codebook={codebook}")
    wq = quantize_gpu(w0, codebook, 16)
    ref = oracle.quantize_groups(w0, levels_of(codebook))
    codes = wq.codes.cpu().numpy()
    bad = np.flatnonzero(codes != ref["packed"])
    assert bad.size == 0, f"{tag}: {bad.size} packed bytes differ, first at {bad[:5]}"
    assert np.array_equal(wq.gscale.cpu().numpy().view(np.uint32), ref["scales"].view(np.uint32))


@pytest.mark.parametrize("codebook", GRIDS + [q.CB_NF4])
@pytest.mark.parametrize("shape", [(4096, 4096), (320, 640), (64, 192)])
def test_group16_quantize(codebook, shape):
    _check_quantize(synth.weights(*shape, workload=8), codebook, f"{shape}")


def test_group16_quantize_edge_values():
    g = np.random.default_rng(31)
    w = (g.standard_normal((128, 256)) * 0.02).astype(np.float32)
    w[0, :16] = 0.0                                   # a zero group
    w[1, 16:48] = -0.0                                # two negative-zero groups
    w[2, :16] = np.float32(1e-40)                     # denormal group
    w[3, 32:48] = np.float32(1e30) * g.standard_normal(16).astype(np.float32)
    for h, cb in ((7, q.CB_INT4), (1, q.CB_TERNARY)):
        k = g.integers(-h, h + 1, (8, 256)).astype(np.float32)
        k[:, ::16] = h                                # absmax h per group: on the grid
        w[8:16] = k / np.float32(h) * np.float32(0.03)
        _check_quantize(w, cb, f"edge values h={h}")


@pytest.mark.parametrize("codebook", GRIDS)
@pytest.mark.parametrize("M,n_in,n_out,r,act,adt", [
    (300, 640, 704, 16, "bf16", "bf16"),    # fused GEMMs, split-K rank passes, ragged tiles
    (1030, 320, 448, 16, "bf16", "bf16"),   # whole-K rank passes, dB in the dX GEMM
    (130, 384, 256, 40, "f32", "f32"),      # fp32 operands, r not a multiple of 16
    (5, 576, 448, 16, "bf16", "f32"),       # few-token forward
    (16, 1088, 192, 64, "f32", "bf16"),     # few tokens, several K chunks, largest r
])
def test_group16_linear(codebook, M, n_in, n_out, r, act, adt):
    L = Layer(19, M, n_in, n_out, r, act=act, adt=adt, codebook=codebook, block=16)
    say(f"[g16 linear] cb={codebook} M={M} in={n_in} out={n_out} r={r} act={act} adt={adt}")
    L.codes_match_oracle()
    Y, XA = L.fwd()
    dX, dA, dB = L.bwd(XA=XA)
    ref = L.ref()
    errs = {"y": rel_err(out_to_f64(Y, act), ref["y"]), "dX": rel_err(out_to_f64(dX, act), ref["dX"]),
            "XA": rel_err(XA.cpu().numpy(), ref["XA"]), "dA": rel_err(dA.cpu().numpy(), ref["dA"]),
            "dB": rel_err(dB.cpu().numpy(), ref["dB"])}
    say(f"    errors {errs}")
    for k, v in errs.items():
        assert v <= TOL, (k, v)


def test_group16_identity_probe():
    """X = I, B = 0: y = bf16(L[code] * c_g), within one bf16 ulp of the
    oracle's dequantized weight (the in-register expansion with 16-entry
    scales)."""
    import torch
    n = 256
    L = Layer(20, n, n, 512, 16, b_zero=True, codebook=q.CB_INT4, block=16)
    L.tX = torch.eye(n, dtype=torch.bfloat16, device="cuda:0")
    Y, _ = L.fwd()
    W = L.w_hat()
    ulp = np.spacing(np.abs(W).astype(np.float32)).astype(np.float64) * 2.0 ** 16
    assert np.all(np.abs(out_to_f64(Y, "bf16") - W) <= ulp)


def test_group16_4096_sampled_rows():
    L = Layer(21, 2048, 4096, 4096, 16, codebook=q.CB_INT4, block=16)
    L.codes_match_oracle()
    rows = np.sort(np.random.default_rng(2).choice(2048, 96, replace=False))
    Y, XA = L.fwd()
    dX, dA, dB = L.bwd(XA=XA)
    ref = L.ref(rows)
    assert rel_err(out_to_f64(Y, "bf16")[rows], ref["y"]) <= TOL
    assert rel_err(out_to_f64(dX, "bf16")[rows], ref["dX"]) <= TOL
    assert rel_err(dA.cpu().numpy(), ref["dA"]) <= TOL
    assert rel_err(dB.cpu().numpy(), ref["dB"]) <= TOL


def test_group16_grouped_few_tokens_equal_single_calls():
    torch, dev = torch_dev()
    M, r = 3, 16
    layers = [Layer(22 + l, M, 576, 448, r, codebook=q.CB_INT3, block=16) for l in range(3)]
    for L in layers[1:]:
        L.tX = layers[0].tX
    ref = [L.fwd() for L in layers]
    Ys = [torch.empty(M, 448, dtype=torch.bfloat16, device=dev) for _ in layers]
    XAs = [torch.empty(M, r, dtype=torch.float32, device=dev) for _ in layers]
    wsb = q.qlora_fwd_group_workspace_bytes(M, [576] * 3, [448] * 3, r)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    q.qlora_linear_fwd_group([L.wq for L in layers], [L.tX for L in layers], M, q.BF16,
                             [L.tA for L in layers], [L.tB for L in layers], r, q.BF16, Ys, XAs,
                             ws, wsb)
    torch.cuda.synchronize()
    for (Y0, XA0), Y, XA in zip(ref, Ys, XAs):
        assert np.array_equal(Y.float().cpu().numpy(), Y0.float().cpu().numpy())
        assert np.array_equal(XA.cpu().numpy(), XA0.cpu().numpy())


@pytest.mark.parametrize("n_in,n_out,r,adt,wdt", [
    (256, 320, 16, "bf16", "f32"),       # matrix cores
    (384, 576, 12, "f32", "f32"),        # FMA kernel (r % 8 != 0)
    (256, 256, 0, "bf16", "f32"),        # the dequantized weight
])
def test_group16_merge(n_in, n_out, r, adt, wdt):
    torch, dev = torch_dev()
    L = Layer(23, 64, n_in, n_out, r, adt=adt, codebook=q.CB_INT4, block=16)
    W = torch.empty(n_in, n_out, dtype=torch.float32, device=dev)
    q.qlora_merge(L.wq, L.tA, L.tB, r, L.qadt, W, q.F32)
    torch.cuda.synchronize()
    A = None if L.A is None else L.A.values
    B = None if L.B is None else L.B.values
    assert rel_err(W.cpu().numpy(), oracle.merge(L.w_hat(), A, B)) <= 1e-6
