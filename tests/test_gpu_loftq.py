"""qlora_loftq_init (adapters from a rank-r SVD of the quantization
residual) against the float64 oracle's exact truncated SVD."""

import numpy as np
import pytest

import oracle
from quantized_rank_fine_amd import qlora as q
from quantized_rank_fine_amd import synth

from gpu_harness import bf16_to_f64, quantize_gpu, say, torch_dev

pytestmark = pytest.mark.gpu


def _w_hat32(wq):
    """deq(Wq) in fp32 as the library forms it (merge with rank 0)."""
    torch, dev = torch_dev()
    W = torch.empty(wq.n_in, wq.n_out, dtype=torch.float32, device=dev)
    q.qlora_merge(wq, None, None, 0, q.F32, W, q.F32)
    torch.cuda.synchronize()
    return W


def _init(W0, wq, k, r, iters, adt="f32", seed=0):
    torch, dev = torch_dev()
    g = torch.Generator(device="cpu").manual_seed(seed)
    omega = torch.randn(wq.n_out, k, generator=g).to(dev)
    dt = torch.bfloat16 if adt == "bf16" else torch.float32
    A = torch.empty(wq.n_in, r, dtype=dt, device=dev)
    B = torch.empty(r, wq.n_out, dtype=dt, device=dev)
    wsb = q.qlora_loftq_workspace_bytes(wq.n_in, wq.n_out, k)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    q.qlora_loftq_init(W0, wq, omega, k, r, iters, A, B, q.BF16 if adt == "bf16" else q.F32, ws, wsb)
    torch.cuda.synchronize()
    return A, B


def test_low_rank_residual_is_recovered():
    """W0 = deq(Wq) + P with P of rank 4: the residual is P (to fp32
    rounding) and A B recovers it."""
    torch, dev = torch_dev()
    wq = quantize_gpu(synth.weights(256, 384, workload=7))
    W_hat = _w_hat32(wq)
    g = np.random.default_rng(51)
    P = (g.standard_normal((256, 4)) @ g.standard_normal((4, 384)) * 0.01).astype(np.float32)
    W0 = W_hat + torch.from_numpy(P).to(dev)
    R = (W0 - W_hat).cpu().numpy().astype(np.float64)      # the exact fp32 residual
    A, B = _init(W0, wq, 12, 4, 2)
    AB = A.cpu().numpy().astype(np.float64) @ B.cpu().numpy().astype(np.float64)
    assert np.abs(AB - R).max() <= 1e-4 * np.abs(R).max()


@pytest.mark.parametrize("codebook", [q.CB_NF4, q.CB_UNIFORM4])
def test_quantization_residual_near_optimal(codebook):
    """On a real quantization residual the rank-16 start removes at least 90 %
    of what the exact truncated SVD removes, and its factors are balanced."""
    torch, dev = torch_dev()
    w0 = synth.weights(512, 768, workload=7)
    wq = quantize_gpu(w0, codebook)
    W_hat = _w_hat32(wq).cpu().numpy().astype(np.float64)
    R = oracle.residual(w0, W_hat)
    say(f"[loftq] 512x768 codebook={codebook}")
    A, B = _init(torch.from_numpy(w0).to(dev), wq, 24, 16, 3)
    An, Bn = A.cpu().numpy().astype(np.float64), B.cpu().numpy().astype(np.float64)
    Ao, Bo = oracle.loftq_init(w0, W_hat, 16)
    full = np.sum(R ** 2)
    e_opt = np.sum((R - Ao @ Bo) ** 2)
    e_gpu = np.sum((R - An @ Bn) ** 2)
    assert e_gpu <= e_opt + 0.1 * (full - e_opt), (full, e_opt, e_gpu)
    ata, bbt = An.T @ An, Bn @ Bn.T
    off = ata - np.diag(np.diag(ata))
    assert np.abs(off).max() <= 1e-3 * np.abs(np.diag(ata)).max()
    assert np.allclose(np.diag(ata), np.diag(bbt), rtol=1e-3)


def test_bf16_output_is_the_rounded_fp32_output():
    torch, dev = torch_dev()
    w0 = synth.weights(256, 256, workload=7)
    wq = quantize_gpu(w0)
    W0 = torch.from_numpy(w0).to(dev)
    A32, B32 = _init(W0, wq, 16, 8, 2)
    A16, B16 = _init(W0, wq, 16, 8, 2, adt="bf16")
    assert torch.equal(A32.to(torch.bfloat16), A16) and torch.equal(B32.to(torch.bfloat16), B16)
