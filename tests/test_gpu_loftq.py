"""qlora_loftq_init (adapters from a rank-r SVD of the quantization
residual) against the float64 oracle's exact truncated SVD."""

import numpy as np
import pytest

import oracle
from quantized_rank_fine_amd import qlora as q
from quantized_rank_fine_amd import synth

from gpu_harness import bf16_to_f64, levels_of, quantize_gpu, say, torch_dev

pytestmark = pytest.mark.gpu


def _w_hat(w0, codebook=q.CB_NF4, block=64):
    """deq(Q(W0)) in float64 from the oracle's own quantization of W0 (block
    16: the lab's 16-entry format)."""
    if block == 16:
        og = oracle.quantize_groups(w0, levels_of(codebook))
        return oracle.dequantize_groups(og["packed"], og["scales"], *w0.shape, levels_of(codebook))
    oq = oracle.quantize(w0, levels_of(codebook))
    return oracle.dequantize(oq["packed"], oq["q8"], oq["s2"], *w0.shape, levels_of(codebook))


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


@pytest.mark.parametrize("n_in,n_out,k", [(256, 384, 12), (192, 320, 12), (256, 384, 13),
                                          (256, 384, 4)])
def test_low_rank_residual_is_recovered(n_in, n_out, k):
    """W0 = fp32(deq(Wq)) + P with P of rank 4: the residual is P (up to
    the fp32 rounding of the dequantized weight) and A B recovers it
    (192 x 320: half-filled last workgroups of both residual products; k =
    13: an odd number of columns for the pairwise rotations of the small
    SVD; the columns past rank 4 are dependent and leave the Cholesky QR as
    zero columns; k = 4 = r: no oversampling)."""
    torch, dev = torch_dev()
    say(f"[loftq] rank-4 residual {n_in}x{n_out} k={k}")
    w0 = synth.weights(n_in, n_out, workload=7)
    wq = quantize_gpu(w0)
    W_hat = _w_hat(w0)
    g = np.random.default_rng(51)
    P = (g.standard_normal((n_in, 4)) @ g.standard_normal((4, n_out)) * 0.01).astype(np.float32)
    W0 = (W_hat.astype(np.float32) + P).astype(np.float32)
    R = W0.astype(np.float64) - W_hat
    A, B = _init(torch.from_numpy(W0).to(dev), wq, k, 4, 2)
    AB = A.cpu().numpy().astype(np.float64) @ B.cpu().numpy().astype(np.float64)
    assert np.abs(AB - R).max() <= 1e-4 * np.abs(R).max()


@pytest.mark.parametrize("codebook,k,r,iters", [(q.CB_NF4, 24, 16, 3), (q.CB_UNIFORM4, 24, 16, 3),
                                                (q.CB_NF4, 96, 64, 4), (q.CB_NF4, 128, 64, 2)])
def test_quantization_residual_near_optimal(codebook, k, r, iters):
    """On a real quantization residual the rank-r start removes at least 90 %
    of what the exact truncated SVD removes, and its factors are balanced
    (k = 96 takes the wide-panel kernels; k = 128 is the largest panel)."""
    torch, dev = torch_dev()
    w0 = synth.weights(512, 768, workload=7)
    wq = quantize_gpu(w0, codebook)
    W_hat = _w_hat(w0, codebook)
    R = oracle.residual(w0, W_hat)
    say(f"[loftq] 512x768 codebook={codebook} k={k} r={r}")
    A, B = _init(torch.from_numpy(w0).to(dev), wq, k, r, iters)
    An, Bn = A.cpu().numpy().astype(np.float64), B.cpu().numpy().astype(np.float64)
    Ao, Bo = oracle.loftq_init(w0, W_hat, r)
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


@pytest.mark.parametrize("n_in,n_out", [(256, 384), (192, 320)])
def test_group16_low_rank_residual_is_recovered(n_in, n_out):
    """The lab's 16-entry format (INT4 levels k/7, one fp32 absmax per 16
    entries): W0 = fp32(deq(Wq)) + P with P of rank 4 is recovered."""
    torch, dev = torch_dev()
    say(f"[loftq] 16-entry format, rank-4 residual {n_in}x{n_out}")
    w0 = synth.weights(n_in, n_out, workload=7)
    wq = quantize_gpu(w0, q.CB_INT4, block=16)
    W_hat = _w_hat(w0, q.CB_INT4, block=16)
    g = np.random.default_rng(52)
    P = (g.standard_normal((n_in, 4)) @ g.standard_normal((4, n_out)) * 0.01).astype(np.float32)
    W0 = (W_hat.astype(np.float32) + P).astype(np.float32)
    R = W0.astype(np.float64) - W_hat
    A, B = _init(torch.from_numpy(W0).to(dev), wq, 12, 4, 2)
    AB = A.cpu().numpy().astype(np.float64) @ B.cpu().numpy().astype(np.float64)
    assert np.abs(AB - R).max() <= 1e-4 * np.abs(R).max()


def test_group16_quantization_residual_near_optimal():
    """On the 16-entry format's real quantization residual the rank-16 start
    removes at least 90 % of what the exact truncated SVD removes."""
    torch, dev = torch_dev()
    w0 = synth.weights(512, 768, workload=7)
    wq = quantize_gpu(w0, q.CB_INT4, block=16)
    W_hat = _w_hat(w0, q.CB_INT4, block=16)
    R = oracle.residual(w0, W_hat)
    A, B = _init(torch.from_numpy(w0).to(dev), wq, 24, 16, 3)
    An, Bn = A.cpu().numpy().astype(np.float64), B.cpu().numpy().astype(np.float64)
    Ao, Bo = oracle.loftq_init(w0, W_hat, 16)
    full = np.sum(R ** 2)
    e_opt = np.sum((R - Ao @ Bo) ** 2)
    e_gpu = np.sum((R - An @ Bn) ** 2)
    assert e_gpu <= e_opt + 0.1 * (full - e_opt), (full, e_opt, e_gpu)


def test_graph_replays_match_eager():
    """The whole start (products, Cholesky QR steps, the small SVD) is
    enqueued on the stream without waiting for the device, so it can be
    captured in a graph: every replay, with eager work between replays, gives
    the bits of the eager call, and two eager calls agree bit for bit."""
    torch, dev = torch_dev()
    say("[loftq] graph capture 256x384 k=24 r=16")
    w0 = synth.weights(256, 384, workload=7)
    wq = quantize_gpu(w0)
    W0 = torch.from_numpy(w0).to(dev)
    g = torch.Generator(device="cpu").manual_seed(3)
    k, r = 24, 16
    omega = torch.randn(wq.n_out, k, generator=g).to(dev)
    A = torch.empty(wq.n_in, r, dtype=torch.float32, device=dev)
    B = torch.empty(r, wq.n_out, dtype=torch.float32, device=dev)
    wsb = q.qlora_loftq_workspace_bytes(wq.n_in, wq.n_out, k)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)

    def call():
        q.qlora_loftq_init(W0, wq, omega, k, r, 2, A, B, q.F32, ws, wsb)

    call()
    torch.cuda.synchronize()
    ref = (A.cpu().numpy().copy(), B.cpu().numpy().copy())
    call()
    torch.cuda.synchronize()
    assert np.array_equal(A.cpu().numpy(), ref[0]) and np.array_equal(B.cpu().numpy(), ref[1])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for rep in range(3):
        A.fill_(float("nan"))                # eager work between replays
        B.fill_(float("nan"))
        ws.fill_(255)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(A.cpu().numpy(), ref[0]), rep
        assert np.array_equal(B.cpu().numpy(), ref[1]), rep


def test_square_panel_is_the_exact_svd():
    """k = in = out = 64: the probe panel spans the whole space, so the start
    is the exact truncated SVD of the residual (up to fp32 rounding): the
    residual energy left matches the oracle's within 1e-4 of the total."""
    torch, dev = torch_dev()
    say("[loftq] 64x64 k=64 r=8")
    w0 = synth.weights(64, 64, workload=7)
    wq = quantize_gpu(w0)
    W_hat = _w_hat(w0)
    R = oracle.residual(w0, W_hat)
    A, B = _init(torch.from_numpy(w0).to(dev), wq, 64, 8, 1)
    An, Bn = A.cpu().numpy().astype(np.float64), B.cpu().numpy().astype(np.float64)
    Ao, Bo = oracle.loftq_init(w0, W_hat, 8)
    full = np.sum(R ** 2)
    e_opt = np.sum((R - Ao @ Bo) ** 2)
    e_gpu = np.sum((R - An @ Bn) ** 2)
    assert abs(e_gpu - e_opt) <= 1e-4 * full, (full, e_opt, e_gpu)
