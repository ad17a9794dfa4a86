"""GPU parity of qlora_adam_step against the float64 oracle (Adam / AdamW
step of an adapter matrix)."""

import numpy as np
import pytest

import oracle
from quantized_rank_fine_amd import qlora as q

from gpu_harness import bf16_to_f64, say, torch_dev

pytestmark = pytest.mark.gpu


def _close(got, ref, lr):
    # fp32 arithmetic: theta to a few fp32 ulps, plus the step's own rounding
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    return np.all(np.abs(got - ref) <= 2.0 ** -21 * np.abs(ref) + 1e-6 * lr)


@pytest.mark.parametrize("n,wd", [(16 * 4096, 0.0), (4096 * 16 + 3, 0.01), (5, 0.0)])
def test_adam_steps_match_oracle(n, wd):
    torch, dev = torch_dev()
    say(f"[adam] n={n} wd={wd}")
    g = np.random.default_rng(31)
    th = (g.standard_normal(n) * 0.05).astype(np.float32)
    tt = torch.from_numpy(th.copy()).to(dev)
    tm = torch.zeros(n, dtype=torch.float32, device=dev)
    tv = torch.zeros(n, dtype=torch.float32, device=dev)
    t16 = torch.empty(n, dtype=torch.bfloat16, device=dev)
    rth, rm, rv = th.astype(np.float64), np.zeros(n), np.zeros(n)
    lr = 1e-3
    # the library takes fp32 hyperparameters: the oracle gets the same values
    f32 = lambda x: float(np.float32(x))
    hp = dict(beta1=f32(0.9), beta2=f32(0.999), eps=f32(1e-8), weight_decay=f32(wd))
    for step in range(1, 4):
        grad = (g.standard_normal(n) * 10.0 ** -step).astype(np.float32)
        tg = torch.from_numpy(grad).to(dev)
        m_prev = rm.copy()
        q.qlora_adam_step(tt, tg, tm, tv, step, lr, theta_bf16=t16, **hp)
        torch.cuda.synchronize()
        # the oracle continues from the GPU's fp32 state, so each step is
        # checked on its own
        gth, gm, gv = tt.cpu().numpy(), tm.cpu().numpy(), tv.cpu().numpy()
        rth, rm, rv = oracle.adam_step(rth, grad, rm, rv, step, f32(lr), **hp)
        assert _close(gth, rth, lr), step
        # m = b1 m + (1 - b1) g can cancel: bound its error by the terms' size
        mtol = 2.0 ** -21 * (hp["beta1"] * np.abs(m_prev) + (1 - hp["beta1"]) * np.abs(grad))
        assert np.all(np.abs(gm - rm) <= mtol), step
        assert np.allclose(gv, rv, rtol=4e-6, atol=0), step
        b = np.asarray(bf16_to_f64(t16))
        exp = torch.from_numpy(gth).to(torch.bfloat16).float().numpy()
        assert np.array_equal(b, exp.astype(np.float64))
        rth, rm, rv = gth.astype(np.float64), gm.astype(np.float64), gv.astype(np.float64)


def test_adam_zero_gradient_and_empty():
    torch, dev = torch_dev()
    th = torch.linspace(-1, 1, 64, device=dev)
    before = th.clone()
    z = torch.zeros(64, device=dev)
    m, v = torch.zeros(64, device=dev), torch.zeros(64, device=dev)
    q.qlora_adam_step(th, z, m, v, 1, 1e-2)
    torch.cuda.synchronize()
    assert torch.equal(th, before)
    q.qlora_adam_step(th, z, m, v, 1, 1e-2, weight_decay=0.5)
    torch.cuda.synchronize()
    exp = before.cpu().numpy().astype(np.float64) * (1 - 1e-2 * 0.5)
    assert np.allclose(th.cpu().numpy(), exp, rtol=2e-7, atol=1e-9)
    q.qlora_adam_step(th, z, m, v, 1, 1e-2, n=0)        # n = 0: nothing happens


# ------------------------------------------------ Adam fused into the backward

from gpu_harness import Layer, out_to_f64   # noqa: E402


def _state(torch, dev, values, seed):
    """theta (the adapter's values in fp32), m, v (nonzero: a later step)."""
    g = np.random.default_rng(seed)
    th = torch.from_numpy(np.asarray(values, np.float32).reshape(-1).copy()).to(dev)
    m = torch.from_numpy((g.standard_normal(th.numel()) * 1e-3).astype(np.float32)).to(dev)
    v = torch.from_numpy((g.random(th.numel()) * 1e-6).astype(np.float32)).to(dev)
    return [th, m, v, torch.empty(th.numel(), dtype=torch.bfloat16, device=dev)]


@pytest.mark.parametrize("M,n_in,n_out,r,act,adt", [
    (1030, 320, 448, 16, "bf16", "bf16"),   # dB in the dX GEMM: both updates in the last launch
    (1100, 1088, 320, 24, "bf16", "f32"),   # G whole, dB in the dY pass
    (300, 640, 704, 16, "bf16", "bf16"),    # split-K: B with G's reduction, A after dX
    (1100, 384, 320, 16, "f32", "f32"),     # fp32 activations and adapters
])
def test_bwd_adam_equals_bwd_then_adam_step(M, n_in, n_out, r, act, adt):
    """Two steps of the fused call give the bits of the backward followed by
    qlora_adam_step on A and B (theta, m, v, the bf16 copy, dX, and dA, dB
    when asked for)."""
    torch, dev = torch_dev()
    say(f"[bwd+adam] M={M} in={n_in} out={n_out} r={r} act={act} adt={adt}")
    L = Layer(41, M, n_in, n_out, r, act=act, adt=adt)
    _, XA = L.fwd()
    sep = [_state(torch, dev, L.A.values, 1), _state(torch, dev, L.B.values, 2)]
    fus = [[t.clone() for t in s] for s in sep]
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    wsb = q.qlora_bwd_workspace_bytes(M, n_in, n_out, r, L.qact)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    for step in (3, 4):
        dX0, dA0, dB0 = L.bwd(XA=XA)
        q.qlora_adam_step(sep[0][0], dA0.reshape(-1), sep[0][1], sep[0][2], step,
                          theta_bf16=sep[0][3], **hp)
        q.qlora_adam_step(sep[1][0], dB0.reshape(-1), sep[1][1], sep[1][2], step,
                          theta_bf16=sep[1][3], **hp)
        dX = torch.empty_like(dX0)
        dA, dB = torch.empty_like(dA0), torch.empty_like(dB0)
        q.qlora_linear_bwd_adam(L.wq, L.tX, L.tdY, M, L.qact, L.tA, L.tB, r, L.qadt, XA, dX,
                                fus[0], fus[1], step, hp["lr"], ws, wsb,
                                beta1=hp["beta1"], beta2=hp["beta2"], eps=hp["eps"],
                                weight_decay=hp["weight_decay"], dA=dA, dB=dB)
        torch.cuda.synchronize()
        assert np.array_equal(out_to_f64(dX, act), out_to_f64(dX0, act))
        assert np.array_equal(dA.cpu().numpy(), dA0.cpu().numpy())
        assert np.array_equal(dB.cpu().numpy(), dB0.cpu().numpy())
        for a, b in zip(sep, fus):
            for x, y in zip(a, b):
                assert np.array_equal(x.float().cpu().numpy(), y.float().cpu().numpy()), step


@pytest.mark.parametrize("M,n_in,n_out", [(1030, 320, 448), (300, 640, 704)])
def test_bwd_adam_updates_the_adapters_it_reads(M, n_in, n_out):
    """bf16 adapters whose bf16 copies are the very A and B the call reads:
    the update comes after every read, so the result is that of separate
    buffers."""
    torch, dev = torch_dev()
    L = Layer(42, M, n_in, n_out, 16)
    _, XA = L.fwd()
    hp = dict(beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0)
    wsb = q.qlora_bwd_workspace_bytes(M, n_in, n_out, 16, L.qact)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    ref = [_state(torch, dev, L.A.values, 5), _state(torch, dev, L.B.values, 6)]
    ali = [[t.clone() for t in s] for s in ref]
    A2, B2 = L.tA.clone(), L.tB.clone()
    ali[0][3], ali[1][3] = A2.view(-1), B2.view(-1)
    dX1 = torch.empty(M, n_in, dtype=torch.bfloat16, device=dev)
    dX2 = torch.empty_like(dX1)
    q.qlora_linear_bwd_adam(L.wq, L.tX, L.tdY, M, L.qact, L.tA, L.tB, 16, L.qadt, XA, dX1,
                            ref[0], ref[1], 1, 1e-3, ws, wsb, **hp)
    q.qlora_linear_bwd_adam(L.wq, L.tX, L.tdY, M, L.qact, A2, B2, 16, L.qadt, XA, dX2,
                            ali[0], ali[1], 1, 1e-3, ws, wsb, **hp)
    torch.cuda.synchronize()
    assert np.array_equal(out_to_f64(dX1, "bf16"), out_to_f64(dX2, "bf16"))
    for a, b in zip(ref, ali):
        for x, y in zip(a, b):
            assert np.array_equal(x.float().cpu().numpy(), y.float().cpu().numpy())
    assert not np.array_equal(A2.float().cpu().numpy(), L.tA.float().cpu().numpy())
