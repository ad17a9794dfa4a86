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
