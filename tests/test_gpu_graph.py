"""The forward and backward captured in a HIP graph and replayed: every
replay, with the program's own eager work and synchronizations between
replays, gives the bits of the eager calls (the library enqueues only
kernels on the caller's stream, allocates nothing and keeps no state)."""

import numpy as np
import pytest

from quantized_rank_fine_amd import qlora as q

from gpu_harness import Layer, say, torch_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,n_in,n_out,r", [
    (1030, 320, 448, 16),    # whole-K rank passes, dB in the dX GEMM
    (300, 640, 704, 16),     # split-K rank passes
    (5, 576, 448, 16),       # few-token forward
])
def test_graph_replays_match_eager(M, n_in, n_out, r):
    torch, dev = torch_dev()
    say(f"[graph] M={M} in={n_in} out={n_out} r={r}")
    L = Layer(51, M, n_in, n_out, r)
    Y = torch.empty(M, n_out, dtype=torch.bfloat16, device=dev)
    XA = torch.empty(M, r, dtype=torch.float32, device=dev)
    dX = torch.empty(M, n_in, dtype=torch.bfloat16, device=dev)
    dA = torch.empty(n_in, r, dtype=torch.float32, device=dev)
    dB = torch.empty(r, n_out, dtype=torch.float32, device=dev)
    fwb = q.qlora_fwd_workspace_bytes(M, n_in, n_out, r, q.BF16)
    bwb = q.qlora_bwd_workspace_bytes(M, n_in, n_out, r, q.BF16)
    wsf = torch.empty(fwb, dtype=torch.uint8, device=dev)
    wsb = torch.empty(bwb, dtype=torch.uint8, device=dev)
    outs = (Y, XA, dX, dA, dB)

    def step():
        q.qlora_linear_fwd(L.wq, L.tX, M, q.BF16, L.tA, L.tB, r, q.BF16, Y, XA, wsf, fwb)
        q.qlora_linear_bwd(L.wq, L.tX, L.tdY, M, q.BF16, L.tA, L.tB, r, q.BF16, XA, dX, dA, dB,
                           wsb, bwb)

    step()
    torch.cuda.synchronize()
    ref = [t.float().cpu().numpy().copy() for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for t in outs:                      # eager work between replays
            t.fill_(float("nan"))
        wsf.zero_()
        wsb.fill_(255)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, t, want in zip(("Y", "XA", "dX", "dA", "dB"), outs, ref):
            assert np.array_equal(t.float().cpu().numpy(), want), (rep, name)
