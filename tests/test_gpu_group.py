"""qlora_linear_fwd_group: up to four independent few-token linears in one
pair of launches give, for each linear, the bits of its own
qlora_linear_fwd call (same kernels, one workgroup per linear's tile)."""

import numpy as np
import pytest

from quantized_rank_fine_amd import qlora as q

from quantized_rank_fine_amd import workloads

from gpu_harness import TOL, Layer, out_to_f64, rel_err, say, torch_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M", [1, 5, 16])
@pytest.mark.parametrize("shapes,shared_x", [
    ([(576, 448), (576, 448), (576, 448)], True),       # q, k, v: one input, three weights
    ([(640, 704), (640, 704)], True),                   # gate, up
    ([(576, 448), (640, 704), (320, 256), (1088, 192)], False),   # four unrelated shapes
])
def test_group_equals_single_calls(M, shapes, shared_x):
    torch, dev = torch_dev()
    say(f"[group] M={M} shapes={shapes} shared_x={shared_x}")
    r = 16
    layers = [Layer(61 + l, M, i, o, r) for l, (i, o) in enumerate(shapes)]
    if shared_x:
        for L in layers[1:]:
            L.tX = layers[0].tX
    ref = [L.fwd() for L in layers]
    Ys = [torch.full((M, o), float("nan"), dtype=torch.bfloat16, device=dev) for (_, o) in shapes]
    XAs = [torch.full((M, r), float("nan"), dtype=torch.float32, device=dev) for _ in shapes]
    wsb = q.qlora_fwd_group_workspace_bytes(M, [i for i, _ in shapes], [o for _, o in shapes], r)
    assert wsb > 0
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    q.qlora_linear_fwd_group([L.wq for L in layers], [L.tX for L in layers], M, q.BF16,
                             [L.tA for L in layers], [L.tB for L in layers], r, q.BF16,
                             Ys, XAs, ws, wsb)
    torch.cuda.synchronize()
    for l, ((Y0, XA0), Y, XA) in enumerate(zip(ref, Ys, XAs)):
        assert np.array_equal(Y.float().cpu().numpy(), Y0.float().cpu().numpy()), l
        assert np.array_equal(XA.cpu().numpy(), XA0.cpu().numpy()), l


@pytest.mark.parametrize("M", [1, 4, 16])
@pytest.mark.parametrize("group", [("q", "k", "v"), ("gate", "up")])
def test_group_7b_shapes_against_oracle(M, group):
    """The grouped calls the decode measurement makes (q/k/v share X, gate/up
    share X) at the 7B shapes, r = 16, bf16: every output against the
    float64 oracle on the oracle's own quantization of each weight."""
    torch, dev = torch_dev()
    names = [l[0] for l in workloads.LLAMA7B_LINEARS]
    shapes = [workloads.LLAMA7B_LINEARS[names.index(nm)][1:] for nm in group]
    say(f"[group] 7b {group} M={M}")
    r = 16
    layers = [Layer(2, M, i, o, r, linear=names.index(nm)) for nm, (i, o) in zip(group, shapes)]
    for L in layers[1:]:
        L.tX, L.X = layers[0].tX, layers[0].X
    Ys = [torch.empty((M, o), dtype=torch.bfloat16, device=dev) for (_, o) in shapes]
    XAs = [torch.empty((M, r), dtype=torch.float32, device=dev) for _ in shapes]
    wsb = q.qlora_fwd_group_workspace_bytes(M, [i for i, _ in shapes], [o for _, o in shapes], r)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    q.qlora_linear_fwd_group([L.wq for L in layers], [L.tX for L in layers], M, q.BF16,
                             [L.tA for L in layers], [L.tB for L in layers], r, q.BF16,
                             Ys, XAs, ws, wsb)
    torch.cuda.synchronize()
    for nm, L, Y, XA in zip(group, layers, Ys, XAs):
        L.codes_match_oracle()
        ref = L.ref()
        ey = rel_err(out_to_f64(Y, "bf16"), ref["y"])
        exa = rel_err(XA.cpu().numpy(), ref["XA"])
        say(f"    {nm}: y {ey:.3g} XA {exa:.3g}")
        assert ey <= TOL and exa <= TOL, nm
