"""Host-side checks of libqlora (no GPU): the library loads and exports every
function its header declares, its own constant tables agree with the oracle,
and argument validation returns the documented status before anything is
enqueued."""

import ctypes

import numpy as np
import pytest

import oracle
from oracle import nf4 as onf4
from quantized_rank_fine_amd import qlora as q
from quantized_rank_fine_amd import workloads


@pytest.fixture(scope="module")
def L():
    return q.lib()


def test_exports_every_declared_symbol(L):
    names = q.header_functions()
    assert {"qlora_quantize", "qlora_linear_fwd", "qlora_linear_bwd"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_level_table_matches_oracle(L):
    lv = np.array(q.qlora_levels(), dtype=np.float32)
    assert np.array_equal(lv.view(np.uint32), oracle.nf4_levels().view(np.uint32))


CODEBOOKS = [(q.CB_NF4, oracle.nf4_levels), (q.CB_UNIFORM4, oracle.uniform4_levels),
             (q.CB_INT4, lambda: oracle.int_levels(7)), (q.CB_INT3, lambda: oracle.int_levels(3)),
             (q.CB_TERNARY, lambda: oracle.int_levels(1))]


def test_codebook_tables(L):
    """Each codebook's level table equals the oracle's bit for bit; the NF4
    entry points agree with codebook 0; an unknown codebook is rejected."""
    for cb, levels in CODEBOOKS:
        lv = np.array(q.qlora_codebook_levels(cb), np.float32)
        assert np.array_equal(lv.view(np.uint32), levels().view(np.uint32))
        assert np.array_equal(lv, -lv[::-1])              # sign-symmetric
    assert q.qlora_codebook_levels(q.CB_NF4) == q.qlora_levels()
    assert q.qlora_codebook_thresholds(q.CB_NF4) == q.qlora_thresholds()
    buf = (ctypes.c_float * 16)()
    assert L.qlora_codebook_levels(5, buf) == -1
    assert L.qlora_codebook_thresholds(-1, buf) == -1


def _x_sweep(T=None, levels=None):
    """fp32 values in [-1, 1]: a strided sweep of bit patterns, the
    neighbourhood of every threshold and level, and the special values."""
    pos = np.arange(0, 0x3F800001, 4099, dtype=np.uint32).view(np.float32)
    xs = [pos, -pos]
    T = np.array(q.qlora_thresholds() if T is None else T, np.float32)
    L = oracle.nf4_levels() if levels is None else levels
    for v in np.concatenate([T, L]):
        b = int(np.array([v], np.float32).view(np.int32)[0])
        nb = np.arange(b - 300, b + 301, dtype=np.int64)
        if v >= 0:
            nb = nb[(nb >= 0) & (nb <= 0x3F800000)]
        else:
            nb = nb[(nb >= np.int64(np.int32(-0x7FFFFFFF) - 1)) & (nb < 0)]
        xs.append(nb.astype(np.int32).view(np.float32))
    xs.append(np.array([0.0, -0.0, 1.0, -1.0, 1e-30, -1e-30, 1.4e-45], np.float32))
    x = np.concatenate(xs).astype(np.float32)
    return x[(x >= -1) & (x <= 1)]


@pytest.mark.parametrize("cb,levels", CODEBOOKS)
def test_thresholds_reproduce_oracle_argmin(L, cb, levels):
    """code = #{j : x >= T_j} equals the oracle's fp32 argmin for every x."""
    T = np.array(q.qlora_codebook_thresholds(cb), np.float32)
    x = _x_sweep(T, levels())
    pad = (-x.size) % 63
    x = np.concatenate([x, np.zeros(pad, np.float32)])
    blocks = x.reshape(-1, 63)
    w = np.concatenate([np.ones((blocks.shape[0], 1), np.float32), blocks], axis=1).reshape(-1)
    c = onf4.block_absmax(w)
    assert np.all(c == 1.0)
    codes = oracle.encode(w, c, levels()).reshape(-1, 64)[:, 1:].reshape(-1)
    mine = np.searchsorted(T, x, side="right")
    assert np.array_equal(codes, mine)


def test_workspace_sizes(L):
    for (M, i, o, r) in [(2048, 4096, 4096, 16), (1, 4096, 11008, 16), (8192, 22016, 8192, 64),
                         (64, 256, 256, 8)]:
        for act in (q.BF16, q.F32):
            f = q.qlora_fwd_workspace_bytes(M, i, o, r, act)
            b = q.qlora_bwd_workspace_bytes(M, i, o, r, act)
            if M <= 16 and r <= 64:
                # few tokens: split-K partials of y and of XA (at least one chunk)
                assert f >= M * o * 4 + M * r * 4
            else:
                # block scales (fp32 per 64 weights) and XA in bf16; below
                # 1024 tokens or above rank 32, split-K partials of XA too
                assert f >= i * o // 16 + M * r * 2
                if M < 1024 or r > 32:
                    assert f >= i * o // 16 + M * r * 4 + M * r * 2
                if act == q.F32:
                    assert f >= M * i * 2
            assert b >= M * r * 4 + i * o // 16
            assert f % 256 == 0 and b % 256 == 0
            if act == q.F32:
                assert b >= M * o * 2
    assert q.qlora_fwd_workspace_bytes(2048, 4096, 4096, 0, q.BF16) == 4096 * 64 * 4
    assert q.qlora_fwd_workspace_bytes(0, 4096, 4096, 16, q.BF16) == 0
    assert q.qlora_bwd_workspace_bytes(64, 100, 256, 8, q.BF16) == 0     # invalid shape
    assert q.qlora_bwd_workspace_bytes(64, 256, 256, 8, 5) == 0          # invalid dtype


def test_addressable_shape_limits(L):
    """Shapes past the kernels' 32-bit addressing are rejected up front: in
    and out at most 2^19, in*out below 2^32 weights, at most 2^24 tokens;
    the largest accepted ones get a workspace size."""
    ok = lambda M, i, o: (q.qlora_fwd_workspace_bytes(M, i, o, 16, q.BF16) > 0 and
                          q.qlora_bwd_workspace_bytes(M, i, o, 16, q.BF16) > 0)
    assert ok(4096, 1 << 19, 4096)
    assert ok(4096, 4096, 1 << 19)
    assert ok(2048, 1 << 19, 8128)             # in*out = 2^32 - 2^25
    assert not ok(4096, (1 << 19) + 64, 64)
    assert not ok(4096, 64, (1 << 19) + 64)
    assert not ok(4096, 1 << 19, 8192)         # in*out = 2^32
    assert not ok(4096, 131072, 131072)
    assert ok(1 << 24, 4096, 4096)
    assert not ok((1 << 24) + 1, 4096, 4096)
    big = _nf4(1 << 19, 8192)
    assert L.qlora_quantize(P, ctypes.byref(big), None) == 2
    assert L.qlora_linear_fwd(ctypes.byref(big), P, 64, q.BF16, P, P, 8, q.BF16, P, P, P,
                              1 << 30, None) == 2
    s = _nf4()
    assert L.qlora_linear_fwd(ctypes.byref(s), P, (1 << 24) + 1, q.BF16, P, P, 8, q.BF16, P, P,
                              P, 1 << 30, None) == 2
    assert L.qlora_linear_bwd(ctypes.byref(s), P, P, (1 << 24) + 1, q.BF16, P, P, 8, q.BF16, P,
                              P, P, P, P, 1 << 30, None) == 2


def test_db_fold_planned_before_launch(L):
    """Where dB is formed inside the dX GEMM (bf16 activations, r <= 16) the
    plan also holds the bf16 XA^T copy; at a token count whose per-block dB
    partials would pass 2^31 bytes the plan falls back to dB in the dY pass,
    so no launch can be refused after an earlier one was queued.  Seen
    through the workspace: fp32 activations never fold and differ from bf16
    only by the bf16 copy of dY."""
    al = lambda b: (b + 255) // 256 * 256
    for (M, i, o, r, fold) in [(2048, 4096, 4096, 16, True), (1 << 24, 4096, 32768, 16, False)]:
        b16 = q.qlora_bwd_workspace_bytes(M, i, o, r, q.BF16)
        b32 = q.qlora_bwd_workspace_bytes(M, i, o, r, q.F32)
        assert b16 > 0 and b32 > 0
        assert (b32 - b16 == al(M * o * 2)) == (not fold), (M, o)


def test_status_strings(L):
    for s in range(8):
        assert q.qlora_status_string(s) == q.STATUS[s]


# ------------------------------------------------------------ validation
# Fake device addresses: validation fails before any pointer is touched or
# any HIP call is made, so these never reach the runtime.
P = 0x10000          # 16-byte aligned
U = 0x10004          # misaligned


def _nf4(i=256, o=256, codes=P, qs=P, gs=P, cb=0):
    return q.nf4_struct(i, o, codes, qs, gs, cb)


def _st(f, *a):
    return f(*a)


def test_quantize_validation(L):
    s = _nf4()
    assert L.qlora_quantize(None, ctypes.byref(s), None) == 1
    assert L.qlora_quantize(U, ctypes.byref(s), None) == 3
    assert L.qlora_quantize(P, None, None) == 1
    for (i, o) in [(100, 256), (256, 100), (0, 256), (-64, 64)]:
        s2 = _nf4(i, o)
        assert L.qlora_quantize(P, ctypes.byref(s2), None) == 2
    assert L.qlora_quantize(P, ctypes.byref(_nf4(codes=None)), None) == 1
    assert L.qlora_quantize(P, ctypes.byref(_nf4(qs=U)), None) == 3
    for cb in (5, -1):                                 # unknown codebook
        assert L.qlora_quantize(P, ctypes.byref(_nf4(cb=cb)), None) == 4


def test_fwd_validation(L):
    s = _nf4()
    f = L.qlora_linear_fwd
    ws = q.qlora_fwd_workspace_bytes(64, 256, 256, 8, q.BF16)
    # M = 0 is a no-op that succeeds without touching the device
    assert f(ctypes.byref(s), P, 0, q.BF16, P, P, 8, q.BF16, P, P, P, ws, None) == 0
    assert f(ctypes.byref(s), P, -1, q.BF16, P, P, 8, q.BF16, P, P, P, ws, None) == 2
    assert f(ctypes.byref(s), P, 64, q.BF16, P, P, 300, q.BF16, P, P, P, ws, None) == 2
    assert f(ctypes.byref(s), P, 64, 7, P, P, 8, q.BF16, P, P, P, ws, None) == 4
    assert f(ctypes.byref(s), P, 64, q.BF16, P, P, 8, 9, P, P, P, ws, None) == 4
    assert f(ctypes.byref(s), None, 64, q.BF16, P, P, 8, q.BF16, P, P, P, ws, None) == 1
    assert f(ctypes.byref(s), P, 64, q.BF16, None, P, 8, q.BF16, P, P, P, ws, None) == 1
    # XA (the saved activation) is optional: a NULL XA passes the pointer
    # checks and is stopped here by the workspace size, before any launch
    assert f(ctypes.byref(s), P, 64, q.BF16, P, P, 8, q.BF16, P, None, P, ws - 1, None) == 5
    assert f(ctypes.byref(s), P, 64, q.BF16, P, P, 8, q.BF16, P, U, P, ws, None) == 3
    assert f(ctypes.byref(s), U, 64, q.BF16, P, P, 8, q.BF16, P, P, P, ws, None) == 3
    assert f(ctypes.byref(s), P, 64, q.BF16, P, P, 8, q.BF16, U, P, P, ws, None) == 3
    assert f(ctypes.byref(s), P, 64, q.BF16, P, P, 8, q.BF16, P, P, P, ws - 1, None) == 5
    assert f(ctypes.byref(s), P, 64, q.BF16, P, P, 8, q.BF16, P, P, None, ws, None) == 1
    bad = _nf4(256, 96)
    assert f(ctypes.byref(bad), P, 64, q.BF16, P, P, 8, q.BF16, P, P, P, ws, None) == 2
    assert f(ctypes.byref(_nf4(cb=5)), P, 64, q.BF16, P, P, 8, q.BF16, P, P, P, ws, None) == 4


def test_bwd_validation(L):
    s = _nf4()
    f = L.qlora_linear_bwd
    ws = q.qlora_bwd_workspace_bytes(64, 256, 256, 8, q.BF16)
    args = lambda **k: [ctypes.byref(k.get("s", s)), k.get("X", P), k.get("dY", P), k.get("M", 64),
                        k.get("act", q.BF16), k.get("A", P), k.get("B", P), k.get("r", 8),
                        k.get("adt", q.BF16), k.get("XA", P), k.get("dX", P), k.get("dA", P),
                        k.get("dB", P), k.get("ws", P), k.get("wsb", ws), None]
    assert f(*args(M=-5)) == 2
    assert f(*args(r=-1)) == 2
    assert f(*args(act=3)) == 4
    assert f(*args(dY=None)) == 1
    assert f(*args(X=None)) == 1
    assert f(*args(dA=None)) == 1
    assert f(*args(dB=U)) == 3
    assert f(*args(XA=U)) == 3
    assert f(*args(wsb=ws - 256)) == 5
    assert f(*args(ws=None)) == 1
    assert f(*args(s=_nf4(192, 100))) == 2


def test_lora_validation(L):
    """Adapter options are checked before anything else; valid ones fall
    through to the usual checks (here M = 0 or a NULL workspace)."""
    s = _nf4()
    ws = q.qlora_fwd_workspace_bytes(64, 256, 256, 8, q.BF16)
    def fwd(o, M=64):
        return L.qlora_linear_fwd_lora(ctypes.byref(s), P, M, q.BF16, P, P, 8, q.BF16,
                                       ctypes.byref(o) if o is not None else None,
                                       P, P, None, ws, None)
    def bwd(o):
        return L.qlora_linear_bwd_lora(ctypes.byref(s), P, P, 64, q.BF16, P, P, 8, q.BF16,
                                       ctypes.byref(o), P, P, P, P, None, ws, None)
    for bad in (q.qlora_lora(1.0, 0.5, None),          # dropout without a mask
                q.qlora_lora(1.0, 1.0, P),             # p = 1
                q.qlora_lora(1.0, -0.1, P),
                q.qlora_lora(1.0, float("nan"), P),
                q.qlora_lora(float("inf"), 0.0, None),
                q.qlora_lora(3e38, 0.9, P)):           # c = scale / (1 - p) overflows fp32
        assert fwd(bad) == 7 and bwd(bad) == 7
        assert fwd(bad, M=0) == 7
    for good in (None, q.qlora_lora(2.0, 0.0, None), q.qlora_lora(0.5, 0.1, P),
                 q.qlora_lora(-1.0, 0.0, P)):
        assert fwd(good) == 1                          # passes to the NULL workspace check
        assert fwd(good, M=0) == 0
    assert bwd(q.qlora_lora(2.0, 0.25, P)) == 1


def test_bwd_adam_validation(L):
    s = _nf4()
    ws = q.qlora_bwd_workspace_bytes(64, 256, 256, 8, q.BF16)
    st = q.qlora_adam_state(P, P, P, None)
    good = q.qlora_adam_hparams(1, 1e-3, 0.9, 0.999, 1e-8, 0.0)
    def call(M=64, sa=st, sb=st, hp=good, wsp=None, lora=None):
        return L.qlora_linear_bwd_adam(ctypes.byref(s), P, P, M, q.BF16, P, P, 8, q.BF16,
                                       ctypes.byref(lora) if lora is not None else None,
                                       P, P, ctypes.byref(sa) if sa is not None else None,
                                       ctypes.byref(sb) if sb is not None else None,
                                       ctypes.byref(hp) if hp is not None else None,
                                       None, None, wsp, ws, None)
    assert call() == 1                                      # NULL workspace, after every check
    assert call(hp=None) == 7
    for bad in (q.qlora_adam_hparams(0, 1e-3, 0.9, 0.999, 1e-8, 0.0),
                q.qlora_adam_hparams(1, 1e-3, 1.0, 0.999, 1e-8, 0.0),
                q.qlora_adam_hparams(1, float("nan"), 0.9, 0.999, 1e-8, 0.0),
                q.qlora_adam_hparams(1, 1e-3, 0.9, 0.999, -1.0, 0.0),
                q.qlora_adam_hparams(1, 1e-3, 0.9, 0.999, 1e-8, -0.1)):
        assert call(hp=bad) == 7
    assert call(lora=q.qlora_lora(1.0, 0.5, None)) == 7
    assert call(M=0) == 2
    assert call(sa=None) == 1 and call(sb=q.qlora_adam_state(P, None, P, None)) == 1
    assert call(sb=q.qlora_adam_state(P, P, U, None)) == 3
    assert call(sa=q.qlora_adam_state(P, P, P, U)) == 3


def test_fwd_group_validation(L):
    n = 2
    ins, outs = [256, 320], [256, 192]
    ws = q.qlora_fwd_group_workspace_bytes(4, ins, outs, 16)
    assert ws > 0
    assert q.qlora_fwd_group_workspace_bytes(17, ins, outs, 16) == 0      # not few-token
    assert q.qlora_fwd_group_workspace_bytes(4, ins, outs, 65) == 0
    assert q.qlora_fwd_group_workspace_bytes(4, [256, 100], outs, 16) == 0
    s = [_nf4(256, 256), _nf4(320, 192)]
    pw = lambda st: (ctypes.POINTER(q.qlora_nf4) * len(st))(*[ctypes.pointer(x) for x in st])
    arr = lambda v, k=n: (ctypes.c_void_p * k)(*([v] * k))
    def call(k=n, M=4, r=16, st=s, X=P, Y=P, wsp=P, wsb=ws):
        return L.qlora_linear_fwd_group(k, pw(st), arr(X, len(st)), M, q.BF16, arr(P, len(st)),
                                        arr(P, len(st)), r, q.BF16, arr(Y, len(st)),
                                        arr(P, len(st)), wsp, wsb, None)
    assert call(k=0) == 2 and call(k=5) == 2
    assert call(M=0) == 2 and call(M=17) == 2 and call(r=65) == 2
    assert call(st=[_nf4(256, 256), _nf4(320, 192, cb=1)]) == 4       # codebooks differ
    assert call(X=None) == 1 and call(Y=U) == 3
    assert call(wsp=None) == 1 and call(wsb=ws - 1) == 5


def test_merge_validation(L):
    s = _nf4()
    f = L.qlora_merge
    assert f(ctypes.byref(s), P, P, 8, q.BF16, None, q.F32, None) == 1
    assert f(ctypes.byref(s), P, P, 8, q.BF16, U, q.F32, None) == 3
    assert f(ctypes.byref(s), None, P, 8, q.BF16, P, q.F32, None) == 1
    assert f(ctypes.byref(s), P, U, 8, q.BF16, P, q.F32, None) == 3
    assert f(ctypes.byref(s), P, P, -1, q.BF16, P, q.F32, None) == 2
    assert f(ctypes.byref(s), P, P, 300, q.BF16, P, q.F32, None) == 2
    assert f(ctypes.byref(s), P, P, 8, 3, P, q.F32, None) == 4
    assert f(ctypes.byref(s), P, P, 8, q.BF16, P, 7, None) == 4
    assert f(ctypes.byref(_nf4(256, 100)), P, P, 8, q.BF16, P, q.F32, None) == 2
    assert f(ctypes.byref(_nf4(cb=7)), P, P, 8, q.BF16, P, q.F32, None) == 4
    assert f(None, P, P, 8, q.BF16, P, q.F32, None) == 1


def test_adam_validation(L):
    f = L.qlora_adam_step
    F = ctypes.c_float
    ok = (P, P, P, P, 64, 1, F(1e-3), F(0.9), F(0.999), F(1e-8), F(0.0), None, None)
    def call(**kw):
        a = list(ok)
        for k, v in kw.items():
            a[["th", "g", "m", "v", "n", "step", "lr", "b1", "b2", "eps", "wd", "t16", "s"].index(k)] = v
        return f(*a)
    assert call(n=0, th=None) == 0                     # no-op before any pointer check
    assert call(th=None) == 1 and call(v=None) == 1
    assert call(g=U) == 3 and call(t16=U) == 3
    assert call(n=-1) == 2 and call(step=0) == 2
    assert call(b1=F(1.0)) == 7 and call(b2=F(-0.1)) == 7
    assert call(eps=F(-1.0)) == 7 and call(wd=F(-1e-3)) == 7
    assert call(lr=F(float("inf"))) == 7


def test_loftq_validation(L):
    f = L.qlora_loftq_init
    s = _nf4(256, 256)
    ws = q.qlora_loftq_workspace_bytes(256, 256, 24)
    assert ws > 0 and q.qlora_loftq_workspace_bytes(256, 256, 0) == 0
    ok = [P, ctypes.byref(s), P, 24, 16, 2, P, P, q.F32, P, ws, None]
    def call(i, v):
        a = list(ok)
        a[i] = v
        return f(*a)
    assert call(0, None) == 1 and call(2, None) == 1 and call(9, None) == 1
    assert call(3, 129) == 2 and call(4, 25) == 2 and call(4, 0) == 2 and call(5, -1) == 2
    assert call(8, 5) == 4
    assert call(6, U) == 3
    assert call(10, ws - 1) == 5
    assert call(1, ctypes.byref(_nf4(256, 100))) == 2
    bad = _nf4(256, 256)
    bad.block = 32                      # neither the 64-weight nor the 16-entry format
    assert call(1, ctypes.byref(bad)) == 4
    # the 16-entry format has no int8 scales: a NULL qscale passes the null
    # check and the call stops at the (too small) workspace, before any
    # device work
    g16 = _nf4(256, 256)
    g16.block = 16
    g16.qscale = None
    a = list(ok)
    a[1], a[10] = ctypes.byref(g16), ws - 1
    assert f(*a) == 5


def test_algorithmic_work_formulas():
    # fwd+bwd FLOP at 4096^2, r = 16, M = 2048 (without the dense dW)
    f = workloads.fwd_flops(2048, 4096, 4096, 16) + workloads.bwd_flops(2048, 4096, 4096, 16)
    assert f == 2 * 2048 * (2 * 4096 * 4096 + 3 * 16 * (4096 + 4096))
    assert workloads.quantize_bytes(4096, 4096) == 75763712


def _bucket_lut(T):
    """The encoder's bucket table, built from its definition: bucket i holds
    x in [-1 + i/32, -1 + (i+1)/32) (bucket 64: x = 1); base = number of
    thresholds below the bucket, T = the one threshold inside (+inf if none)."""
    T = np.asarray(T, np.float64)
    T = T[np.isfinite(T) & (T <= 1.0)]     # x = w / absmax never exceeds 1
    lut = []
    for i in range(128):
        a = -1.0 + i / 32.0
        b = a + 1.0 / 32.0 if i < 64 else np.inf
        inside = T[(T >= a) & (T < b)]
        assert inside.size <= 1, (i, inside)
        lut.append((np.float32(inside[0]) if inside.size else np.float32(np.inf), int(np.sum(T < a))))
    return lut


@pytest.mark.parametrize("cb,levels", CODEBOOKS)
def test_bucket_lookup_reproduces_oracle_argmin(L, cb, levels):
    """code = base + (x >= T_bucket), with the bucket read off the fp32 bits of
    x + 3, equals the oracle's fp32 argmin on the threshold sweep and around
    every bucket boundary (where x + 3 rounds up into the next bucket)."""
    T = np.array(q.qlora_codebook_thresholds(cb), np.float32)
    lut = _bucket_lut(T)
    edges = []
    for i in range(65):
        b = np.array([-1.0 + i / 32.0], np.float32).view(np.int32)[0]
        nb = np.arange(b - 4000, b + 4001, dtype=np.int64)
        nb = nb[(nb >= np.int64(np.int32(-0x7FFFFFFF) - 1)) & (nb <= 0x7FFFFFFF)]
        edges.append(nb.astype(np.int32).view(np.float32))
        edges.append(-edges[-1])
    x = np.concatenate([_x_sweep(T, levels())] + edges)
    x = x[(x >= -1) & (x <= 1)]
    key = ((x + np.float32(3.0)).astype(np.float32).view(np.uint32) >> 17) & 127
    Tb = np.array([e[0] for e in lut], np.float32)[key]
    base = np.array([e[1] for e in lut], np.int64)[key]
    mine = base + (x >= Tb)
    pad = (-x.size) % 63
    xx = np.concatenate([x, np.zeros(pad, np.float32)])
    w = np.concatenate([np.ones((xx.size // 63, 1), np.float32), xx.reshape(-1, 63)], axis=1).reshape(-1)
    codes = oracle.encode(w, onf4.block_absmax(w), levels()).reshape(-1, 64)[:, 1:].reshape(-1)[: x.size]
    assert np.array_equal(codes, mine)


def test_fp64_reciprocal_product_rounds_like_fp32_division():
    """The encoder forms x = RN32(w * RN64(1/c)) in fp64.  For fp32 w, c this
    equals the IEEE fp32 quotient w / c: random pairs over many binades, and
    pairs whose quotient sits next to an fp32 rounding midpoint."""
    rng = np.random.default_rng(7)
    n = 1 << 20
    c = (rng.random(n) * 2.0 ** rng.integers(-60, 60, n)).astype(np.float32)
    c = c[c > 0]
    w = (c * (rng.random(c.size) * 2 - 1)).astype(np.float32)
    # quotients near midpoints: w = RN32(c * mid) for a random fp32 midpoint
    mid_base = (rng.random(c.size) * 0.999 + 0.001).astype(np.float32)
    up = np.nextafter(mid_base, np.float32(2.0))
    mid = (mid_base.astype(np.float64) + up.astype(np.float64)) / 2
    w2 = (c.astype(np.float64) * mid).astype(np.float32)
    for ww in (w, w2, -w2):
        exact = (ww / c).astype(np.float32)
        y = 1.0 / c.astype(np.float64)
        mine = (ww.astype(np.float64) * y).astype(np.float32)
        assert np.array_equal(exact.view(np.uint32), mine.view(np.uint32))


def test_noalloc_forward_validation(L):
    """The forward that allocates nothing refuses a shape whose workspace
    exceeds its device-resident array before any HIP call (so this runs
    without a GPU), and validates like qlora_linear_fwd."""
    import re
    text = open(q.HEADER).read()
    m = re.search(r"#define QLORA_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == q.NOALLOC_SCRATCH_BYTES
    f = L.qlora_linear_fwd_noalloc
    s = _nf4(4096, 256)
    assert q.qlora_fwd_workspace_bytes(8192, 4096, 256, 16, q.F32) > q.NOALLOC_SCRATCH_BYTES
    assert f(ctypes.byref(s), P, 8192, q.F32, P, P, 16, q.F32, P, P, None) == 5
    assert f(ctypes.byref(s), P, 0, q.BF16, P, P, 16, q.BF16, P, P, None) == 0
    assert f(ctypes.byref(s), P, -1, q.BF16, P, P, 16, q.BF16, P, P, None) == 2
    assert f(ctypes.byref(_nf4(256, 100)), P, 64, q.BF16, P, P, 8, q.BF16, P, P, None) == 2
    assert f(ctypes.byref(s), P, 64, 9, P, P, 8, q.BF16, P, P, None) == 4


def test_scale_format_validation(L):
    """qlora_nf4.block: 0 / 64 (double-quantized 64-weight blocks) or 16 (the
    lab's 16-entry groups, qscale unused and may be NULL); anything else is
    refused as a dtype error before any launch."""
    for blk in (8, 32, 128, -16):
        s = q.nf4_struct(256, 256, P, P, P, 0, blk)
        assert L.qlora_quantize(P, ctypes.byref(s), None) == 4
    s = q.nf4_struct(256, 256, P, None, P, q.CB_INT4, 16)     # no qscale: accepted
    assert L.qlora_linear_fwd(ctypes.byref(s), P, 0, q.BF16, P, P, 8, q.BF16, P, P, P, 0, None) == 0
    s = q.nf4_struct(256, 256, P, None, P, q.CB_INT4, 64)     # 64-weight format needs qscale
    assert L.qlora_quantize(P, ctypes.byref(s), None) == 1
    s = q.nf4_struct(256, 256, P, None, U, q.CB_INT4, 16)
    assert L.qlora_quantize(P, ctypes.byref(s), None) == 3
