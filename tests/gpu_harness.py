"""Shared helpers of the GPU parity tests: run the library through its C ABI
on seeded synthetic inputs and compute what the oracle says about them."""

import sys

import numpy as np

import oracle
from quantized_rank_fine_amd import qlora as q
from quantized_rank_fine_amd import synth

TOL = 1e-2          # max|gpu - ref| / max|ref| for float outputs (bf16 compute)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def torch_dev():
    import torch
    return torch, torch.device("cuda:0")


def to_dev(a, dtype=None):
    torch, dev = torch_dev()
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.to(dev)


def rel_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.abs(ref).max()
    if den == 0:
        return float(np.abs(got).max())
    return float(np.abs(got - ref).max() / den)


def bf16_to_f64(t):
    """device bf16 tensor (torch) -> numpy float64."""
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32).__lshift__(16) \
        .view(np.float32).astype(np.float64)


def out_to_f64(t, dtype):
    import torch
    if dtype == "bf16":
        return bf16_to_f64(t)
    return t.float().cpu().numpy().astype(np.float64)


def levels_of(codebook):
    """The oracle's level table of a codebook."""
    return {q.CB_NF4: oracle.nf4_levels, q.CB_UNIFORM4: oracle.uniform4_levels,
            q.CB_INT4: lambda: oracle.int_levels(7), q.CB_INT3: lambda: oracle.int_levels(3),
            q.CB_TERNARY: lambda: oracle.int_levels(1)}[codebook]()


def quantize_gpu(w0, codebook=q.CB_NF4, block=64):
    """Quantize an fp32 (in, out) numpy matrix on the GPU; returns the
    NF4Weight (device buffers).  block = 16: the lab's 16-entry format."""
    torch, dev = torch_dev()
    n_in, n_out = w0.shape
    wq = q.NF4Weight(n_in, n_out, dev, codebook, block)
    tw = to_dev(w0)
    q.qlora_quantize(tw, wq)
    torch.cuda.synchronize()
    del tw
    return wq


class Layer:
    """Seeded inputs of one adapted linear, on host and device."""

    def __init__(self, workload, M, n_in, n_out, r, act="bf16", adt="bf16", b_zero=False,
                 layer=0, linear=0, w0=None, codebook=q.CB_NF4, block=64):
        torch, dev = torch_dev()
        self.M, self.n_in, self.n_out, self.r = M, n_in, n_out, r
        self.codebook = codebook
        self.block = block
        self.act, self.adt = act, adt
        self.w0 = synth.weights(n_in, n_out, workload, layer, linear) if w0 is None else w0
        self._okey = (workload, n_in, n_out, layer, linear, codebook, block) if w0 is None else None
        self._oq = None
        self.X = synth.activations(M, n_in, workload, act, layer, linear)
        self.dY = synth.activations(M, n_out, workload, act, layer, linear, tensor=synth.T_DY)
        if r > 0:
            self.A, self.B = synth.adapters(n_in, n_out, r, workload, adt, b_zero, layer, linear)
        else:
            self.A = self.B = None
        self.tdt = torch.bfloat16 if act == "bf16" else torch.float32
        self.adt_t = torch.bfloat16 if adt == "bf16" else torch.float32
        self.qact = q.BF16 if act == "bf16" else q.F32
        self.qadt = q.BF16 if adt == "bf16" else q.F32

        def dv(tensor, dt):
            if tensor is None:
                return None
            if tensor.dtype == "bf16":
                return to_dev(tensor.raw.view(np.int16)).view(torch.bfloat16)
            return to_dev(tensor.raw)

        self.tX = dv(self.X, self.tdt)
        self.tdY = dv(self.dY, self.tdt)
        self.tA = dv(self.A, self.adt_t)
        self.tB = dv(self.B, self.adt_t)
        self.wq = quantize_gpu(self.w0, codebook, block)

    # ---------------------------------------------------------------- runs
    def fwd(self, lora=None, save_xa=True):
        """lora: None, or (scale, dropout_p, keep) with keep a device uint8
        [M, r] tensor or None -- then the call goes through the options entry
        point.  save_xa=False passes a NULL XA (not saved)."""
        torch, dev = torch_dev()
        M, r = self.M, self.r
        Y = torch.empty(M, self.n_out, dtype=self.tdt, device=dev)
        XA = torch.empty(M, max(r, 1), dtype=torch.float32, device=dev) if r and save_xa else None
        wsb = q.qlora_fwd_workspace_bytes(M, self.n_in, self.n_out, r, self.qact)
        ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev) if wsb else None
        if lora is None:
            q.qlora_linear_fwd(self.wq, self.tX, M, self.qact, self.tA, self.tB, r, self.qadt,
                               Y, XA, ws, wsb)
        else:
            q.qlora_linear_fwd_lora(self.wq, self.tX, M, self.qact, self.tA, self.tB, r,
                                    self.qadt, *lora, Y, XA, ws, wsb)
        torch.cuda.synchronize()
        return Y, XA

    def bwd(self, XA=None, want_dx=True, lora=None):
        torch, dev = torch_dev()
        M, r = self.M, self.r
        dX = torch.empty(M, self.n_in, dtype=self.tdt, device=dev) if want_dx else None
        dA = torch.empty(self.n_in, max(r, 1), dtype=torch.float32, device=dev) if r else None
        dB = torch.empty(max(r, 1), self.n_out, dtype=torch.float32, device=dev) if r else None
        wsb = q.qlora_bwd_workspace_bytes(M, self.n_in, self.n_out, r, self.qact)
        ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev) if wsb else None
        if lora is None:
            q.qlora_linear_bwd(self.wq, self.tX, self.tdY, M, self.qact, self.tA, self.tB, r,
                               self.qadt, XA, dX, dA, dB, ws, wsb)
        else:
            q.qlora_linear_bwd_lora(self.wq, self.tX, self.tdY, M, self.qact, self.tA, self.tB,
                                    r, self.qadt, *lora, XA, dX, dA, dB, ws, wsb)
        torch.cuda.synchronize()
        return dX, dA, dB

    # -------------------------------------------------------------- oracle
    def oracle_q(self):
        """The oracle's quantization of this layer's W0 (cached per seeded
        weight): codes, q8 and s2 computed on the CPU from the same input."""
        if self._oq is None:
            key = self._okey
            if key is not None and key in _ORACLE_Q:
                self._oq = _ORACLE_Q[key]
            else:
                if self.block == 16:
                    self._oq = oracle.quantize_groups(self.w0, levels_of(self.codebook))
                else:
                    self._oq = oracle.quantize(self.w0, levels_of(self.codebook))
                if key is not None:
                    _ORACLE_Q.clear()          # keep one large weight at a time
                    _ORACLE_Q[key] = self._oq
        return self._oq

    def w_hat(self):
        """deq(Q(W0)) in float64, from the oracle's own quantization of W0
        (nothing read back from the device)."""
        oq = self.oracle_q()
        if self.block == 16:
            return oracle.dequantize_groups(oq["packed"], oq["scales"], self.n_in, self.n_out,
                                            levels_of(self.codebook))
        return oracle.dequantize(oq["packed"], oq["q8"], oq["s2"], self.n_in, self.n_out,
                                 levels_of(self.codebook))

    def codes_match_oracle(self):
        """The device's packed codes, q8 and s2 against the oracle's."""
        oq = self.oracle_q()
        assert np.array_equal(self.wq.codes.cpu().numpy(), oq["packed"])
        if self.block == 16:
            assert np.array_equal(self.wq.gscale.cpu().numpy().view(np.uint32),
                                  oq["scales"].view(np.uint32))
            return
        assert np.array_equal(self.wq.qscale.cpu().numpy(), oq["q8"])
        assert np.array_equal(self.wq.gscale.cpu().numpy().view(np.uint32),
                              oq["s2"].view(np.uint32))

    def ref(self, rows=None):
        """Oracle forward/backward (float64) on the oracle's quantized weight.
        With `rows`, y and dX only for those rows."""
        W = self.w_hat()
        X = self.X.values.astype(np.float64)
        dY = self.dY.values.astype(np.float64)
        A = None if self.A is None else self.A.values
        B = None if self.B is None else self.B.values
        out = {}
        if A is not None:
            XA = X @ A.astype(np.float64)
            out["XA"] = XA
        sel = slice(None) if rows is None else rows
        _, y = oracle.forward(X[sel], W, A, B)
        out["y"] = y
        g = oracle.backward(X[sel], dY[sel], W, A, B)
        out["dX"] = g["dX"]
        if A is not None:
            G = dY @ B.astype(np.float64).T
            out["dA"] = X.T @ G
            out["dB"] = XA.T @ dY
        return out


# The oracle's quantization of the most recent seeded weight, keyed by
# (workload, in, out, layer, linear, codebook).
_ORACLE_Q = {}
