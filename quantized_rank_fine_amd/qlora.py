"""Thin Python binding of libqlora (argument marshalling only).

Every function here has the name of the C entry point it calls and does no
arithmetic of its own: it turns torch tensors into device pointers, takes the
current HIP stream, calls the library and raises on a non-OK status.  Every
step of the hot path runs in the HIP kernels of ``libqlora.so``; if the
library is missing the import fails loudly.
"""

import ctypes
import os
import re

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqlora.so")
HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "qlora.h")

F32, BF16 = 0, 1
LAB_GROUP = 16                        # QLORA_LAB_GROUP: 16-entry scale groups
NOALLOC_SCRATCH_BYTES = 32 << 20      # QLORA_NOALLOC_SCRATCH_BYTES
CB_NF4, CB_UNIFORM4, CB_INT4, CB_INT3, CB_TERNARY = 0, 1, 2, 3, 4   # qlora_codebook
STATUS = {0: "ok", 1: "null pointer", 2: "invalid shape", 3: "pointer not 16-byte aligned",
          4: "invalid dtype", 5: "workspace too small", 6: "HIP runtime error",
          7: "invalid value"}
KERNELS = ("quantize", "xa_rowdot", "fwd_gemm", "dy_pass", "dx_gemm", "da_pass", "reduce",
           "fwd_smallm")


class QloraError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} (status {status})")


class qlora_nf4(ctypes.Structure):
    _fields_ = [("in_", ctypes.c_int64), ("out", ctypes.c_int64),
                ("codes", ctypes.c_void_p), ("qscale", ctypes.c_void_p),
                ("gscale", ctypes.c_void_p), ("codebook", ctypes.c_int32),
                ("block", ctypes.c_int32)]


class qlora_lora(ctypes.Structure):
    _fields_ = [("scale", ctypes.c_float), ("dropout_p", ctypes.c_float),
                ("keep", ctypes.c_void_p)]


class qlora_adam_state(ctypes.Structure):
    _fields_ = [("theta", ctypes.c_void_p), ("m", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("theta_bf16", ctypes.c_void_p)]


class qlora_adam_hparams(ctypes.Structure):
    _fields_ = [("step", ctypes.c_int64), ("lr", ctypes.c_float), ("beta1", ctypes.c_float),
                ("beta2", ctypes.c_float), ("eps", ctypes.c_float),
                ("weight_decay", ctypes.c_float)]


_lib = None


def lib():
    """Load libqlora.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                           "(or python quantized_rank_fine_amd/build.py)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    pnf4 = ctypes.POINTER(qlora_nf4)
    L.qlora_quantize.argtypes = [vp, pnf4, vp]
    L.qlora_linear_fwd.argtypes = [pnf4, vp, i64, ctypes.c_int, vp, vp, i32, ctypes.c_int, vp, vp,
                                   vp, sz, vp]
    L.qlora_linear_fwd_noalloc.argtypes = [pnf4, vp, i64, ctypes.c_int, vp, vp, i32,
                                           ctypes.c_int, vp, vp, vp]
    L.qlora_linear_fwd_noalloc.restype = ctypes.c_int
    L.qlora_linear_bwd.argtypes = [pnf4, vp, vp, i64, ctypes.c_int, vp, vp, i32, ctypes.c_int, vp,
                                   vp, vp, vp, vp, sz, vp]
    plora = ctypes.POINTER(qlora_lora)
    L.qlora_linear_fwd_lora.argtypes = [pnf4, vp, i64, ctypes.c_int, vp, vp, i32, ctypes.c_int,
                                        plora, vp, vp, vp, sz, vp]
    L.qlora_linear_bwd_lora.argtypes = [pnf4, vp, vp, i64, ctypes.c_int, vp, vp, i32,
                                        ctypes.c_int, plora, vp, vp, vp, vp, vp, sz, vp]
    pst, php = ctypes.POINTER(qlora_adam_state), ctypes.POINTER(qlora_adam_hparams)
    L.qlora_linear_bwd_adam.argtypes = [pnf4, vp, vp, i64, ctypes.c_int, vp, vp, i32,
                                        ctypes.c_int, plora, vp, vp, pst, pst, php, vp, vp, vp,
                                        sz, vp]
    L.qlora_linear_fwd_group.argtypes = [i32, ctypes.POINTER(pnf4), ctypes.POINTER(vp), i64,
                                         ctypes.c_int, ctypes.POINTER(vp), ctypes.POINTER(vp),
                                         i32, ctypes.c_int, ctypes.POINTER(vp),
                                         ctypes.POINTER(vp), vp, sz, vp]
    L.qlora_linear_fwd_group.restype = ctypes.c_int
    L.qlora_fwd_group_workspace_bytes.argtypes = [i32, i64, ctypes.POINTER(i64),
                                                  ctypes.POINTER(i64), i32, ctypes.c_int]
    L.qlora_fwd_group_workspace_bytes.restype = sz
    L.qlora_merge.argtypes = [pnf4, vp, vp, i32, ctypes.c_int, vp, ctypes.c_int, vp]
    f32 = ctypes.c_float
    L.qlora_adam_step.argtypes = [vp, vp, vp, vp, i64, i64, f32, f32, f32, f32, f32, vp, vp]
    L.qlora_loftq_init.argtypes = [vp, pnf4, vp, i32, i32, i32, vp, vp, ctypes.c_int, vp, sz, vp]
    L.qlora_loftq_workspace_bytes.argtypes = [i64, i64, i32]
    L.qlora_loftq_workspace_bytes.restype = sz
    for f in (L.qlora_quantize, L.qlora_linear_fwd, L.qlora_linear_bwd, L.qlora_merge,
              L.qlora_adam_step, L.qlora_loftq_init, L.qlora_linear_fwd_lora,
              L.qlora_linear_bwd_lora, L.qlora_linear_bwd_adam):
        f.restype = ctypes.c_int
    for f in (L.qlora_fwd_workspace_bytes, L.qlora_bwd_workspace_bytes):
        f.argtypes = [i64, i64, i64, i32, ctypes.c_int]
        f.restype = sz
    L.qlora_status_string.argtypes = [ctypes.c_int]
    L.qlora_status_string.restype = ctypes.c_char_p
    L.qlora_levels.argtypes = [ctypes.POINTER(ctypes.c_float)]
    L.qlora_levels.restype = None
    L.qlora_thresholds.argtypes = [ctypes.POINTER(ctypes.c_float)]
    L.qlora_thresholds.restype = None
    for f in (L.qlora_codebook_levels, L.qlora_codebook_thresholds):
        f.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_float)]
        f.restype = ctypes.c_int
    L.qlora_timing_enable.argtypes = [ctypes.c_int]
    L.qlora_timing_enable.restype = ctypes.c_int
    L.qlora_timing_read.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_double),
                                    ctypes.POINTER(ctypes.c_int64)]
    L.qlora_timing_read.restype = ctypes.c_int
    L.qlora_timing_reset.argtypes = []
    L.qlora_timing_reset.restype = None
    L.qlora_kernel_name.argtypes = [ctypes.c_int]
    L.qlora_kernel_name.restype = ctypes.c_char_p
    _lib = L
    return L


def header_functions():
    """Names of the functions include/qlora.h declares."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(qlora_[a-z0-9_]+)\s*\(",
                       text, flags=re.M)
    inline = set(re.findall(r"static\s+inline\s+\w+\s+(qlora_[a-z0-9_]+)\s*\(", text))
    return sorted(set(names) - inline)


# ------------------------------------------------------------------ helpers

def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(status, where):
    if status != 0:
        raise QloraError(status, where)


def nf4_struct(n_in, n_out, codes, qscale, gscale, codebook=CB_NF4, block=0):
    """qlora_nf4 describing caller-owned buffers (tensors or raw pointers)."""
    return qlora_nf4(int(n_in), int(n_out), _ptr(codes), _ptr(qscale), _ptr(gscale),
                     int(codebook), int(block))


class NF4Weight:
    """Caller-owned device buffers of one quantized (in, out) weight, the
    codebook its codes index and its scale format: block 64 (int8 block
    scales, double-quantized) or LAB_GROUP (one fp32 scale per 16 entries)."""

    def __init__(self, n_in, n_out, device="cuda", codebook=CB_NF4, block=64):
        import torch
        n = n_in * n_out
        self.n_in, self.n_out = n_in, n_out
        self.codebook = codebook
        self.block = block
        self.codes = torch.empty(n // 2, dtype=torch.uint8, device=device)
        if block == LAB_GROUP:
            self.qscale = None
            self.gscale = torch.empty(n // LAB_GROUP, dtype=torch.float32, device=device)
        else:
            self.qscale = torch.empty(n // 64, dtype=torch.int8, device=device)
            self.gscale = torch.empty((n // 64 + 255) // 256, dtype=torch.float32, device=device)

    def struct(self):
        return nf4_struct(self.n_in, self.n_out, self.codes, self.qscale, self.gscale,
                          self.codebook, 0 if self.block == 64 else self.block)


# ------------------------------------------------------------- entry points

def qlora_quantize(W0, wq, stream=None):
    s = wq.struct() if isinstance(wq, NF4Weight) else wq
    _check(lib().qlora_quantize(_ptr(W0), ctypes.byref(s), _stream(stream)), "qlora_quantize")


def qlora_merge(wq, A, B, r, adt, W, wdt, stream=None):
    s = wq.struct() if isinstance(wq, NF4Weight) else wq
    _check(lib().qlora_merge(ctypes.byref(s), _ptr(A), _ptr(B), int(r), int(adt), _ptr(W),
                             int(wdt), _stream(stream)), "qlora_merge")


def qlora_adam_step(theta, grad, m, v, step, lr, beta1=0.9, beta2=0.999, eps=1e-8,
                    weight_decay=0.0, theta_bf16=None, n=None, stream=None):
    n = theta.numel() if n is None else int(n)
    _check(lib().qlora_adam_step(_ptr(theta), _ptr(grad), _ptr(m), _ptr(v), n, int(step),
                                 float(lr), float(beta1), float(beta2), float(eps),
                                 float(weight_decay), _ptr(theta_bf16), _stream(stream)),
           "qlora_adam_step")


def qlora_loftq_workspace_bytes(n_in, n_out, k):
    return int(lib().qlora_loftq_workspace_bytes(int(n_in), int(n_out), int(k)))


def qlora_loftq_init(W0, wq, omega, k, r, iters, A, B, adt, ws, ws_bytes, stream=None):
    s = wq.struct() if isinstance(wq, NF4Weight) else wq
    _check(lib().qlora_loftq_init(_ptr(W0), ctypes.byref(s), _ptr(omega), int(k), int(r),
                                  int(iters), _ptr(A), _ptr(B), int(adt), _ptr(ws),
                                  int(ws_bytes), _stream(stream)), "qlora_loftq_init")


def qlora_fwd_workspace_bytes(M, n_in, n_out, r, act=BF16):
    return int(lib().qlora_fwd_workspace_bytes(M, n_in, n_out, r, int(act)))


def qlora_bwd_workspace_bytes(M, n_in, n_out, r, act=BF16):
    return int(lib().qlora_bwd_workspace_bytes(M, n_in, n_out, r, int(act)))


def qlora_linear_fwd(wq, X, M, act, A, B, r, adt, Y, XA, ws, ws_bytes, stream=None):
    s = wq.struct() if isinstance(wq, NF4Weight) else wq
    _check(lib().qlora_linear_fwd(ctypes.byref(s), _ptr(X), int(M), int(act), _ptr(A), _ptr(B),
                                  int(r), int(adt), _ptr(Y), _ptr(XA), _ptr(ws), int(ws_bytes),
                                  _stream(stream)), "qlora_linear_fwd")


def qlora_linear_fwd_noalloc(wq, X, M, act, A, B, r, adt, Y, XA, stream=None):
    """qlora_linear_fwd with the library's device-resident scratch (no
    workspace argument; nothing is allocated)."""
    s = wq.struct() if isinstance(wq, NF4Weight) else wq
    _check(lib().qlora_linear_fwd_noalloc(ctypes.byref(s), _ptr(X), int(M), int(act), _ptr(A),
                                          _ptr(B), int(r), int(adt), _ptr(Y), _ptr(XA),
                                          _stream(stream)), "qlora_linear_fwd_noalloc")


def qlora_linear_bwd(wq, X, dY, M, act, A, B, r, adt, XA, dX, dA, dB, ws, ws_bytes,
                     stream=None):
    s = wq.struct() if isinstance(wq, NF4Weight) else wq
    _check(lib().qlora_linear_bwd(ctypes.byref(s), _ptr(X), _ptr(dY), int(M), int(act), _ptr(A),
                                  _ptr(B), int(r), int(adt), _ptr(XA), _ptr(dX), _ptr(dA),
                                  _ptr(dB), _ptr(ws), int(ws_bytes), _stream(stream)),
           "qlora_linear_bwd")


def _lora(scale, dropout_p, keep):
    return qlora_lora(float(scale), float(dropout_p), _ptr(keep))


def qlora_linear_fwd_lora(wq, X, M, act, A, B, r, adt, scale, dropout_p, keep, Y, XA, ws,
                          ws_bytes, stream=None):
    """qlora_linear_fwd with the alpha/r factor `scale` and dropout on X.A
    (`keep`: [M, r] uint8 device mask or None, `dropout_p` its probability)."""
    s = wq.struct() if isinstance(wq, NF4Weight) else wq
    o = _lora(scale, dropout_p, keep)
    _check(lib().qlora_linear_fwd_lora(ctypes.byref(s), _ptr(X), int(M), int(act), _ptr(A),
                                       _ptr(B), int(r), int(adt), ctypes.byref(o), _ptr(Y),
                                       _ptr(XA), _ptr(ws), int(ws_bytes), _stream(stream)),
           "qlora_linear_fwd_lora")


def qlora_linear_bwd_lora(wq, X, dY, M, act, A, B, r, adt, scale, dropout_p, keep, XA, dX, dA,
                          dB, ws, ws_bytes, stream=None):
    """qlora_linear_bwd with the same adapter options as the forward."""
    s = wq.struct() if isinstance(wq, NF4Weight) else wq
    o = _lora(scale, dropout_p, keep)
    _check(lib().qlora_linear_bwd_lora(ctypes.byref(s), _ptr(X), _ptr(dY), int(M), int(act),
                                       _ptr(A), _ptr(B), int(r), int(adt), ctypes.byref(o),
                                       _ptr(XA), _ptr(dX), _ptr(dA), _ptr(dB), _ptr(ws),
                                       int(ws_bytes), _stream(stream)),
           "qlora_linear_bwd_lora")


def qlora_linear_bwd_adam(wq, X, dY, M, act, A, B, r, adt, XA, dX, state_A, state_B, step, lr,
                          ws, ws_bytes, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0,
                          lora=None, dA=None, dB=None, stream=None):
    """The backward with one Adam step of A and B fused into its last launch.
    state_A / state_B: (theta, m, v, theta_bf16 or None) device tensors;
    lora: None or (scale, dropout_p, keep)."""
    s = wq.struct() if isinstance(wq, NF4Weight) else wq
    sa = qlora_adam_state(*[_ptr(t) for t in state_A])
    sb = qlora_adam_state(*[_ptr(t) for t in state_B])
    hp = qlora_adam_hparams(int(step), float(lr), float(beta1), float(beta2), float(eps),
                            float(weight_decay))
    o = _lora(*lora) if lora is not None else None
    _check(lib().qlora_linear_bwd_adam(ctypes.byref(s), _ptr(X), _ptr(dY), int(M), int(act),
                                       _ptr(A), _ptr(B), int(r), int(adt),
                                       ctypes.byref(o) if o is not None else None, _ptr(XA),
                                       _ptr(dX), ctypes.byref(sa), ctypes.byref(sb),
                                       ctypes.byref(hp), _ptr(dA), _ptr(dB), _ptr(ws),
                                       int(ws_bytes), _stream(stream)),
           "qlora_linear_bwd_adam")


def qlora_fwd_group_workspace_bytes(M, ins, outs, r, act=None):
    n = len(ins)
    act = BF16 if act is None else act
    return int(lib().qlora_fwd_group_workspace_bytes(n, int(M), (ctypes.c_int64 * n)(*ins),
                                                     (ctypes.c_int64 * n)(*outs), int(r),
                                                     int(act)))


def qlora_linear_fwd_group(wqs, Xs, M, act, As, Bs, r, adt, Ys, XAs, ws, ws_bytes, stream=None):
    """Forward of up to 4 independent few-token linears in one pair of
    launches (lists of the per-linear weights and tensors)."""
    n = len(wqs)
    structs = [w.struct() if isinstance(w, NF4Weight) else w for w in wqs]
    pw = (ctypes.POINTER(qlora_nf4) * n)(*[ctypes.pointer(st) for st in structs])
    arr = lambda ts: (ctypes.c_void_p * n)(*[_ptr(t) for t in ts])
    _check(lib().qlora_linear_fwd_group(n, pw, arr(Xs), int(M), int(act), arr(As), arr(Bs),
                                        int(r), int(adt), arr(Ys), arr(XAs), _ptr(ws),
                                        int(ws_bytes), _stream(stream)),
           "qlora_linear_fwd_group")


def qlora_levels():
    buf = (ctypes.c_float * 16)()
    lib().qlora_levels(buf)
    return list(buf)


def qlora_thresholds():
    buf = (ctypes.c_float * 15)()
    lib().qlora_thresholds(buf)
    return list(buf)


def qlora_codebook_levels(codebook):
    buf = (ctypes.c_float * 16)()
    _check(0 if lib().qlora_codebook_levels(int(codebook), buf) == 0 else 4,
           "qlora_codebook_levels")
    return list(buf)


def qlora_codebook_thresholds(codebook):
    buf = (ctypes.c_float * 15)()
    _check(0 if lib().qlora_codebook_thresholds(int(codebook), buf) == 0 else 4,
           "qlora_codebook_thresholds")
    return list(buf)


def qlora_status_string(status):
    return lib().qlora_status_string(int(status)).decode()


def qlora_timing_enable(kinds=None):
    """Time the given kernel kinds (indices into KERNELS); None = all."""
    if kinds is None:
        mask = (1 << len(KERNELS)) - 1
    else:
        mask = 0
        for k in kinds:
            mask |= 1 << (KERNELS.index(k) if isinstance(k, str) else int(k))
    return lib().qlora_timing_enable(mask)


def qlora_timing_disable():
    return lib().qlora_timing_enable(0)


def qlora_timing_read(kind):
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    rc = lib().qlora_timing_read(int(kind), ctypes.byref(ms), ctypes.byref(n))
    if rc != 0:
        raise RuntimeError(f"qlora_timing_read failed ({rc})")
    return ms.value, n.value


def qlora_timing_reset():
    lib().qlora_timing_reset()


def qlora_kernel_name(kind):
    return lib().qlora_kernel_name(int(kind)).decode()
