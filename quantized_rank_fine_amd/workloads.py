"""The workloads this library is measured and tested on (shapes only).

Each linear is (in, out) with adapters of rank r; M is the number of tokens.
"""

LLAMA7B_LINEARS = (            # q, k, v, o, gate, up, down
    ("q", 4096, 4096), ("k", 4096, 4096), ("v", 4096, 4096), ("o", 4096, 4096),
    ("gate", 4096, 11008), ("up", 4096, 11008), ("down", 11008, 4096),
)

LLAMA65B_LINEARS = (
    ("q", 8192, 8192), ("k", 8192, 8192), ("v", 8192, 8192), ("o", 8192, 8192),
    ("gate", 8192, 22016), ("up", 8192, 22016), ("down", 22016, 8192),
)

WORKLOADS = {
    0: dict(name="linear-256x256-r8-M64-f32", linears=(("w", 256, 256),),
            rank=8, tokens=(64,), act="f32", adt="f32", layers=1, backward=True),
    1: dict(name="linear-4096x4096-r16-M2048-bf16", linears=(("w", 4096, 4096),),
            rank=16, tokens=(2048,), act="bf16", adt="bf16", layers=1, backward=True),
    2: dict(name="7b-layer-decode-r16-M1-4-16-bf16", linears=LLAMA7B_LINEARS,
            rank=16, tokens=(1, 4, 16), act="bf16", adt="bf16", layers=1,
            backward=False),
    3: dict(name="7b-layer-train-r64-M4096-bf16", linears=LLAMA7B_LINEARS,
            rank=64, tokens=(4096,), act="bf16", adt="bf16", layers=1, backward=True),
    4: dict(name="65b-80-layers-r64-M8192-bf16", linears=LLAMA65B_LINEARS,
            rank=64, tokens=(8192,), act="bf16", adt="bf16", layers=80,
            backward=True),
}


def fwd_flops(m, n_in, n_out, r):
    """Algorithmic forward FLOP: X.Wq plus the two rank-r products."""
    return 2 * m * (n_in * n_out + r * (n_in + n_out))


def bwd_flops(m, n_in, n_out, r):
    """Algorithmic backward FLOP: dY.Wq^T plus G, G.A^T, dA, dB (XA saved).
    The dense dW = X^T.dY is not formed and not counted."""
    return 2 * m * (n_in * n_out + 2 * r * (n_in + n_out))


def quantize_bytes(n_in, n_out):
    """Algorithmic bytes of one quantize pass: fp32 read, packed codes,
    int8 block scales and fp32 group scales written."""
    n = n_in * n_out
    return 4 * n + n // 2 + n // 64 + 4 * ((n // 64 + 255) // 256)


def nf4_bytes(n_in, n_out):
    """Bytes of the frozen quantized weight (codes + q8 + s2)."""
    n = n_in * n_out
    return n // 2 + n // 64 + 4 * ((n // 64 + 255) // 256)
