"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle
checks.

This module holds no arithmetic of the method: it only draws random numbers
and rounds them to the storage type of the input (fp32 or bf16).  Both the
HIP path and the CPU oracle receive exactly these values.

Recipe (the workloads' stated distributions):
* frozen weights W0 ~ N(0, 0.02^2), fp32, stored (in, out) row-major;
* activations X and upstream gradients dY ~ N(0, 1), cast to bf16 with
  round-to-nearest-even (kept fp32 for the small fp32 workload);
* adapters A ~ N(0, 1) / sqrt(in) and B ~ N(0, 0.01^2) or B = 0
  ("QLoRA (low-rank adapters on a quantized model)", "How it works": A random,
  B zero at the start);
* every tensor has its own generator, numpy ``default_rng`` seeded with
  ``[0, workload, layer, linear, tensor_id]`` (seeds rooted at 0 as in the
  pages' snippets).
"""

import numpy as np

W_STD = 0.02
B_STD = 0.01

# tensor ids inside a seed key
T_W0, T_X, T_DY, T_A, T_B = 0, 1, 2, 3, 4


def rng(workload, layer=0, linear=0, tensor=0):
    return np.random.default_rng([0, int(workload), int(layer), int(linear), int(tensor)])


def bf16_bits(x):
    """fp32 array -> uint16 bf16 bit patterns, round to nearest even.
    Inputs must be finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits):
    """uint16 bf16 bit patterns -> exact fp32 values."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32)
    return (b << np.uint32(16)).view(np.float32)


class Tensor:
    """A synthetic input: ``values`` are the exact fp32 numbers; ``raw`` is
    what goes to the device (fp32 array, or uint16 bf16 bits)."""

    def __init__(self, values, raw, dtype):
        self.values = values
        self.raw = raw
        self.dtype = dtype          # "f32" or "bf16"

    @property
    def shape(self):
        return self.values.shape


def _as(x, dtype):
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return Tensor(x, x, "f32")
    if dtype == "bf16":
        bits = bf16_bits(x)
        return Tensor(bf16_to_f32(bits), bits, "bf16")
    raise ValueError(dtype)


def weights(n_in, n_out, workload, layer=0, linear=0):
    """W0 ~ N(0, 0.02^2), fp32, shape (in, out)."""
    g = rng(workload, layer, linear, T_W0)
    w = g.standard_normal((n_in, n_out), dtype=np.float32)
    w *= np.float32(W_STD)
    return w


def activations(m, dim, workload, dtype, layer=0, linear=0, tensor=T_X):
    """X (tensor=T_X) or dY (tensor=T_DY) ~ N(0, 1), shape (m, dim)."""
    g = rng(workload, layer, linear, tensor)
    return _as(g.standard_normal((m, dim), dtype=np.float32), dtype)


def adapters(n_in, n_out, rank, workload, dtype, b_zero=False, layer=0, linear=0):
    """A ~ N(0,1)/sqrt(in) (in x r); B ~ N(0, 0.01^2) or zeros (r x out)."""
    ga = rng(workload, layer, linear, T_A)
    a = ga.standard_normal((n_in, rank), dtype=np.float32)
    a = (a / np.float32(np.sqrt(n_in))).astype(np.float32)
    if b_zero:
        b = np.zeros((rank, n_out), dtype=np.float32)
    else:
        gb = rng(workload, layer, linear, T_B)
        b = gb.standard_normal((rank, n_out), dtype=np.float32) * np.float32(B_STD)
    return _as(a, dtype), _as(b, dtype)


def p2_sample():
    """The weight sample of the reconstruction experiment on "LLMs · QLoRA"
    (NormalFloat section): 262,144 standard-normal draws from torch's CPU
    generator started at seed 0, scaled to a standard deviation of 0.02, fp32."""
    import torch
    gen = torch.Generator().manual_seed(0)
    draws = torch.randn(64 * 4096, generator=gen, dtype=torch.float32).numpy()
    return draws * np.float32(W_STD)
