"""CPU oracle for the QLoRA adapted linear layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call, link
or execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table or
constant generator with the HIP library; both sides receive the same seeded
inputs from ``quantized_rank_fine_amd.synth`` and nothing else.

What it computes (plain, slow, obviously correct):

* ``levels``  -- the 16 NormalFloat-style levels (normal quantiles at 16 evenly
  spaced probabilities in [0.02, 0.98], divided by the largest magnitude), and
  the uniform 4-bit grid used as the comparison in the same write-up, and
  the symmetric integer grids (4, 3 bits and ternary) of the QLoRA lab.
* ``nf4``     -- blockwise absmax (64 weights per block), nearest-level
  encoding, two-codes-per-byte packing, double quantization of the block
  scales to int8 with one fp32 scale per 256 blocks, and dequantization;
  the lab's variant with one fp32 scale per 16 entries and no double
  quantization.
  The encoding runs in fp32 because its decision rule is an fp32 argmin;
  dequantization is exact in float64.
* ``linear``  -- forward y = X.deq(Wq) + (X.A).B and the backward
  dX, dA, dB in float64, both in factored form and (for tiny shapes) through
  the dense weight gradient dW = X^T.dY exactly as the chain rule is written;
  the same with the alpha/r factor and dropout on X.A (mask given);
  the merged dense weight deq(Wq) + A.B; adapters initialised from the
  best rank-r approximation of the quantization residual W0 - deq(Q(W0)).
* ``optim``   -- one Adam (AdamW) step of an adapter matrix, in float64.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
against values the pages print or against closed forms; no function is
"parity unpinned".
"""

from .levels import nf4_levels, uniform4_levels, int_levels, adapter_params
from .nf4 import (
    BLOCK,
    GROUP,
    QMAX,
    block_absmax,
    encode,
    pack_codes,
    unpack_codes,
    double_quantize,
    quantize,
    dequantize,
    storage_bits_per_weight,
    LAB_GROUP,
    quantize_groups,
    dequantize_groups,
    group_storage_bits_per_weight,
)
from .linear import (
    forward,
    backward,
    backward_via_dense_dw,
    forward_lora,
    backward_lora,
    lora_factor,
    merge,
    residual,
    loftq_init,
)
from .optim import adam_step

__all__ = [
    "nf4_levels",
    "uniform4_levels",
    "int_levels",
    "adapter_params",
    "BLOCK",
    "GROUP",
    "QMAX",
    "block_absmax",
    "encode",
    "pack_codes",
    "unpack_codes",
    "double_quantize",
    "quantize",
    "dequantize",
    "storage_bits_per_weight",
    "LAB_GROUP",
    "quantize_groups",
    "dequantize_groups",
    "group_storage_bits_per_weight",
    "forward",
    "backward",
    "merge",
    "residual",
    "loftq_init",
    "adam_step",
    "backward_via_dense_dw",
    "forward_lora",
    "backward_lora",
    "lora_factor",
]
