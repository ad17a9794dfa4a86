"""Blockwise NF4 quantization with double-quantized scales (oracle).

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.

Steps, in the order the pages give them:

1. Blocks.  The frozen weight W0 is stored (in, out) row-major ("QLoRA
   (low-rank adapters on a quantized model)", "How it works") and flattened;
   a block is 64 consecutive entries ("What QLoRA adds": each block of 64
   weights has its own absmax scale; "LLMs · QLoRA", code listing: reshape
   to rows of 64).
2. Absmax per block, c_b = max |w| (same listing), exact in fp32.
3. Encode: x = w / c_b in IEEE fp32, then the index of the nearest level,
   argmin_i fp32(|x - L_i|) (same listing).  Ties go to the lower index,
   which is what an argmin returning the first minimum does.  A block whose
   absmax is 0 encodes every entry as if x = 0.
4. Pack two 4-bit codes per byte: flat element 2j in the low nibble, 2j+1 in
   the high nibble (the pages only say "4 bits"; this order is our reading).
5. Double quantization ("What QLoRA adds": the per-block scales are quantized
   again, to 8 bits).  Reading: symmetric int8 with q_max = 127 and one fp32
   scale per 256 consecutive block scales; s2_g = fp32(max_b c_b) / 127 in
   fp32, q_b = round-half-even(fp32(c_b / s2_g)) clamped to [-127, 127].  The
   codes in step 3 use the exact c_b, not the double-quantized one.
6. Dequantize: w_hat = L[code] * (q_b * s2_g), evaluated in float64.
"""

import numpy as np

from .levels import nf4_levels

BLOCK = 64          # weights per absmax block
GROUP = 256         # block scales per double-quantization group
QMAX = 127          # symmetric int8 range for the block scales

_CHUNK = 1 << 18    # weights encoded per numpy pass (bounds the n x 16 temporary)


def block_absmax(w_flat):
    """c_b = max |w| over each block of 64 consecutive weights (fp32, exact)."""
    w = np.asarray(w_flat, dtype=np.float32).reshape(-1, BLOCK)
    return np.abs(w).max(axis=1)


def encode(w_flat, c, levels=None, block=BLOCK):
    """4-bit codes: argmin_i fp32(|fp32(w / c_b) - L_i|), first minimum wins.

    ``w_flat`` fp32 [n], ``c`` fp32 [n/block] (one scale per ``block``
    consecutive weights); returns uint8 [n] in 0..15.
    A table in sign-magnitude order (the integer grids) holds zero twice,
    -0 then +0, one value: there the tie goes by the sign of x (x > 0 takes
    +0), so that the codes rise with x.  The NF4 and uniform tables have no
    zero entry.
    """
    L = nf4_levels() if levels is None else np.asarray(levels, np.float32)
    w = np.asarray(w_flat, dtype=np.float32).reshape(-1, block)
    c = np.asarray(c, dtype=np.float32).reshape(-1, 1)
    out = np.empty(w.shape, dtype=np.uint8)
    rows_per_chunk = max(1, _CHUNK // block)
    for r0 in range(0, w.shape[0], rows_per_chunk):
        wb = w[r0:r0 + rows_per_chunk]
        cb = c[r0:r0 + rows_per_chunk]
        safe = np.where(cb == 0, np.float32(1), cb)
        x = (wb / safe).astype(np.float32)           # IEEE fp32 division
        x = np.where(cb == 0, np.float32(0), x)       # zero block -> x = 0
        d = np.abs(x[..., None] - L)                  # fp32 distances
        idx = np.argmin(d, axis=-1)
        nxt = np.minimum(idx + 1, L.size - 1)
        zero_pair = ((L[idx] == 0) & np.signbit(L[idx]) & (L[nxt] == 0) & ~np.signbit(L[nxt])
                     & (nxt == idx + 1))
        out[r0:r0 + rows_per_chunk] = np.where(zero_pair & (x > 0), nxt, idx)
    return out.reshape(-1)


def pack_codes(codes):
    """byte j = code[2j] | code[2j+1] << 4."""
    codes = np.asarray(codes, dtype=np.uint8).reshape(-1, 2)
    return (codes[:, 0] | (codes[:, 1] << 4)).astype(np.uint8)


def unpack_codes(packed):
    """Inverse of :func:`pack_codes`."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.size * 2, dtype=np.uint8)
    out[0::2] = packed & 0x0F
    out[1::2] = packed >> 4
    return out


def double_quantize(c):
    """Block scales -> (q8 int8 [nb], s2 fp32 [ceil(nb/256)])."""
    c = np.asarray(c, dtype=np.float32)
    nb = c.size
    ng = (nb + GROUP - 1) // GROUP
    q8 = np.zeros(nb, dtype=np.int8)
    s2 = np.zeros(ng, dtype=np.float32)
    for g in range(ng):
        cg = c[g * GROUP:(g + 1) * GROUP]
        s = np.float32(cg.max()) / np.float32(QMAX)   # fp32 division
        s2[g] = s
        if s == 0:
            continue                                   # all-zero group: q = 0
        q = np.rint((cg / s).astype(np.float32))       # half to even
        q8[g * GROUP:(g + 1) * GROUP] = np.clip(q, -QMAX, QMAX).astype(np.int8)
    return q8, s2


def quantize(w0, levels=None):
    """Full quantize pass of an (in, out) fp32 matrix.

    Returns a dict with ``codes`` (uint8 [n]), ``packed`` (uint8 [n/2]),
    ``absmax`` (fp32 [n/64]), ``q8`` (int8 [n/64]) and ``s2`` (fp32 [n/16384]).
    Requires n % 64 == 0 (every shape here has out % 64 == 0).
    """
    w = np.ascontiguousarray(w0, dtype=np.float32).reshape(-1)
    if w.size % BLOCK:
        raise ValueError("number of weights must be a multiple of 64")
    c = block_absmax(w)
    codes = encode(w, c, levels)
    q8, s2 = double_quantize(c)
    return {"codes": codes, "packed": pack_codes(codes), "absmax": c,
            "q8": q8, "s2": s2}


def dequantize(packed, q8, s2, n_in, n_out, levels=None):
    """w_hat[k, n] = L[code] * q_b * s2_g in float64, shape (in, out)."""
    L = (nf4_levels() if levels is None else np.asarray(levels, np.float32))
    L = L.astype(np.float64)
    codes = unpack_codes(packed)
    q = np.asarray(q8, dtype=np.int8).astype(np.float64)
    s = np.asarray(s2, dtype=np.float32).astype(np.float64)
    scale_block = q * np.repeat(s, GROUP)[:q.size]
    w = L[codes].reshape(-1, BLOCK) * scale_block[:, None]
    return w.reshape(n_in, n_out)


# --------------------------------------------------------------------------
# The lab's quantizer ("QLoRA (low-rank adapters on a quantized model)", "The
# code, line by line" and its Simplifications paragraph): symmetric uniform
# integers with one scale per 16 consecutive entries of the flattened
# (in, out) matrix, and no double quantization.  Reading: the scale of a
# group is its absmax c_g (fp32, exact), the level set is k/h for |k| <= h
# (h = 7, 3, 1 for 4, 3 and 2 bits; "2-bit" is ternary), and a weight's
# code is the nearest level of fp32(w / c_g) with the rule of ``encode``;
# the dequantized weight is L[code] * c_g.  Any 16-entry level table works
# the same way.

LAB_GROUP = 16


def quantize_groups(w0, levels, group=LAB_GROUP):
    """Per-group quantize of an (in, out) fp32 matrix: returns ``codes``
    (uint8 [n]), ``packed`` (uint8 [n/2]) and ``scales`` (fp32 [n/group],
    group g = flat entries group*g .. group*g + group - 1)."""
    w = np.ascontiguousarray(w0, dtype=np.float32).reshape(-1)
    if w.size % group:
        raise ValueError("number of weights must be a multiple of the group size")
    c = np.abs(w.reshape(-1, group)).max(axis=1)
    codes = encode(w, c, levels, block=group)
    return {"codes": codes, "packed": pack_codes(codes), "scales": c}


def dequantize_groups(packed, scales, n_in, n_out, levels, group=LAB_GROUP):
    """w_hat = L[code] * c_g in float64, shape (in, out)."""
    L = np.asarray(levels, np.float32).astype(np.float64)
    codes = unpack_codes(packed)
    c = np.asarray(scales, dtype=np.float32).astype(np.float64)
    return (L[codes].reshape(-1, group) * c[:, None]).reshape(n_in, n_out)


def group_storage_bits_per_weight(group=LAB_GROUP):
    """4-bit code + one fp32 scale per group."""
    return 4.0 + 32.0 / group


def storage_bits_per_weight():
    """4-bit code + int8 per 64 weights + fp32 per 64*256 weights."""
    return 4.0 + 8.0 / BLOCK + 32.0 / (BLOCK * GROUP)
