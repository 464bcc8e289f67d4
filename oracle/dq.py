"""Double quantization of the NF4 block statistics (test infrastructure only).

What the pages fix: the 4-bit loading config of bitsandbytes issue #1849
(*Reproduction*, Qwen3-30B-A3B) switches double quantization on, and in the
maintainer thread the per-expert ``compress_statistics`` (the absmax itself
quantized) is the part deferred from the first version.  The pages name the
idea and print no format for it.

Readings taken here (the plainest 8-bit blockwise form of "the absmax
quantized"; bitsandbytes' own format is not on the pages and is not
reproduced):

* Each expert's absmax vector ``[blocks_per_expert]`` (blocks in row order,
  as stored for NF4) is cut into groups of ``GROUP = 256`` consecutive
  blocks; the last group of an expert may be shorter.  Groups never cross an
  expert, so one expert's slice still stands alone.
* Per group with largest absmax ``m``: the group scale is
  ``s2 = fp32(m / 255)`` (IEEE division) and each absmax ``a`` becomes the
  8-bit code ``c = round_half_even(fp32(fp32(255 a) / m))`` in [0, 255]
  (absmax is never negative).  This is the row-wise int8 rule of the same
  library with 255 in place of 127, unsigned.  A group of zeros stores
  ``s2 = 0`` and codes 0.
* The absmax the weights are decoded with is ``a' = fp32(c * s2)``; the NF4
  codes are unchanged and dequantize as ``bf16_rne(fp32(level * a'))``.
* Storage per expert: codes ``uint8 [E, blocks_per_expert]`` and group
  scales ``fp32 [E, ceil(blocks_per_expert / 256)]``.
"""

import numpy as np

from .nf4 import nf4_dequantize

GROUP = 256
LEVELS = 255


def groups_per_expert(nblocks):
    """Number of absmax groups of one expert with ``nblocks`` NF4 blocks."""
    return (nblocks + GROUP - 1) // GROUP


def dq_compress(absmax):
    """fp32 absmax ``[E, nb]`` -> ``(codes uint8 [E, nb], scale2 fp32 [E, ng])``."""
    a = np.asarray(absmax, dtype=np.float32)
    if a.ndim != 2:
        raise ValueError("absmax must be [E, blocks_per_expert]")
    if np.any(a < 0) or not np.all(np.isfinite(a)):
        raise ValueError("absmax must be finite and non-negative")
    E, nb = a.shape
    ng = groups_per_expert(nb)
    codes = np.zeros((E, nb), dtype=np.uint8)
    scale2 = np.zeros((E, ng), dtype=np.float32)
    for e in range(E):
        for g in range(ng):
            part = a[e, GROUP * g:GROUP * (g + 1)]
            m = part.max()
            if m == 0:
                continue                                       # codes 0, scale 0
            scale2[e, g] = np.float32(m) / np.float32(LEVELS)  # IEEE fp32 division
            x = (part * np.float32(LEVELS)).astype(np.float32)
            ratio = (x / m).astype(np.float32)                 # IEEE fp32 division
            codes[e, GROUP * g:GROUP * (g + 1)] = np.rint(ratio).astype(np.uint8)
    return codes, scale2


def dq_decompress(codes, scale2):
    """``(codes [E, nb], scale2 [E, ng])`` -> fp32 absmax' ``[E, nb]`` = fp32(c * s2)."""
    c = np.asarray(codes, dtype=np.uint8)
    s2 = np.asarray(scale2, dtype=np.float32)
    E, nb = c.shape
    if s2.shape != (E, groups_per_expert(nb)):
        raise ValueError("scale2 must be [E, ceil(blocks_per_expert / 256)]")
    per_block = np.repeat(s2, GROUP, axis=1)[:, :nb]
    return (c.astype(np.float32) * per_block).astype(np.float32)


def nf4_dq_dequantize(qdata, codes, scale2):
    """Packed NF4 codes ``[E, R, C/2]`` with double-quantized absmax -> bf16 ``[E, R, C]``."""
    return nf4_dequantize(qdata, dq_decompress(codes, scale2))
