"""Blockwise NF4 quantization of fused expert tensors (test infrastructure only).

What the pages fix:

* "MoE Expert Quantization" (Axolotl docs), *Implementation details*: in
  4-bit mode each 3-D+ expert tensor is quantized on load with the NF4
  format of bitsandbytes.
* bitsandbytes issue #1849, maintainer comment thread: the packed codes are
  a plain tensor; the per-block absmax is kept beside it as
  ``[num_experts, blocks_per_expert]``; the blocksize is 64 and
  ``in_features`` must be divisible by it, so that blocks never straddle an
  expert (or a row); no double quantization of the absmax.
* bitsandbytes issue #1849, *Description*: ``gate_up_proj [E, 2I, H]`` and
  ``down_proj [E, H, I]``; each ``[e]`` slice is an ``[out, in]`` weight, so a
  64-block runs along the last (in_features) axis.

What the pages leave open, and the reading taken here:

* The 16 NF4 levels are not printed.  They are built as in the QLoRA paper's
  4-bit NormalFloat: standard-normal quantiles at evenly spaced
  probabilities, asymmetric so that zero is a level (8 positive, 7 negative,
  one zero), normalised so the extremes are exactly -1 and +1.  The outermost
  probability is ``delta = ((1 - 1/30) + (1 - 1/32)) / 2``; the levels are
  formed in fp64 and rounded once to fp32.
* ``n = w / absmax`` is an IEEE fp32 division (round to nearest even).
* The code is the index of the level nearest to ``n``; an exact tie goes to
  the lower index.  Distances are taken in fp64, where they are exact for
  these operands.  (With bf16 weights no ratio ``fp32(w/absmax)`` lands
  exactly on a midpoint between two levels, so the tie rule only matters for
  the scalar decision :func:`nf4_code_of_ratio`.)
* An all-zero block stores absmax 0 and every code 7 (the zero level).
* Two codes share a byte with the even column in the high nibble.
* Dequantization is ``bf16_RNE(fp32(level[code] * absmax))``: the fp32
  product first, then round to bf16.
"""

import math

import numpy as np
from scipy.stats import norm

from .bf16 import bf16_to_f32, f32_to_bf16

BLOCKSIZE = 64
ZERO_CODE = 7


def nf4_levels_f64():
    """The 16 NormalFloat levels in fp64, ascending, extremes exactly -1 and +1."""
    delta = 0.5 * ((1.0 - 1.0 / 30.0) + (1.0 - 1.0 / 32.0))
    # 8 positive levels: quantiles at 8 evenly spaced probabilities from delta
    # down to (but excluding) 1/2.
    p_pos = np.linspace(delta, 0.5, 9)[:-1]
    # 7 negative levels: mirror of 7 evenly spaced probabilities.
    p_neg = np.linspace(delta, 0.5, 8)[:-1]
    positive = norm.ppf(p_pos)
    negative = -norm.ppf(p_neg)
    levels = np.sort(np.concatenate([positive, [0.0], negative]))
    return levels / np.max(np.abs(levels))


def nf4_codebook():
    """The NF4 codebook as fp32 (levels rounded once from fp64)."""
    return nf4_levels_f64().astype(np.float32)


def _check_shape(shape):
    if len(shape) != 3:
        raise ValueError("expert tensor must be 3-D [E, rows, cols]")
    if shape[2] % BLOCKSIZE != 0:
        raise ValueError("cols (in_features) must be divisible by the blocksize 64")


def nf4_quantize(w_bits):
    """Quantize bf16 expert weights ``[E, R, C]`` (uint16 patterns) to NF4.

    Returns ``(qdata uint8 [E, R, C/2], absmax float32 [E, R*C/64])``.
    """
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    _check_shape(w_bits.shape)
    E, R, C = w_bits.shape
    # Blocks are independent; rows are processed a slab at a time only to
    # bound the memory of the [.., 64, 16] distance array.
    slab = max(1, (1 << 22) // (C * 16))
    if E * R > slab:
        flat = w_bits.reshape(E * R, 1, C)
        parts = [nf4_quantize(flat[i:i + slab].reshape(1, -1, C)) for i in range(0, E * R, slab)]
        qdata = np.concatenate([p[0].reshape(-1, C // 2) for p in parts]).reshape(E, R, C // 2)
        absmax = np.concatenate([p[1].reshape(-1) for p in parts]).reshape(E, R * (C // BLOCKSIZE))
        return qdata, absmax
    nb = C // BLOCKSIZE
    w = bf16_to_f32(w_bits).reshape(E, R, nb, BLOCKSIZE)

    # absmax of each 64-block (exact in fp32: it is one of the inputs)
    absmax = np.max(np.abs(w), axis=-1)

    # normalise: IEEE fp32 division; an all-zero block is handled below
    safe = np.where(absmax == 0, np.float32(1), absmax).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        n = (w / safe[..., None]).astype(np.float32)

    # nearest level, distances in fp64, ties -> lower index (argmin keeps the first)
    levels = nf4_codebook().astype(np.float64)
    dist = np.abs(n.astype(np.float64)[..., None] - levels)
    codes = np.argmin(dist, axis=-1).astype(np.uint8)
    codes[absmax == 0] = ZERO_CODE

    # two codes per byte, even column in the high nibble
    codes = codes.reshape(E, R, C)
    qdata = (codes[..., 0::2] << 4) | codes[..., 1::2]
    return qdata.astype(np.uint8), absmax.reshape(E, R * nb).astype(np.float32)


def nf4_unpack(qdata):
    """uint8 [E, R, C/2] -> codes uint8 [E, R, C] (even column from the high nibble)."""
    q = np.asarray(qdata, dtype=np.uint8)
    codes = np.empty(q.shape[:-1] + (q.shape[-1] * 2,), dtype=np.uint8)
    codes[..., 0::2] = q >> 4
    codes[..., 1::2] = q & 0x0F
    return codes


def nf4_dequantize(qdata, absmax):
    """NF4 -> bf16 (uint16 patterns) ``[E, R, C]``: bf16_RNE(fp32(level * absmax))."""
    codes = nf4_unpack(qdata)
    E, R, C = codes.shape
    nb = C // BLOCKSIZE
    a = np.asarray(absmax, dtype=np.float32).reshape(E, R, nb, 1)
    levels = nf4_codebook()
    vals = levels[codes].reshape(E, R, nb, BLOCKSIZE)
    prod = (vals * a).astype(np.float32)          # fp32 product, round to nearest
    return f32_to_bf16(prod).reshape(E, R, C)


def nf4_packed_nbytes(E, R, C):
    """Bytes of packed codes for one ``[E, R, C]`` tensor (absmax excluded)."""
    _check_shape((E, R, C))
    return E * R * C // 2


def nf4_absmax_nbytes(E, R, C):
    """Bytes of fp32 absmax for one ``[E, R, C]`` tensor."""
    _check_shape((E, R, C))
    return E * R * (C // BLOCKSIZE) * 4


def nf4_code_of_ratio(n):
    """Reference decision for one fp32 ratio: nearest level, ties to the lower index.

    Pure-Python version of the vectorised decision in :func:`nf4_quantize`,
    for hand-checked cases.
    """
    levels = [float(x) for x in nf4_codebook()]
    n = float(np.float32(n))
    best, best_d = 0, math.inf
    for i, c in enumerate(levels):
        d = abs(n - c)
        if d < best_d:
            best, best_d = i, d
    return best
