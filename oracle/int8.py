"""Row-wise int8 quantization of fused expert tensors (test infrastructure only).

What the pages fix: "MoE Expert Quantization" (Axolotl docs), *Implementation
details*: in 8-bit mode each 3-D+ expert tensor is quantized on load with a
row-wise int8 parametrization and dequantized back for the forward.  A row is
one ``[e][r]`` slice along in_features (the ``[out, in]`` orientation of
bitsandbytes issue #1849's *Description* code).

What the pages leave open, and the reading taken here:

* ``absmax`` is the largest |w| of the row; the stored scale is
  ``fp32(absmax / 127)`` (IEEE division).
* ``q = round_half_even(fp32(fp32(127 * w) / absmax))``: the code comes from
  ``127 * w / absmax`` (``127 * w`` is exact in fp32 for bf16 w), not from
  ``w / scale``.  The range is [-127, 127]; -128 is never produced.
* A zero row stores scale 0 and all codes 0.
* Dequantization is ``bf16_RNE(fp32(q * scale))``.
"""

import numpy as np

from .bf16 import bf16_to_f32, f32_to_bf16


def int8_quantize_rowwise(w_bits):
    """bf16 ``[E, R, C]`` (uint16 patterns) -> ``(q int8 [E, R, C], scale float32 [E, R])``."""
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    if w_bits.ndim != 3:
        raise ValueError("expert tensor must be 3-D [E, rows, cols]")
    w = bf16_to_f32(w_bits)
    absmax = np.max(np.abs(w), axis=-1)                       # [E, R], exact
    scale = (absmax / np.float32(127)).astype(np.float32)     # IEEE fp32 division

    safe = np.where(absmax == 0, np.float32(1), absmax).astype(np.float32)
    x = (w * np.float32(127)).astype(np.float32)              # exact
    ratio = (x / safe[..., None]).astype(np.float32)          # IEEE fp32 division
    q = np.rint(ratio)                                        # round half to even
    q[absmax == 0] = 0
    return q.astype(np.int8), scale


def int8_dequantize_rowwise(q, scale):
    """int8 ``[E, R, C]`` + scale ``[E, R]`` -> bf16 patterns: bf16_RNE(fp32(q * scale))."""
    q = np.asarray(q, dtype=np.int8)
    s = np.asarray(scale, dtype=np.float32)[..., None]
    prod = (q.astype(np.float32) * s).astype(np.float32)
    return f32_to_bf16(prod)
