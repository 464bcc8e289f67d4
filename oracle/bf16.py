"""bf16 <-> fp32 conversions used by the oracle (test infrastructure only).

bf16 is the upper half of an IEEE binary32.  Widening is exact: shift the 16
bits into the high half.  Narrowing rounds the fp32 value to the nearest bf16,
ties to even (round-to-nearest-even on the dropped 16 bits).  NaN inputs are
outside the scope of the method (finite weights and activations only).

The pages fix bf16 as the dtype of the unquantized expert weights
("MoE Expert Quantization", intro: experts load "in full bf16 precision") and
of the dequantized weights the forward consumes.
"""

import numpy as np


def bf16_to_f32(bits):
    """uint16 bf16 patterns -> float32 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16(x):
    """float32 values -> uint16 bf16 patterns, round to nearest, ties to even.

    Written as the definition: keep the upper 16 bits and round on the lower
    16 by comparing them with the halfway value 0x8000; on an exact tie round
    so that the kept part is even.
    """
    u = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32).astype(np.uint64)
    upper = u >> np.uint64(16)
    lower = u & np.uint64(0xFFFF)
    round_up = (lower > 0x8000) | ((lower == 0x8000) & ((upper & np.uint64(1)) == 1))
    out = upper + round_up.astype(np.uint64)
    return out.astype(np.uint16)


def f64_to_bf16_via_f32(x):
    """float64 -> fp32 (RN) -> bf16 (RNE): the two-step rounding the forward output uses."""
    return f32_to_bf16(np.asarray(x, dtype=np.float64).astype(np.float32))
