"""Per-expert views for the oracle on large shapes (tests only).

The oracle quantizes and dequantizes only the experts (and down rows) a
test's sampled tokens need, from the same bf16 bytes the GPU received.
"""

import numpy as np

from moeq_synth import bf16_bits
from oracle.dq import dq_compress, nf4_dq_dequantize
from oracle.int8 import int8_dequantize_rowwise, int8_quantize_rowwise
from oracle.nf4 import nf4_dequantize, nf4_quantize


def oracle_roundtrip(bits, fmt):
    """bf16 bits [E, R, C] -> the oracle's dequantized bf16 bits [E, R, C]."""
    if fmt == "nf4":
        return nf4_dequantize(*nf4_quantize(bits))
    if fmt == "nf4_dq":
        q, absmax = nf4_quantize(bits)
        return nf4_dq_dequantize(q, *dq_compress(absmax))
    return int8_dequantize_rowwise(*int8_quantize_rowwise(bits))


class LazyDequant:
    """``obj[e]`` -> oracle-dequantized bf16 bits of expert e (optionally some rows only)."""

    def __init__(self, w, fmt, rows=None):
        self.w, self.fmt, self.rows = w, fmt, rows
        self.cache = {}

    def __len__(self):
        return int(self.w.shape[0])

    def __getitem__(self, e):
        e = int(e)
        if e not in self.cache:
            we = self.w[e]
            if self.rows is not None and self.fmt == "nf4_dq":
                # absmax groups span rows: quantize the whole expert, then pick
                bits = bf16_bits(we).reshape(1, *we.shape)
                self.cache[e] = oracle_roundtrip(bits, self.fmt)[0][self.rows.cpu().numpy()]
                return self.cache[e]
            if self.rows is not None:
                we = we[self.rows]
            bits = bf16_bits(we).reshape(1, *we.shape)
            self.cache[e] = oracle_roundtrip(bits, self.fmt)[0]
        return self.cache[e]
