"""Pins for oracle.bf16: library conversion (torch) and exact rational rounding."""

import numpy as np
import torch

from oracle.bf16 import bf16_to_f32, f32_to_bf16
from tests.exact import bf16_from_frac_rne


def _torch_bf16_bits(x):
    t = torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_widen_is_exact_over_all_finite_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = bf16_to_f32(bits)
    finite = np.isfinite(f)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(f[finite].view(np.uint32), ref[finite].view(np.uint32))
    # narrowing a widened value gives the pattern back
    assert np.array_equal(f32_to_bf16(f[finite]), bits[finite])


def test_narrow_matches_torch_rne():
    rng = np.random.default_rng(11)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * 0.02,
        rng.standard_normal(200000).astype(np.float32) * 1e4,
        (rng.integers(0, 2**31, 200000, dtype=np.uint64).astype(np.uint32)).view(np.float32),
    ])
    x = x[np.isfinite(x)]
    assert np.array_equal(f32_to_bf16(x), _torch_bf16_bits(x))


def test_narrow_ties_go_to_even():
    # lower 16 bits exactly 0x8000: even upper stays, odd upper rounds up
    even = np.array([0x3F808000], dtype=np.uint32).view(np.float32)    # upper 0x3F80 (even)
    odd = np.array([0x3F818000], dtype=np.uint32).view(np.float32)     # upper 0x3F81 (odd)
    assert f32_to_bf16(even)[0] == 0x3F80
    assert f32_to_bf16(odd)[0] == 0x3F82
    neg = np.array([0xBF818000], dtype=np.uint32).view(np.float32)
    assert f32_to_bf16(neg)[0] == 0xBF82


def test_narrow_matches_exact_rational_rounding():
    rng = np.random.default_rng(12)
    x = rng.standard_normal(3000).astype(np.float32)
    got = f32_to_bf16(x)
    for xi, gi in zip(x, got):
        assert bf16_from_frac_rne(xi) == int(gi)
