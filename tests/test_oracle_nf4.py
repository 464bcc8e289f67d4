"""Pins for oracle.nf4: codebook construction, decision, packing, dequantize.

Each check is tied to something other than the oracle itself: the inverse
normal CDF, exact rational arithmetic, exhaustive enumeration over bf16
ratios, hand-worked blocks and the byte count printed on the pages.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
from scipy.stats import norm

from oracle.bf16 import bf16_to_f32, f32_to_bf16
from oracle.nf4 import (BLOCKSIZE, nf4_codebook, nf4_code_of_ratio, nf4_dequantize,
                        nf4_packed_nbytes, nf4_quantize, nf4_unpack)
from tests.exact import bf16_from_frac_rne, frac, rn32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
DELTA = 0.5 * ((1 - 1 / 30) + (1 - 1 / 32))


def _bits(x):
    return f32_to_bf16(np.asarray(x, dtype=np.float32))


# ---------------------------------------------------------------- codebook

def test_codebook_structure():
    c = nf4_codebook()
    assert c.dtype == np.float32 and c.shape == (16,)
    assert np.all(np.diff(c) > 0)
    assert c[0] == -1.0 and c[15] == 1.0
    assert c[7] == 0.0 and not np.signbit(c[7])
    assert np.sum(c < 0) == 7 and np.sum(c > 0) == 8


def test_codebook_levels_sit_at_evenly_spaced_normal_probabilities():
    # Inverse check through the CDF: the positive levels scaled by the largest
    # quantile land at probabilities delta, delta - s, ..., 8 of them, step
    # s = (delta - 1/2)/8; the negative ones mirror 7 probabilities, step /7.
    c = nf4_codebook().astype(np.float64)
    M = norm.ppf(DELTA)
    for j in range(8):
        p = norm.cdf(c[15 - j] * M)
        assert abs(p - (DELTA - j * (DELTA - 0.5) / 8)) < 1e-7
    for j in range(7):
        p = norm.cdf(-c[j] * M)
        assert abs(p - (DELTA - j * (DELTA - 0.5) / 7)) < 1e-7


# ---------------------------------------------------------------- decision

def _exact_code(n32):
    """argmin over levels of |n - c_i| in exact rationals, ties to the lower index."""
    q = frac(n32)
    levels = [frac(x) for x in nf4_codebook()]
    d = [abs(q - c) for c in levels]
    return d.index(min(d))


def _exact_thresholds():
    """t_i = largest fp32 <= (c_i + c_{i+1})/2, from exact rationals."""
    c = [frac(x) for x in nf4_codebook()]
    out = []
    for i in range(15):
        mid = (c[i] + c[i + 1]) / 2
        t = np.float32(float(mid))
        while frac(t) > mid:
            t = np.nextafter(t, np.float32(-np.inf))
        while frac(np.nextafter(t, np.float32(np.inf))) <= mid:
            t = np.nextafter(t, np.float32(np.inf))
        out.append(np.float32(t))
    return np.array(out, dtype=np.float32)


def test_decision_matches_exact_argmin_on_random_pairs():
    rng = np.random.default_rng(3)
    w = rng.standard_normal((40, 64)).astype(np.float32) * 0.02
    bits = _bits(w).reshape(1, 40, 64)
    q, a = nf4_quantize(bits)
    codes = nf4_unpack(q).reshape(40, 64)
    wf = bf16_to_f32(bits).reshape(40, 64)
    for r in range(40):
        amax = max(abs(frac(x)) for x in wf[r])
        assert frac(a[0, r]) == amax
        for j in range(64):
            n = rn32(frac(wf[r, j]) / amax)           # exact RN32 of the quotient
            assert codes[r, j] == _exact_code(n)


def test_decision_around_every_midpoint_and_ties_to_lower():
    t = _exact_thresholds()
    c = [frac(x) for x in nf4_codebook()]
    ties = 0
    for i in range(15):
        mid = (c[i] + c[i + 1]) / 2
        n = t[i]
        for _ in range(40):                          # walk down from the threshold
            n = np.nextafter(n, np.float32(-np.inf))
        for _ in range(81):
            expect = i + 1 if frac(n) > mid else i   # exact tie (== mid) -> lower index
            ties += frac(n) == mid
            assert nf4_code_of_ratio(n) == expect, (i, n)
            n = np.nextafter(n, np.float32(np.inf))
    assert ties >= 3                                 # several midpoints are fp32 values


def test_decision_vectorised_equals_scalar_on_dense_grid():
    rng = np.random.default_rng(4)
    n = np.concatenate([rng.uniform(-1, 1, 3000), np.linspace(-1, 1, 2001)]).astype(np.float32)
    # embed each ratio as w with absmax 1: block [1, n, n, ...]
    n = n[: (len(n) // 63) * 63].reshape(-1, 63)
    blocks = np.concatenate([np.ones((n.shape[0], 1), np.float32), n], axis=1)
    w = bf16_to_f32(_bits(blocks))                   # the ratios actually quantized
    q, _ = nf4_quantize(_bits(blocks).reshape(1, -1, 64))
    codes = nf4_unpack(q).reshape(-1, 64)
    for r in range(0, w.shape[0], 7):
        for j in range(64):
            assert codes[r, j] == nf4_code_of_ratio(w[r, j])


def test_exhaustive_over_all_bf16_ratios():
    """Every (w, absmax) bf16 pair with absmax in [1, 2) and |w| <= absmax.

    The code depends on w/absmax only, and every bf16 ratio occurs with an
    absmax in [1, 2), so this covers the whole decision.  Expected codes come
    from exact fp64 products: RN32(w/a) > t_i exactly when w > a * mu_i, where
    mu_i is the midpoint between t_i and the next fp32 (a 25-bit value, so
    a*mu_i is exact in fp64 and no bf16 ratio equals it).
    """
    t = _exact_thresholds().astype(np.float64)
    up = np.nextafter(_exact_thresholds(), np.float32(np.inf)).astype(np.float64)
    mu = (t + up) / 2
    allw = bf16_to_f32(np.arange(65536, dtype=np.uint32).astype(np.uint16))
    allw = allw[np.isfinite(allw)]
    blocks, expect = [], []
    for A in range(128, 256):
        a = np.float32(bf16_to_f32(np.array([0x3F00 + A], dtype=np.uint16))[0])
        assert 1.0 <= a < 2.0
        w = allw[np.abs(allw) <= a]
        pad = (-len(w)) % 63
        w = np.concatenate([w, np.zeros(pad, np.float32)]).reshape(-1, 63)
        blk = np.concatenate([np.full((w.shape[0], 1), a, np.float32), w], axis=1)
        blocks.append(blk)
        e = (blk.astype(np.float64)[..., None] > np.float64(a) * mu).sum(-1)
        expect.append(e)
    blocks = np.concatenate(blocks)
    expect = np.concatenate(expect)
    q, absmax = nf4_quantize(_bits(blocks).reshape(1, -1, 64))
    assert np.array_equal(absmax.reshape(-1), blocks[:, 0])
    codes = nf4_unpack(q).reshape(-1, 64)
    assert np.array_equal(codes, expect)


# ---------------------------------------------------------------- packing & edge blocks

def test_hand_worked_block_packing():
    # absmax 1.0; w = [1, 0, -1, 0.5, 0.25, -0.25, 0...]:
    #   1 -> level 15; 0 -> level 7; -1 -> level 0;
    #   0.5: |0.5-0.4407|=0.0593 < |0.5626-0.5|=0.0626 -> level 12;
    #   0.25: nearest is 0.2461 (level 10); -0.25: nearest is -0.2844 (level 4)
    #   since |-0.25+0.2844|=0.0344 < |-0.25+0.1848|=0.0652.
    # Bytes, even column in the high nibble: F7 0C A4 then 77 x 29.
    w = np.zeros(64, np.float32)
    w[:6] = [1.0, 0.0, -1.0, 0.5, 0.25, -0.25]
    q, a = nf4_quantize(_bits(w).reshape(1, 1, 64))
    assert a.shape == (1, 1) and a[0, 0] == 1.0
    assert list(q.reshape(-1)[:3]) == [0xF7, 0x0C, 0xA4]
    assert np.all(q.reshape(-1)[3:] == 0x77)


def test_zero_block_and_negative_zero():
    w = np.zeros((1, 2, 128), np.float32)
    w[0, 1, 64:] = 0.5
    w[0, 1, 65] = -0.0
    q, a = nf4_quantize(_bits(w))
    assert a.tolist() == [[0.0, 0.0, 0.0, 0.5]]
    assert np.all(q[0, 0] == 0x77)                   # zero blocks: code 7 everywhere
    assert np.all(q[0, 1, :32] == 0x77)
    assert q[0, 1, 32] == 0xF7                        # [0.5 -> 15, -0.0 -> 7]
    d = nf4_dequantize(q, a)
    assert d[0, 1, 65] == 0x0000                      # -0 dequantizes to +0


def test_absmax_layout_is_block_major_in_row_order():
    rng = np.random.default_rng(5)
    w = rng.standard_normal((3, 5, 192)).astype(np.float32)
    bits = _bits(w)
    _, a = nf4_quantize(bits)
    wf = bf16_to_f32(bits)
    assert a.shape == (3, 5 * 3)
    for e in range(3):
        for r in range(5):
            for b in range(3):
                assert a[e, r * 3 + b] == max(abs(float(x)) for x in wf[e, r, 64 * b:64 * b + 64])


def test_blocksize_rule():
    with pytest.raises(ValueError):
        nf4_quantize(np.zeros((1, 2, 96), np.uint16))
    with pytest.raises(ValueError):
        nf4_quantize(np.zeros((2, 64), np.uint16))


# ---------------------------------------------------------------- dequantize

def test_dequantize_matches_exact_two_step_rounding():
    rng = np.random.default_rng(6)
    bits = _bits(rng.standard_normal((2, 3, 128)).astype(np.float32) * 0.02)
    q, a = nf4_quantize(bits)
    d = nf4_dequantize(q, a)
    codes = nf4_unpack(q)
    c = nf4_codebook()
    for e in range(2):
        for r in range(3):
            for j in range(128):
                s = a[e, r * 2 + j // 64]
                p = rn32(frac(c[codes[e, r, j]]) * frac(s))
                assert d[e, r, j] == bf16_from_frac_rne(p)


def test_constant_blocks_reconstruct_exactly():
    for v in [0.02, -0.0137, 1.5, -3.0e-5]:
        w = np.full((1, 1, 64), v, np.float32)
        bits = _bits(w)
        q, a = nf4_quantize(bits)
        assert np.all(q == (0xFF if v > 0 else 0x00))
        assert np.array_equal(nf4_dequantize(q, a), bits)


def test_round_trip_is_idempotent():
    rng = np.random.default_rng(7)
    w = rng.standard_normal((4, 16, 256)).astype(np.float32) * 0.02
    w[0, 0, 5] = 0.4                                  # an outlier block
    q, a = nf4_quantize(_bits(w))
    q2, a2 = nf4_quantize(nf4_dequantize(q, a))
    assert np.array_equal(q, q2) and np.array_equal(a, a2)


# ---------------------------------------------------------------- byte count from the pages

def test_packed_bytes_match_the_pages_olmoe_figure():
    with open(os.path.join(GOLDEN, "olmoe_nf4_expert_bytes.json")) as f:
        g = json.load(f)
    E, H, I, L = g["E"], g["H"], g["I"], g["layers"]
    total = L * (nf4_packed_nbytes(E, 2 * I, H) + nf4_packed_nbytes(E, H, I))
    assert total == int(g["packed_gib"] * 2**30)
    params = L * E * 3 * H * I
    assert abs(params / 1e9 - g["expert_params_billion_approx"]) < 0.05
    # the oracle's own arrays have exactly that size per element count
    q, a = nf4_quantize(np.zeros((2, 4, 128), np.uint16))
    assert q.nbytes == nf4_packed_nbytes(2, 4, 128) and a.nbytes == 2 * 4 * 2 * 4
