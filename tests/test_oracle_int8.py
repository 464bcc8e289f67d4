"""Pins for oracle.int8: exact rational rounding, error bound, edge rows, dequantize."""

from fractions import Fraction

import numpy as np

from oracle.bf16 import bf16_to_f32, f32_to_bf16
from oracle.int8 import int8_dequantize_rowwise, int8_quantize_rowwise
from tests.exact import bf16_from_frac_rne, frac, rn32, round_half_even


def _bits(x):
    return f32_to_bf16(np.asarray(x, dtype=np.float32))


def test_codes_equal_exact_round_half_even_of_127w_over_absmax():
    rng = np.random.default_rng(21)
    w = rng.standard_normal((2, 6, 50)).astype(np.float32) * 0.02
    w[1, 3] *= 1e-30                                  # tiny (subnormal-range) row
    bits = _bits(w)
    q, s = int8_quantize_rowwise(bits)
    wf = bf16_to_f32(bits)
    for e in range(2):
        for r in range(6):
            amax = max(abs(frac(x)) for x in wf[e, r])
            assert frac(s[e, r]) == frac(rn32(amax / 127))
            for j in range(50):
                assert q[e, r, j] == round_half_even(127 * frac(wf[e, r, j]) / amax)


def test_exact_ties_round_to_even():
    # absmax 127 makes 127*w/absmax == w: halves must go to the even integer
    w = np.array([[[127.0, 2.5, 3.5, -2.5, -3.5, 0.5, -0.5, 1.5, 126.5]]], np.float32)
    q, s = int8_quantize_rowwise(_bits(w))
    assert q.tolist() == [[[127, 2, 4, -2, -4, 0, 0, 2, 126]]]
    assert s[0, 0] == 1.0


def test_error_bound_and_extremes():
    rng = np.random.default_rng(22)
    w = rng.standard_normal((3, 20, 300)).astype(np.float32) * 0.02
    bits = _bits(w)
    q, s = int8_quantize_rowwise(bits)
    wf = bf16_to_f32(bits).astype(np.float64)
    amax = np.max(np.abs(wf), axis=-1)
    err = np.abs(wf - q.astype(np.float64) * s[..., None].astype(np.float64))
    assert np.all(err <= s[..., None] / 2 + 2.0**-24 * amax[..., None])
    assert q.min() >= -127 and q.max() <= 127
    # the largest |w| of each row maps to +-127 exactly
    arg = np.argmax(np.abs(wf), axis=-1)
    top = np.take_along_axis(q, arg[..., None], axis=-1)[..., 0]
    assert np.all(np.abs(top.astype(int)) == 127)


def test_zero_row():
    w = np.zeros((1, 2, 16), np.float32)
    w[0, 1, 3] = -0.5
    q, s = int8_quantize_rowwise(_bits(w))
    assert s[0, 0] == 0 and np.all(q[0, 0] == 0)
    assert q[0, 1, 3] == -127 and np.all(np.delete(q[0, 1], 3) == 0)


def test_dequantize_exact_and_round_trip():
    rng = np.random.default_rng(23)
    bits = _bits(rng.standard_normal((2, 4, 40)).astype(np.float32) * 0.02)
    q, s = int8_quantize_rowwise(bits)
    d = int8_dequantize_rowwise(q, s)
    for e in range(2):
        for r in range(4):
            for j in range(40):
                p = rn32(Fraction(int(q[e, r, j])) * frac(s[e, r]))
                assert d[e, r, j] == bf16_from_frac_rne(p)
    q2, s2 = int8_quantize_rowwise(d)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)


def _exact_q(w, a):
    """round_half_even(127*w/a) for bf16 w, a>0 in exact int64 arithmetic (vectorised)."""
    wb = f32_to_bf16(w).astype(np.int64)
    ab = int(f32_to_bf16(np.array([a], np.float32))[0])
    def split(b):
        e = (b >> 7) & 0xFF
        m = b & 0x7F
        mant = np.where(e > 0, m | 0x80, m)
        exp = np.where(e > 0, e, 1)
        return mant, exp
    mw, ew = split(wb & 0x7FFF)
    ma, ea = split(np.array([ab & 0x7FFF], np.int64))
    d = ew - ea[0]
    sh_up = np.clip(d, 0, 62)
    sh_dn = np.clip(-d, 0, 62)
    num = 127 * mw * (np.int64(1) << sh_up)
    den = ma[0] * (np.int64(1) << np.minimum(sh_dn, 40))
    num = np.where(sh_dn > 40, 0, num)           # ratio below 127*255/2^40: rounds to 0
    q0 = num // den
    rem = num - q0 * den
    up = (2 * rem > den) | ((2 * rem == den) & (q0 % 2 == 1))
    q = q0 + up
    return np.where((wb >> 15) & 1, -q, q)


def test_exhaustive_over_all_bf16_ratios():
    """Every bf16 (w, absmax) pair with absmax in [1, 2) and |w| <= absmax.

    q depends on w/absmax only and every bf16 ratio occurs with such an
    absmax; the expectation is the exact integer round-half-even of 127w/a.
    """
    allw = bf16_to_f32(np.arange(65536, dtype=np.uint32).astype(np.uint16))
    allw = allw[np.isfinite(allw)]
    rows, expect = [], []
    for A in range(128, 256):
        a = np.float32(bf16_to_f32(np.array([0x3F00 + A], np.uint16))[0])
        w = allw[np.abs(allw) <= a]
        pad = (-len(w)) % 255
        w = np.concatenate([w, np.zeros(pad, np.float32)]).reshape(-1, 255)
        r = np.concatenate([np.full((w.shape[0], 1), a, np.float32), w], axis=1)
        rows.append(r)
        expect.append(_exact_q(r.reshape(-1), a).reshape(r.shape))
    rows = np.concatenate(rows)
    expect = np.concatenate(expect)
    q, s = int8_quantize_rowwise(f32_to_bf16(rows).reshape(1, -1, 256))
    assert np.array_equal(q.reshape(-1, 256).astype(np.int64), expect)
    assert s.shape == (1, rows.shape[0])
