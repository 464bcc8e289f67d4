"""Pins for oracle.dq: the 8-bit codes against exact rational rounding per
expert-local group, constructed exact ties, an exact grid round trip, the
error bound, zero and ragged groups, and the decoded weights against exact
two-step rounding of level x absmax'."""

import numpy as np

from oracle.bf16 import bf16_to_f32, f32_to_bf16
from oracle.dq import GROUP, dq_compress, dq_decompress, groups_per_expert, nf4_dq_dequantize
from oracle.nf4 import nf4_codebook, nf4_quantize, nf4_unpack
from tests.exact import bf16_from_frac_rne, frac, rn32, round_half_even


def _bf16_values(x):
    """fp32 values that are exactly bf16 (absmax of bf16 weights always is)."""
    return bf16_to_f32(f32_to_bf16(np.asarray(x, dtype=np.float32)))


def test_codes_equal_exact_rounding_within_expert_groups():
    rng = np.random.default_rng(31)
    E, nb = 2, 300                                   # groups of 256 and 44 per expert
    a = _bf16_values(np.abs(rng.standard_normal((E, nb))) * 0.05 + 0.01)
    a[1, 0] = 7.0                                    # would dominate expert 0's last group if groups crossed experts
    a[0, 10] = 0.0
    codes, s2 = dq_compress(a)
    assert codes.shape == (E, nb) and s2.shape == (E, 2)
    for e in range(E):
        for g in range(2):
            blk = a[e, GROUP * g:GROUP * (g + 1)]
            m = max(frac(v) for v in blk)
            assert frac(s2[e, g]) == frac(rn32(m / 255))
            for j, v in enumerate(blk):
                assert codes[e, GROUP * g + j] == round_half_even(255 * frac(v) / m)
    assert codes[0, 10] == 0


def test_exact_ties_round_to_even():
    # group max 255 makes 255 a / m == a: halves go to the even integer
    a = np.array([[255.0, 2.5, 3.5, 0.5, 1.5, 254.5, 100.5, 0.0]], np.float32)
    codes, s2 = dq_compress(a)
    assert codes.tolist() == [[255, 2, 4, 0, 2, 254, 100, 0]]
    assert s2[0, 0] == 1.0


def test_grid_round_trips_exactly():
    # m = 255 * 2^j and a = c * 2^j: every code is c and absmax' is a exactly
    rng = np.random.default_rng(32)
    for j in (-12, -3, 0, 5):
        c = rng.integers(0, 256, size=(3, 512)).astype(np.float32)
        c[:, 0] = 255
        c[:, 256] = 255
        a = (c * np.float32(2.0 ** j)).astype(np.float32)
        codes, s2 = dq_compress(a)
        np.testing.assert_array_equal(codes, c.astype(np.uint8))
        np.testing.assert_array_equal(s2, np.full((3, 2), 2.0 ** j, np.float32))
        np.testing.assert_array_equal(dq_decompress(codes, s2), a)


def test_error_bound_monotone_and_maximum():
    rng = np.random.default_rng(33)
    a = _bf16_values(np.abs(rng.standard_normal((4, 1000))) * 0.03)
    codes, s2 = dq_compress(a)
    back = dq_decompress(codes, s2)
    for e in range(4):
        for g in range(groups_per_expert(1000)):
            sl = slice(GROUP * g, GROUP * (g + 1))
            m = float(a[e, sl].max())
            # half a code step, plus the two fp32 roundings of s2 and c * s2
            assert np.max(np.abs(back[e, sl].astype(np.float64) - a[e, sl])) <= m / 510 + m * 2.0 ** -21
            assert codes[e, sl][np.argmax(a[e, sl])] == 255
            order = np.argsort(a[e, sl], kind="stable")
            assert np.all(np.diff(codes[e, sl][order].astype(int)) >= 0)


def test_zero_single_and_ragged_groups():
    a = np.zeros((3, 257), np.float32)
    a[1, :] = 0.5
    a[2, 256] = 0.25                                 # a one-block last group
    codes, s2 = dq_compress(a)
    assert s2.shape == (3, 2)
    assert np.all(codes[0] == 0) and np.all(s2[0] == 0)
    assert np.all(codes[1] == 255) and s2[1, 0] == np.float32(0.5) / np.float32(255)
    assert np.all(codes[2, :256] == 0) and s2[2, 0] == 0 and codes[2, 256] == 255
    np.testing.assert_array_equal(dq_decompress(codes, s2)[0], 0.0)
    one, s1 = dq_compress(np.array([[0.125]], np.float32))
    assert one.tolist() == [[255]] and s1.shape == (1, 1)


def test_decoded_weights_equal_exact_two_step_rounding():
    rng = np.random.default_rng(34)
    E, R, C = 2, 6, 128                              # 12 blocks per expert
    w = f32_to_bf16((rng.standard_normal((E, R, C)) * 0.02).astype(np.float32))
    q, absmax = nf4_quantize(w)
    codes, s2 = dq_compress(absmax)
    out = nf4_dq_dequantize(q, codes, s2)
    lev = nf4_codebook()
    nib = nf4_unpack(q)
    for e in range(E):
        for r in range(R):
            for col in range(0, C, 5):
                b = r * (C // 64) + col // 64
                a_dec = rn32(frac(np.float32(codes[e, b])) * frac(s2[e, b // GROUP]))
                val = rn32(frac(lev[nib[e, r, col]]) * frac(a_dec))
                assert int(out[e, r, col]) == bf16_from_frac_rne(val)
