"""Pins for oracle.backward: central finite differences of the forward oracle
(an independent function), exact linearity in the routing weights and in the
incoming gradient, and the unrouted / zero-weight / duplicate special cases."""

import numpy as np

from oracle.backward import experts_backward, experts_backward_f64
from oracle.bf16 import bf16_to_f32, f32_to_bf16
from oracle.forward import experts_forward, experts_forward_f64


def _case(rng, E=4, H=12, I=6, T=5, K=3, scale=0.4):
    gu = [rng.standard_normal((2 * I, H)) * scale for _ in range(E)]
    dn = [rng.standard_normal((H, I)) * scale for _ in range(E)]
    x = rng.standard_normal((T, H))
    idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)])
    wts = rng.uniform(-1.0, 1.0, (T, K))
    dout = rng.standard_normal((T, H))
    return gu, dn, x, idx, wts, dout


def _loss(x, idx, wts, gu, dn, dout):
    return float(np.sum(dout * experts_forward_f64(x, idx, wts, gu, dn)))


def test_grad_hidden_matches_central_differences():
    rng = np.random.default_rng(7)
    gu, dn, x, idx, wts, dout = _case(rng)
    gx, _ = experts_backward_f64(x, idx, wts, gu, dn, dout)
    eps = 1e-5
    # every coordinate of a tiny case
    num = np.zeros_like(x)
    for t in range(x.shape[0]):
        for j in range(x.shape[1]):
            xp, xm = x.copy(), x.copy()
            xp[t, j] += eps
            xm[t, j] -= eps
            num[t, j] = (_loss(xp, idx, wts, gu, dn, dout) - _loss(xm, idx, wts, gu, dn, dout)) / (2 * eps)
    assert np.max(np.abs(num - gx)) <= 1e-7 * max(1.0, np.max(np.abs(gx)))


def test_grad_hidden_directional_derivative_larger_case():
    rng = np.random.default_rng(8)
    gu, dn, x, idx, wts, dout = _case(rng, E=6, H=32, I=16, T=9, K=4)
    gx, _ = experts_backward_f64(x, idx, wts, gu, dn, dout)
    for _ in range(4):
        v = rng.standard_normal(x.shape)
        eps = 1e-5
        d = (_loss(x + eps * v, idx, wts, gu, dn, dout) - _loss(x - eps * v, idx, wts, gu, dn, dout)) / (2 * eps)
        assert abs(d - np.sum(gx * v)) <= 1e-7 * max(1.0, abs(d))


def test_grad_weights_exact_by_linearity():
    """The output is linear in each routing weight, so a difference quotient
    with any step is exact up to rounding."""
    rng = np.random.default_rng(9)
    gu, dn, x, idx, wts, dout = _case(rng)
    _, gw = experts_backward_f64(x, idx, wts, gu, dn, dout)
    for t in range(wts.shape[0]):
        for k in range(wts.shape[1]):
            wp, wm = wts.copy(), wts.copy()
            wp[t, k] += 0.5
            wm[t, k] -= 0.5
            d = _loss(x, idx, wp, gu, dn, dout) - _loss(x, idx, wm, gu, dn, dout)
            assert abs(d - gw[t, k]) <= 1e-12 * max(1.0, abs(d))


def test_linear_in_incoming_gradient():
    rng = np.random.default_rng(10)
    gu, dn, x, idx, wts, dout = _case(rng)
    a = experts_backward_f64(x, idx, wts, gu, dn, dout)
    b = experts_backward_f64(x, idx, wts, gu, dn, 3.0 * dout)
    np.testing.assert_allclose(b[0], 3.0 * a[0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(b[1], 3.0 * a[1], rtol=1e-12, atol=1e-12)


def test_unrouted_zero_weight_and_duplicates():
    rng = np.random.default_rng(11)
    gu, dn, x, idx, wts, dout = _case(rng, T=3, K=2)
    E = len(gu)
    idx[0] = [-1, E]                      # token 0 routed nowhere
    wts[1, 1] = 0.0                       # a zero weight
    idx[2] = [1, 1]                       # the same expert twice
    gx, gw = experts_backward_f64(x, idx, wts, gu, dn, dout)
    assert np.all(gx[0] == 0.0) and np.all(gw[0] == 0.0)
    # a zero weight still has a weight gradient, but adds nothing to gx:
    only = idx.copy()
    only[1, 1] = -1
    gx2, gw2 = experts_backward_f64(x, only, wts, gu, dn, dout)
    np.testing.assert_allclose(gx2[1], gx[1], rtol=1e-13, atol=1e-13)
    assert gw[1, 1] != 0.0 and gw2[1, 1] == 0.0
    # a duplicated expert acts once with the summed weight
    one = idx.copy()
    one[2] = [1, -1]
    w1 = wts.copy()
    w1[2, 0] = wts[2, 0] + wts[2, 1]
    gx3, _ = experts_backward_f64(x, one, w1, gu, dn, dout)
    np.testing.assert_allclose(gx3[2], gx[2], rtol=1e-12, atol=1e-12)
    assert abs(gw[2, 0] - gw[2, 1]) <= 1e-12 * max(1.0, abs(gw[2, 0]))


def test_bits_entry_point_agrees_with_real_valued_core():
    rng = np.random.default_rng(12)
    E, H, I, T, K = 3, 16, 8, 4, 2
    gu = f32_to_bf16((rng.standard_normal((E, 2 * I, H)) * 0.1).astype(np.float32))
    dn = f32_to_bf16((rng.standard_normal((E, H, I)) * 0.1).astype(np.float32))
    x = f32_to_bf16(rng.standard_normal((T, H)).astype(np.float32))
    dout = f32_to_bf16(rng.standard_normal((T, H)).astype(np.float32))
    idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)])
    wts = rng.uniform(0, 1, (T, K)).astype(np.float32)
    gx, gw = experts_backward(x, idx, wts, gu, dn, dout)
    f64 = lambda b: bf16_to_f32(b).astype(np.float64)
    gx2, gw2 = experts_backward_f64(f64(x), idx, wts.astype(np.float64), list(map(f64, gu)), list(map(f64, dn)),
                                    f64(dout))
    np.testing.assert_array_equal(gx, gx2)
    np.testing.assert_array_equal(gw, gw2)
    # and the forward's bits entry point agrees with its core on the same data
    np.testing.assert_array_equal(experts_forward(x, idx, wts, gu, dn),
                                  experts_forward_f64(f64(x), idx, wts.astype(np.float64), list(map(f64, gu)),
                                                      list(map(f64, dn))))
