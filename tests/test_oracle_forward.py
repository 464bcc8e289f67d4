"""Pins for oracle.forward: closed forms on permutation-structured experts,
linearity, expert relabelling, duplicates and a scalar brute force."""

import math

import numpy as np

from oracle.bf16 import bf16_to_f32, f32_to_bf16
from oracle.forward import experts_forward, rel_frobenius, silu


def _bits(x):
    return f32_to_bf16(np.asarray(x, dtype=np.float32))


def _silu_scalar(z):
    return z / (1.0 + math.exp(-z))


def test_silu_values():
    assert silu(np.array([0.0]))[0] == 0.0
    assert abs(silu(np.array([1.0]))[0] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-15
    assert abs(silu(np.array([-40.0]))[0]) < 1e-15
    assert silu(np.array([-1000.0]))[0] == 0.0            # no overflow warning/NaN
    assert abs(silu(np.array([30.0]))[0] - 30.0) < 1e-10


def _perm_experts(E, H, I, rng):
    """Experts whose gate, up and down are scaled permutation-like selections.

    gate row j picks x[pg[j]] * ag, up row j picks x[pu[j]] * au, down row n
    picks h[pd[n]] * ad (pd maps H outputs onto I inputs, many-to-one).  H = 2I
    makes gate_up square, the case where a transposed operand is not caught
    by shapes.
    """
    gu = np.zeros((E, 2 * I, H), np.float32)
    dn = np.zeros((E, H, I), np.float32)
    meta = []
    for e in range(E):
        pg, pu = rng.permutation(H)[:I], rng.permutation(H)[:I]
        pd = rng.integers(0, I, H)
        ag, au, ad = [float(2.0 ** rng.integers(-2, 3)) * s for s in (1, -1, 1)]
        gu[e, np.arange(I), pg] = ag
        gu[e, I + np.arange(I), pu] = au
        dn[e, np.arange(H), pd] = ad
        meta.append((pg, pu, pd, ag, au, ad))
    return _bits(gu), _bits(dn), meta


def test_closed_form_on_permutation_experts():
    rng = np.random.default_rng(41)
    E, H, I, T, K = 4, 16, 8, 6, 3
    gu, dn, meta = _perm_experts(E, H, I, rng)
    x = _bits(rng.standard_normal((T, H)))
    idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)])
    wts = rng.uniform(0.1, 1.0, (T, K)).astype(np.float32)
    out = experts_forward(x, idx, wts, gu, dn)
    xf = bf16_to_f32(x).astype(np.float64)
    for t in range(T):
        for n in range(H):
            acc = 0.0
            for k in range(K):
                pg, pu, pd, ag, au, ad = meta[idx[t, k]]
                j = pd[n]
                g = ag * xf[t, pg[j]]
                u = au * xf[t, pu[j]]
                acc += float(wts[t, k]) * ad * _silu_scalar(g) * u
            assert abs(out[t, n] - acc) <= 1e-12 * (1 + abs(acc))


def test_linear_in_weights_and_duplicates_add():
    rng = np.random.default_rng(42)
    E, H, I, T = 3, 32, 16, 5
    gu = _bits(rng.standard_normal((E, 2 * I, H)) * 0.1)
    dn = _bits(rng.standard_normal((E, H, I)) * 0.1)
    x = _bits(rng.standard_normal((T, H)))
    idx = np.array([[0, 1]] * T)
    w1 = np.full((T, 2), 0.25, np.float32)
    w2 = np.full((T, 2), 0.5, np.float32)
    o1 = experts_forward(x, idx, w1, gu, dn)
    o2 = experts_forward(x, idx, w2, gu, dn)
    assert np.allclose(o2, 2 * o1, rtol=1e-13, atol=0)
    # the same expert twice with weights a, b equals it once with a + b
    dup = experts_forward(x, np.array([[2, 2]] * T), np.array([[0.25, 0.5]] * T, np.float32), gu, dn)
    one = experts_forward(x, np.array([[2]] * T), np.array([[0.75]] * T, np.float32), gu, dn)
    assert np.allclose(dup, one, rtol=1e-13, atol=1e-15)


def test_relabelling_experts_changes_nothing():
    rng = np.random.default_rng(43)
    E, H, I, T, K = 6, 32, 16, 9, 2
    gu = _bits(rng.standard_normal((E, 2 * I, H)) * 0.1)
    dn = _bits(rng.standard_normal((E, H, I)) * 0.1)
    x = _bits(rng.standard_normal((T, H)))
    idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)])
    wts = rng.uniform(0, 1, (T, K)).astype(np.float32)
    p = rng.permutation(E)                      # new storage slot of old expert e is p[e]
    gu2, dn2 = np.empty_like(gu), np.empty_like(dn)
    gu2[p], dn2[p] = gu, dn
    assert np.array_equal(experts_forward(x, idx, wts, gu, dn),
                          experts_forward(x, p[idx], wts, gu2, dn2))


def test_scalar_brute_force_single_expert():
    # E = 1, K = 1, weight 1: a dense SwiGLU MLP, evaluated with scalar loops
    rng = np.random.default_rng(44)
    H, I, T = 8, 4, 3
    gu = _bits(rng.standard_normal((1, 2 * I, H)))
    dn = _bits(rng.standard_normal((1, H, I)))
    x = _bits(rng.standard_normal((T, H)))
    out = experts_forward(x, np.zeros((T, 1), np.int64), np.ones((T, 1), np.float32), gu, dn)
    G, D, X = (bf16_to_f32(a).astype(np.float64) for a in (gu[0], dn[0], x))
    for t in range(T):
        h = []
        for j in range(I):
            g = sum(G[j, c] * X[t, c] for c in range(H))
            u = sum(G[I + j, c] * X[t, c] for c in range(H))
            h.append(_silu_scalar(g) * u)
        for n in range(H):
            y = sum(D[n, j] * h[j] for j in range(I))
            assert abs(out[t, n] - y) <= 1e-12 * (1 + abs(y))


def test_unrouted_index_contributes_nothing():
    rng = np.random.default_rng(45)
    E, H, I, T = 2, 16, 8, 4
    gu = _bits(rng.standard_normal((E, 2 * I, H)))
    dn = _bits(rng.standard_normal((E, H, I)))
    x = _bits(rng.standard_normal((T, H)))
    a = experts_forward(x, np.array([[1, -1]] * T), np.ones((T, 2), np.float32), gu, dn)
    b = experts_forward(x, np.array([[1]] * T), np.ones((T, 1), np.float32), gu, dn)
    assert np.array_equal(a, b)


def test_rel_frobenius():
    assert rel_frobenius(np.array([1.0, 1.0]), np.array([1.0, 1.0])) == 0.0
    assert abs(rel_frobenius(np.array([3.0, 4.0]) * 1.01, np.array([3.0, 4.0])) - 0.01) < 1e-12
