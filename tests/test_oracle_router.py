"""Pins for oracle.router: the selection against numpy's stable argsort, the
softmax against its defining identities, the tie-break on constructed exact
ties, and renormalisation as a softmax over the selected logits."""

import numpy as np

from oracle.bf16 import bf16_to_f32, f32_to_bf16
from oracle.router import router_logits, router_topk


def _bits(a):
    return f32_to_bf16(np.asarray(a, dtype=np.float32))


def test_selection_matches_stable_argsort():
    rng = np.random.default_rng(21)
    T, H, E, K = 40, 64, 16, 4
    x, g = _bits(rng.standard_normal((T, H))), _bits(rng.standard_normal((E, H)) * 0.1)
    idx, w, logits = router_topk(x, g, K)
    ref = np.argsort(-logits, axis=1, kind="stable")[:, :K]
    np.testing.assert_array_equal(idx, ref)
    # logits are the plain product of the widened operands
    xf, gf = bf16_to_f32(x).astype(np.float64), bf16_to_f32(g).astype(np.float64)
    np.testing.assert_array_equal(logits, xf @ gf.T)
    assert np.all(np.diff(np.take_along_axis(logits, idx, 1), axis=1) <= 0)


def test_softmax_identities_and_renormalisation():
    rng = np.random.default_rng(22)
    T, H, E, K = 12, 32, 8, 3
    x, g = _bits(rng.standard_normal((T, H))), _bits(rng.standard_normal((E, H)) * 0.2)
    idx, w, logits = router_topk(x, g, K)
    _, wall, _ = router_topk(x, g, E)                  # K = E: every probability
    np.testing.assert_allclose(wall.sum(axis=1), 1.0, rtol=1e-14)
    # ratios of probabilities are exp of logit differences
    for t in range(T):
        a, b = idx[t, 0], idx[t, 1]
        assert abs(w[t, 0] / w[t, 1] - np.exp(logits[t, a] - logits[t, b])) <= 1e-12 * w[t, 0] / w[t, 1]
    _, wr, _ = router_topk(x, g, K, renormalize=True)
    np.testing.assert_allclose(wr.sum(axis=1), 1.0, rtol=1e-14)
    sel = np.take_along_axis(logits, idx, 1)
    soft = np.exp(sel - sel.max(1, keepdims=True))
    np.testing.assert_allclose(wr, soft / soft.sum(1, keepdims=True), rtol=1e-13)


def test_exact_ties_go_to_the_lower_index():
    H, E = 16, 6
    g = np.zeros((E, H), np.float32)
    g[1, 0] = g[4, 0] = 1.0      # experts 1 and 4 tie
    g[2, 0] = 2.0                # expert 2 is the largest
    g[3, 0] = g[5, 0] = -1.0     # 0 (logit 0) beats 3 and 5
    x = np.zeros((2, H), np.float32)
    x[:, 0] = 1.0
    idx, _, _ = router_topk(_bits(x), _bits(g), 4)
    np.testing.assert_array_equal(idx, [[2, 1, 4, 0], [2, 1, 4, 0]])


def test_single_expert_and_logit_values():
    x = _bits([[1.0, 2.0, 0.5, -1.0]])
    g = _bits([[0.5, 0.25, 2.0, 1.0], [-1.0, 0.0, 0.0, 0.0]])
    idx, w, logits = router_topk(x, g, 1)
    np.testing.assert_array_equal(logits, [[0.5 + 0.5 + 1.0 - 1.0, -1.0]])
    assert idx[0, 0] == 0
    assert abs(w[0, 0] - 1.0 / (1.0 + np.exp(-2.0))) < 1e-15
    np.testing.assert_array_equal(router_logits(x, g), logits)
