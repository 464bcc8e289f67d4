"""The routed experts forward in fp64 (test infrastructure only).

What the pages fix:

* bitsandbytes issue #1849, *Description*: the experts module holds
  ``gate_up_proj [E, 2I, H]`` and ``down_proj [E, H, I]`` with an activation
  ``act_fn`` applied between them; each ``[e]`` slice is an ``[out, in]``
  weight (the maintainer thread names the stack
  ``[num_experts, out_features, in_features]``).
* unsloth-zoo issue #850, *Suggested fix*: the forward takes
  ``(hidden_states, top_k_index, top_k_weights)``.
* bitsandbytes issue #1849, maintainer thread: the correctness-first forward
  dequantizes each expert and multiplies, expert by expert.

Readings taken here (the pages leave them open):

* The first I rows of ``gate_up_proj[e]`` are the gate, the last I the up
  projection (the order in the name ``gate_up``).
* The activation is SiLU, ``h = silu(g) * u`` with ``silu(z) = z / (1 + exp(-z))``.
* ``top_k_weights`` are used as given (no renormalisation); a token's output
  is ``sum_k w[t, k] * down[e_k] @ h_{t,k}``.  A repeated expert within a
  token's row counts once per occurrence.
* Everything is computed in fp64 from the dequantized bf16 weights and the
  bf16 hidden states, so the result is the exact value the GPU's fp32
  accumulation approximates.
"""

import numpy as np

from .bf16 import bf16_to_f32


def silu(z):
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def experts_forward(hidden_bits, top_k_index, top_k_weights, gate_up, down):
    """Routed experts forward.

    ``hidden_bits`` uint16 bf16 ``[T, H]``; ``top_k_index`` int ``[T, K]``;
    ``top_k_weights`` float32 ``[T, K]``; ``gate_up[e]`` -> uint16 bf16
    ``[2I, H]`` and ``down[e]`` -> uint16 bf16 ``[H, I]`` for each expert
    (a 3-D array or any object with ``len`` and indexable by expert).  An
    index outside ``[0, E)`` is not routed and contributes nothing.  Returns
    fp64 ``[T, H]``.  ``down[e]`` may hold only some rows of the down weight
    (the same rows for every expert); the result then holds the matching
    output columns, since output column n depends only on down row n.
    """
    x = bf16_to_f32(hidden_bits).astype(np.float64)
    wts = np.asarray(top_k_weights, dtype=np.float32).astype(np.float64)
    return experts_forward_f64(x, top_k_index, wts, _Widen(gate_up), _Widen(down),
                               lambda: H_of(down, x.shape[1]))


class _Widen:
    """Expert -> its bf16 weight widened to fp64, on demand."""

    def __init__(self, w):
        self.w = w

    def __len__(self):
        return len(self.w)

    def __getitem__(self, e):
        return bf16_to_f32(self.w[e]).astype(np.float64)


def H_of(down, H):
    """Output width when nothing is routed: the down rows held per expert."""
    if isinstance(down, np.ndarray) and down.ndim == 3:
        return down.shape[1]
    return down[0].shape[0] if len(down) else H


def experts_forward_f64(x, top_k_index, top_k_weights, gate_up, down, n_empty=None):
    """The same forward on real-valued operands: ``x`` fp64 ``[T, H]``,
    ``top_k_weights`` ``[T, K]``, ``gate_up[e]`` ``[2I, H]`` and ``down[e]``
    ``[H', I]`` as fp64 arrays.  ``n_empty``: a callable giving the output
    width when nothing is routed (default: H)."""
    x = np.asarray(x, dtype=np.float64)
    idx = np.asarray(top_k_index, dtype=np.int64)
    wts = np.asarray(top_k_weights, dtype=np.float64)
    T, H = x.shape
    K = idx.shape[1]
    y = None

    E = len(gate_up)
    for e in np.unique(idx):
        if e < 0 or e >= E:                         # not routed: contributes nothing
            continue
        tok, kk = np.nonzero(idx == e)              # every (t, k) served by expert e
        w_gu = np.asarray(gate_up[int(e)], dtype=np.float64)   # [2I, H]
        w_d = np.asarray(down[int(e)], dtype=np.float64)       # [H', I]
        I = w_gu.shape[0] // 2
        assert w_gu.shape == (2 * I, H) and w_d.shape[1] == I
        X = x[tok]                                  # [n, H]
        g = X @ w_gu[:I].T                          # gate: first I rows
        u = X @ w_gu[I:].T                          # up: last I rows
        h = silu(g) * u                             # [n, I]
        if y is None:
            y = np.zeros((T, K, w_d.shape[0]), dtype=np.float64)
        y[tok, kk] = h @ w_d.T                      # [n, H']

    if y is None:                                   # nothing routed
        y = np.zeros((T, K, H if n_empty is None else n_empty()), dtype=np.float64)
    out = np.zeros((T, y.shape[2]), dtype=np.float64)
    for k in range(K):
        out += wts[:, k:k + 1] * y[:, k]
    return out


def rel_frobenius(approx, exact):
    """||approx - exact||_F / ||exact||_F in fp64."""
    a = np.asarray(approx, dtype=np.float64)
    b = np.asarray(exact, dtype=np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / den) if den > 0 else float(np.linalg.norm(a - b))
