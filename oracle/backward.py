"""Gradients of the routed experts forward with respect to its inputs, in fp64
(test infrastructure only).

What the pages fix: the workload the quantized experts serve is adapter
training over frozen quantized expert weights ("MoE Expert Quantization",
Axolotl docs, intro and *Expert LoRA targeting*; Axolotl issue #3787,
*Use case* and *Evidence*: QLoRA training steps over frozen 4-bit experts).
Training needs the gradient of the experts block with respect to what flows
into it, the hidden states and the routing weights, while the packed weights
stay frozen.  The pages print no backward; this is the chain rule of the
forward in ``oracle.forward`` (its readings: gate = first I rows of gate_up,
SiLU, weights used as given):

    g = G_e x_t,  u = U_e x_t,  h = silu(g) * u,  z = D_e h,  out_t = sum_k w_tk z
    d w_tk  = dout_t . z
    dh      = w_tk * D_e^T dout_t
    dg      = dh * u * silu'(g),   silu'(g) = s (1 + g (1 - s)),  s = sigmoid(g)
    du      = dh * silu(g)
    dx_t   += G_e^T dg + U_e^T du          (summed over k)

Everything is fp64 on the dequantized bf16 weights and the bf16 inputs; the
roundings the GPU applies between stages are not part of the function, so
this is the exact value they approximate.
"""

import numpy as np

from .bf16 import bf16_to_f32
from .forward import _Widen, silu


def sigmoid(z):
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def experts_backward(hidden_bits, top_k_index, top_k_weights, gate_up, down, grad_out_bits):
    """Gradients of ``sum(grad_out * experts_forward(...))``.

    Arguments as in ``oracle.forward.experts_forward`` plus ``grad_out_bits``
    uint16 bf16 ``[T, H]``.  Returns ``(grad_hidden fp64 [T, H],
    grad_weights fp64 [T, K])``; an unrouted assignment (index outside
    ``[0, E)``) gets weight gradient 0 and adds nothing to ``grad_hidden``.
    """
    x = bf16_to_f32(hidden_bits).astype(np.float64)
    dout = bf16_to_f32(grad_out_bits).astype(np.float64)
    wts = np.asarray(top_k_weights, dtype=np.float32).astype(np.float64)
    return experts_backward_f64(x, top_k_index, wts, _Widen(gate_up), _Widen(down), dout)


def experts_backward_f64(x, top_k_index, top_k_weights, gate_up, down, grad_out):
    """The same gradients on real-valued operands (fp64 arrays, as in
    ``oracle.forward.experts_forward_f64``)."""
    x = np.asarray(x, dtype=np.float64)
    dout = np.asarray(grad_out, dtype=np.float64)
    idx = np.asarray(top_k_index, dtype=np.int64)
    wts = np.asarray(top_k_weights, dtype=np.float64)
    T, H = x.shape
    K = idx.shape[1]
    gx = np.zeros((T, H), dtype=np.float64)
    gw = np.zeros((T, K), dtype=np.float64)

    E = len(gate_up)
    for e in np.unique(idx):
        if e < 0 or e >= E:                          # not routed
            continue
        tok, kk = np.nonzero(idx == e)               # every (t, k) served by expert e
        w_gu = np.asarray(gate_up[int(e)], dtype=np.float64)   # [2I, H]
        w_d = np.asarray(down[int(e)], dtype=np.float64)       # [H, I]
        I = w_gu.shape[0] // 2
        assert w_gu.shape == (2 * I, H) and w_d.shape == (H, I)
        X, G = x[tok], dout[tok]                     # [n, H]
        w = wts[tok, kk][:, None]                    # [n, 1]
        g = X @ w_gu[:I].T
        u = X @ w_gu[I:].T
        s = sigmoid(g)
        h = silu(g) * u
        z = h @ w_d.T                                # [n, H]: y before the weight
        gw[tok, kk] = np.sum(G * z, axis=1)
        dh = w * (G @ w_d)                           # [n, I]
        dg = dh * u * s * (1.0 + g * (1.0 - s))
        du = dh * silu(g)
        dx = dg @ w_gu[:I] + du @ w_gu[I:]           # [n, H]
        np.add.at(gx, tok, dx)
    return gx, gw
