"""The router in front of the experts, in fp64 (test infrastructure only).

What the pages fix: the MoE block has a router weight ``mlp.gate.weight``
next to the fused experts ("MoE Expert Quantization", Axolotl docs, *Expert
LoRA targeting*, where it is the commented-out adapter target), it stays in
bf16 while the experts are quantized and can be the only trained part
(bitsandbytes issue #1849, maintainer thread: router-only training over NF4
experts), and its output is the ``(top_k_index, top_k_weights)`` pair the
experts interface takes (unsloth-zoo issue #850, *Suggested fix*).

Readings taken here (the pages print no router):

* ``gate`` is ``[E, H]`` (``[out, in]`` like the experts); the logits of
  token t are ``l_t = gate @ x_t``.
* Probabilities are the softmax of the logits over all E experts.
* The K experts with the largest logits are selected, in descending logit
  order; equal logits go to the lower expert index.
* ``top_k_weights`` are the selected probabilities, or, with
  ``renormalize``, those probabilities divided by their sum (which equals a
  softmax over the K selected logits).
"""

import numpy as np

from .bf16 import bf16_to_f32


def router_logits(hidden_bits, gate_bits):
    """fp64 ``[T, E]`` logits from bf16 hidden ``[T, H]`` and gate ``[E, H]``."""
    x = bf16_to_f32(hidden_bits).astype(np.float64)
    g = bf16_to_f32(gate_bits).astype(np.float64)
    return x @ g.T


def router_topk(hidden_bits, gate_bits, K, renormalize=False):
    """``(top_k_index int64 [T, K], top_k_weights fp64 [T, K], logits fp64 [T, E])``."""
    logits = router_logits(hidden_bits, gate_bits)
    T, E = logits.shape
    m = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - m)
    p /= p.sum(axis=1, keepdims=True)
    idx = np.empty((T, K), dtype=np.int64)
    for t in range(T):
        # descending logit, ascending index among equals
        order = sorted(range(E), key=lambda e: (-logits[t, e], e))
        idx[t] = order[:K]
    w = np.take_along_axis(p, idx, axis=1)
    if renormalize:
        w = w / w.sum(axis=1, keepdims=True)
    return idx, w, logits
