"""Per-expert bucketing of top-k assignments (test infrastructure only).

What the pages fix: unsloth-zoo issue #850, *Suggested fix*: the experts
forward takes ``(hidden_states, top_k_index, top_k_weights)`` uniformly across
fused-expert architectures, so one generic routine must group the (token, k)
assignments by the expert that serves them.

Reading taken here (the pages give no order): assignment ``a = t*K + k``;
``perm`` lists the assignments of expert 0, then expert 1, ..., each expert's
in ascending ``a``; ``slot[a]`` is the position of ``a`` in ``perm``.
Indices outside ``[0, E)`` are not routed: they are absent from ``counts``
and ``perm``, and their ``slot`` is -1.
"""

import numpy as np


def route_buckets(top_k_index, num_experts):
    """Return ``(counts [E], offsets [E+1], perm [n_routed], slot [T*K])`` as int32."""
    idx = np.asarray(top_k_index, dtype=np.int64).reshape(-1)
    E = int(num_experts)
    n = idx.shape[0]

    counts = np.zeros(E, dtype=np.int64)
    for e in range(E):
        counts[e] = np.count_nonzero(idx == e)

    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]

    perm = np.empty(offsets[E], dtype=np.int64)
    slot = np.full(n, -1, dtype=np.int64)
    for e in range(E):
        members = np.nonzero(idx == e)[0]            # ascending assignment index
        perm[offsets[e]:offsets[e + 1]] = members
        slot[members] = np.arange(offsets[e], offsets[e + 1])

    return (counts.astype(np.int32), offsets.astype(np.int32),
            perm.astype(np.int32), slot.astype(np.int32))
