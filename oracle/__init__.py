"""Plain CPU oracle for MoE expert weight quantization and the packed-experts forward.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, headers,
tables or constant generators with the HIP library; the NF4 codebook is
re-derived here from its construction, not read from the kernel sources.

Everything is numpy (fp64 where the arithmetic is floating point and the
sources fix no precision) and deliberately slow and literal, so that each
function can be checked against the pages by eye.

Sources (page title, then section):

* "MoE Expert Quantization" (Axolotl docs), *Implementation details*: 3-D+
  expert tensors are quantized on load; 4-bit mode uses NF4, 8-bit mode a
  row-wise int8 parametrization.
* bitsandbytes issue #1849 "Failed to quant MoE models with fused expert
  weights in transformers v5", *Description* (the fused ``gate_up_proj
  [E, 2I, H]`` / ``down_proj [E, H, I]`` layout and the ``act_fn``) and the
  maintainer comment thread (plain packed storage plus a module-owned absmax
  ``[num_experts, blocks_per_expert]``; in_features divisible by the
  blocksize 64; no double quantization; a per-expert dequantize + matmul
  loop as the correctness-first forward).
* unsloth-zoo issue #850, *Suggested fix*: the experts interface
  ``(hidden_states, top_k_index, top_k_weights)``.
* Axolotl issue #3787 "Expert-granularity CPU offload for quantized MoE",
  *Use case*: adapter training steps over frozen 4-bit experts, the
  workload the backward serves.

Modules:

* :mod:`oracle.bf16`    -- bf16 <-> fp32 conversions.
* :mod:`oracle.nf4`     -- NF4 codebook, blockwise quantize, dequantize.
* :mod:`oracle.int8`    -- row-wise int8 quantize, dequantize.
* :mod:`oracle.routing` -- per-expert bucketing of top-k assignments.
* :mod:`oracle.forward` -- the routed experts forward in fp64.
* :mod:`oracle.backward` -- its gradients with respect to the hidden states
  and the routing weights (frozen weights), in fp64.
* :mod:`oracle.router`  -- the router front-end (logits, softmax, top-K) in fp64.
* :mod:`oracle.dq`      -- double quantization of the NF4 absmax (8-bit codes
  per 256-block group of one expert, fp32 group scales).

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against closed forms, brute force, exact rational arithmetic or library
routines; none is "parity unpinned".
"""

from . import bf16, nf4, int8, routing, forward  # noqa: F401
