"""Shared helpers for the GPU parity tests."""

import sys

import numpy as np
import torch

import bit_weight_quantization_moeq_amd as moeq
from moeq_synth import bf16_bits

DEV = "cuda"


def say(msg):
    """Name the case before any GPU step (flushed, so a fault still shows it)."""
    print(f"[case] {msg}", file=sys.stderr, flush=True)


def dev_bf16(bits):
    """uint16 bf16 patterns (numpy) -> bf16 device tensor."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(DEV)


def host(t):
    return t.detach().cpu().numpy()


def host_bits(t):
    return bf16_bits(t)


def require_native():
    """The HIP library must be the code that runs: fail loudly if it is absent."""
    import os
    assert os.path.exists(moeq.library_path()), "libmoeq.so not built"
    assert torch.cuda.is_available(), "no GPU visible"
