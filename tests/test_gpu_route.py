"""GPU parity: routing buckets (counts, offsets, perm, slot) bit-exact against the oracle."""

import numpy as np
import pytest
import torch

import bit_weight_quantization_moeq_amd as moeq
import moeq_synth as syn
from oracle.routing import route_buckets
from tests.gpu_common import host, require_native, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _native():
    require_native()


def _check(idx, E, label):
    say(f"route {label} T={idx.shape[0]} K={idx.shape[1]} E={E}")
    c, o, p, s = moeq.moeq_route_buckets(torch.from_numpy(np.ascontiguousarray(idx, np.int32)).cuda(), E)
    torch.cuda.synchronize()
    rc, ro, rp, rs = route_buckets(idx, E)
    assert np.array_equal(host(c), rc), label
    assert np.array_equal(host(o), ro), label
    gp = host(p)
    assert np.array_equal(gp[: len(rp)], rp), label
    assert np.all(gp[len(rp):] == -1), label                  # untouched past offsets[E]
    assert np.array_equal(host(s), rs), label


@pytest.mark.parametrize("name,T", [("tiny", 64), ("olmoe", 1), ("olmoe", 32), ("olmoe", 4096),
                                    ("qwen3", 64), ("qwen3", 8192), ("gptoss", 16), ("gptoss", 2048),
                                    ("mixtral", 1), ("mixtral", 16384)])
def test_route_workloads(name, T):
    s = syn.SHAPES[name]
    idx, _ = syn.routing(T, s.K, s.E, kind=s.routing)
    _check(idx.numpy(), s.E, f"{name} T={T}")


def test_route_ragged_duplicates_and_unrouted():
    rng = np.random.default_rng(201)
    for T, K, E in [(333, 3, 17), (1, 1, 1), (257, 1, 1000), (1000, 6, 5), (5000, 13, 1024)]:
        idx = rng.integers(0, E, (T, K)).astype(np.int32)    # duplicates within rows allowed
        _check(idx, E, f"random T={T} K={K} E={E}")
    idx = rng.integers(-3, 12, (700, 4)).astype(np.int32)    # some unrouted (<0 or >= E)
    _check(idx, 9, "unrouted entries")
    skew = np.zeros((4096, 8), np.int32)                     # every assignment on one expert
    _check(skew, 64, "all on expert 0")


def test_route_empty():
    _check(np.zeros((0, 4), np.int32), 8, "empty")


def test_route_is_deterministic():
    s = syn.SHAPES["qwen3"]
    idx, _ = syn.routing(8192, s.K, s.E, kind="zipf", device="cuda")
    a = moeq.moeq_route_buckets(idx, s.E)
    b = moeq.moeq_route_buckets(idx, s.E)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
