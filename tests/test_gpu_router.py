"""GPU parity: the router front-end against the fp64 oracle (oracle.router).

The logits are fp32 sums on the GPU, so where two logits are closer than the
fp32 accumulation bound either order is a correct top-K: the test requires
the GPU's selection to match the oracle's exactly wherever the oracle's
logit gaps exceed that bound, and to be a valid top-K (each pick within the
bound of the oracle's logit of that rank) everywhere.  Weights: relative
error <= 1e-4 against the oracle's probabilities of the experts the GPU
picked."""

import numpy as np
import pytest
import torch

import bit_weight_quantization_moeq_amd as moeq
import moeq_synth as syn
from oracle.bf16 import bf16_to_f32
from oracle.router import router_topk
from oracle.routing import route_buckets
from tests.gpu_common import host, host_bits, require_native, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _native():
    require_native()


def _check(x, gate, K, renorm, idx, wts, label):
    xb, gb = host_bits(x), host_bits(gate)
    ref_i, ref_w, logits = router_topk(xb, gb, K, renormalize=renorm)
    xf, gf = bf16_to_f32(xb).astype(np.float64), bf16_to_f32(gb).astype(np.float64)
    bound = 2.0 ** -18 * (np.abs(xf) @ np.abs(gf).T).max(axis=1)          # per token
    gi, gw = host(idx).astype(np.int64), host(wts).astype(np.float64)
    T, E = logits.shape
    order = np.argsort(-logits, axis=1, kind="stable")
    sorted_l = np.take_along_axis(logits, order, 1)
    picked_l = np.take_along_axis(logits, gi, 1)
    assert np.all((gi >= 0) & (gi < E)), label
    assert all(len(set(r)) == K for r in gi.tolist()), (label, "repeated expert")
    assert np.all(np.abs(picked_l - sorted_l[:, :K]) <= bound[:, None]), (label, "not a top-K")
    # unique where the oracle's neighbouring gaps (through rank K) exceed 2 * bound
    gaps = -np.diff(sorted_l[:, :min(K + 1, E)], axis=1)
    clear = np.all(gaps > 2 * bound[:, None], axis=1)
    assert np.array_equal(gi[clear], ref_i[clear]), (label, "selection differs on a clear token")
    p = np.exp(logits - logits.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    pw = np.take_along_axis(p, gi, 1)
    if renorm:
        pw = pw / pw.sum(1, keepdims=True)
    err = np.max(np.abs(gw - pw) / np.maximum(pw, 1e-30))
    print(f"{label}: {clear.mean():.4f} of tokens clear, max weight rel err {err:.2e}")
    assert err <= 1e-4, (label, err)


CASES = [("tiny", 53, False), ("olmoe", 4096, False), ("qwen3", 1000, True), ("mixtral", 77, True)]


@pytest.mark.parametrize("name,T,renorm", CASES)
def test_router_workloads(name, T, renorm):
    s = syn.SHAPES[name]
    x = syn.hidden_states(T, s.H, device="cuda")
    gate = syn.router_weight(s.E, s.H, device="cuda")
    say(f"router {name} T={T} E={s.E} K={s.K} renorm={renorm}")
    idx, wts = moeq.moeq_router_topk(x, gate, s.K, renormalize=renorm)
    torch.cuda.synchronize()
    _check(x, gate, s.K, renorm, idx, wts, f"{name} T={T}")


@pytest.mark.parametrize("E,K", [(1000, 17), (1024, 1), (33, 33), (5, 3)])
def test_router_expert_counts(E, K):
    T, H = 21, 128
    x = syn.hidden_states(T, H, device="cuda", layer=3)
    gate = syn.router_weight(E, H, std=0.1, device="cuda", layer=3)
    say(f"router E={E} K={K}")
    idx, wts = moeq.moeq_router_topk(x, gate, K, renormalize=(K % 2 == 1))
    torch.cuda.synchronize()
    _check(x, gate, K, K % 2 == 1, idx, wts, f"E={E} K={K}")


def test_router_ties_and_determinism():
    # experts 1 and 4 have identical rows: exact ties, lower index first
    E, H, T, K = 6, 64, 40, 4
    gate = syn.router_weight(E, H, std=0.1, device="cuda", layer=4)
    gate[4] = gate[1]
    x = syn.hidden_states(T, H, device="cuda", layer=4)
    a = moeq.moeq_router_topk(x, gate, K)
    b = moeq.moeq_router_topk(x, gate, K)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    gi = host(a[0])
    for r in gi.tolist():
        if 1 in r and 4 in r:
            assert r.index(1) < r.index(4)
        assert not (4 in r and 1 not in r)
    _check(x, gate, K, False, a[0], a[1], "ties")


def test_router_feeds_the_experts_forward():
    s = syn.SHAPES["tiny"]
    T = 64
    gu, dn, x, _, _ = syn.layer_inputs(s, T, device="cuda")
    gate = syn.router_weight(s.E, s.H, device="cuda")
    idx, wts = moeq.moeq_router_topk(x, gate, s.K, renormalize=True)
    out = moeq.moeq_experts_forward(x, idx, wts, moeq.moeq_quantize_nf4(gu), moeq.moeq_quantize_nf4(dn))
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    with pytest.raises(moeq.MoeqError):
        moeq.moeq_router_topk(x, gate, s.E + 1)


# ---------------------------------------------------------------------------
# The router fused with the routing stage (moeq_router_route)
# ---------------------------------------------------------------------------
def _check_routing(idx, r, E, label):
    """The fused routing equals the oracle's bucketing of the selections the
    router made (bit-exact), and those selections are a valid top-K."""
    ref = route_buckets(host(idx), E)
    got = [host(t) for t in r]
    for name, a, b in zip(("counts", "offsets", "perm", "slot"), got, ref):
        assert np.array_equal(a, b), (label, name)


ROUTE_CASES = [("tiny", 53, False), ("olmoe", 4096, False), ("qwen3", 1000, True), ("mixtral", 77, True),
               ("mixtral", 16384, False), ("gptoss", 2048, True)]


@pytest.mark.parametrize("name,T,renorm", ROUTE_CASES)
def test_router_route_matches_oracle_and_unfused(name, T, renorm):
    s = syn.SHAPES[name]
    x = syn.hidden_states(T, s.H, device="cuda")
    gate = syn.router_weight(s.E, s.H, device="cuda")
    say(f"router_route {name} T={T} E={s.E} K={s.K} renorm={renorm}")
    idx, wts, r = moeq.moeq_router_route(x, gate, s.K, renormalize=renorm)
    i2, w2 = moeq.moeq_router_topk(x, gate, s.K, renormalize=renorm)
    torch.cuda.synchronize()
    assert torch.equal(idx, i2) and torch.equal(wts, w2), "fused router selections differ from the router's"
    if T <= 4096:
        _check(x, gate, s.K, renorm, idx, wts, f"{name} T={T}")
    _check_routing(idx, r, s.E, f"{name} T={T}")
    c, o, p, sl = moeq.moeq_route_buckets(idx, s.E)
    torch.cuda.synchronize()
    assert torch.equal(c, r.counts) and torch.equal(o, r.offsets) and torch.equal(p, r.perm) \
        and torch.equal(sl, r.slot)


@pytest.mark.parametrize("E,K", [(1000, 17), (1024, 1), (33, 33), (5, 3), (64, 64)])
def test_router_route_expert_counts(E, K):
    T, H = 37, 128
    x = syn.hidden_states(T, H, device="cuda", layer=3)
    gate = syn.router_weight(E, H, std=0.1, device="cuda", layer=3)
    say(f"router_route E={E} K={K}")
    idx, wts, r = moeq.moeq_router_route(x, gate, K, renormalize=(K % 2 == 1))
    torch.cuda.synchronize()
    _check(x, gate, K, K % 2 == 1, idx, wts, f"E={E} K={K}")
    _check_routing(idx, r, E, f"E={E} K={K}")


def test_router_route_rejects_large_k_and_handles_empty():
    H = 128
    x = syn.hidden_states(4, H, device="cuda")
    gate = syn.router_weight(100, H, device="cuda")
    with pytest.raises(moeq.MoeqError) as ei:
        moeq.moeq_router_route(x, gate, 65)
    assert ei.value.status == -2
    idx, wts, r = moeq.moeq_router_route(x[:0], gate, 3)
    torch.cuda.synchronize()
    assert idx.shape == (0, 3) and int(r.counts.abs().sum()) == 0 and int(r.offsets.abs().sum()) == 0


# T*K = 64 takes the few-assignment path; the others the tiled one
@pytest.mark.parametrize("name,T,fmt", [("tiny", 32, "nf4"), ("tiny", 300, "int8"), ("olmoe", 4096, "nf4"),
                                        ("qwen3", 1000, "nf4_dq"), ("mixtral", 512, "nf4")])
def test_forward_routed_is_bit_identical(name, T, fmt):
    s = syn.SHAPES[name]
    gu = syn.expert_weights(s.gate_up_shape, tensor=syn.GATE_UP, outliers=s.outliers, device="cuda")
    dn = syn.expert_weights(s.down_shape, tensor=syn.DOWN, outliers=s.outliers, device="cuda")
    if fmt == "int8":
        qg, qd = moeq.moeq_quantize_int8_rowwise(gu), moeq.moeq_quantize_int8_rowwise(dn)
    else:
        qg = moeq.moeq_quantize_nf4(gu, double_quant=fmt == "nf4_dq")
        qd = moeq.moeq_quantize_nf4(dn, double_quant=fmt == "nf4_dq")
    del gu, dn
    x = syn.hidden_states(T, s.H, device="cuda")
    gate = syn.router_weight(s.E, s.H, device="cuda")
    say(f"forward_routed {name} T={T} fmt={fmt}")
    idx, wts, r = moeq.moeq_router_route(x, gate, s.K, renormalize=True)
    a = moeq.moeq_experts_forward(x, idx, wts, qg, qd)
    b = moeq.moeq_experts_forward_routed(x, idx, wts, qg, qd, r)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
