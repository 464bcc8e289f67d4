"""GPU parity: gradients of the experts block through the frozen packed
weights against the fp64 oracle (oracle.backward) on the same dequantized
weights.  Bar: relative Frobenius error <= 5e-3 for both gradients (the
forward's bound: the backward adds the bf16 rounding of dg|du and of the
output, each ~2^-9/sqrt(3) relative rms); runs are bit-identical."""

import numpy as np
import pytest
import torch

import bit_weight_quantization_moeq_amd as moeq
import moeq_synth as syn
from oracle.backward import experts_backward
from oracle.bf16 import bf16_to_f32
from oracle.forward import rel_frobenius
from tests.gpu_common import host, host_bits, require_native, say
from tests.oracle_lazy import LazyDequant

pytestmark = pytest.mark.gpu
TOL = 5e-3


@pytest.fixture(scope="module", autouse=True)
def _native():
    require_native()


def _quantize(w, fmt):
    return moeq.moeq_quantize_nf4(w) if fmt == "nf4" else moeq.moeq_quantize_int8_rowwise(w)


def _compare(x, idx, wts, gu, dn, dout, fmt, gx, gw, tokens, label):
    tokens = np.asarray(tokens)
    ref_x, ref_w = experts_backward(host_bits(x)[tokens], host(idx)[tokens], host(wts)[tokens],
                                    LazyDequant(gu, fmt), LazyDequant(dn, fmt), host_bits(dout)[tokens])
    got_x = bf16_to_f32(host_bits(gx)[tokens]).astype(np.float64)
    got_w = host(gw)[tokens].astype(np.float64)
    ex, ew = rel_frobenius(got_x, ref_x), rel_frobenius(got_w, ref_w)
    print(f"{label}: grad_hidden rel Frobenius {ex:.3e}, grad_weights {ew:.3e}")
    assert ex <= TOL, (label, "grad_hidden", ex)
    assert ew <= TOL, (label, "grad_weights", ew)
    # an unrouted assignment has weight gradient exactly 0
    unrouted = (host(idx)[tokens] < 0) | (host(idx)[tokens] >= gu.shape[0])
    assert np.all(got_w[unrouted] == 0.0)


def _layer(name, T, fmt=None, device="cpu"):
    s = syn.SHAPES[name]
    fmt = fmt or s.fmt
    gu, dn, x, idx, wts = syn.layer_inputs(s, T, device=device)
    dout = syn.grad_output(T, s.H, device=device)
    return s, fmt, *(t.cuda() for t in (gu, dn, x, idx, wts, dout))


@pytest.mark.parametrize("fmt", ["nf4", "int8"])
def test_backward_tiny_full(fmt):
    s, fmt, gu, dn, x, idx, wts, dout = _layer("tiny", 64, fmt)
    say(f"backward tiny fmt={fmt}")
    qg, qd = _quantize(gu, fmt), _quantize(dn, fmt)
    gx, gw = moeq.moeq_experts_backward(x, idx, wts, qg, qd, dout)
    torch.cuda.synchronize()
    _compare(x, idx, wts, gu, dn, dout, fmt, gx, gw, np.arange(64), f"tiny {fmt}")


# NF4 rows with an odd number of 64-blocks (H = 320, I = 192) and with an even
# number that is not a multiple of 4 (H = 384, I = 128): ragged column tiles in
# the transposed GEMMs.
@pytest.mark.parametrize("H,I", [(320, 192), (384, 128)])
def test_backward_nf4_block_counts(H, I):
    s = syn.MoEShape("blocks", E=4, H=H, I=I, K=2, fmt="nf4")
    T = 200
    gu, dn, x, idx, wts = syn.layer_inputs(s, T, device="cpu")
    dout = syn.grad_output(T, s.H, device="cpu")
    gu, dn, x, idx, wts, dout = (t.cuda() for t in (gu, dn, x, idx, wts, dout))
    say(f"backward nf4 H={H} I={I} T={T}")
    qg, qd = moeq.moeq_quantize_nf4(gu), moeq.moeq_quantize_nf4(dn)
    gx, gw = moeq.moeq_experts_backward(x, idx, wts, qg, qd, dout)
    torch.cuda.synchronize()
    _compare(x, idx, wts, gu, dn, dout, "nf4", gx, gw, np.arange(T), f"nf4 H={H} I={I}")


# (shape, T, sampled tokens): gpt-oss has an odd number of 64-row K steps in
# the down-projection transpose (H = 2880)
CASES = [("olmoe", 512, 3), ("qwen3", 256, 3), ("gptoss", 64, 3), ("mixtral", 32, 2)]


@pytest.mark.parametrize("name,T,ns", CASES)
def test_backward_workloads_sampled(name, T, ns):
    dev = "cuda" if name in ("olmoe", "qwen3", "mixtral", "gptoss") else "cpu"
    s, fmt, gu, dn, x, idx, wts, dout = _layer(name, T, device=dev)
    say(f"backward {name} T={T} fmt={fmt}")
    qg, qd = _quantize(gu, fmt), _quantize(dn, fmt)
    gx, gw = moeq.moeq_experts_backward(x, idx, wts, qg, qd, dout)
    torch.cuda.synchronize()
    tokens = np.random.default_rng(5).choice(T, ns, replace=False)
    _compare(x, idx, wts, gu, dn, dout, fmt, gx, gw, tokens, f"{name} T={T}")


@pytest.mark.parametrize("fmt", ["nf4", "int8"])
def test_backward_edge_routing(fmt):
    s = syn.SHAPES["tiny"]
    T = 97
    gu, dn, x, _, _ = syn.layer_inputs(s, T, device="cpu")
    dout = syn.grad_output(T, s.H)
    gu, dn, x, dout = gu.cuda(), dn.cuda(), x.cuda(), dout.cuda()
    qg, qd = _quantize(gu, fmt), _quantize(dn, fmt)
    rng = np.random.default_rng(303)
    idx = rng.integers(-2, s.E + 2, (T, 3)).astype(np.int32)       # duplicates and unrouted
    idx[5] = [4, 4, 4]
    idx[6] = [-1, s.E, 77]                                          # a token routed nowhere
    wts = rng.uniform(-1, 1, (T, 3)).astype(np.float32)
    # zero weights: their hidden-state contribution vanishes, but dL/dw is
    # still dout . (down h), taken from the unweighted down^T product
    wts[7:17, 1] = 0.0
    idx[7:17, 1] = np.arange(10) % s.E
    idx_d, wts_d = torch.from_numpy(idx).cuda(), torch.from_numpy(wts).cuda()
    say(f"backward edge routing fmt={fmt}")
    gx, gw = moeq.moeq_experts_backward(x, idx_d, wts_d, qg, qd, dout)
    torch.cuda.synchronize()
    _compare(x, idx_d, wts_d, gu, dn, dout, fmt, gx, gw, np.arange(T), f"edge {fmt}")
    assert torch.count_nonzero(gx[6]) == 0
    assert bool((host(gw)[7:17, 1] != 0.0).all()), "zero routing weights still have a weight gradient"


def test_backward_is_bit_identical_and_empty_batch():
    s, fmt, gu, dn, x, idx, wts, dout = _layer("olmoe", 300, device="cuda")
    qg, qd = _quantize(gu, fmt), _quantize(dn, fmt)
    say("backward determinism olmoe T=300")
    a = moeq.moeq_experts_backward(x, idx, wts, qg, qd, dout)
    b = moeq.moeq_experts_backward(x, idx, wts, qg, qd, dout)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    e = moeq.moeq_experts_backward(x[:0].contiguous(), idx[:0].contiguous(), wts[:0].contiguous(), qg, qd,
                                   dout[:0].contiguous())
    assert e[0].shape == (0, s.H) and e[1].shape == (0, s.K)
