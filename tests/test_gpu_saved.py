"""GPU: the training pair that keeps the gate and up pre-activations
(moeq_experts_forward_save, moeq_experts_backward_saved) against the plain
calls.  The saved backward skips only the recompute of the gate_up GEMM, so
its gradients must equal moeq_experts_backward's bit for bit; the saving
forward's output equals moeq_experts_forward's bit for bit on the tiled path
and is held to the oracle (5e-3 relative Frobenius) where the plain forward
takes the few-assignment path instead."""

import numpy as np
import pytest
import torch

import bit_weight_quantization_moeq_amd as moeq
import moeq_synth as syn
from tests.gpu_common import require_native, say
from tests.test_gpu_forward import _compare

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _native():
    require_native()


def _quantize(w, fmt):
    if fmt == "int8":
        return moeq.moeq_quantize_int8_rowwise(w)
    return moeq.moeq_quantize_nf4(w, double_quant=(fmt == "nf4_dq"))


# T*K = 128 (the plain forward takes the few-assignment path), 1200 (tiled,
# several tiles per expert with a ragged last one)
@pytest.mark.parametrize("fmt", ["nf4", "nf4_dq", "int8"])
@pytest.mark.parametrize("T", [64, 600])
def test_saved_pair_matches_plain_calls(fmt, T):
    s = syn.MoEShape("saved", E=8, H=512, I=256, K=2, fmt="nf4")
    gu, dn, x, idx, wts = (t.cuda() for t in syn.layer_inputs(s, T, device="cpu"))
    if T == 600:  # unrouted assignments (index -1 and E) and zero weights among them
        idx[5, 0], idx[77, 1], idx[301, 0] = -1, s.E, -1
        wts[9, 1], wts[450, 0] = 0.0, 0.0
    dout = syn.grad_output(T, s.H, device="cpu").cuda()
    say(f"saved pair fmt={fmt} T={T}")
    qg, qd = _quantize(gu, fmt), _quantize(dn, fmt)
    out_s, gsv = moeq.moeq_experts_forward_save(x, idx, wts, qg, qd)
    out_f = moeq.moeq_experts_forward(x, idx, wts, qg, qd)
    gx_s, gw_s = moeq.moeq_experts_backward_saved(idx, wts, qg, qd, gsv, dout)
    gx, gw = moeq.moeq_experts_backward(x, idx, wts, qg, qd, dout)
    torch.cuda.synchronize()
    assert torch.equal(gx_s, gx), "grad_hidden differs from the recomputing backward"
    assert torch.equal(gw_s, gw), "grad_weights differ from the recomputing backward"
    if T * s.K > 512:
        assert torch.equal(out_s, out_f), "output differs from the plain tiled forward"
    oracle_fmt = "int8" if fmt == "int8" else "nf4"
    if fmt != "nf4_dq":  # the double-quantized format's oracle parity lives in its own tests
        _compare(x, idx, wts, gu, dn, oracle_fmt, out_s, np.arange(0, T, 7), label=f"saved {fmt} T={T}")


def test_saved_pair_second_call_smaller_batch():
    """Buffers reused across calls: a smaller batch after a larger one still
    matches the recomputing backward bit for bit."""
    s = syn.MoEShape("saved", E=8, H=512, I=256, K=2, fmt="nf4")
    for T in (900, 300):
        gu, dn, x, idx, wts = (t.cuda() for t in syn.layer_inputs(s, T, device="cpu"))
        dout = syn.grad_output(T, s.H, device="cpu").cuda()
        say(f"saved pair reuse T={T}")
        qg, qd = _quantize(gu, "nf4"), _quantize(dn, "nf4")
        _, gsv = moeq.moeq_experts_forward_save(x, idx, wts, qg, qd)
        gx_s, gw_s = moeq.moeq_experts_backward_saved(idx, wts, qg, qd, gsv, dout)
        gx, gw = moeq.moeq_experts_backward(x, idx, wts, qg, qd, dout)
        torch.cuda.synchronize()
        assert torch.equal(gx_s, gx) and torch.equal(gw_s, gw)
