"""GPU: the experts forward, and the training pair that keeps the gate/up
pre-activations, captured in a HIP graph and replayed give the eager results
bit for bit on every replay (the library records no memset, so a captured
call is the same sequence of kernels).  Replays are separated by eager work
and synchronisations, as a serving or training loop would run them."""

import pytest
import torch

import bit_weight_quantization_moeq_amd as moeq
import moeq_synth as syn
from tests.gpu_common import require_native, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _native():
    require_native()


# T*K = 8 and 64 take the few-assignment path, 1024 the tiled one
@pytest.mark.parametrize("fmt", ["nf4", "int8", "nf4_dq"])
@pytest.mark.parametrize("T", [4, 32, 512])
def test_forward_graph_replays_match_eager(fmt, T):
    s = syn.SHAPES["tiny"]
    gu, dn, x, idx, wts = (t.cuda() for t in syn.layer_inputs(s, T, device="cpu"))
    if fmt == "int8":
        qg, qd = moeq.moeq_quantize_int8_rowwise(gu), moeq.moeq_quantize_int8_rowwise(dn)
    else:
        qg = moeq.moeq_quantize_nf4(gu, double_quant=fmt == "nf4_dq")
        qd = moeq.moeq_quantize_nf4(dn, double_quant=fmt == "nf4_dq")
    say(f"graph replay fmt={fmt} T={T}")
    out = torch.empty((T, s.H), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(moeq.moeq_experts_forward_workspace_bytes(T, s.K, qg, qd), dtype=torch.uint8, device="cuda")
    ref = moeq.moeq_experts_forward(x, idx, wts, qg, qd)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        moeq.moeq_experts_forward(x, idx, wts, qg, qd, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moeq.moeq_experts_forward(x, idx, wts, qg, qd, out=out, workspace=ws)
    for r in range(4):
        out.fill_(0)
        ws.fill_(0xFF)                       # stale workspace contents must not matter
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), (fmt, T, r)
        moeq.moeq_experts_forward(x[:1].contiguous(), idx[:1].contiguous(), wts[:1].contiguous(), qg, qd)


@pytest.mark.parametrize("fmt", ["nf4", "int8"])
def test_saved_training_step_graph_replays_match_eager(fmt):
    """moeq_experts_forward_save then moeq_experts_backward_saved captured as
    one graph: every replay reproduces the eager outputs, saved rows and
    gradients bit for bit."""
    s = syn.SHAPES["tiny"]
    T = 512
    gu, dn, x, idx, wts = (t.cuda() for t in syn.layer_inputs(s, T, device="cpu"))
    dout = syn.grad_output(T, s.H, device="cpu").cuda()
    if fmt == "int8":
        qg, qd = moeq.moeq_quantize_int8_rowwise(gu), moeq.moeq_quantize_int8_rowwise(dn)
    else:
        qg, qd = moeq.moeq_quantize_nf4(gu), moeq.moeq_quantize_nf4(dn)
    say(f"graph replay of the saved training step fmt={fmt} T={T}")
    ref_out, ref_gsv = moeq.moeq_experts_forward_save(x, idx, wts, qg, qd)
    ref_gx, ref_gw = moeq.moeq_experts_backward_saved(idx, wts, qg, qd, ref_gsv, dout)
    routed = int(((idx >= 0) & (idx < s.E)).sum())
    out, gsv = torch.empty_like(ref_out), torch.empty_like(ref_gsv)
    gx, gw = torch.empty_like(ref_gx), torch.empty_like(ref_gw)
    fws = torch.empty(moeq.moeq_experts_forward_workspace_bytes(T, s.K, qg, qd), dtype=torch.uint8, device="cuda")
    bws = torch.empty(moeq.moeq_experts_backward_saved_workspace_bytes(T, s.K, qg, qd), dtype=torch.uint8,
                      device="cuda")

    def step():
        moeq.moeq_experts_forward_save(x, idx, wts, qg, qd, out=out, gu_saved=gsv, workspace=fws)
        moeq.moeq_experts_backward_saved(idx, wts, qg, qd, gsv, dout, grad_hidden=gx, grad_weights=gw,
                                         workspace=bws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(4):
        for t in (out, gsv, gx, gw):
            t.fill_(0)
        fws.fill_(0xFF)
        bws.fill_(0xFF)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), (fmt, r, "out")
        assert torch.equal(gsv[:routed], ref_gsv[:routed]), (fmt, r, "gu_saved")
        assert torch.equal(gx, ref_gx) and torch.equal(gw, ref_gw), (fmt, r, "gradients")
        moeq.moeq_experts_forward(x[:1].contiguous(), idx[:1].contiguous(), wts[:1].contiguous(), qg, qd)
