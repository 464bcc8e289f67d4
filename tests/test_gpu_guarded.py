"""GPU parity on a shape whose experts span several full 256-row token tiles,
compared output by output against the fp64 oracle, with every output and
workspace buffer surrounded by guard bytes that must come back untouched
(an epilogue store past the last row or column, or past the end of the
workspace, would otherwise pass every numeric check).  unsloth-zoo issue
#850, Suggested fix: failures must be loud.

Shape: E = 4, H = 256, I = 128, top-2, T = 2048 -> 1024 assignments per expert
on average: four full 256-row tiles each, the 8-block (256-row) tile form and
the token-tile split with several tiles per expert on every column tile."""

import numpy as np
import pytest
import torch

import bit_weight_quantization_moeq_amd as moeq
import moeq_synth as syn
from oracle.backward import experts_backward
from oracle.bf16 import bf16_to_f32
from oracle.forward import experts_forward, rel_frobenius
from tests.gpu_common import host, host_bits, require_native, say
from tests.oracle_lazy import LazyDequant

pytestmark = pytest.mark.gpu
TOL = 5e-3
GUARD = 4096          # guard bytes on each side (a multiple of 256: keeps the buffer aligned)
PATTERN = 0xA5


@pytest.fixture(scope="module", autouse=True)
def _native():
    require_native()


class Guarded:
    """A tensor of `shape` / `dtype` inside a byte buffer with GUARD bytes of
    PATTERN on each side."""

    def __init__(self, shape, dtype, fill=None):
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        self.n = n
        self.buf = torch.full((n + 2 * GUARD,), PATTERN, dtype=torch.uint8, device="cuda")
        self.t = self.buf[GUARD:GUARD + n].view(dtype).view(shape)
        if fill is not None:
            self.t.fill_(fill)

    def check(self, label):
        torch.cuda.synchronize()
        lo, hi = self.buf[:GUARD], self.buf[GUARD + self.n:]
        assert bool((lo == PATTERN).all()), (label, "guard below the buffer overwritten")
        assert bool((hi == PATTERN).all()), (label, "guard above the buffer overwritten")


def _guarded_qweight(fmt, E, R, C):
    f = {"nf4": moeq.FMT_NF4, "nf4_dq": moeq.FMT_NF4_DQ, "int8": moeq.FMT_INT8_ROWWISE}[fmt]
    probe = moeq.QWeight(f, E, R, C, None, None)
    gs = [Guarded(shape, dtype) for _, shape, dtype in probe.layout()]
    q = moeq.QWeight(f, E, R, C, gs[0].t, gs[1].t, gs[2].t if len(gs) == 3 else None)
    return q, gs


def _quantize_guarded(w, fmt, label):
    q, gs = _guarded_qweight(fmt, *w.shape)
    if fmt == "int8":
        moeq.moeq_quantize_int8_rowwise(w, out=q)
    else:
        moeq.moeq_quantize_nf4(w, out=q)
    for g in gs:
        g.check(f"{label} quantize")
    return q


SHAPE = syn.MoEShape("tiles", E=4, H=256, I=128, K=2, fmt="nf4")
T_FULL = 2048


@pytest.mark.parametrize("fmt", ["nf4", "nf4_dq", "int8"])
def test_forward_full_output_multi_tile_guarded(fmt):
    s = SHAPE
    gu, dn, x, idx, wts = (t.cuda() for t in syn.layer_inputs(s, T_FULL, device="cpu"))
    say(f"guarded forward {fmt} E={s.E} H={s.H} I={s.I} T={T_FULL}")
    qg = _quantize_guarded(gu, fmt, fmt)
    qd = _quantize_guarded(dn, fmt, fmt)
    out = Guarded((T_FULL, s.H), torch.bfloat16, fill=0)
    need = moeq.moeq_experts_forward_workspace_bytes(T_FULL, s.K, qg, qd)
    ws = Guarded((need,), torch.uint8)
    moeq.moeq_experts_forward(x, idx, wts, qg, qd, out=out.t, workspace=ws.t)
    out.check(f"{fmt} out")
    ws.check(f"{fmt} workspace")
    counts = np.bincount(host(idx).reshape(-1), minlength=s.E)
    assert counts.min() > 3 * 256, counts                        # several full tiles per expert
    oracle_fmt = "nf4_dq" if fmt == "nf4_dq" else fmt
    ref = experts_forward(host_bits(x), host(idx), host(wts), LazyDequant(gu, oracle_fmt), LazyDequant(dn, oracle_fmt))
    got = bf16_to_f32(host_bits(out.t)).astype(np.float64)
    err = rel_frobenius(got, ref)
    # every token, not just the bulk: the worst token also stays close
    tok_err = np.linalg.norm(got - ref, axis=1) / np.linalg.norm(ref, axis=1)
    print(f"{fmt}: rel Frobenius {err:.3e}, worst token {tok_err.max():.3e}")
    assert err <= TOL and tok_err.max() <= 4 * TOL, (fmt, err, tok_err.max())


@pytest.mark.parametrize("fmt", ["nf4", "nf4_dq", "int8"])
def test_backward_full_output_multi_tile_guarded(fmt):
    s = SHAPE
    gu, dn, x, idx, wts = (t.cuda() for t in syn.layer_inputs(s, T_FULL, device="cpu"))
    dout = syn.grad_output(T_FULL, s.H, device="cuda")
    say(f"guarded backward {fmt} T={T_FULL}")
    qg = _quantize_guarded(gu, fmt, fmt)
    qd = _quantize_guarded(dn, fmt, fmt)
    gx = Guarded((T_FULL, s.H), torch.bfloat16, fill=0)
    gw = Guarded((T_FULL, s.K), torch.float32, fill=0)
    need = moeq.moeq_experts_backward_workspace_bytes(T_FULL, s.K, qg, qd)
    ws = Guarded((need,), torch.uint8)
    moeq.moeq_experts_backward(x, idx, wts, qg, qd, dout, grad_hidden=gx.t, grad_weights=gw.t, workspace=ws.t)
    for g, n in ((gx, "grad_hidden"), (gw, "grad_weights"), (ws, "workspace")):
        g.check(f"{fmt} {n}")
    of = "nf4_dq" if fmt == "nf4_dq" else fmt
    ref_x, ref_w = experts_backward(host_bits(x), host(idx), host(wts), LazyDequant(gu, of), LazyDequant(dn, of),
                                    host_bits(dout))
    ex = rel_frobenius(bf16_to_f32(host_bits(gx.t)).astype(np.float64), ref_x)
    ew = rel_frobenius(host(gw.t).astype(np.float64), ref_w)
    print(f"{fmt}: grad_hidden {ex:.3e}, grad_weights {ew:.3e}")
    assert ex <= TOL and ew <= TOL, (fmt, ex, ew)


# few-assignment path (T*K <= 512) and a ragged tiled case, all formats
@pytest.mark.parametrize("fmt", ["nf4", "nf4_dq", "int8"])
@pytest.mark.parametrize("T", [1, 16, 255, 777])
def test_forward_guarded_small(fmt, T):
    s = syn.SHAPES["tiny"]
    gu, dn, x, idx, wts = (t.cuda() for t in syn.layer_inputs(s, T, device="cpu"))
    say(f"guarded forward tiny {fmt} T={T}")
    qg = _quantize_guarded(gu, fmt, fmt)
    qd = _quantize_guarded(dn, fmt, fmt)
    out = Guarded((T, s.H), torch.bfloat16, fill=0)
    need = moeq.moeq_experts_forward_workspace_bytes(T, s.K, qg, qd)
    ws = Guarded((need,), torch.uint8)
    moeq.moeq_experts_forward(x, idx, wts, qg, qd, out=out.t, workspace=ws.t)
    out.check(f"{fmt} T={T} out")
    ws.check(f"{fmt} T={T} workspace")
    ref = experts_forward(host_bits(x), host(idx), host(wts), LazyDequant(gu, fmt), LazyDequant(dn, fmt))
    err = rel_frobenius(bf16_to_f32(host_bits(out.t)).astype(np.float64), ref)
    assert err <= TOL, (fmt, T, err)


@pytest.mark.parametrize("fmt", ["nf4", "nf4_dq", "int8"])
def test_dequantize_guarded(fmt):
    s = SHAPE
    w = syn.expert_weights(s.gate_up_shape, device="cuda")
    q = _quantize_guarded(w, fmt, fmt)
    out = Guarded(s.gate_up_shape, torch.bfloat16)
    moeq.moeq_dequantize(q, out=out.t)
    out.check(f"{fmt} dequantize")
    assert torch.isfinite(out.t.float()).all()


def test_router_and_routing_guarded():
    s = syn.SHAPES["olmoe"]
    T = 1000
    x = syn.hidden_states(T, s.H, device="cuda")
    gate = syn.router_weight(s.E, s.H, device="cuda")
    gi = Guarded((T, s.K), torch.int32)
    gwt = Guarded((T, s.K), torch.float32)
    moeq.moeq_router_topk(x, gate, s.K, top_k_index=gi.t, top_k_weights=gwt.t)
    gi.check("router idx")
    gwt.check("router weights")
    need = moeq.moeq_route_workspace_bytes(T, s.K, s.E)
    ws = Guarded((need,), torch.uint8)
    moeq.moeq_route_buckets(gi.t, s.E, workspace=ws.t)
    ws.check("route workspace")
