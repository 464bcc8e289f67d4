"""GPU parity: the routed experts forward from packed storage against the fp64
oracle on the same dequantized weights.  Bar: relative Frobenius error <= 5e-3
(the accuracy bound the method's forward is held to); runs are bit-identical."""

import numpy as np
import pytest
import torch

import bit_weight_quantization_moeq_amd as moeq
import moeq_synth as syn
from oracle.bf16 import bf16_to_f32
from oracle.forward import experts_forward, rel_frobenius
from tests.gpu_common import host, host_bits, require_native, say
from tests.oracle_lazy import LazyDequant

pytestmark = pytest.mark.gpu
TOL = 5e-3


@pytest.fixture(scope="module", autouse=True)
def _native():
    require_native()


def _quantize(w, fmt):
    return moeq.moeq_quantize_nf4(w) if fmt == "nf4" else moeq.moeq_quantize_int8_rowwise(w)


def _compare(x, idx, wts, gu, dn, fmt, out, tokens, cols=None, label=""):
    """Oracle on the sampled tokens (and output columns) vs the GPU output."""
    tokens = np.asarray(tokens)
    xs = host_bits(x)[tokens]
    ids = host(idx)[tokens]
    ws = host(wts)[tokens]
    rows = None if cols is None else torch.from_numpy(np.asarray(cols)).to(gu.device)
    ref = experts_forward(xs, ids, ws, LazyDequant(gu, fmt), LazyDequant(dn, fmt, rows=rows))
    got = bf16_to_f32(host_bits(out)[tokens]).astype(np.float64)
    if cols is not None:
        got = got[:, np.asarray(cols)]
    err = rel_frobenius(got, ref)
    print(f"{label}: rel Frobenius error {err:.3e}")
    assert err <= TOL, (label, err)
    return err


def _layer(name, T, device, fmt=None):
    s = syn.SHAPES[name]
    fmt = fmt or s.fmt
    gu, dn, x, idx, wts = syn.layer_inputs(s, T, device=device)
    gu, dn, x, idx, wts = (t.cuda() for t in (gu, dn, x, idx, wts))
    return s, fmt, gu, dn, x, idx, wts


@pytest.mark.parametrize("fmt", ["nf4", "int8"])
def test_forward_tiny_full(fmt):
    s, fmt, gu, dn, x, idx, wts = _layer("tiny", 64, "cpu", fmt)
    say(f"forward tiny fmt={fmt}")
    qg, qd = _quantize(gu, fmt), _quantize(dn, fmt)
    out = moeq.moeq_experts_forward(x, idx, wts, qg, qd)
    torch.cuda.synchronize()
    _compare(x, idx, wts, gu, dn, fmt, out, np.arange(64), label=f"tiny {fmt}")


# (shape, T, sampled tokens, sampled output columns or None)
CASES = [
    ("olmoe", 1, 1, None), ("olmoe", 32, 3, None), ("olmoe", 4096, 2, 512),
    ("qwen3", 1, 1, None), ("qwen3", 64, 2, None), ("qwen3", 8192, 2, 512),
    ("gptoss", 16, 3, None), ("gptoss", 2048, 2, 720),
    ("mixtral", 1, 1, 256), ("mixtral", 512, 1, 256), ("mixtral", 16384, 1, 256),
]


@pytest.mark.parametrize("name,T,ns,nc", CASES)
def test_forward_workloads_sampled(name, T, ns, nc):
    s, fmt, gu, dn, x, idx, wts = _layer(name, T, "cuda")
    say(f"forward {name} T={T} fmt={fmt}")
    qg, qd = _quantize(gu, fmt), _quantize(dn, fmt)
    out = moeq.moeq_experts_forward(x, idx, wts, qg, qd)
    torch.cuda.synchronize()
    rng = np.random.default_rng(T)
    tokens = np.sort(rng.choice(T, ns, replace=False))
    cols = None if nc is None else np.sort(rng.choice(s.H, nc, replace=False))
    _compare(x, idx, wts, gu, dn, fmt, out, tokens, cols, label=f"{name} T={T}")
    assert torch.isfinite(out.float()).all()


# NF4 rows with an odd number of 64-blocks (H = 320: 5, I = 192: 3) and with
# an even number that is not a multiple of 4 (H = 384: 6, I = 128: 2): the
# few-assignment path loads the absmax of two K steps at once only when the
# count is even.  T*K = 2 and 32 take the few-assignment path, 600 the tiled one.
@pytest.mark.parametrize("H,I", [(320, 192), (384, 128)])
@pytest.mark.parametrize("T", [1, 16, 300])
def test_forward_nf4_block_counts(H, I, T):
    s = syn.MoEShape("blocks", E=4, H=H, I=I, K=2, fmt="nf4")
    gu, dn, x, idx, wts = (t.cuda() for t in syn.layer_inputs(s, T, device="cpu"))
    say(f"forward nf4 H={H} I={I} T={T}")
    qg, qd = moeq.moeq_quantize_nf4(gu), moeq.moeq_quantize_nf4(dn)
    out = moeq.moeq_experts_forward(x, idx, wts, qg, qd)
    torch.cuda.synchronize()
    _compare(x, idx, wts, gu, dn, "nf4", out, np.arange(T), label=f"nf4 H={H} I={I} T={T}")


# Few touched experts and a long down K (E = 2, H = 256, I = 4096, top-1):
# the down launch splits K across workgroups as well (4 ways here), each
# writing its own slice of y for the combine to add; every output element.
@pytest.mark.parametrize("fmt", ["nf4", "int8"])
@pytest.mark.parametrize("T", [1, 2])
def test_forward_down_split_full(fmt, T):
    s = syn.MoEShape("longk", E=2, H=256, I=4096, K=1, fmt=fmt)
    gu, dn, x, idx, wts = (t.cuda() for t in syn.layer_inputs(s, T, device="cpu"))
    say(f"forward down split fmt={fmt} T={T}")
    out = moeq.moeq_experts_forward(x, idx, wts, _quantize(gu, fmt), _quantize(dn, fmt))
    torch.cuda.synchronize()
    _compare(x, idx, wts, gu, dn, fmt, out, np.arange(T), label=f"down split {fmt} T={T}")


# The down GEMM splits each token tile's rows in two when it has at most one
# work item per CU even at the upper bound on token tiles (E = 8 wide experts
# and 600 tokens here: 12 tiles x 16 column tiles); with 4096 tokens it does
# not.  An output element keeps one writer and one K order, so the tokens of
# the small batch come out bit-identical inside the large one; the split batch
# also meets the oracle.
@pytest.mark.parametrize("fmt", ["nf4", "int8"])
def test_forward_down_row_split_keeps_bits(fmt):
    s = syn.MoEShape("wide", E=8, H=4096, I=256, K=2, fmt=fmt)
    gu, dn, x, idx, wts = (t.cuda() for t in syn.layer_inputs(s, 4096, device="cpu"))
    qg, qd = _quantize(gu, fmt), _quantize(dn, fmt)
    say(f"forward down row split fmt={fmt}")
    small = moeq.moeq_experts_forward(x[:600].contiguous(), idx[:600].contiguous(), wts[:600].contiguous(), qg, qd)
    large = moeq.moeq_experts_forward(x, idx, wts, qg, qd)
    torch.cuda.synchronize()
    assert torch.equal(small, large[:600])
    _compare(x, idx, wts, gu, dn, fmt, small, np.arange(0, 600, 9), label=f"down row split {fmt}")


# The path boundary: T*K = 512 is the last few-assignment batch, 514 the
# first tiled one; every output element of both is checked.
@pytest.mark.parametrize("T", [256, 257])
@pytest.mark.parametrize("fmt", ["nf4", "int8"])
def test_forward_path_boundary_full(fmt, T):
    s = syn.SHAPES["tiny"]
    gu, dn, x, idx, wts = (t.cuda() for t in syn.layer_inputs(s, T, device="cpu"))
    say(f"forward path boundary fmt={fmt} T={T} (T*K={T * s.K})")
    qg, qd = _quantize(gu, fmt), _quantize(dn, fmt)
    out = moeq.moeq_experts_forward(x, idx, wts, qg, qd)
    torch.cuda.synchronize()
    _compare(x, idx, wts, gu, dn, fmt, out, np.arange(T), label=f"boundary {fmt} T={T}")


# The expert-count extremes on both paths, every output element: 1024
# experts (32 bitmap words in the few-assignment path, 1024 per-expert tile
# counts in the routing) and a single expert with top-1 (every assignment in
# one expert: one workgroup's list holds them all, the tiles cover them all).
@pytest.mark.parametrize("T", [100, 600])
@pytest.mark.parametrize("E,K", [(1024, 2), (1, 1)])
def test_forward_expert_count_extremes_full(E, K, T):
    s = syn.MoEShape("wide", E=E, H=128, I=64, K=K, fmt="nf4")
    gu, dn, x, idx, wts = (t.cuda() for t in syn.layer_inputs(s, T, device="cpu"))
    if E > 1:
        assert int(idx.max()) >= 900  # the high experts are used
    say(f"forward E={s.E} K={K} T={T}")
    qg, qd = moeq.moeq_quantize_nf4(gu), moeq.moeq_quantize_nf4(dn)
    out = moeq.moeq_experts_forward(x, idx, wts, qg, qd)
    torch.cuda.synchronize()
    _compare(x, idx, wts, gu, dn, "nf4", out, np.arange(T), label=f"E={s.E} K={K} T={T}")


# T*K = 387 takes the few-assignment path, 900 the tiled one
@pytest.mark.parametrize("T", [129, 300])
@pytest.mark.parametrize("fmt", ["nf4", "int8"])
def test_forward_edge_routing(fmt, T):
    s = syn.SHAPES["tiny"]
    gu, dn, x, _, _ = syn.layer_inputs(s, T, device="cpu")
    gu, dn, x = gu.cuda(), dn.cuda(), x.cuda()
    qg, qd = _quantize(gu, fmt), _quantize(dn, fmt)
    rng = np.random.default_rng(301)
    idx = rng.integers(-2, s.E + 2, (T, 3)).astype(np.int32)      # duplicates and unrouted
    idx[5] = [4, 4, 4]
    wts = rng.uniform(-1, 1, (T, 3)).astype(np.float32)
    idx_d, wts_d = torch.from_numpy(idx).cuda(), torch.from_numpy(wts).cuda()
    say(f"forward edge routing fmt={fmt} T={T}")
    out = moeq.moeq_experts_forward(x, idx_d, wts_d, qg, qd)
    torch.cuda.synchronize()
    _compare(x, idx_d, wts_d, gu, dn, fmt, out, np.arange(T), label=f"edge {fmt} T={T}")
    # a token with no routed assignment gets exactly zero
    idx[7] = [-1, s.E, 99]
    out2 = moeq.moeq_experts_forward(x, torch.from_numpy(idx).cuda(), wts_d, qg, qd)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out2[7]) == 0
    # K = 1, T = 1
    out1 = moeq.moeq_experts_forward(x[:1].contiguous(), idx_d[:1, :1].contiguous(),
                                     wts_d[:1, :1].contiguous(), qg, qd)
    torch.cuda.synchronize()
    _compare(x[:1], idx_d[:1, :1], wts_d[:1, :1], gu, dn, fmt, out1, [0], label=f"T=1 K=1 {fmt}")


# K larger than a wave: T*K = 280 takes the few-assignment path, 560 the tiled one
@pytest.mark.parametrize("T", [4, 8])
def test_forward_large_top_k(T):
    s = syn.SHAPES["tiny"]
    gu, dn, x, _, _ = syn.layer_inputs(s, T, device="cpu")
    gu, dn, x = gu.cuda(), dn.cuda(), x.cuda()
    qg, qd = moeq.moeq_quantize_nf4(gu), moeq.moeq_quantize_nf4(dn)
    rng = np.random.default_rng(17)
    K = 70
    idx = rng.integers(-1, s.E + 1, (T, K)).astype(np.int32)
    wts = rng.uniform(-0.2, 0.2, (T, K)).astype(np.float32)
    idx_d, wts_d = torch.from_numpy(idx).cuda(), torch.from_numpy(wts).cuda()
    say(f"forward large top-k T={T} K={K}")
    out = moeq.moeq_experts_forward(x, idx_d, wts_d, qg, qd)
    torch.cuda.synchronize()
    _compare(x, idx_d, wts_d, gu, dn, "nf4", out, np.arange(T), label=f"K={K} T={T}")


def test_forward_empty_batch():
    s = syn.SHAPES["tiny"]
    gu, dn = syn.expert_weights(s.gate_up_shape, device="cuda"), syn.expert_weights(s.down_shape, device="cuda")
    qg, qd = moeq.moeq_quantize_nf4(gu), moeq.moeq_quantize_nf4(dn)
    x = torch.empty((0, s.H), dtype=torch.bfloat16, device="cuda")
    idx = torch.empty((0, 2), dtype=torch.int32, device="cuda")
    w = torch.empty((0, 2), dtype=torch.float32, device="cuda")
    out = moeq.moeq_experts_forward(x, idx, w, qg, qd)
    assert out.shape == (0, s.H)


def test_forward_is_bit_identical_run_to_run():
    s, fmt, gu, dn, x, idx, wts = _layer("olmoe", 4096, "cuda")
    qg, qd = _quantize(gu, fmt), _quantize(dn, fmt)
    say("forward determinism olmoe T=4096")

    def fwd(lo, hi):
        return moeq.moeq_experts_forward(x[lo:hi].contiguous(), idx[lo:hi].contiguous(),
                                         wts[lo:hi].contiguous(), qg, qd)
    a = moeq.moeq_experts_forward(x, idx, wts, qg, qd)
    b = moeq.moeq_experts_forward(x, idx, wts, qg, qd)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    # Within each path a token's output does not depend on the batch it is in:
    # tiled path (T*K > 512) ...
    c = fwd(100, 400)
    torch.cuda.synchronize()
    assert torch.equal(c[:64], a[100:164])
    # ... and the few-assignment path (T*K <= 512), run to run as well
    d1, d2, d3 = fwd(100, 164), fwd(100, 164), fwd(100, 132)
    torch.cuda.synchronize()
    assert torch.equal(d1, d2)
    assert torch.equal(d3, d1[:32])
    # The two paths add the K products in different orders, and the tiled
    # path rounds each weighted product to bf16 before the sum.  Each is
    # within TOL of the oracle (tested above), which by the triangle
    # inequality only bounds their gap by 2 TOL.  The gap itself is that
    # rounding: independent errors of at most 2^-8 of each weighted row
    # (bf16 round to nearest), about 2^-8 / sqrt(3) = 2.3e-3 of the rows in
    # root mean square, and the K rows of a token add with little
    # cancellation here (positive softmax weights over independent
    # experts), so the gap is expected near 2.3e-3 (measured 2.7e-3).  The
    # assertion allows twice that expectation (4.5e-3, inside TOL).
    err = rel_frobenius(bf16_to_f32(host_bits(d1)).astype(np.float64),
                        bf16_to_f32(host_bits(a[100:164])).astype(np.float64))
    print(f"few-assignment vs tiled path: rel Frobenius {err:.3e}")
    assert err <= 2 * 2.0 ** -8 / np.sqrt(3.0)


def test_forward_rejects_mixed_formats():
    s = syn.SHAPES["tiny"]
    gu, dn = syn.expert_weights(s.gate_up_shape, device="cuda"), syn.expert_weights(s.down_shape, device="cuda")
    qg, qd = moeq.moeq_quantize_nf4(gu), moeq.moeq_quantize_int8_rowwise(dn)
    x = syn.hidden_states(4, s.H, device="cuda")
    idx, w = syn.routing(4, 2, s.E, device="cuda")
    with pytest.raises(moeq.MoeqError) as ei:
        moeq.moeq_experts_forward(x, idx, w, qg, qd)
    assert ei.value.status == -4
