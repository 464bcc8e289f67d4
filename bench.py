#!/usr/bin/env python3
"""Benchmark of the NF4 MoE-experts hot path on one MI355X.

One step = quantize-on-load of one OLMoE-1B-7B-shaped MoE layer (gate_up
[64, 2048, 2048] and down [64, 2048, 1024] bf16 ~ N(0, 0.02) -> NF4,
blocksize 64) followed by the routed experts forward of T = 4096 tokens with
top-8 uniform routing straight from that packed storage (routing buckets,
gate_up grouped GEMM + SwiGLU, down grouped GEMM, k-ordered combine).

Printed (one JSON line): ``value`` = experts-forward tokens/s (HIP events
around the forward of the timed steps that record no stage events),
``quantize_GBps`` = quantize algorithmic bytes / quantize time (events),
``ms_per_step`` = wall time per whole step; ``roofline`` for the dominant
kernel of the step, from the stage events recorded on every other timed step;
``device_copy_GBps`` = a plain 1 GiB device copy, the measured HBM ceiling;
``decode`` = forward-only figures at T = 1 and 32, streaming the weights from
HBM; ``backward`` = the gradients through the frozen packed experts for the
same batch; ``router`` = the router front-end (gate GEMM, softmax, top-K)
on the same batch; ``offload`` = the forward with the packed experts in
pinned host memory and the next layer prefetched; ``double_quant`` = the
same quantize, forward, decode and backward with double-quantized absmax;
``codec`` = row-wise int8 quantize and the two dequantizes; ``load`` = the
quantize-on-load pass over 16 OLMoE-shaped and 48 Qwen3-shaped layers;
``cpu_baseline`` = the CPU oracle on a bounded sample of the same workload.
Inputs are seeded synthetic tensors resident in HBM before the timed region.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "NF4 experts-forward tokens/s + quantize GB/s, fraction of HBM/MFMA peak"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
NF4_BYTES_PER_ELEM = 2.0 + 0.5 + 4.0 / 64   # bf16 read + packed code + absmax share
NF4_PACKED_BYTES_PER_ELEM = 0.5 + 4.0 / 64  # what the forward streams per weight element
# NF4 with double-quantized absmax: one code byte per 64-block, 4 bytes per 256 blocks
DQ_PACKED_BYTES_PER_ELEM = 0.5 + 1.0 / 64 + 4.0 / (64 * 256)
DQ_BYTES_PER_ELEM = 2.0 + DQ_PACKED_BYTES_PER_ELEM


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="olmoe")
    ap.add_argument("--T", type=int, default=4096)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-codec", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-router", action="store_true")
    ap.add_argument("--no-offload", action="store_true")
    ap.add_argument("--no-double-quant", action="store_true")
    ap.add_argument("--no-load", action="store_true")
    ap.add_argument("--configs", action="store_true",
                    help="also time the experts forward at every configured shape and batch (off by default)")
    return ap.parse_args()


def forward_bytes_flops(s, idx_np, T, packed_bpe=NF4_PACKED_BYTES_PER_ELEM):
    """Algorithmic bytes and flops of one forward: touched experts' packed weights
    once, x in and out once, the routing inputs once; 6*T*K*H*I flops."""
    U = len(set(idx_np.reshape(-1).tolist()))
    wbytes = U * 3 * s.H * s.I * packed_bpe
    abytes = 2 * T * s.H * 2 + T * s.K * 8
    flops = 6.0 * T * s.K * s.H * s.I
    return wbytes + abytes, flops, U


PROFILE_KERNEL = {"g1_gate_up_swiglu": "g1_kernel<1>", "g2_down": "g2_kernel<1>",
                  "quantize_gate_up": "nf4_quantize_kernel", "quantize_down": "nf4_quantize_kernel",
                  "combine": "combine_kernel"}


def measured_traffic(stage):
    """HBM bytes per launch of the stage's kernel from the committed
    FETCH_SIZE/WRITE_SIZE summaries under profiles/, or None when there is
    none or the kernel sources changed since the counters were taken."""
    import glob
    import re

    from profsum import source_hash
    want = PROFILE_KERNEL.get(stage)
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*_traffic.md"))):
        m = re.search(r"```json\n(.*?)\n```", open(path).read(), re.S)
        if not m:
            continue
        block = json.loads(m.group(1))
        if block.get("kernel") == want and block.get("source_sha256") == source_hash():
            return float(block["traffic_bytes"])
    return None


def new_events(torch, n):
    """n timing events on torch's current stream, created now (one record each)
    so their raw hipEvent_t handles can be handed to the library."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in ev:
        e.record()
    return ev


def cpu_baseline(s, gu, dn, x, idx, wts, T, n_quant=32):
    """The oracle, untuned, on a bounded sample (~10 s of CPU work): NF4
    quantize of the first `n_quant` experts' gate_up and down, and the forward
    of all T tokens with their expert indices folded onto experts 0 and 1
    (identical work per assignment)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import moeq_synth as syn
    from oracle.forward import experts_forward
    from oracle.nf4 import nf4_dequantize, nf4_quantize

    gbits = syn.bf16_bits(gu[:n_quant])
    dbits = syn.bf16_bits(dn[:n_quant])
    t0 = time.perf_counter()
    qg = nf4_quantize(gbits)
    qd = nf4_quantize(dbits)
    tq = time.perf_counter() - t0
    qelems = gbits.size + dbits.size
    del gbits, dbits
    dg = nf4_dequantize(qg[0][:2], qg[1][:2])
    dd = nf4_dequantize(qd[0][:2], qd[1][:2])
    xs = syn.bf16_bits(x)
    ids = idx.cpu().numpy() % 2
    ws = wts.cpu().numpy()
    t0 = time.perf_counter()
    experts_forward(xs, ids, ws, dg, dd)
    tf = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {
        "value": T / tf, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
        "quantize_GBps": qelems * NF4_BYTES_PER_ELEM / tq / 1e9,
        "sample": (f"NF4 quantize of experts 0-{n_quant - 1} of gate_up and down ({qelems} elements, "
                   f"{tq:.1f} s); fp64 forward of all T={T} tokens of the top-{s.K} workload with expert "
                   f"indices folded onto experts 0 and 1 ({tf:.1f} s); numpy/BLAS threads={threads}, "
                   f"host cpu_count={os.cpu_count()}"),
    }


def device_copy_GBps(torch, dev, nbytes=1 << 30, reps=10):
    """Measured HBM bandwidth of a plain device copy (read + write bytes / time)."""
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    del src, dst
    return 2.0 * nbytes / (ms * 1e-3) / 1e9


def clone_q(moeq, q):
    t = [u.clone() for u in q._tensors()]
    return moeq.QWeight(q.format, q.num_experts, q.rows, q.cols, t[0], t[1], t[2] if len(t) == 3 else None)


def decode_figures(torch, np, moeq, syn, s, qg, qd, dev, copy_GBps, layers=4, calls=48,
                   packed_bpe=NF4_PACKED_BYTES_PER_ELEM):
    """Forward-only figures at T = 1 and 32.  The calls rotate over `layers`
    copies of the quantized layer (together larger than the last-level cache),
    so every call streams its experts' codes from HBM as in a many-layer model;
    `calls` back-to-back calls sit between one pair of events.  A second pass
    with stage events gives the per-kernel split."""
    stack = [(qg, qd)]
    for _ in range(layers - 1):
        stack.append((clone_q(moeq, qg), clone_q(moeq, qd)))
    dec = {}
    for Td in (1, 32):
        xd = syn.hidden_states(Td, s.H, device=dev, layer=1)
        idd, wd = syn.routing(Td, s.K, s.E, kind=s.routing, device=dev, layer=1)
        od = torch.empty((Td, s.H), dtype=torch.bfloat16, device=dev)
        wsd = torch.empty(moeq.moeq_experts_forward_workspace_bytes(Td, s.K, qg, qd), dtype=torch.uint8, device=dev)
        for r in range(2 * layers):
            g, d = stack[r % layers]
            moeq.moeq_experts_forward(xd, idd, wd, g, d, out=od, workspace=wsd)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for r in range(calls):
            g, d = stack[r % layers]
            moeq.moeq_experts_forward(xd, idd, wd, g, d, out=od, workspace=wsd)
        b.record()
        torch.cuda.synchronize()
        tms = a.elapsed_time(b) / calls
        reps = 4 * layers
        evd = [new_events(torch, 5) for _ in range(reps)]
        for r in range(reps):
            g, d = stack[r % layers]
            moeq.moeq_experts_forward(xd, idd, wd, g, d, out=od, workspace=wsd,
                                      stage_events=[h.cuda_event for h in evd[r]])
        torch.cuda.synchronize()
        kms = {n: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evd[layers:]]))
               for j, n in enumerate(["route", "g1_gate_up_swiglu", "g2_down", "combine"])}
        nb, fl, Ud = forward_bytes_flops(s, idd.cpu().numpy(), Td, packed_bpe)
        dec[f"T{Td}"] = {"tokens_per_s": Td / (tms * 1e-3), "forward_ms": tms,
                         "packed_GBps": nb / (tms * 1e-3) / 1e9,
                         "hbm_frac": nb / (tms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                         "copy_frac": nb / (tms * 1e-3) / 1e9 / copy_GBps,
                         "touched_experts": Ud, "stage_ms_with_events": kms,
                         "timing": f"{calls} back-to-back calls over {layers} layer copies"}
    return dec


def backward_figures(torch, np, moeq, syn, s, qg, qd, x, idx, wts, dev, reps=10):
    """Gradients of the experts block (hidden states and routing weights, the
    packed weights frozen) for the same layer and batch: events around
    back-to-back calls.  Work: the gate_up GEMM recomputed (4 T K H I flops),
    the unweighted down GEMM (2), the down^T GEMM (2) and the gate_up^T GEMM
    (4): 12 T K H I flops."""
    T = x.shape[0]
    dout = syn.grad_output(T, s.H, device=dev)
    ws = torch.empty(moeq.moeq_experts_backward_workspace_bytes(T, s.K, qg, qd), dtype=torch.uint8, device=dev)
    gx = torch.empty((T, s.H), dtype=torch.bfloat16, device=dev)
    gw = torch.empty((T, s.K), dtype=torch.float32, device=dev)
    for _ in range(2):
        moeq.moeq_experts_backward(x, idx, wts, qg, qd, dout, grad_hidden=gx, grad_weights=gw, workspace=ws)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        moeq.moeq_experts_backward(x, idx, wts, qg, qd, dout, grad_hidden=gx, grad_weights=gw, workspace=ws)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    flops = 12.0 * T * s.K * s.H * s.I
    return {"workload": f"same layer and batch (T={T}), incoming gradient ~ N(0, 1) bf16",
            "ms": ms, "tokens_per_s": T / (ms * 1e-3), "TFLOPs": flops / (ms * 1e-3) / 1e12,
            "mfma_frac": flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            "flops": "12 T K H I (gate_up recompute 4, unweighted down 2, down^T 2, gate_up^T 4)"}


def router_figures(torch, np, moeq, syn, s, x, dev, copy_GBps, reps=20):
    """Router front-end on the benchmark batch: a bf16 gate [E, H] -> top-K
    indices and weights.  HBM-bound: the hidden states are read once
    (T H 2 B), the gate once, the outputs written once (8 T K B)."""
    T = x.shape[0]
    gate = syn.router_weight(s.E, s.H, device=dev)
    idx = torch.empty((T, s.K), dtype=torch.int32, device=dev)
    w = torch.empty((T, s.K), dtype=torch.float32, device=dev)
    moeq.moeq_router_topk(x, gate, s.K, top_k_index=idx, top_k_weights=w)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        moeq.moeq_router_topk(x, gate, s.K, top_k_index=idx, top_k_weights=w)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    nbytes = 2.0 * T * s.H + 2.0 * s.E * s.H + 8.0 * T * s.K
    return {"workload": f"T={T}, gate [{s.E}, {s.H}] bf16, top-{s.K}", "ms": ms,
            "GBps": nbytes / (ms * 1e-3) / 1e9, "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "TFLOPs": 2.0 * T * s.E * s.H / (ms * 1e-3) / 1e12}


def offload_figures(torch, np, moeq, s, qg, qd, x, idx, wts, dev, fwd_ms, layers=4, passes=2):
    """Expert-granularity offload: `layers` copies of the benchmark layer in
    pinned host memory, two device slots, layer N+1 prefetched on a side
    stream during layer N's forward.  Reported per layer: the resident
    forward, the host-to-device copy alone, and the offloaded forward in
    steady state; `overlap` = (resident + copy - offloaded) / min(resident,
    copy), 1 when the shorter of the two is fully hidden."""
    from bit_weight_quantization_moeq_amd.offload import ExpertOffload
    off = ExpertOffload([(qg, qd)] * layers, dev)
    out = torch.empty((x.shape[0], s.H), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(moeq.moeq_experts_forward_workspace_bytes(x.shape[0], s.K, qg, qd), dtype=torch.uint8,
                     device=dev)
    # the copy alone (side stream)
    hg, hd = off.host[1]
    dg, dd = off.slots[1]
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(off.copy_stream):
        a.record()
        for _ in range(3):
            moeq.moeq_qweight_copy_async(hg, dg)
            moeq.moeq_qweight_copy_async(hd, dd)
        b.record()
    torch.cuda.synchronize()
    copy_ms = a.elapsed_time(b) / 3
    off.filled = [None, None]
    for layer in range(layers):                      # warm
        off.forward(layer, x, idx, wts, out=out, workspace=ws)
    torch.cuda.synchronize()
    a.record()
    for _ in range(passes):
        for layer in range(layers):
            off.forward(layer, x, idx, wts, out=out, workspace=ws)
    b.record()
    torch.cuda.synchronize()
    off_ms = a.elapsed_time(b) / (passes * layers)
    nbytes = off.layer_bytes(0)
    return {"workload": f"{layers} copies of the benchmark layer in pinned host memory, T={x.shape[0]}",
            "layer_bytes": nbytes, "copy_ms": copy_ms, "copy_GBps": nbytes / (copy_ms * 1e-3) / 1e9,
            "resident_forward_ms": fwd_ms, "offloaded_forward_ms": off_ms,
            "overlap": (fwd_ms + copy_ms - off_ms) / min(fwd_ms, copy_ms)}


def double_quant_figures(torch, np, moeq, syn, s, gu, dn, x, idx, wts, dev, copy_GBps, reps=10):
    """The same layer with double-quantized absmax: quantize-on-load into that
    format, the T-token forward, the decode forwards and the backward, each
    decoding the absmax inside its kernels; plus the storage of both formats."""
    qg = moeq.QWeight.empty(moeq.FMT_NF4_DQ, *s.gate_up_shape, device=dev)
    qd = moeq.QWeight.empty(moeq.FMT_NF4_DQ, *s.down_shape, device=dev)
    T = x.shape[0]
    out = torch.empty((T, s.H), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(moeq.moeq_experts_forward_workspace_bytes(T, s.K, qg, qd), dtype=torch.uint8, device=dev)

    def timed(fn):
        fn()
        fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    q_ms = timed(lambda: (moeq.moeq_quantize_nf4(gu, out=qg), moeq.moeq_quantize_nf4(dn, out=qd)))
    nel = gu.numel() + dn.numel()
    qb = nel * DQ_BYTES_PER_ELEM
    f_ms = timed(lambda: moeq.moeq_experts_forward(x, idx, wts, qg, qd, out=out, workspace=ws))
    nf4_bytes = nel * NF4_PACKED_BYTES_PER_ELEM
    return {"workload": "same layer and batch, absmax double-quantized (8-bit code per block, fp32 per 256 blocks)",
            "quantize_ms": q_ms, "quantize_GBps": qb / (q_ms * 1e-3) / 1e9,
            "quantize_hbm_frac": qb / (q_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "quantize_copy_frac": qb / (q_ms * 1e-3) / 1e9 / copy_GBps,
            "forward_ms": f_ms, "tokens_per_s": T / (f_ms * 1e-3),
            "decode": decode_figures(torch, np, moeq, syn, s, qg, qd, dev, copy_GBps,
                                     packed_bpe=DQ_PACKED_BYTES_PER_ELEM),
            "backward": backward_figures(torch, np, moeq, syn, s, qg, qd, x, idx, wts, dev),
            "layer_bytes": {"nf4": nf4_bytes, "nf4_double_quant": float(qg.nbytes() + qd.nbytes()),
                            "bits_per_weight_nf4": 8 * NF4_PACKED_BYTES_PER_ELEM,
                            "bits_per_weight_double_quant": 8.0 * (qg.nbytes() + qd.nbytes()) / nel}}


def load_figures(torch, np, moeq, syn, dev, copy_GBps):
    """Quantize-on-load of whole models' expert stacks: the OLMoE shape's 16
    layers and the Qwen3 shape's 48 layers, NF4.  One layer's bf16 weights
    are generated once and quantized `layers` times back-to-back (every layer
    streams the same bytes from HBM; a layer's 1.2 GB outgrows every cache),
    with events around the whole pass."""
    out = {}
    for name, layers in (("olmoe", 16), ("qwen3", 48)):
        s = syn.SHAPES[name]
        gu = syn.expert_weights(s.gate_up_shape, tensor=syn.GATE_UP, device=dev)
        dn = syn.expert_weights(s.down_shape, tensor=syn.DOWN, device=dev)
        qg = moeq.QWeight.empty(moeq.FMT_NF4, *s.gate_up_shape, device=dev)
        qd = moeq.QWeight.empty(moeq.FMT_NF4, *s.down_shape, device=dev)
        moeq.moeq_quantize_nf4(gu, out=qg)
        moeq.moeq_quantize_nf4(dn, out=qd)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(layers):
            moeq.moeq_quantize_nf4(gu, out=qg)
            moeq.moeq_quantize_nf4(dn, out=qd)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        nel = layers * (gu.numel() + dn.numel())
        out[name] = {"layers": layers, "ms": ms, "bf16_GB": nel * 2 / 1e9,
                     "packed_GB": layers * (qg.nbytes() + qd.nbytes()) / 1e9,
                     "GBps": nel * NF4_BYTES_PER_ELEM / (ms * 1e-3) / 1e9,
                     "hbm_frac": nel * NF4_BYTES_PER_ELEM / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS}
        del gu, dn, qg, qd
    return out


def codec_figures(torch, np, moeq, syn, dev, copy_GBps, reps=5):
    """Row-wise int8 quantize on the gpt-oss-shaped experts and dequantize of
    both formats: algorithmic bytes / event time."""
    out = {}

    def timed(fn):
        fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    g = syn.SHAPES["gptoss"]
    wg = syn.expert_weights(g.gate_up_shape, tensor=syn.GATE_UP, device=dev)
    wd = syn.expert_weights(g.down_shape, tensor=syn.DOWN, device=dev)
    q8g = moeq.QWeight.empty(moeq.FMT_INT8_ROWWISE, *g.gate_up_shape, device=dev)
    q8d = moeq.QWeight.empty(moeq.FMT_INT8_ROWWISE, *g.down_shape, device=dev)
    ms = timed(lambda: (moeq.moeq_quantize_int8_rowwise(wg, out=q8g), moeq.moeq_quantize_int8_rowwise(wd, out=q8d)))
    nel = wg.numel() + wd.numel()
    nrow = g.E * (g.gate_up_shape[1] + g.down_shape[1])
    b = 3.0 * nel + 4.0 * nrow
    out["int8_quantize"] = {"workload": f"gpt-oss-shaped gate_up {list(g.gate_up_shape)} + down {list(g.down_shape)}",
                            "ms": ms, "GBps": b / (ms * 1e-3) / 1e9, "hbm_frac": b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                            "copy_frac": b / (ms * 1e-3) / 1e9 / copy_GBps}
    dq = torch.empty(g.gate_up_shape, dtype=torch.bfloat16, device=dev)
    ms = timed(lambda: moeq.moeq_dequantize(q8g, out=dq))
    b = 3.0 * wg.numel() + 4.0 * g.E * g.gate_up_shape[1]
    out["int8_dequantize"] = {"workload": f"gpt-oss-shaped gate_up {list(g.gate_up_shape)}", "ms": ms,
                              "GBps": b / (ms * 1e-3) / 1e9, "hbm_frac": b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS}
    q4 = moeq.moeq_quantize_nf4(wg)
    ms = timed(lambda: moeq.moeq_dequantize(q4, out=dq))
    b = wg.numel() * NF4_BYTES_PER_ELEM
    out["nf4_dequantize"] = {"workload": f"gpt-oss-shaped gate_up {list(g.gate_up_shape)}", "ms": ms,
                             "GBps": b / (ms * 1e-3) / 1e9, "hbm_frac": b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS}
    del wg, wd, q8g, q8d, dq, q4
    return out


def configs_figures(torch, moeq, syn, dev, reps=20):
    """The experts forward at every configured shape and batch size: the
    shape's format, weights quantized on the device, 20 back-to-back calls
    between one pair of events (routing included); TFLOP/s over 6 T K H I and
    GB/s over the touched experts' packed weights."""
    out = []
    for name, s in syn.SHAPES.items():
        if name == "tiny":
            continue
        gu = syn.expert_weights(s.gate_up_shape, tensor=syn.GATE_UP, outliers=s.outliers, device=dev)
        dn = syn.expert_weights(s.down_shape, tensor=syn.DOWN, outliers=s.outliers, device=dev)
        quant = moeq.moeq_quantize_nf4 if s.fmt == "nf4" else moeq.moeq_quantize_int8_rowwise
        qg, qd = quant(gu), quant(dn)
        del gu, dn
        bpe = NF4_PACKED_BYTES_PER_ELEM if s.fmt == "nf4" else 1.0
        for T in s.tokens:
            x = syn.hidden_states(T, s.H, device=dev)
            idx, wts = syn.routing(T, s.K, s.E, kind=s.routing, device=dev)
            o = torch.empty((T, s.H), dtype=torch.bfloat16, device=dev)
            ws = torch.empty(moeq.moeq_experts_forward_workspace_bytes(T, s.K, qg, qd), dtype=torch.uint8, device=dev)
            for _ in range(3):
                moeq.moeq_experts_forward(x, idx, wts, qg, qd, out=o, workspace=ws)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(reps):
                moeq.moeq_experts_forward(x, idx, wts, qg, qd, out=o, workspace=ws)
            b.record()
            torch.cuda.synchronize()
            ms = a.elapsed_time(b) / reps
            flops = 6.0 * T * s.K * s.H * s.I
            u = int(torch.unique(idx[(idx >= 0) & (idx < s.E)]).numel())
            packed = u * 3.0 * s.H * s.I * bpe
            out.append({"config": name, "format": s.fmt, "T": T, "forward_ms": ms, "tokens_per_s": T / (ms * 1e-3),
                        "TFLOPs": flops / (ms * 1e-3) / 1e12, "mfma_frac": flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                        "touched_experts": u, "packed_GBps": packed / (ms * 1e-3) / 1e9})
            del x, idx, wts, o, ws
        del qg, qd
        torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import bit_weight_quantization_moeq_amd as moeq
    import moeq_synth as syn

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    s = syn.SHAPES[args.config]
    T = args.T
    if s.fmt != "nf4":
        raise SystemExit("the benchmarked path is NF4")

    gu = syn.expert_weights(s.gate_up_shape, tensor=syn.GATE_UP, outliers=s.outliers, device=dev)
    dn = syn.expert_weights(s.down_shape, tensor=syn.DOWN, outliers=s.outliers, device=dev)
    x = syn.hidden_states(T, s.H, device=dev)
    idx, wts = syn.routing(T, s.K, s.E, kind=s.routing, device=dev)
    qg = moeq.QWeight.empty(moeq.FMT_NF4, *s.gate_up_shape, device=dev)
    qd = moeq.QWeight.empty(moeq.FMT_NF4, *s.down_shape, device=dev)
    out = torch.empty((T, s.H), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(moeq.moeq_experts_forward_workspace_bytes(T, s.K, qg, qd), dtype=torch.uint8, device=dev)
    copy_GBps = device_copy_GBps(torch, dev)

    nsteps = args.warmup + args.steps
    ev = [new_events(torch, 8) for _ in range(nsteps)]

    def step(i):
        # Every library call runs on torch's current stream, where these events
        # are recorded.  Even steps also record the forward's stage boundaries
        # (per-kernel durations); odd steps record only its start and end, so
        # the forward time carries no event gaps between its kernels.
        e = ev[i]
        e[0].record()
        moeq.moeq_quantize_nf4(gu, out=qg)
        e[1].record()
        moeq.moeq_quantize_nf4(dn, out=qd)
        e[2].record()
        if i % 2 == 0:
            moeq.moeq_experts_forward(x, idx, wts, qg, qd, out=out, workspace=ws,
                                      stage_events=[h.cuda_event for h in e[3:8]])
        else:
            e[3].record()
            moeq.moeq_experts_forward(x, idx, wts, qg, qd, out=out, workspace=ws)
            e[7].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.warmup, nsteps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    names = ["quantize_gate_up", "quantize_down", None, "route", "g1_gate_up_swiglu", "g2_down", "combine"]
    stage = {n: [] for n in names if n}
    fwd_plain, fwd_staged, q_ms = [], [], []
    for i in range(args.warmup, nsteps):
        e = ev[i]
        q_ms.append(e[0].elapsed_time(e[2]))
        stage["quantize_gate_up"].append(e[0].elapsed_time(e[1]))
        stage["quantize_down"].append(e[1].elapsed_time(e[2]))
        if i % 2 == 0:
            for j in range(3, 7):
                stage[names[j]].append(e[j].elapsed_time(e[j + 1]))
            fwd_staged.append(e[3].elapsed_time(e[7]))
        else:
            fwd_plain.append(e[3].elapsed_time(e[7]))
    avg = {n: float(np.mean(v)) for n, v in stage.items() if v}
    fwd = float(np.mean(fwd_plain or fwd_staged))
    qt = float(np.mean(q_ms))

    n_gu, n_dn = int(np.prod(s.gate_up_shape)), int(np.prod(s.down_shape))
    q_bytes = (n_gu + n_dn) * NF4_BYTES_PER_ELEM
    idx_np = idx.cpu().numpy()
    f_bytes, f_flops, U = forward_bytes_flops(s, idx_np, T)
    n_assign = T * s.K

    # dominant kernel of the step and its roofline (algorithmic work per launch / event time)
    dom = max(avg, key=avg.get)
    work = {
        "quantize_gate_up": ("hbm", n_gu * NF4_BYTES_PER_ELEM),
        "quantize_down": ("hbm", n_dn * NF4_BYTES_PER_ELEM),
        "g1_gate_up_swiglu": ("mfma", 4.0 * n_assign * s.H * s.I),
        "g2_down": ("mfma", 2.0 * n_assign * s.H * s.I),
        "route": ("hbm", n_assign * 4 * 4.0),
        "combine": ("hbm", n_assign * s.H * 4.0 + T * s.H * 2.0),
    }
    bound, amount = work[dom]
    if bound == "hbm":
        achieved = amount / (avg[dom] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBPS, "traffic": None}
    else:
        achieved = amount / (avg[dom] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / MFMA_BF16_PEAK_TFLOPS, "traffic": None}
    roof["traffic"] = measured_traffic(dom)
    roof["kernel"] = dom
    roof["ms_per_launch"] = avg[dom]

    result = {
        "metric": METRIC,
        "value": T / (fwd * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": (f"{s.name}-shaped MoE layer E={s.E} H={s.H} I={s.I} top-{s.K} "
                                f"{s.routing} routing, T={T}: NF4 quantize-on-load of gate_up+down, "
                                f"then the experts forward from packed storage"),
                   "E": s.E, "H": s.H, "I": s.I, "K": s.K, "T": T, "format": "nf4", "blocksize": 64},
        "forward_ms": fwd,
        "forward_ms_with_stage_events": float(np.mean(fwd_staged)) if fwd_staged else None,
        "forward_TFLOPs": f_flops / (fwd * 1e-3) / 1e12,
        "forward_mfma_frac": f_flops / (fwd * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
        "quantize_ms": qt,
        "quantize_GBps": q_bytes / (qt * 1e-3) / 1e9,
        "quantize_hbm_frac": q_bytes / (qt * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "quantize_copy_frac": q_bytes / (qt * 1e-3) / 1e9 / copy_GBps,
        "device_copy_GBps": copy_GBps,
        "stage_ms": avg,
        "touched_experts": U,
        "roofline": roof,
    }

    if not args.no_decode:
        result["decode"] = decode_figures(torch, np, moeq, syn, s, qg, qd, dev, copy_GBps)
    if not args.no_offload:
        result["offload"] = offload_figures(torch, np, moeq, s, qg, qd, x, idx, wts, dev, fwd)
    if not args.no_router:
        result["router"] = router_figures(torch, np, moeq, syn, s, x, dev, copy_GBps)
    if not args.no_backward:
        result["backward"] = backward_figures(torch, np, moeq, syn, s, qg, qd, x, idx, wts, dev)
    if not args.no_double_quant:
        result["double_quant"] = double_quant_figures(torch, np, moeq, syn, s, gu, dn, x, idx, wts, dev, copy_GBps)
    if not args.no_codec:
        result["codec"] = codec_figures(torch, np, moeq, syn, dev, copy_GBps)
    if not args.no_load:
        result["load"] = load_figures(torch, np, moeq, syn, dev, copy_GBps)

    if args.configs:
        result["configs"] = configs_figures(torch, moeq, syn, dev)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(s, gu, dn, x, idx, wts, T)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
