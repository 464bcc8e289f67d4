#!/usr/bin/env python3
"""Benchmark of the NF4 MoE-experts hot path on one MI355X.

Headline step (the largest configured layer that fits one GPU): quantize-on-load
of one Mixtral-8x7B-shaped MoE layer (gate_up [8, 28672, 4096] and down
[8, 4096, 14336] bf16 ~ N(0, 0.02) with 0.1 % +-20-sigma outliers -> NF4,
blocksize 64), then the routed experts forward of T = 16384 tokens with top-2
uniform routing straight from packed storage (routing buckets, gate_up grouped
GEMM + SwiGLU, down grouped GEMM, k-ordered combine).  Two packed slots
alternate: step i quantizes into slot i % 2 and runs the forward from the
slot quantized one step earlier, so the forward never reads weights the
quantize has just written through the caches.

Printed (one JSON line): ``value`` = experts-forward tokens/s of the headline
(HIP events around the forward of the timed steps that record no stage
events); ``roofline`` = the step's dominant kernel (algorithmic flops or bytes
per launch / its event-timed duration), with HBM traffic and the MFMA-busy
counter read from the committed rocprofv3 summaries when they match the
current kernel sources; ``forward_configs`` = the forward at every configured
shape and batch size; ``quantize_configs`` = quantize-on-load of every shape,
against the measured device copy and the same-byte-mix streaming reference;
few-assignment (decode) cases also as a HIP-graph replay with a per-kernel
split; ``olmoe_T4096``, ``backward``, ``router``, ``offload``,
``double_quant``, ``codec`` = the secondary records; ``cpu_baseline`` = the
CPU oracle on a bounded sample of the headline workload.  Inputs are seeded
synthetic tensors resident in HBM before every timed region.

``--parts`` picks records (comma list; default all) for profiler runs.
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
LLC_BYTES = 256 << 20           # MI355X last-level (Infinity) cache
NF4_BYTES_PER_ELEM = 2.0 + 0.5 + 4.0 / 64   # bf16 read + packed code + absmax share
NF4_PACKED_BYTES_PER_ELEM = 0.5 + 4.0 / 64  # what the forward streams per weight element
# NF4 with double-quantized absmax: one code byte per 64-block, 4 bytes per 256 blocks
DQ_PACKED_BYTES_PER_ELEM = 0.5 + 1.0 / 64 + 4.0 / (64 * 256)
DQ_BYTES_PER_ELEM = 2.0 + DQ_PACKED_BYTES_PER_ELEM

PARTS = ("headline", "configs", "decode", "quantize", "olmoe", "backward", "router", "offload",
         "double_quant", "codec", "cpu_baseline")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--parts", default=",".join(PARTS),
                    help=f"comma list of records to produce (default all: {','.join(PARTS)})")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cases", default="",
                    help="comma list of shape:T forward cases (e.g. olmoe:32) to run instead of every configured "
                         "one, plain back-to-back calls only (for counter runs of one case)")
    return ap.parse_args()


def packed_bpe(fmt):
    return {"nf4": NF4_PACKED_BYTES_PER_ELEM, "nf4_dq": DQ_PACKED_BYTES_PER_ELEM, "int8": 1.0}[fmt]


def touched_bytes(s, idx, fmt):
    """(packed bytes of the experts a batch touches, each read once; those
    plus the activations in and out and the routing inputs; touched experts)."""
    import torch
    flat = idx.reshape(-1)
    U = int(torch.unique(flat[(flat >= 0) & (flat < s.E)]).numel())
    if fmt == "int8":
        w = U * (3 * s.H * s.I + 4 * (2 * s.I + s.H))
    else:
        w = U * 3 * s.H * s.I * packed_bpe(fmt)
    T, K = idx.shape
    return float(w), float(w + 4 * T * s.H + 8 * T * K), U


def measured_profile(kind, kernel):
    """The JSON block of a committed profiles/ summary of `kind` ("traffic" or
    "counters") for `kernel`, or None when there is none or the kernel
    sources changed since the counters were taken."""
    import glob
    import re

    from profsum import source_hash
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", f"*_{kind}.md"))):
        m = re.search(r"```json\n(.*?)\n```", open(path).read(), re.S)
        if not m:
            continue
        block = json.loads(m.group(1))
        if block.get("kernel") == kernel and block.get("source_sha256") == source_hash(kernel):
            block["summary"] = os.path.relpath(path, ROOT)
            return block
    return None


def new_events(torch, n):
    """n timing events on torch's current stream, created now (one record each)
    so their raw hipEvent_t handles can be handed to the library."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in ev:
        e.record()
    return ev


def timed(torch, fn, reps, warm=2):
    """Mean ms of `reps` back-to-back calls between one pair of events."""
    for _ in range(warm):
        fn()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def clone_q(moeq, q):
    t = [u.clone() for u in q._tensors()]
    return moeq.QWeight(q.format, q.num_experts, q.rows, q.cols, t[0], t[1], t[2] if len(t) == 3 else None)


def quantize_fn(moeq, fmt):
    if fmt == "int8":
        return moeq.moeq_quantize_int8_rowwise
    return lambda w, out=None: moeq.moeq_quantize_nf4(w, out=out, double_quant=(fmt == "nf4_dq"))


def layer_weights(torch, moeq, syn, s, dev, fmt=None, layer=0):
    """A quantized layer of shape `s` (its own format unless `fmt`), the bf16
    source freed."""
    fmt = fmt or s.fmt
    gu = syn.expert_weights(s.gate_up_shape, tensor=syn.GATE_UP, outliers=s.outliers, device=dev, layer=layer)
    qg = quantize_fn(moeq, fmt)(gu)
    del gu
    dn = syn.expert_weights(s.down_shape, tensor=syn.DOWN, outliers=s.outliers, device=dev, layer=layer)
    qd = quantize_fn(moeq, fmt)(dn)
    del dn
    return qg, qd


def device_copy_GBps(torch, dev, nbytes=1 << 30, reps=10):
    """Measured HBM bandwidth of a plain device copy (read + write bytes / time)."""
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    ms = timed(torch, lambda: dst.copy_(src), reps)
    del src, dst
    return 2.0 * nbytes / (ms * 1e-3) / 1e9


# ---------------------------------------------------------------------------
# One step: quantize-on-load + forward of one layer, stage events on even steps
# ---------------------------------------------------------------------------
def step_record(torch, np, moeq, syn, s, T, dev, steps, warmup, copy_GBps):
    gu = syn.expert_weights(s.gate_up_shape, tensor=syn.GATE_UP, outliers=s.outliers, device=dev)
    dn = syn.expert_weights(s.down_shape, tensor=syn.DOWN, outliers=s.outliers, device=dev)
    x = syn.hidden_states(T, s.H, device=dev)
    idx, wts = syn.routing(T, s.K, s.E, kind=s.routing, device=dev)
    slots = [(moeq.QWeight.empty(moeq.FMT_NF4, *s.gate_up_shape, device=dev),
              moeq.QWeight.empty(moeq.FMT_NF4, *s.down_shape, device=dev)) for _ in range(2)]
    for qg, qd in slots:
        moeq.moeq_quantize_nf4(gu, out=qg)
        moeq.moeq_quantize_nf4(dn, out=qd)
    out = torch.empty((T, s.H), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(moeq.moeq_experts_forward_workspace_bytes(T, s.K, *slots[0]), dtype=torch.uint8, device=dev)

    nsteps = warmup + steps
    ev = [new_events(torch, 8) for _ in range(nsteps)]

    def step(i):
        # Every library call runs on torch's current stream, where these events
        # are recorded.  Even steps also record the forward's stage boundaries
        # (per-kernel durations); odd steps record only its start and end.
        e = ev[i]
        qg, qd = slots[i % 2]
        fg, fd = slots[(i + 1) % 2]           # quantized one step earlier
        e[0].record()
        moeq.moeq_quantize_nf4(gu, out=qg)
        e[1].record()
        moeq.moeq_quantize_nf4(dn, out=qd)
        e[2].record()
        if i % 2 == 0:
            moeq.moeq_experts_forward(x, idx, wts, fg, fd, out=out, workspace=ws,
                                      stage_events=[h.cuda_event for h in e[3:8]])
        else:
            e[3].record()
            moeq.moeq_experts_forward(x, idx, wts, fg, fd, out=out, workspace=ws)
            e[7].record()

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(warmup, nsteps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    names = ["quantize_gate_up", "quantize_down", None, "route", "g1_gate_up_swiglu", "g2_down", "combine"]
    stage = {n: [] for n in names if n}
    fwd_plain, fwd_staged, q_ms = [], [], []
    for i in range(warmup, nsteps):
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
    _, f_bytes, U = touched_bytes(s, idx, "nf4")
    n_assign = T * s.K
    flops = 6.0 * n_assign * s.H * s.I
    rec = {
        "workload": (f"{s.name}-shaped MoE layer E={s.E} H={s.H} I={s.I} top-{s.K} {s.routing} routing"
                     f"{' (0.1% +-20-sigma outliers)' if s.outliers else ''}, NF4 blocksize 64, T={T}: "
                     f"quantize-on-load of gate_up+down, then the experts forward from packed storage"),
        "E": s.E, "H": s.H, "I": s.I, "K": s.K, "T": T, "format": "nf4",
        "ms_per_step": wall * 1e3 / steps,
        "forward_ms": fwd, "tokens_per_s": T / (fwd * 1e-3),
        "forward_ms_with_stage_events": float(np.mean(fwd_staged)) if fwd_staged else None,
        "forward_TFLOPs": flops / (fwd * 1e-3) / 1e12,
        "forward_mfma_frac": flops / (fwd * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
        "forward_flops": flops, "forward_algorithmic_bytes": f_bytes, "touched_experts": U,
        "quantize_ms": qt, "quantize_bytes": q_bytes,
        "quantize_GBps": q_bytes / (qt * 1e-3) / 1e9,
        "quantize_hbm_frac": q_bytes / (qt * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "quantize_copy_frac": q_bytes / (qt * 1e-3) / 1e9 / copy_GBps,
        "stage_ms": avg,
    }
    # dominant kernel of the step and its roofline (algorithmic work per launch / event time)
    work = {
        "quantize_gate_up": ("hbm", n_gu * NF4_BYTES_PER_ELEM, "nf4_quantize_kernel"),
        "quantize_down": ("hbm", n_dn * NF4_BYTES_PER_ELEM, "nf4_quantize_kernel"),
        "g1_gate_up_swiglu": ("mfma", 4.0 * n_assign * s.H * s.I, "g1_kernel<1>"),
        "g2_down": ("mfma", 2.0 * n_assign * s.H * s.I, "g2_kernel<1>"),
        "route": ("hbm", n_assign * 4 * 4.0, "route_rank_kernel"),
        "combine": ("hbm", n_assign * s.H * 2.0 + T * s.H * 2.0, "combine_kernel<unsigned short>"),
    }
    dom = max(avg, key=avg.get)
    bound, amount, kname = work[dom]
    if bound == "hbm":
        achieved = amount / (avg[dom] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBPS}
    else:
        achieved = amount / (avg[dom] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / MFMA_BF16_PEAK_TFLOPS}
    tag = f"{s.name}_T{T}"
    traffic = measured_profile("traffic", f"{kname}@{tag}")
    counters = measured_profile("counters", f"{kname}@{tag}")
    roof["traffic"] = traffic["traffic_bytes"] if traffic else None
    roof.update({"kernel": kname, "stage": dom, "ms_per_launch": avg[dom],
                 "algorithmic_per_launch": amount,
                 "traffic_summary": traffic["summary"] if traffic else None,
                 "mfma_busy_counter": counters.get("mfma_util") if counters else None,
                 "counter_summary": counters["summary"] if counters else None})
    rec["roofline"] = roof
    del gu, dn, slots, ws
    return rec, (x, idx, wts)


# ---------------------------------------------------------------------------
# The forward at every configured shape and batch size
# ---------------------------------------------------------------------------
def forward_case(torch, moeq, syn, s, fmt, stack, T, dev, copy_GBps, graph=False, stage=False):
    """The forward of T tokens over `stack` (copies of the quantized layer, used
    in turn so that the distinct packed bytes of a rotation exceed the
    last-level cache): back-to-back calls between one pair of events; with
    `graph`, the same calls captured once in a HIP graph and replayed (the
    launches then cost no host time); with `stage`, the per-kernel split from
    stage events."""
    import numpy as np
    x = syn.hidden_states(T, s.H, device=dev, layer=1)
    idx, wts = syn.routing(T, s.K, s.E, kind=s.routing, device=dev, layer=1)
    out = torch.empty((T, s.H), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(moeq.moeq_experts_forward_workspace_bytes(T, s.K, *stack[0]), dtype=torch.uint8, device=dev)
    L = len(stack)
    wbytes, nbytes, U = touched_bytes(s, idx, fmt)
    flops = 6.0 * T * s.K * s.H * s.I
    # about 50 ms of calls, whole rotations
    est_ms = max(nbytes / 4e12, flops / 8e14) * 1e3 + 0.01
    reps = max(1, min(8, int(50.0 / (est_ms * L)))) * L
    state = {"r": 0}

    def call():
        g, d = stack[state["r"] % L]
        state["r"] += 1
        moeq.moeq_experts_forward(x, idx, wts, g, d, out=out, workspace=ws)

    ms = timed(torch, call, reps, warm=L)
    rec = {"config": s.name, "format": fmt, "T": T, "K": s.K, "forward_ms": ms,
           "tokens_per_s": T / (ms * 1e-3), "TFLOPs": flops / (ms * 1e-3) / 1e12,
           "mfma_frac": flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
           "touched_experts": U, "packed_MB": wbytes / 1e6, "algorithmic_MB": nbytes / 1e6,
           "GBps": nbytes / (ms * 1e-3) / 1e9, "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
           "copy_frac": nbytes / (ms * 1e-3) / 1e9 / copy_GBps,
           "path": "few-assignment" if T * s.K <= 512 else "tiled",
           "timing": f"{reps} back-to-back calls over {L} layer copies "
                     f"({L * wbytes / 1e6:.0f} MB of distinct packed weights per rotation)"}
    if graph:
        torch.cuda.synchronize()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(L):
                call()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        ref = out.clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(L):
                call()
        gm = timed(torch, g.replay, max(2, reps // L)) / L
        rec["graph_forward_ms"] = gm
        rec["graph_tokens_per_s"] = T / (gm * 1e-3)
        rec["graph_GBps"] = nbytes / (gm * 1e-3) / 1e9
        rec["graph_hbm_frac"] = nbytes / (gm * 1e-3) / 1e9 / HBM_PEAK_GBPS
        rec["graph_matches_eager"] = bool(torch.equal(out, ref))
        del g
    if stage:
        evs = [new_events(torch, 5) for _ in range(2 * L)]
        for r in range(2 * L):
            gq, dq = stack[r % L]
            moeq.moeq_experts_forward(x, idx, wts, gq, dq, out=out, workspace=ws,
                                      stage_events=[h.cuda_event for h in evs[r]])
        torch.cuda.synchronize()
        kms = {n: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs[L:]]))
               for j, n in enumerate(["route", "gate_up", "down", "combine"])}
        rec["stage_ms_with_events"] = kms
        if U:
            if fmt == "int8":
                gb = U * (2 * s.I * s.H + 8 * s.I)
                db = U * (s.H * s.I + 4 * s.H)
            else:
                gb = U * 2 * s.I * s.H * packed_bpe(fmt)
                db = U * s.H * s.I * packed_bpe(fmt)
            rec["gate_up_packed_GBps"] = gb / (kms["gate_up"] * 1e-3) / 1e9
            rec["down_packed_GBps"] = db / (kms["down"] * 1e-3) / 1e9
    del x, idx, wts, out, ws
    return rec


def layer_stack(torch, moeq, syn, s, fmt, dev, per_call_bytes, target=4 * LLC_BYTES, cap_bytes=24e9):
    """The quantized layer plus copies, so that a rotation touches `target`
    distinct packed bytes (at least 2 copies, at most `cap_bytes` of them)."""
    qg, qd = layer_weights(torch, moeq, syn, s, dev, fmt)
    lb = qg.nbytes() + qd.nbytes()
    n = int(min(max(2, -(-target // max(int(per_call_bytes), 1))), max(2, cap_bytes // lb)))
    return [(qg, qd)] + [(clone_q(moeq, qg), clone_q(moeq, qd)) for _ in range(n - 1)]


def config_records(torch, moeq, syn, dev, copy_GBps, log, decode_only=False, cases=None):
    """Every configured shape and batch size in the shape's format: the
    forward (tokens/s, TFLOP/s, GB/s over the touched experts' packed bytes);
    few-assignment batches also as a HIP-graph replay and split per kernel.
    `cases`: only these (shape, T) pairs, back-to-back calls only."""
    out = []
    for name, s in syn.SHAPES.items():
        Ts = tuple(T for T in s.tokens if T * s.K <= 512) if decode_only else s.tokens
        if cases is not None:
            Ts = tuple(T for (n, T) in cases if n == name)
        for T in Ts:
            log(f"forward {name} T={T}")
            idx, _ = syn.routing(T, s.K, s.E, kind=s.routing, device=dev, layer=1)
            wbytes, _, _ = touched_bytes(s, idx, s.fmt)
            stack = layer_stack(torch, moeq, syn, s, s.fmt, dev, wbytes)
            dec = T * s.K <= 512 and cases is None
            out.append(forward_case(torch, moeq, syn, s, s.fmt, stack, T, dev, copy_GBps, graph=dec, stage=dec))
            del stack
            torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------------------
# Quantize-on-load of every shape, against the measured ceilings
# ---------------------------------------------------------------------------
def quantize_records(torch, np, moeq, syn, dev, copy_GBps, log, reps=5):
    out = {}
    # The attainable rate for the quantize kernel's byte mix and access
    # pattern: its launch, loads and stores without the NF4 arithmetic.
    s = syn.SHAPES["mixtral"]
    w = syn.expert_weights(s.gate_up_shape, tensor=syn.GATE_UP, device=dev)
    q = moeq.QWeight.empty(moeq.FMT_NF4, *s.gate_up_shape, device=dev)
    ref_ms = timed(torch, lambda: moeq.moeq_stream_reference(w, q), reps)
    ceil = w.numel() * NF4_BYTES_PER_ELEM / (ref_ms * 1e-3) / 1e9
    q_ms = timed(torch, lambda: moeq.moeq_quantize_nf4(w, out=q), reps)
    out["stream_reference"] = {
        "workload": f"mixtral-shaped gate_up {list(s.gate_up_shape)}: the NF4 quantize kernel's launch, "
                    f"loads and stores without the NF4 arithmetic (2 B read, 0.5625 B written per element)",
        "ms": ref_ms, "GBps": ceil, "hbm_frac": ceil / HBM_PEAK_GBPS, "copy_frac": ceil / copy_GBps,
        "quantize_ms_same_tensor": q_ms, "quantize_frac_of_reference": ref_ms / q_ms}
    del w, q
    torch.cuda.empty_cache()

    def one(name, fmt, layers=1):
        log(f"quantize {name} x{layers} ({fmt})")
        s = syn.SHAPES[name]
        gu = syn.expert_weights(s.gate_up_shape, tensor=syn.GATE_UP, outliers=s.outliers, device=dev)
        dn = syn.expert_weights(s.down_shape, tensor=syn.DOWN, outliers=s.outliers, device=dev)
        f = moeq.FMT_INT8_ROWWISE if fmt == "int8" else moeq.FMT_NF4
        qg = moeq.QWeight.empty(f, *s.gate_up_shape, device=dev)
        qd = moeq.QWeight.empty(f, *s.down_shape, device=dev)
        qfn = quantize_fn(moeq, fmt)

        def run():
            for _ in range(layers):
                qfn(gu, out=qg)
                qfn(dn, out=qd)
        ms = timed(torch, run, 1 if layers > 1 else reps, warm=1)
        nel = gu.numel() + dn.numel()
        if fmt == "int8":
            b = layers * (3.0 * nel + 4.0 * s.E * (s.gate_up_shape[1] + s.down_shape[1]))
        else:
            b = layers * nel * NF4_BYTES_PER_ELEM
        rec = {"layers": layers, "format": fmt, "elements": layers * nel, "ms": ms,
               "bf16_GB": layers * nel * 2 / 1e9, "packed_GB": layers * (qg.nbytes() + qd.nbytes()) / 1e9,
               "algorithmic_GB": b / 1e9, "GBps": b / (ms * 1e-3) / 1e9,
               "hbm_frac": b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, "copy_frac": b / (ms * 1e-3) / 1e9 / copy_GBps}
        if fmt == "nf4":
            rec["stream_reference_frac"] = b / (ms * 1e-3) / 1e9 / ceil
        if layers > 1:
            rec["timing"] = (f"one layer's bf16 weights ({nel * 2 / 1e9:.2f} GB, larger than every cache) "
                             f"quantized {layers} times back to back between one pair of events")
        del gu, dn, qg, qd
        torch.cuda.empty_cache()
        return rec

    out["mixtral_layer"] = one("mixtral", "nf4")
    out["olmoe_layer"] = one("olmoe", "nf4")
    out["olmoe_16_layers"] = one("olmoe", "nf4", 16)
    out["qwen3_layer"] = one("qwen3", "nf4")
    out["qwen3_48_layers"] = one("qwen3", "nf4", 48)
    out["gptoss_int8_layer"] = one("gptoss", "int8")
    out["tiny_layer"] = one("tiny", "nf4")
    return out


# ---------------------------------------------------------------------------
# Secondary records
# ---------------------------------------------------------------------------
def backward_record(torch, moeq, syn, s, qg, qd, x, idx, wts, dev, reps=10):
    """Gradients of the experts block (hidden states and routing weights, the
    packed weights frozen): the gate_up GEMM recomputed (4 T K H I flops), the
    down^T GEMM (2), the gate_up^T GEMM (4); the routing-weight gradient comes
    from the down^T product, with no down GEMM of its own."""
    T = x.shape[0]
    dout = syn.grad_output(T, s.H, device=dev)
    ws = torch.empty(moeq.moeq_experts_backward_workspace_bytes(T, s.K, qg, qd), dtype=torch.uint8, device=dev)
    gx = torch.empty((T, s.H), dtype=torch.bfloat16, device=dev)
    gw = torch.empty((T, s.K), dtype=torch.float32, device=dev)
    ms = timed(torch, lambda: moeq.moeq_experts_backward(x, idx, wts, qg, qd, dout, grad_hidden=gx,
                                                         grad_weights=gw, workspace=ws), reps)
    flops = 10.0 * T * s.K * s.H * s.I
    # the training pair that keeps g and u: the forward writes them beside its
    # output, the backward skips the recompute (the same gradients, bit for bit)
    gsv = torch.empty((T * s.K, 2 * s.I), dtype=torch.float32, device=dev)
    out = torch.empty((T, s.H), dtype=torch.bfloat16, device=dev)
    fws = torch.empty(moeq.moeq_experts_forward_workspace_bytes(T, s.K, qg, qd), dtype=torch.uint8, device=dev)
    save_ms = timed(torch, lambda: moeq.moeq_experts_forward_save(x, idx, wts, qg, qd, out=out, gu_saved=gsv,
                                                                  workspace=fws), reps)
    sws = torch.empty(moeq.moeq_experts_backward_saved_workspace_bytes(T, s.K, qg, qd), dtype=torch.uint8,
                      device=dev)
    saved_ms = timed(torch, lambda: moeq.moeq_experts_backward_saved(idx, wts, qg, qd, gsv, dout, grad_hidden=gx,
                                                                     grad_weights=gw, workspace=sws), reps)
    sflops = 6.0 * T * s.K * s.H * s.I
    return {"workload": f"{s.name}-shaped layer, T={T}, incoming gradient ~ N(0, 1) bf16",
            "ms": ms, "tokens_per_s": T / (ms * 1e-3), "TFLOPs": flops / (ms * 1e-3) / 1e12,
            "mfma_frac": flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            "flops": "10 T K H I (gate_up recompute 4, down^T 2, gate_up^T 4)",
            "saved_pre_activations": {
                "forward_save_ms": save_ms, "backward_ms": saved_ms,
                "TFLOPs": sflops / (saved_ms * 1e-3) / 1e12,
                "mfma_frac": sflops / (saved_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                "flops": "6 T K H I (down^T 2, gate_up^T 4)", "saved_bytes": 8 * T * s.K * s.I}}


def router_record(torch, moeq, syn, s, x, dev, copy_GBps, reps=20):
    """Router front-end on the batch: a bf16 gate [E, H] -> top-K indices and
    weights.  HBM-bound: the hidden states are read once (T H 2 B), the gate
    once, the outputs written once (8 T K B)."""
    T = x.shape[0]
    gate = syn.router_weight(s.E, s.H, device=dev)
    idx = torch.empty((T, s.K), dtype=torch.int32, device=dev)
    w = torch.empty((T, s.K), dtype=torch.float32, device=dev)
    ms = timed(torch, lambda: moeq.moeq_router_topk(x, gate, s.K, top_k_index=idx, top_k_weights=w), reps)
    nbytes = 2.0 * T * s.H + 2.0 * s.E * s.H + 8.0 * T * s.K
    # the router fused with the routing stage, against the router followed by
    # the routing stage on its output (the same counts, offsets, perm, slot)
    ws = torch.empty(moeq.moeq_router_route_workspace_bytes(T, s.H, s.E, s.K), dtype=torch.uint8, device=dev)
    fused_ms = timed(torch, lambda: moeq.moeq_router_route(x, gate, s.K, workspace=ws), reps)
    rws = torch.empty(moeq.moeq_route_workspace_bytes(T, s.K, s.E), dtype=torch.uint8, device=dev)
    split_ms = timed(torch, lambda: moeq.moeq_route_buckets(
        moeq.moeq_router_topk(x, gate, s.K, top_k_index=idx, top_k_weights=w)[0], s.E, workspace=rws), reps)
    return {"workload": f"T={T}, gate [{s.E}, {s.H}] bf16, top-{s.K}", "ms": ms,
            "GBps": nbytes / (ms * 1e-3) / 1e9, "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "TFLOPs": 2.0 * T * s.E * s.H / (ms * 1e-3) / 1e12,
            "fused_with_routing_ms": fused_ms, "router_then_routing_ms": split_ms}


def offload_record(torch, moeq, s, qg, qd, x, idx, wts, dev, fwd_ms, layers=4, passes=2):
    """Expert-granularity offload: `layers` copies of the layer in pinned host
    memory, two device slots, layer N+1 prefetched on a side stream during
    layer N's forward.  `overlap` = (resident + copy - offloaded) /
    min(resident, copy), 1 when the shorter of the two is fully hidden."""
    from bit_weight_quantization_moeq_amd.offload import ExpertOffload
    off = ExpertOffload([(qg, qd)] * layers, dev)
    out = torch.empty((x.shape[0], s.H), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(moeq.moeq_experts_forward_workspace_bytes(x.shape[0], s.K, qg, qd), dtype=torch.uint8,
                     device=dev)
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
    for layer in range(layers):
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
    return {"workload": f"{layers} copies of the {s.name}-shaped layer in pinned host memory, T={x.shape[0]}",
            "layer_bytes": nbytes, "copy_ms": copy_ms, "copy_GBps": nbytes / (copy_ms * 1e-3) / 1e9,
            "resident_forward_ms": fwd_ms, "offloaded_forward_ms": off_ms,
            "overlap": (fwd_ms + copy_ms - off_ms) / min(fwd_ms, copy_ms)}


def double_quant_record(torch, moeq, syn, s, x, idx, wts, dev, copy_GBps, reps=10):
    """The layer with double-quantized absmax: quantize-on-load into that
    format, the T-token forward, the few-assignment forwards and the backward,
    each decoding the absmax inside its kernels; plus both formats' storage."""
    gu = syn.expert_weights(s.gate_up_shape, tensor=syn.GATE_UP, device=dev)
    dn = syn.expert_weights(s.down_shape, tensor=syn.DOWN, device=dev)
    qg = moeq.QWeight.empty(moeq.FMT_NF4_DQ, *s.gate_up_shape, device=dev)
    qd = moeq.QWeight.empty(moeq.FMT_NF4_DQ, *s.down_shape, device=dev)
    q_ms = timed(torch, lambda: (moeq.moeq_quantize_nf4(gu, out=qg), moeq.moeq_quantize_nf4(dn, out=qd)), reps)
    nel = gu.numel() + dn.numel()
    del gu, dn
    qb = nel * DQ_BYTES_PER_ELEM
    T = x.shape[0]
    idxs, _ = syn.routing(T, s.K, s.E, kind=s.routing, device=dev, layer=1)
    wb, _, _ = touched_bytes(s, idxs, "nf4_dq")
    n = int(max(2, -(-4 * LLC_BYTES // int(wb))))
    stack = [(qg, qd)] + [(clone_q(moeq, qg), clone_q(moeq, qd)) for _ in range(n - 1)]
    fwd = forward_case(torch, moeq, syn, s, "nf4_dq", stack, T, dev, copy_GBps)
    del stack
    dec = []
    for Td in (t for t in s.tokens if t * s.K <= 512):
        idd, _ = syn.routing(Td, s.K, s.E, kind=s.routing, device=dev, layer=1)
        wb, _, _ = touched_bytes(s, idd, "nf4_dq")
        n = int(max(2, -(-4 * LLC_BYTES // int(wb))))
        st = [(qg, qd)] + [(clone_q(moeq, qg), clone_q(moeq, qd)) for _ in range(n - 1)]
        dec.append(forward_case(torch, moeq, syn, s, "nf4_dq", st, Td, dev, copy_GBps, graph=True, stage=True))
        del st
    rec = {"workload": f"{s.name}-shaped layer, absmax double-quantized (8-bit code per block, fp32 per 256 blocks)",
           "quantize_ms": q_ms, "quantize_GBps": qb / (q_ms * 1e-3) / 1e9,
           "quantize_hbm_frac": qb / (q_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
           "quantize_copy_frac": qb / (q_ms * 1e-3) / 1e9 / copy_GBps,
           "forward": fwd, "decode": dec,
           "backward": backward_record(torch, moeq, syn, s, qg, qd, x, idx, wts, dev),
           "layer_bytes": {"nf4": nel * NF4_PACKED_BYTES_PER_ELEM, "nf4_double_quant": float(qg.nbytes() + qd.nbytes()),
                           "bits_per_weight_nf4": 8 * NF4_PACKED_BYTES_PER_ELEM,
                           "bits_per_weight_double_quant": 8.0 * (qg.nbytes() + qd.nbytes()) / nel}}
    torch.cuda.empty_cache()
    return rec


def codec_record(torch, moeq, syn, dev, reps=5):
    """Dequantize of both formats on the gpt-oss-shaped gate_up: algorithmic
    bytes / event time."""
    out = {}
    g = syn.SHAPES["gptoss"]
    wg = syn.expert_weights(g.gate_up_shape, tensor=syn.GATE_UP, device=dev)
    q8g = moeq.moeq_quantize_int8_rowwise(wg)
    dq = torch.empty(g.gate_up_shape, dtype=torch.bfloat16, device=dev)
    ms = timed(torch, lambda: moeq.moeq_dequantize(q8g, out=dq), reps)
    b = 3.0 * wg.numel() + 4.0 * g.E * g.gate_up_shape[1]
    out["int8_dequantize"] = {"workload": f"gpt-oss-shaped gate_up {list(g.gate_up_shape)}", "ms": ms,
                              "GBps": b / (ms * 1e-3) / 1e9, "hbm_frac": b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS}
    q4 = moeq.moeq_quantize_nf4(wg)
    ms = timed(torch, lambda: moeq.moeq_dequantize(q4, out=dq), reps)
    b = wg.numel() * NF4_BYTES_PER_ELEM
    out["nf4_dequantize"] = {"workload": f"gpt-oss-shaped gate_up {list(g.gate_up_shape)}", "ms": ms,
                             "GBps": b / (ms * 1e-3) / 1e9, "hbm_frac": b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS}
    del wg, q8g, dq, q4
    torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------------------
# The CPU oracle beside it
# ---------------------------------------------------------------------------
def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(s, T, dev_x, dev_idx, dev_wts, sample_tokens=512):
    """The oracle, untuned, on a bounded sample of the headline workload:
    NF4 quantize of expert 0's first 2048 gate_up rows (8.4 M elements) as it
    runs, and again under a 1-thread limit; then the fp64
    forward of the first `sample_tokens` tokens with every assignment folded
    onto expert 0 (identical work per assignment), which gives tokens/s."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info, threadpool_limits

    import moeq_synth as syn
    from oracle.forward import experts_forward
    from oracle.nf4 import nf4_dequantize, nf4_quantize

    gu = syn.expert_weights((1,) + tuple(s.gate_up_shape[1:]), tensor=syn.GATE_UP, outliers=s.outliers,
                            device=dev_x.device)
    dn = syn.expert_weights((1,) + tuple(s.down_shape[1:]), tensor=syn.DOWN, outliers=s.outliers,
                            device=dev_x.device)
    gbits, dbits = syn.bf16_bits(gu), syn.bf16_bits(dn)
    del gu, dn
    torch.cuda.empty_cache()
    part = np.ascontiguousarray(gbits[:, :2048])
    t0 = time.perf_counter()
    nf4_quantize(part)
    tq = time.perf_counter() - t0
    one = part
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        nf4_quantize(one)
        tq1 = time.perf_counter() - t0
    dg = nf4_dequantize(*nf4_quantize(gbits))
    dd = nf4_dequantize(*nf4_quantize(dbits))
    xs = syn.bf16_bits(dev_x[:sample_tokens])
    ids = np.zeros((sample_tokens, s.K), dtype=np.int32)
    ws = dev_wts[:sample_tokens].cpu().numpy()
    t0 = time.perf_counter()
    experts_forward(xs, ids, ws, dg, dd)
    tf = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {
        "value": sample_tokens / tf, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
        "cpu_model": cpu_model(), "host_cpu_count": os.cpu_count(),
        "quantize_GBps": part.size * NF4_BYTES_PER_ELEM / tq / 1e9,
        "quantize_GBps_1_thread": one.size * NF4_BYTES_PER_ELEM / tq1 / 1e9,
        "extrapolated_forward_ms_full_T": tf / sample_tokens * T * 1e3,
        "sample": (f"fp64 oracle forward of the first {sample_tokens} of the T={T} tokens of the headline "
                   f"workload with every assignment folded onto expert 0 ({tf:.1f} s, the same work per "
                   f"assignment; tokens/s extrapolated to the full batch); NF4 quantize of expert 0's first 2048 "
                   f"gate_up rows ({part.size} elements, {tq:.1f} s; numpy elementwise code, one thread in "
                   f"practice) and the same rows again under a 1-thread limit ({tq1:.1f} s); "
                   f"numpy/BLAS threads={threads}"),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    parts = set(p for p in args.parts.split(",") if p)
    unknown = parts - set(PARTS)
    if unknown:
        raise SystemExit(f"unknown --parts {sorted(unknown)}; choose from {PARTS}")
    if args.no_cpu_baseline:
        parts.discard("cpu_baseline")

    import numpy as np
    import torch

    import bit_weight_quantization_moeq_amd as moeq
    import moeq_synth as syn

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    t_start = time.perf_counter()

    def log(msg):
        print(f"[bench {time.perf_counter() - t_start:6.1f}s] {msg}", file=sys.stderr, flush=True)

    copy_GBps = device_copy_GBps(torch, dev)
    s = syn.SHAPES["mixtral"]
    T = s.tokens[-1]
    result = {"metric": METRIC, "value": None, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
              "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True, "scaling": "weak",
              "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
              "config": {"workload": f"{s.name}-shaped MoE layer, T={T}", "E": s.E, "H": s.H, "I": s.I,
                         "K": s.K, "T": T, "format": "nf4", "blocksize": 64},
              "device_copy_GBps": copy_GBps}
    hx = None
    if "headline" in parts:
        log(f"headline: {s.name} T={T} step")
        rec, hx = step_record(torch, np, moeq, syn, s, T, dev, args.steps, args.warmup, copy_GBps)
        result["value"] = rec["tokens_per_s"]
        result["ms_per_step"] = rec["ms_per_step"]
        result["config"]["workload"] = rec["workload"]
        result["roofline"] = rec.pop("roofline")
        for k in ("forward_ms", "forward_TFLOPs", "forward_mfma_frac", "forward_flops", "forward_algorithmic_bytes",
                  "quantize_ms", "quantize_bytes", "quantize_GBps", "quantize_hbm_frac", "quantize_copy_frac",
                  "stage_ms", "touched_experts", "forward_ms_with_stage_events"):
            result[k] = rec[k]
        torch.cuda.empty_cache()
    if args.cases:
        cases = [(c.split(":")[0], int(c.split(":")[1])) for c in args.cases.split(",")]
        bad = [c for c in cases if c[0] not in syn.SHAPES]
        if bad:
            raise SystemExit(f"unknown shapes in --cases: {bad}; choose from {sorted(syn.SHAPES)}")
        log(f"forward cases {cases}")
        result["forward_configs"] = config_records(torch, moeq, syn, dev, copy_GBps, log, cases=cases)
    elif "configs" in parts or "decode" in parts:
        log("forward at every configured shape and batch size")
        result["forward_configs"] = config_records(torch, moeq, syn, dev, copy_GBps, log,
                                                   decode_only="configs" not in parts)
    if "quantize" in parts:
        log("quantize-on-load of every shape")
        qc = quantize_records(torch, np, moeq, syn, dev, copy_GBps, log)
        result["quantize_configs"] = qc
        if result.get("quantize_GBps"):
            result["quantize_stream_reference_frac"] = result["quantize_GBps"] / qc["stream_reference"]["GBps"]
    o = syn.SHAPES["olmoe"]
    if parts & {"olmoe", "backward", "router", "offload", "double_quant"}:
        To = o.tokens[-1]
        log(f"olmoe T={To} step")
        orec, (ox, oidx, owts) = step_record(torch, np, moeq, syn, o, To, dev, args.steps, args.warmup, copy_GBps)
        if "olmoe" in parts:
            result["olmoe_T4096"] = orec
        qg, qd = layer_weights(torch, moeq, syn, o, dev)
        if "backward" in parts:
            log("backward")
            result["backward"] = backward_record(torch, moeq, syn, o, qg, qd, ox, oidx, owts, dev)
        if "router" in parts:
            log("router")
            result["router"] = router_record(torch, moeq, syn, o, ox, dev, copy_GBps)
        if "offload" in parts:
            log("offload")
            result["offload"] = offload_record(torch, moeq, o, qg, qd, ox, oidx, owts, dev, orec["forward_ms"])
        if "double_quant" in parts:
            log("double-quantized absmax")
            result["double_quant"] = double_quant_record(torch, moeq, syn, o, ox, oidx, owts, dev, copy_GBps)
        del qg, qd
        torch.cuda.empty_cache()
    if "codec" in parts:
        log("dequantize")
        result["codec"] = codec_record(torch, moeq, syn, dev)
    if "cpu_baseline" in parts:
        log("cpu baseline")
        if hx is None:
            hx = (syn.hidden_states(T, s.H, device=dev),) + syn.routing(T, s.K, s.E, kind=s.routing, device=dev)
        result["cpu_baseline"] = cpu_baseline(s, T, *hx)
    log("done")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
