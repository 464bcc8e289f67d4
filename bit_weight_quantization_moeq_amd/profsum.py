"""Condense rocprofv3 CSV output into the short Markdown summaries kept under
``profiles/``.

    python -m bit_weight_quantization_moeq_amd.profsum stats <kernel_stats.csv> "<command>"
    python -m bit_weight_quantization_moeq_amd.profsum traffic <fetch_dir> <write_dir> <kernel> <copy_bytes> \
        <algorithmic_bytes> "<fetch command>" "<write command>"
    python -m bit_weight_quantization_moeq_amd.profsum decode <kernel_trace.csv> <H> <I> \
        <format>=<bytes_per_weight>[,...] <grid_x>=<touched experts>[,...] "<command>"

``stats`` prints a per-kernel duration table.  ``traffic`` reads two
``--pmc FETCH_SIZE`` / ``--pmc WRITE_SIZE`` runs (KiB per dispatch), takes the
mean per dispatch of ``kernel`` and calibrates each counter against the
largest plain device copy in the same run (``copy_bytes`` bytes read and
written by ``__amd_rocclr_copyBuffer``), then prints the table plus a JSON
block that bench.py reads; the block carries the SHA-256 of the kernel
sources so that a changed kernel reports no stale traffic.  ``decode`` splits
the few-assignment kernels' dispatches by launch grid (one grid per batch
size) and prices each against the packed bytes of the experts it touches.
"""

import csv
import glob
import hashlib
import json
import os
import re
import sys

SOURCES = ("csrc/experts.hip", "csrc/quant.hip", "csrc/route.hip", "csrc/api.hip", "csrc/moeq_internal.h")


def _code_only(text):
    """The source with comments and blank space removed (the sources hold no
    string literal containing a comment marker)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_hash():
    """SHA-256 of the kernel sources' code (comments and layout ignored)."""
    here = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha256()
    for rel in SOURCES:
        with open(os.path.join(here, rel)) as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()


def short(name):
    name = name.replace("moeq::(anonymous namespace)::", "").replace("void ", "")
    name = name.replace("(anonymous namespace)::", "")
    depth, out = 0, []
    for ch in name:                      # drop the argument list, keep template arguments
        if ch == "(" and depth == 0:
            break
        depth += ch == "<"
        depth -= ch == ">"
        out.append(ch)
    return "".join(out)[:70]


def stats(path, command):
    rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    print(f"command: `{command}`\n")
    print("| kernel | calls | avg us | min us | max us | % of GPU time |")
    print("|---|---:|---:|---:|---:|---:|")
    for r in rows:
        print(f"| {short(r['Name'])} | {r['Calls']} | {float(r['AverageNs'])/1e3:.1f} | "
              f"{float(r['MinNs'])/1e3:.1f} | {float(r['MaxNs'])/1e3:.1f} | {float(r['Percentage']):.1f} |")


def _per_dispatch(d, counter):
    """kernel short name -> list of per-dispatch counter values (KiB)."""
    out = {}
    for p in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        acc = {}
        for r in csv.DictReader(open(p)):
            if r["Counter_Name"] != counter:
                continue
            key = (r["Dispatch_Id"], r["Kernel_Name"])
            acc[key] = acc.get(key, 0.0) + float(r["Counter_Value"])
        for (_, name), v in acc.items():
            out.setdefault(short(name), []).append(v)
    return out


def traffic(fetch_dir, write_dir, kernel, copy_bytes, algo_bytes, cmd_f, cmd_w):
    copy_bytes, algo_bytes = float(copy_bytes), float(algo_bytes)
    f, w = _per_dispatch(fetch_dir, "FETCH_SIZE"), _per_dispatch(write_dir, "WRITE_SIZE")
    cf = max(f["__amd_rocclr_copyBuffer"]) * 1024.0 / copy_bytes   # counter bytes per copied byte
    cw = max(w["__amd_rocclr_copyBuffer"]) * 1024.0 / copy_bytes
    fk = sum(f[kernel]) / len(f[kernel]) * 1024.0 / cf
    wk = sum(w[kernel]) / len(w[kernel]) * 1024.0 / cw
    print(f"FETCH_SIZE command: `{cmd_f}`\n\nWRITE_SIZE command: `{cmd_w}`\n")
    print(f"Calibration: the largest `__amd_rocclr_copyBuffer` dispatch copies {copy_bytes:.0f} bytes; "
          f"FETCH_SIZE reads {cf:.3f} and WRITE_SIZE {cw:.3f} counter bytes per copied byte.\n")
    print("| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM read MB (cal.) | HBM write MB (cal.) "
          "| algorithmic MB | traffic / algorithmic |")
    print("|---|---:|---:|---:|---:|---:|---:|---:|")
    print(f"| {kernel} | {len(f[kernel])} | {sum(f[kernel]) / len(f[kernel]):.0f} | {sum(w[kernel]) / len(w[kernel]):.0f} "
          f"| {fk / 1e6:.1f} | {wk / 1e6:.1f} | {algo_bytes / 1e6:.1f} | {(fk + wk) / algo_bytes:.3f} |")
    block = {"kernel": kernel, "hbm_read_bytes": fk, "hbm_write_bytes": wk, "traffic_bytes": fk + wk,
             "algorithmic_bytes": algo_bytes, "source_sha256": source_hash()}
    print("\n```json\n" + json.dumps(block) + "\n```")


def decode(trace, H, I, bpw, grids, command):
    """Per-launch-grid durations of the few-assignment kernels from a
    --kernel-trace CSV, and GB/s over the touched experts' packed weights
    (gate_up 2I x H for the G1 launch, down H x I for G2; bpw maps the
    kernel's format tag, its first template argument, to packed bytes per
    weight)."""
    H, I = int(H), int(I)
    bpw = {int(k): float(v) for k, v in (g.split("=") for g in bpw.split(","))}
    touched = {int(k): int(v) for k, v in (g.split("=") for g in grids.split(","))}
    groups = {}
    for r in csv.DictReader(open(trace)):
        name = short(r["Kernel_Name"])
        if not name.startswith("decode"):
            continue
        key = (name, int(r["Grid_Size_X"]), int(r["Grid_Size_Y"]))
        groups.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    print(f"command: `{command}`\n")
    print("| kernel | grid (threads x, y) | touched experts | dispatches | avg us | min us | max us "
          "| packed MB | GB/s (avg) |")
    print("|---|---|---:|---:|---:|---:|---:|---:|---:|")
    for (name, gx, gy), v in sorted(groups.items()):
        avg = sum(v) / len(v)
        u = touched.get(gx)
        mb = gbs = ""
        if u is not None and name.startswith("decode_kernel"):
            args = name[name.index("<") + 1:].split(",")
            g1 = args[1].strip() == "true"
            b = u * (2 * I * H if g1 else H * I) * bpw[int(args[0])]
            mb, gbs = f"{b / 1e6:.1f}", f"{b / avg / 1e3:.0f}"
        print(f"| {name} | {gx} x {gy} | {'' if u is None else u} | {len(v)} | {avg:.2f} | {min(v):.2f} "
              f"| {max(v):.2f} | {mb} | {gbs} |")


if __name__ == "__main__":
    if sys.argv[1] == "stats":
        stats(sys.argv[2], sys.argv[3])
    elif sys.argv[1] == "traffic":
        traffic(*sys.argv[2:9])
    elif sys.argv[1] == "decode":
        decode(*sys.argv[2:8])
    else:
        raise SystemExit(__doc__)
