"""Condense rocprofv3 CSV output into the short Markdown summaries kept under
``profiles/``.

    python profsum.py stats <kernel_stats.csv> "<command>"
    python profsum.py traffic <fetch_dir> <write_dir> <kernel> <copy_bytes> \
        <algorithmic_bytes> "<fetch command>" "<write command>"
    python profsum.py decode <kernel_trace.csv> <H> <I> \
        <format>=<bytes_per_weight>[,...] <grid_x>=<touched experts>[,...] "<command>"
    python profsum.py counters <pmc_dir> <kernel>[@<workload>] <simd_count|0> \
        <algorithmic_flops> "<command>"
    python profsum.py kernels <pmc_dir> "<command>"

``stats`` prints a per-kernel duration table.  ``traffic`` reads two
``--pmc FETCH_SIZE`` / ``--pmc WRITE_SIZE`` runs (KiB per dispatch), takes the
mean per dispatch of ``kernel`` and calibrates each counter against the
largest plain device copy in the same run (``copy_bytes`` bytes read and
written by ``__amd_rocclr_copyBuffer``), then prints the table plus a JSON
block that bench.py reads; the block carries the SHA-256 of the kernel
sources so that a changed kernel reports no stale traffic.  ``decode`` splits
the few-assignment kernels' dispatches by launch grid (one grid per batch
size) and prices each against the packed bytes of the experts it touches.
``counters`` averages every counter of one ``--pmc`` run per dispatch of
``kernel`` and derives the MFMA busy fraction (the summed per-SIMD
SQ_VALU_MFMA_BUSY_CYCLES over the GPU's busy cycles times the SIMD count, the
definition rocprofv3 gives MfmaUtil; GRBM_GUI_ACTIVE arrives summed over the
XCDs, so one XCD's busy cycles are that sum over the agent's Num_Xcc), the
shader clock the busy cycles imply over the dispatch's duration, and the flops
the MFMA op counter implies (SQ_INSTS_VALU_MFMA_MOPS_BF16 counts units of 512
flops).  ``simd_count`` 0 takes the SIMD count from the agent info.
``kernels`` prints those derived figures, and the SQ stall fractions when
the run counted them, for every kernel of the library in one run.

A kernel argument may carry ``@<workload>`` (e.g. ``g1_kernel<1>@mixtral_T16384``):
the tag names the workload in the JSON block, which bench.py matches against
the configuration it measures; the counters are read for the bare kernel
name, so the profiled command must run that kernel on that workload only.
"""

import csv
import glob
import hashlib
import json
import os
import re
import sys

PKG = "bit_weight_quantization_moeq_amd"
SOURCES = tuple(f"{PKG}/csrc/{n}" for n in (
    "experts.hip", "decode.hip", "quant.hip", "route.hip", "api.hip", "router.hip", "experts_core.h",
    "moeq_internal.h"))


def _code_only(text):
    """The source with comments and blank space removed (the sources hold no
    string literal containing a comment marker)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def _kernel_file(kernel):
    """The source under csrc/ that defines `kernel` (bare name, template
    arguments and any @workload tag dropped), or None."""
    here = os.path.dirname(os.path.abspath(__file__))
    base = kernel.split("@", 1)[0].split("<", 1)[0].strip()
    for rel in SOURCES:
        with open(os.path.join(here, rel)) as f:
            if re.search(r"__global__[^;{]*\b" + re.escape(base) + r"\s*\(", f.read()):
                return rel
    return None


def _with_includes(rel):
    """`rel` and the csrc headers it includes, transitively, in first-seen order."""
    here = os.path.dirname(os.path.abspath(__file__))
    out = [rel]
    for cur in out:
        with open(os.path.join(here, cur)) as f:
            for name in re.findall(r'#include "([^"]+)"', f.read()):
                inc = f"{PKG}/csrc/{name}"
                if inc not in out and os.path.exists(os.path.join(here, inc)):
                    out.append(inc)
    return out


def source_hash(kernel=None):
    """SHA-256 of the kernel sources' code (comments and layout ignored): of
    the file that defines `kernel` plus the csrc headers it includes, or of
    every source when no kernel is named (or its file is not found)."""
    here = os.path.dirname(os.path.abspath(__file__))
    f = _kernel_file(kernel) if kernel else None
    files = _with_includes(f) if f else SOURCES
    h = hashlib.sha256()
    for rel in files:
        with open(os.path.join(here, rel)) as fh:
            h.update(_code_only(fh.read()).encode())
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


def _bare(kernel):
    return kernel.split("@", 1)[0]


def traffic(fetch_dir, write_dir, kernel, copy_bytes, algo_bytes, cmd_f, cmd_w):
    copy_bytes, algo_bytes = float(copy_bytes), float(algo_bytes)
    k = _bare(kernel)
    f, w = _per_dispatch(fetch_dir, "FETCH_SIZE"), _per_dispatch(write_dir, "WRITE_SIZE")
    cf = max(f["__amd_rocclr_copyBuffer"]) * 1024.0 / copy_bytes   # counter bytes per copied byte
    cw = max(w["__amd_rocclr_copyBuffer"]) * 1024.0 / copy_bytes
    fk = sum(f[k]) / len(f[k]) * 1024.0 / cf
    wk = sum(w[k]) / len(w[k]) * 1024.0 / cw
    print(f"FETCH_SIZE command: `{cmd_f}`\n\nWRITE_SIZE command: `{cmd_w}`\n")
    print(f"Calibration: the largest `__amd_rocclr_copyBuffer` dispatch copies {copy_bytes:.0f} bytes; "
          f"FETCH_SIZE reads {cf:.3f} and WRITE_SIZE {cw:.3f} counter bytes per copied byte.\n")
    print("| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM read MB (cal.) | HBM write MB (cal.) "
          "| algorithmic MB | traffic / algorithmic |")
    print("|---|---:|---:|---:|---:|---:|---:|---:|")
    print(f"| {k} | {len(f[k])} | {sum(f[k]) / len(f[k]):.0f} | {sum(w[k]) / len(w[k]):.0f} "
          f"| {fk / 1e6:.1f} | {wk / 1e6:.1f} | {algo_bytes / 1e6:.1f} | {(fk + wk) / algo_bytes:.3f} |")
    block = {"kernel": kernel, "hbm_read_bytes": fk, "hbm_write_bytes": wk, "traffic_bytes": fk + wk,
             "algorithmic_bytes": algo_bytes, "source_sha256": source_hash(kernel)}
    print("\n```json\n" + json.dumps(block) + "\n```")


def _all_counters(d):
    """kernel short name -> list of {counter: value} per dispatch (plus the
    dispatch's duration in ns under "duration_ns")."""
    out = {}
    for p in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        acc = {}
        for r in csv.DictReader(open(p)):
            key = (r["Dispatch_Id"], r["Kernel_Name"])
            c = acc.setdefault(key, {})
            c[r["Counter_Name"]] = c.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            c["duration_ns"] = float(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
        for (_, name), c in acc.items():
            out.setdefault(short(name), []).append(c)
    return out


def _gpu_agent(d):
    """The GPU row of the run's agent info (Num_Xcc, Simd_Count, ...), or {}."""
    for p in glob.glob(os.path.join(d, "**", "*agent_info.csv"), recursive=True):
        for r in csv.DictReader(open(p)):
            if r.get("Name", "").startswith("gfx"):
                return r
    return {}


def counters(pmc_dir, kernel, simds, algo_flops, command):
    algo_flops = float(algo_flops)
    agent = _gpu_agent(pmc_dir)
    simds = int(simds) or int(agent.get("Simd_Count", 0))
    nxcc = int(agent.get("Num_Xcc", 1) or 1)
    k = _bare(kernel)
    per = _all_counters(pmc_dir)[k]
    names = sorted({n for c in per for n in c})
    mean = {n: sum(c.get(n, 0.0) for c in per) / len(per) for n in names}
    print(f"command: `{command}`\n")
    print(f"{len(per)} dispatches of `{k}`; mean per dispatch:\n")
    print("| counter | mean per dispatch |")
    print("|---|---:|")
    for n in names:
        print(f"| {n} | {mean[n]:.6g} |")
    block = {"kernel": kernel, "dispatches": len(per), "counters": mean, "source_sha256": source_hash(kernel)}
    if "MfmaUtil" in mean:
        block["mfma_util"] = mean["MfmaUtil"] / 100.0
        print(f"\nMFMA busy (rocprofv3's MfmaUtil: the summed per-SIMD SQ_VALU_MFMA_BUSY_CYCLES over the "
              f"largest GRBM_GUI_ACTIVE instance times the SIMD count): {mean['MfmaUtil']:.1f} % "
              f"(mean over dispatches).")
    elif "SQ_VALU_MFMA_BUSY_CYCLES" in mean and "GRBM_GUI_ACTIVE" in mean and simds > 0:
        util = [c["SQ_VALU_MFMA_BUSY_CYCLES"] / (c["GRBM_GUI_ACTIVE"] / nxcc * simds) for c in per]
        clk = [c["GRBM_GUI_ACTIVE"] / nxcc / c["duration_ns"] for c in per]
        block["mfma_util"] = sum(util) / len(util)
        block["shader_clock_GHz"] = sum(clk) / len(clk)
        print(f"\nMFMA busy: SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / {nxcc} XCDs x {simds} SIMDs) = "
              f"{100 * block['mfma_util']:.1f} % of the busy cycles (mean over dispatches); those cycles over "
              f"the dispatch duration give a shader clock of {block['shader_clock_GHz']:.3f} GHz.")
    if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in mean and algo_flops > 0:
        block["counter_flops"] = mean["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512.0
        block["algorithmic_flops"] = algo_flops
        print(f"\nbf16 MFMA flops from the op counter (x 512): {block['counter_flops']:.4g} per dispatch, "
              f"against {algo_flops:.4g} algorithmic ({block['counter_flops'] / algo_flops:.3f} x).")
    print("\n```json\n" + json.dumps(block) + "\n```")


def kernels(pmc_dir, command, prefix="moeq::"):
    """One row per kernel of the library (names starting with `prefix`) in a
    --pmc run: dispatches, mean duration, and whichever derived figures its
    counters allow -- the MFMA busy fraction and shader clock (as in
    ``counters``) and, from the SQ stall counters, the fractions of the
    waves' cycles spent waiting on a counter (SQ_WAIT_INST_ANY), waiting for
    anything (SQ_WAIT_ANY), issuing VALU (SQ_ACTIVE_INST_VALU, MFMA included)
    and LDS (SQ_ACTIVE_INST_LDS) instructions; with SQ_WAVES in the same run,
    the instructions each wave issued (SQ_INSTS_VALU, MFMA included;
    SQ_INSTS_VMEM_RD; SQ_INSTS_MFMA)."""
    agent = _gpu_agent(pmc_dir)
    simds = int(agent.get("Simd_Count", 0) or 0)
    nxcc = int(agent.get("Num_Xcc", 1) or 1)
    per = {}
    for p in glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True):
        acc = {}
        for r in csv.DictReader(open(p)):
            if not r["Kernel_Name"].replace("void ", "").startswith(prefix):
                continue
            c = acc.setdefault((r["Dispatch_Id"], r["Kernel_Name"]), {})
            c[r["Counter_Name"]] = c.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            c["duration_ns"] = float(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
        for (_, name), c in acc.items():
            per.setdefault(short(name), []).append(c)
    print(f"command: `{command}`\n")
    print("| kernel | dispatches | mean us | MFMA busy | clock GHz | wait on counter | wait any | VALU issue | LDS issue "
          "| VALU instr / wave | VMEM reads / wave | MFMA / wave |")
    print("|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|")
    rows = {}
    for k in sorted(per, key=lambda k: -sum(c["duration_ns"] for c in per[k])):
        cs = per[k]
        tot = lambda n: sum(c.get(n, 0.0) for c in cs)
        row = {"dispatches": len(cs), "mean_us": tot("duration_ns") / len(cs) / 1e3}
        if tot("SQ_VALU_MFMA_BUSY_CYCLES") > 0 and tot("GRBM_GUI_ACTIVE") > 0 and simds:
            row["mfma_busy"] = tot("SQ_VALU_MFMA_BUSY_CYCLES") / (tot("GRBM_GUI_ACTIVE") / nxcc * simds)
            row["clock_GHz"] = tot("GRBM_GUI_ACTIVE") / nxcc / tot("duration_ns")
        if tot("SQ_WAVE_CYCLES") > 0:
            for n, key in (("SQ_WAIT_INST_ANY", "wait_counter"), ("SQ_WAIT_ANY", "wait_any"),
                           ("SQ_ACTIVE_INST_VALU", "valu"), ("SQ_ACTIVE_INST_LDS", "lds")):
                if n in cs[0]:
                    row[key] = tot(n) / tot("SQ_WAVE_CYCLES")
        if tot("SQ_WAVES") > 0:
            for n, key in (("SQ_INSTS_VALU", "valu_per_wave"), ("SQ_INSTS_VMEM_RD", "vmem_rd_per_wave"),
                           ("SQ_INSTS_MFMA", "mfma_per_wave")):
                if n in cs[0]:
                    row[key] = tot(n) / tot("SQ_WAVES")
        f = lambda key, fmt: (fmt.format(row[key]) if key in row else "")
        print(f"| {k} | {row['dispatches']} | {row['mean_us']:.1f} | {f('mfma_busy', '{:.1%}')} | {f('clock_GHz', '{:.2f}')} "
              f"| {f('wait_counter', '{:.1%}')} | {f('wait_any', '{:.1%}')} | {f('valu', '{:.1%}')} | {f('lds', '{:.1%}')} "
              f"| {f('valu_per_wave', '{:.0f}')} | {f('vmem_rd_per_wave', '{:.0f}')} | {f('mfma_per_wave', '{:.0f}')} |")
        rows[k] = row
    return rows


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
    elif sys.argv[1] == "counters":
        counters(*sys.argv[2:7])
    elif sys.argv[1] == "kernels":
        kernels(sys.argv[2], sys.argv[3])
    else:
        raise SystemExit(__doc__)
