"""Condense a rocprofv3 --kernel-trace --stats CSV into a short Markdown table.

usage: python profiles/summarize.py <kernel_stats.csv> "<command that produced it>" > profiles/<name>.md
"""

import csv
import re
import sys


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


def main(path, command):
    rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    print(f"command: `{command}`\n")
    print("| kernel | calls | avg us | min us | max us | % of GPU time |")
    print("|---|---:|---:|---:|---:|---:|")
    for r in rows:
        print(f"| {short(r['Name'])} | {r['Calls']} | {float(r['AverageNs'])/1e3:.1f} | "
              f"{float(r['MinNs'])/1e3:.1f} | {float(r['MaxNs'])/1e3:.1f} | {float(r['Percentage']):.1f} |")


if __name__ == "__main__":
    main(sys.argv[1], sys.argv[2])
