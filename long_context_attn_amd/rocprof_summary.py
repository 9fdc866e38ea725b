"""Summarise a rocprofv3 kernel trace of this library's kernels as Markdown.

    python -m long_context_attn_amd.rocprof_summary TRACE_CSV [--title T] [--command C]

Groups the dispatches of the library's kernels (names in namespace la::) by
kernel and launch grid, so that calls of one workload are averaged together
and calls of another (for example the prefills that build the decode
workload's initial states) are kept apart.  Durations are in microseconds.
"""
from __future__ import annotations

import argparse
import csv
import re
import shutil
import statistics
import subprocess
from collections import OrderedDict

_demangled = {}


def demangle(name: str) -> str:
    """rocprofv3 leaves some names mangled; c++filt restores them when present."""
    if not name.startswith("_Z") or shutil.which("c++filt") is None:
        return name
    if name not in _demangled:
        _demangled[name] = subprocess.run(["c++filt", name], capture_output=True,
                                          text=True).stdout.strip() or name
    return _demangled[name]


def short_name(name: str) -> str:
    n = demangle(name).replace("void ", "")
    m = re.match(r"_ZN2la(\d+)", n)
    if m:  # still mangled (bf16 template arguments): keep namespace and identifier
        k = int(m.group(1))
        ident = n[m.end():m.end() + k]
        return "la::" + ident + ("<bf16>" if "DF16b" in n else "")
    return n.split("(")[0]


def summarize(path: str):
    groups = OrderedDict()
    with open(path) as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"]
            if "la::" not in name and not name.startswith("_ZN2la"):
                continue
            grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
            wg = int(r["Workgroup_Size_X"]) * int(r["Workgroup_Size_Y"]) * int(r["Workgroup_Size_Z"])
            key = (short_name(name), grid // max(wg, 1), wg)
            dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            g = groups.setdefault(key, dict(durs=[], vgpr=r.get("VGPR_Count"),
                                            agpr=r.get("Accum_VGPR_Count"),
                                            lds=r.get("LDS_Block_Size")))
            g["durs"].append(dur)
    return groups


def markdown(groups, title, command, min_calls=1):
    out = ["# " + title, "", "Command (repo root, one MI355X):", "", "    " + command, "",
           "| kernel | workgroups x threads | calls | avg us | median us | min us | max us | VGPR | AGPR | LDS B |",
           "|---|---|---|---|---|---|---|---|---|---|"]
    for (name, nwg, wg), g in groups.items():
        d = g["durs"]
        if len(d) < min_calls:
            continue
        out.append("| %s | %d x %d | %d | %.1f | %.1f | %.1f | %.1f | %s | %s | %s |" % (
            name, nwg, wg, len(d), statistics.mean(d), statistics.median(d), min(d), max(d),
            g["vgpr"], g["agpr"], g["lds"]))
    return "\n".join(out) + "\n"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("trace")
    ap.add_argument("--title", default="rocprofv3 kernel trace summary")
    ap.add_argument("--command", default="")
    ap.add_argument("--min-calls", type=int, default=1)
    a = ap.parse_args()
    print(markdown(summarize(a.trace), a.title, a.command, a.min_calls), end="")


if __name__ == "__main__":
    main()
