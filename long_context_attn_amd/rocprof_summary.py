"""Summaries of rocprofv3 output for this library's kernels, as Markdown.

    python -m long_context_attn_amd.rocprof_summary TRACE_CSV [--title T] [--command C]
    python -m long_context_attn_amd.rocprof_summary pmc --fetch CSV --write CSV
           --workload NAME --copy-bytes N [--kernel-workload K=W ...] [--update JSON]
           [--title T] [--command C]
    python -m long_context_attn_amd.rocprof_summary counters CSV [--title T] [--command C]

The first form groups the dispatches of the library's kernels (names in
namespace la::) of a --kernel-trace run by kernel and launch grid, so that
calls of one workload are averaged together and calls of another (for
example the prefills that build the decode workload's initial states) are
kept apart.  Durations are in microseconds.

The second form reads two --pmc runs (FETCH_SIZE, then WRITE_SIZE, in KiB per
dispatch) of `bench.py --pmc-pass`, whose first large dispatch is a device
copy of exactly --copy-bytes bytes.  The counters do not count bytes one to
one, so each is scaled by what it reads for that copy (known bytes read and
written); the result is the HBM traffic per launch of each kernel, recorded
in --update (a JSON file keyed "kernel@workload") with the hash of the
kernel sources it was measured on.
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
    m = re.match(r"_ZN2la(?:12_GLOBAL__N_1)?(\d+)", n)
    if m:  # still mangled (bf16 template arguments): keep namespace and identifier
        k = int(m.group(1))
        ident = n[m.end():m.end() + k]
        # literal template arguments (bool and int), e.g. ILb1ELb0EE -> <true, false>
        t = re.match(r"I((?:L[bi]\d+E)+)E", n[m.end() + k:])
        if t:
            args = re.findall(r"L([bi])(\d+)E", t.group(1))
            return "la::%s<%s>" % (ident, ", ".join(
                ("true" if v == "1" else "false") if ty == "b" else v for ty, v in args))
        return "la::" + ident + ("<bf16>" if "DF16b" in n else "")
    # kernels in an anonymous namespace: "la::(anonymous namespace)::name(args)"
    n = n.replace("(anonymous namespace)::", "")
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
    out += ["", "VGPR and AGPR are rocprofv3's VGPR_Count and Accum_VGPR_Count fields as the tool "
            "reports them; for the large kernels they read about half of the register count in "
            "the compiled code object (the walk: 124 here, .vgpr_count 242)."]
    return "\n".join(out) + "\n"


def _pmc_values(path):
    """{kernel short name: [values]} and the copy kernel's values of one --pmc csv."""
    vals, copy = {}, []
    with open(path) as f:
        for r in csv.DictReader(f):
            name, x = r["Kernel_Name"], float(r["Counter_Value"])
            if "la::" in name or name.startswith("_ZN2la"):
                vals.setdefault(short_name(name).replace("la::", "").split("<")[0], []).append(x)
            elif "copyBuffer" in name:
                copy.append(x)
    return vals, copy


def counters_summary(path, title, command, simds=1024):
    """Median per dispatch of every counter of a --pmc csv, per kernel."""
    vals = OrderedDict()
    with open(path) as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"]
            if "la::" not in name and not name.startswith("_ZN2la"):
                continue
            # one row per kernel and launch shape (a kernel launched on two
            # shapes, such as the two projection GEMMs, gets two rows)
            wg = int(r.get("Workgroup_Size") or 0)
            grid = int(r.get("Grid_Size") or 0)
            k = short_name(name).replace("la::", "")
            k = "%s | %s" % (k, "%d x %d" % (grid // wg, wg) if wg > 0 else "-")
            vals.setdefault(k, OrderedDict()).setdefault(r["Counter_Name"], []).append(
                float(r["Counter_Value"]))
    names = []
    for d in vals.values():
        for c in d:
            if c not in names:
                names.append(c)
    out = ["# " + title, "", "Command (repo root, one MI355X):", ""]
    out += ["    " + c for c in command.split(" ;; ")]
    note = "Median per dispatch."
    if "MfmaUtil" in names or "VALUBusy" in names:
        note += ("  MfmaUtil and VALUBusy are rocprofv3's derived metrics, in percent: the MFMA "
                 "unit's busy cycles over all %d SIMDs, and the cycles the CUs spend issuing "
                 "vector-ALU instructions, each against the GPU's active cycles." % simds)
    out += ["", note, "",
            "| kernel | workgroups x threads | dispatches | " + " | ".join(names) + " |",
            "|---|---|---|" + "---|" * len(names)]
    for k, d in vals.items():
        row = [k, str(max(len(v) for v in d.values()))]
        for c in names:
            row.append("%.4g" % statistics.median(d[c]) if c in d else "")
        out.append("| " + " | ".join(row) + " |")
    return "\n".join(out) + "\n"


def pmc_summary(fetch_csv, write_csv, workload, copy_bytes, title, command, update=None,
                kernel_workloads=None):
    import json
    import os
    from .build import source_sha
    fv, fc = _pmc_values(fetch_csv)
    wv, wc = _pmc_values(write_csv)
    if not fc or not wc:
        raise SystemExit("no device-copy dispatch in the counter runs: no calibration")
    # the copy reads and writes copy_bytes each; counters are KiB per dispatch
    f_fetch = copy_bytes / (max(fc) * 1024.0)
    f_write = copy_bytes / (max(wc) * 1024.0)
    sha = source_sha()
    out = ["# " + title, "", "Commands (repo root, one MI355X):", ""]
    out += ["    " + c for c in command.split(" ;; ")]
    out += ["", "Calibration: for a device copy of %d bytes FETCH_SIZE counts 1/%.3f of the bytes "
            "read and WRITE_SIZE 1/%.3f of the bytes written; the byte columns scale the counters "
            "by those factors.  Kernel sources %s." % (copy_bytes, f_fetch, f_write, sha), "",
            "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM read MB | HBM write MB | "
            "HBM total MB |", "|---|---|---|---|---|---|---|"]
    entries = {}
    for k in sorted(set(fv) & set(wv)):
        fk = statistics.median(fv[k])
        wk = statistics.median(wv[k])
        rd, wr = fk * 1024 * f_fetch, wk * 1024 * f_write
        out.append("| %s | %d | %.0f | %.0f | %.1f | %.1f | %.1f |" % (
            k, len(fv[k]), fk, wk, rd / 1e6, wr / 1e6, (rd + wr) / 1e6))
        wl = (kernel_workloads or {}).get(k, workload)
        entries["%s@%s" % (k, wl)] = dict(
            hbm_bytes_per_launch=int(rd + wr), read_bytes=int(rd), write_bytes=int(wr),
            fetch_factor=round(f_fetch, 4), write_factor=round(f_write, 4), source_sha=sha)
    if update:
        doc = json.load(open(update)) if os.path.exists(update) else {}
        doc.update(entries)
        with open(update, "w") as f:
            json.dump(doc, f, indent=1, sort_keys=True)
            f.write("\n")
    return "\n".join(out) + "\n"


def main():
    import sys
    if len(sys.argv) > 1 and sys.argv[1] == "pmc":
        ap = argparse.ArgumentParser()
        ap.add_argument("pmc")
        ap.add_argument("--fetch", required=True)
        ap.add_argument("--write", required=True)
        ap.add_argument("--workload", required=True)
        ap.add_argument("--copy-bytes", type=int, required=True)
        ap.add_argument("--update")
        ap.add_argument("--kernel-workload", action="append", default=[],
                        help="KERNEL=WORKLOAD: the workload a kernel's dispatches belong to")
        ap.add_argument("--title", default="rocprofv3 traffic counters")
        ap.add_argument("--command", default="")
        a = ap.parse_args()
        kw = dict(x.split("=", 1) for x in a.kernel_workload)
        print(pmc_summary(a.fetch, a.write, a.workload, a.copy_bytes, a.title, a.command,
                          a.update, kw), end="")
        return
    if len(sys.argv) > 1 and sys.argv[1] == "counters":
        ap = argparse.ArgumentParser()
        ap.add_argument("counters")
        ap.add_argument("csv")
        ap.add_argument("--title", default="rocprofv3 counters")
        ap.add_argument("--command", default="")
        a = ap.parse_args()
        print(counters_summary(a.csv, a.title, a.command), end="")
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("trace")
    ap.add_argument("--title", default="rocprofv3 kernel trace summary")
    ap.add_argument("--command", default="")
    ap.add_argument("--min-calls", type=int, default=1)
    a = ap.parse_args()
    print(markdown(summarize(a.trace), a.title, a.command, a.min_calls), end="")


if __name__ == "__main__":
    main()
