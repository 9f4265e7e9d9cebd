"""Per-kernel summary of rocprofv3 shader counters (``--pmc``, CSV output).

Each ``--csv`` is one counter pass of the same command (rocprofv3 collects a
limited set per pass).  For every kernel name given by ``--kernel`` (a
substring of the dispatched kernel's name), the summary lists each counter's
median value per dispatch over all matching dispatches, then a few ratios:

  VALU / MFMA       SQ_INSTS_VALU / SQ_INSTS_MFMA (SQ_INSTS_VALU counts the
                    MFMA instructions too)
  MOPS / MFMA       SQ_INSTS_VALU_MFMA_MOPS_<type> / SQ_INSTS_MFMA (the
                    counter's matrix-op units per instruction; the unit
                    differs between operand types, so flops are taken from
                    the instruction count instead)
  MFMA flops        SQ_INSTS_MFMA x the flops of the kernel's one MFMA shape,
                    when given with --mfma-flops KERNEL=FLOPS
  MfmaUtil          rocprofv3's derived metric: MFMA-busy cycles over the
                    dispatch's GPU-active cycles times the SIMD count, percent
  VALUBusy          rocprofv3's derived metric: VALU-active cycles per CU over
                    the GPU-active cycles, percent
  LdsBankConflict   rocprofv3's derived metric: bank-conflict cycles per LDS
                    access cycle

Usage:
  python -m long_context_compressed_compress_amd.counters --csv A.csv --csv B.csv \\
      --kernel indexer_mx_kernel --title "..." --command "..." --out profiles/NAME.md
"""
from __future__ import annotations

import argparse
import collections
import csv


def per_kernel(paths, kernels):
    """{kernel substring: ({counter: [value per dispatch]}, dispatch count)}."""
    out = {}
    for k in kernels:
        vals = collections.defaultdict(list)
        n = 0
        for p in paths:
            disp = collections.defaultdict(lambda: collections.defaultdict(float))
            with open(p, newline="") as f:
                for r in csv.DictReader(f):
                    if k in r["Kernel_Name"]:
                        disp[r["Dispatch_Id"]][r["Counter_Name"]] += float(r["Counter_Value"])
            for d in disp.values():
                for c, v in d.items():
                    vals[c].append(v)
            n = max(n, len(disp))
        out[k] = (vals, n)
    return out


def _median(v):
    v = sorted(v)
    return v[len(v) // 2]


def summarize(paths, kernels, title, command, notes=(), mfma_flops=None):
    mfma_flops = mfma_flops or {}
    res = per_kernel(paths, kernels)
    lines = [f"# {title}", "", "Commands (one counter pass each):", "", "```", command, "```", ""]
    for k, (vals, n) in res.items():
        if not vals:
            lines += [f"## `{k}`", "", "no dispatch found", ""]
            continue
        med = {c: _median(v) for c, v in vals.items()}
        lines += [f"## `{k}` ({n} dispatches, median per dispatch)", "", "| counter | value |", "|---|---:|"]
        for c in sorted(med):
            v = med[c]
            lines.append(f"| {c} | {v:,.0f} |" if abs(v) >= 100 else f"| {c} | {v:.4g} |")
        derived = []
        if med.get("SQ_INSTS_MFMA"):
            if "SQ_INSTS_VALU" in med:
                derived.append(("VALU instructions per MFMA instruction", f"{med['SQ_INSTS_VALU'] / med['SQ_INSTS_MFMA']:.2f}"))
            for c, v in med.items():
                if c.startswith("SQ_INSTS_VALU_MFMA_MOPS_") and v > 0:
                    derived.append((f"{c} per MFMA instruction", f"{v / med['SQ_INSTS_MFMA']:.1f}"))
            if k in mfma_flops:
                derived.append((f"MFMA flops per dispatch (SQ_INSTS_MFMA x {mfma_flops[k]:,})",
                                f"{med['SQ_INSTS_MFMA'] * mfma_flops[k]:.4g}"))
        if derived:
            lines += ["", "| derived | value |", "|---|---:|"] + [f"| {a} | {b} |" for a, b in derived]
        lines.append("")
    lines += list(notes)
    return "\n".join(lines) + "\n"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--csv", action="append", required=True)
    ap.add_argument("--kernel", action="append", required=True)
    ap.add_argument("--title", required=True)
    ap.add_argument("--command", required=True)
    ap.add_argument("--note", action="append", default=[])
    ap.add_argument("--mfma-flops", action="append", default=[], metavar="KERNEL=FLOPS")
    ap.add_argument("--out", required=True)
    a = ap.parse_args()
    mf = {kv.split("=")[0]: int(kv.split("=")[1]) for kv in a.mfma_flops}
    text = summarize(a.csv, a.kernel, a.title, a.command, a.note, mf)
    with open(a.out, "w") as f:
        f.write(text)
    print(text)


if __name__ == "__main__":
    main()
