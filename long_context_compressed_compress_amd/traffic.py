"""HBM traffic of one kernel from rocprofv3 byte counters.

Two counter runs of the same command (``rocprofv3 --pmc FETCH_SIZE`` and
``rocprofv3 --pmc WRITE_SIZE``, CSV output) give KiB per dispatch.  Each
counter is calibrated on a plain device copy of known size recorded in the
same runs (``bench.py --calibrate-copy`` copies 1 GiB): factor = copy bytes /
counter bytes of the copy.  traffic = FETCH * f_fetch + WRITE * f_write, in
bytes per dispatch.

The summary written to ``profiles/`` records a digest of the kernel's source
files; ``bench.py`` reports the traffic only while the sources still match.

Usage (after the two runs, on this machine):
  python -m long_context_compressed_compress_amd.traffic --fetch F.csv --write W.csv \
      --kernel indexer_mx_kernel --out profiles/NAME.md --command "..."
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
COPY_BYTES = 1 << 30
# sources that define each measured kernel (a change voids the measurement)
KERNEL_SOURCES = {
    "indexer_mx_kernel": ["csrc/indexer.hip", "csrc/common.h"],
    "decode_step": ["csrc/indexer.hip", "csrc/topk.hip", "csrc/attention.hip", "csrc/decode.hip", "csrc/common.h",
                    "csrc/api.cpp"],
}
# "decode_step" is not one kernel: the traffic of every kernel a decode step
# launches, summed per step (steps counted by the indexer's dispatches)
STEP_KERNELS = ("decode_append_kernel", "indexer_mx_kernel", "topk_split_", "attn_mfma_", "attn_merge_")


def source_digest(kernel: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(HERE, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _per_dispatch(path: str, counter: str):
    """{dispatch id: (kernel name, summed counter value)} from a rocprofv3 counter CSV."""
    out = collections.OrderedDict()
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            d = r["Dispatch_Id"]
            name, val = out.get(d, (r["Kernel_Name"], 0.0))
            out[d] = (name, val + float(r["Counter_Value"]))
    return out


def _median(v):
    v = sorted(v)
    return v[len(v) // 2]


def measure(fetch_csv: str, write_csv: str, kernel: str):
    res = {}
    breakdown = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        disp = _per_dispatch(path, counter)
        if kernel == "decode_step":
            steps = sum(1 for n, _ in disp.values() if "indexer_mx_kernel" in n)
            tot = sum(v for n, v in disp.values() if any(k in n for k in STEP_KERNELS))
            ker = [tot / steps] if steps else []
            n_ker = steps
            parts = collections.OrderedDict()
            for n, v in disp.values():
                for k in STEP_KERNELS:
                    if k in n:
                        short = n.split("(")[0].replace("void ", "").replace("csa::", "")
                        parts[short] = parts.get(short, 0.0) + (v / steps if steps else 0.0)
            breakdown[counter] = parts
        else:
            ker = [v for n, v in disp.values() if kernel in n]
            n_ker = len(ker)
        # the calibration copies: the dispatches that moved about 1 GiB
        big = [v for n, v in disp.values() if v * 1024 > 0.5 * COPY_BYTES and not any(k in n for k in STEP_KERNELS)]
        if not ker or not big:
            raise SystemExit(f"{counter}: found {len(ker)} {kernel} dispatches and {len(big)} copy dispatches")
        res[counter] = (_median(ker), _median(big), n_ker)
    f_fetch = COPY_BYTES / (res["FETCH_SIZE"][1] * 1024)
    f_write = COPY_BYTES / (res["WRITE_SIZE"][1] * 1024)
    fetch_b = res["FETCH_SIZE"][0] * 1024 * f_fetch
    write_b = res["WRITE_SIZE"][0] * 1024 * f_write
    return {"kernel": kernel, "fetch_kib": res["FETCH_SIZE"][0], "write_kib": res["WRITE_SIZE"][0],
            "copy_fetch_kib": res["FETCH_SIZE"][1], "copy_write_kib": res["WRITE_SIZE"][1],
            "f_fetch": f_fetch, "f_write": f_write, "dispatches": res["FETCH_SIZE"][2],
            "traffic_bytes": fetch_b + write_b, "fetch_bytes": fetch_b, "write_bytes": write_b,
            "source_digest": source_digest(kernel),
            "breakdown": {n: (breakdown["FETCH_SIZE"].get(n, 0.0) * 1024 * f_fetch,
                              breakdown["WRITE_SIZE"].get(n, 0.0) * 1024 * f_write)
                          for n in breakdown.get("FETCH_SIZE", {})}}


def write_summary(m: dict, out: str, command: str, algorithmic_bytes: float | None = None):
    lines = [
        f"# HBM traffic of `{m['kernel']}` (rocprofv3 byte counters)",
        "",
        f"Commands (each a separate counter pass; output CSV under the -d folder):",
        "",
        "```",
        command,
        "```",
        "",
        "| quantity | value |",
        "|---|---|",
        f"| {m['kernel']} {'steps' if m['kernel'] == 'decode_step' else 'dispatches'} measured | "
        f"{m['dispatches']} |",
        f"| FETCH_SIZE per {'step (every kernel of the step, mean)' if m['kernel'] == 'decode_step' else 'dispatch (median)'}"
        f" | {m['fetch_kib']:.1f} KiB |",
        f"| WRITE_SIZE per {'step (every kernel of the step, mean)' if m['kernel'] == 'decode_step' else 'dispatch (median)'}"
        f" | {m['write_kib']:.1f} KiB |",
        f"| 1 GiB copy: FETCH_SIZE / WRITE_SIZE | {m['copy_fetch_kib']:.1f} / {m['copy_write_kib']:.1f} KiB |",
        f"| calibration factors (fetch, write) | {m['f_fetch']:.4f}, {m['f_write']:.4f} |",
        f"| traffic per dispatch | {m['traffic_bytes'] / 1e6:.3f} MB "
        f"(read {m['fetch_bytes'] / 1e6:.3f} MB, write {m['write_bytes'] / 1e6:.3f} MB) |",
    ]
    if algorithmic_bytes:
        lines.append(f"| algorithmic bytes per {'step' if m['kernel'] == 'decode_step' else 'dispatch'} | "
                     f"{algorithmic_bytes / 1e6:.3f} MB "
                     f"(traffic / algorithmic = {m['traffic_bytes'] / algorithmic_bytes:.3f}) |")
    if m.get("breakdown"):
        lines += ["", "Per kernel, calibrated, per step (a kernel launched twice a step is summed):", "",
                  "| kernel | read MB | write MB |", "|---|---:|---:|"]
        for n, (fb, wb) in m["breakdown"].items():
            lines.append(f"| `{n}` | {fb / 1e6:.3f} | {wb / 1e6:.3f} |")
    lines += ["", "Machine-readable:", "", "```",
              f"kernel={m['kernel']} traffic_bytes={m['traffic_bytes']:.0f} source_digest={m['source_digest']}",
              "```", ""]
    with open(out, "w") as f:
        f.write("\n".join(lines))


def load(path: str, kernel: str):
    """Traffic bytes per dispatch from a summary, or None if absent or stale."""
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"kernel=(\S+) traffic_bytes=(\d+) source_digest=(\w+)", text)
    if not m or m.group(1) != kernel or m.group(3) != source_digest(kernel):
        return None
    return float(m.group(2))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--kernel", default="indexer_mx_kernel")
    ap.add_argument("--out", required=True)
    ap.add_argument("--command", required=True)
    ap.add_argument("--algorithmic-bytes", type=float, default=None)
    a = ap.parse_args()
    m = measure(a.fetch, a.write, a.kernel)
    write_summary(m, a.out, a.command, a.algorithmic_bytes)
    print(m)


if __name__ == "__main__":
    main()
