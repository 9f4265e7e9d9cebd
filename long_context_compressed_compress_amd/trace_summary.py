"""Per-kernel durations from a rocprofv3 kernel trace (``--kernel-trace``,
default rocpd output: an SQLite ``*_results.db`` with a ``kernels`` view).

For every kernel name: dispatch count, mean / min / max duration, and the
time per step (total over the run / steps), where the number of steps is the
dispatch count of ``--step-kernel`` divided by ``--per-step`` (how many times
a step launches that kernel).

Usage:
  python -m long_context_compressed_compress_amd.trace_summary --db RUN_results.db \\
      --step-kernel indexer_mx_kernel --title "..." --command "..." --out profiles/NAME.md
"""
from __future__ import annotations

import argparse
import collections
import sqlite3


def durations(db_path):
    db = sqlite3.connect(db_path)
    cols = [r[1] for r in db.execute("pragma table_info(kernels)")]
    name_col = "name" if "name" in cols else "kernel_name"
    d = collections.defaultdict(list)
    for name, start, end in db.execute(f"select {name_col}, start, end from kernels order by start"):
        d[name].append((end - start) / 1000.0)
    return d


def short(name: str) -> str:
    n = name.split("(")[0]
    return n[5:] if n.startswith("void ") else n


def summarize(db_path, step_kernel, per_step, title, command, notes=()):
    d = durations(db_path)
    n_step = sum(len(v) for k, v in d.items() if step_kernel in k) // max(1, per_step)
    rows = sorted(d.items(), key=lambda kv: -sum(kv[1]))
    lines = [f"# {title}", "", "Command:", "", "```", command, "```", "",
             f"Per-kernel durations over every dispatch of the run (set-up included); steps = "
             f"{n_step} (dispatches of `{step_kernel}` / {per_step}); per step = total / steps.", "",
             "| kernel | calls | avg us | min us | max us | us per step |", "|---|---:|---:|---:|---:|---:|"]
    step_sum = 0.0
    for name, v in rows:
        per = sum(v) / n_step if n_step else 0.0
        step_sum += per if len(v) >= n_step else 0.0
        lines.append(f"| `{short(name)}` | {len(v)} | {sum(v) / len(v):.2f} | {min(v):.2f} | {max(v):.2f} | "
                     f"{per:.2f} |")
        if n_step and len(v) == 2 * n_step:   # launched twice a step: each launch of the step on its own
            for j, which in ((0, "1st"), (1, "2nd")):
                u = v[j::2]
                lines.append(f"| &nbsp;&nbsp;{which} launch of the step | {len(u)} | {sum(u) / len(u):.2f} | "
                             f"{min(u):.2f} | {max(u):.2f} | {sum(u) / n_step:.2f} |")
    lines += ["", f"Sum of kernel time per step over the kernels launched every step: {step_sum:.1f} us.", ""]
    lines += list(notes)
    return "\n".join(lines) + "\n"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--db", required=True)
    ap.add_argument("--step-kernel", default="indexer_mx_kernel")
    ap.add_argument("--per-step", type=int, default=1)
    ap.add_argument("--title", required=True)
    ap.add_argument("--command", required=True)
    ap.add_argument("--note", action="append", default=[])
    ap.add_argument("--out", required=True)
    a = ap.parse_args()
    text = summarize(a.db, a.step_kernel, a.per_step, a.title, a.command, a.note)
    with open(a.out, "w") as f:
        f.write(text)
    print(text)


if __name__ == "__main__":
    main()
