"""Prefix reuse at 1M context: the time to save and to restore one sequence's
decode cache (prefix_save / prefix_load), against recomputing what a restore
replaces on this path — the CSA entries with their MXFP4 keys and the HCA
entries of 2^20 raw tokens (csa_compress + hca_compress on the GPU).

One sequence of a CSA + HCA layer pair at position 2^20: 262,144 CSA entries
(256 B each) with 34-byte keys and 8,192 HCA entries, ≈ 78 MB; with the rings
(window and compressor state) ≈ 0.5 MB more.  The snapshot files go to --dir
(host I/O: what the numbers include is the file system under that folder).

  python -m long_context_compressed_compress_amd.prefix_report --dir /tmp --out profiles/prefix_reuse_1m.md
"""
from __future__ import annotations

import argparse
import json
import os
import time

import numpy as np

CTX = 1 << 20
W = 128


def _wall(torch, fn, reps):
    ts = []
    for _ in range(reps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        r = fn()
        torch.cuda.synchronize()
        ts.append(time.perf_counter() - t0)
    return float(np.median(ts)), r


def measure(folder: str, reps: int):
    import torch

    from . import libcsa as L
    from . import workloads as WL
    dev = torch.device("cuda:0")

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    wts = WL.hybrid_prefill_weights()
    weights = {"csa_w_gate": up(wts["w_gate"]), "csa_pos_bias": up(wts["pos_bias"]), "csa_w_idx": up(wts["w_idx"]),
               "hca_w_gate": up(wts["w_gate_hca"]), "hca_pos_bias": up(wts["pos_bias_hca"])}
    n_c, n_h = CTX // 4, CTX // 128
    cache = L.DecodeCache(1, 128, 64, 64, 1024, W, n_c + 64, n_h + 64, 1.0 / np.sqrt(192), weights, device=dev)
    csa = WL.csa_decode_1m(batch_rows=[0])
    hca = WL.hca_decode_1m(batch_rows=[0])
    L.kv_pack(up(csa["entries"][0]), cache.csa_kv[0, :n_c])
    L.mxfp4_quantize(up(csa["k_idx"][0]), cache.csa_keys[0, :n_c], cache.csa_key_scales[0, :n_c])
    L.kv_pack(up(hca["entries"][0]), cache.hca_kv[0, :n_h])
    cache.pos.fill_(CTX)
    cache.csa_entries.fill_(n_c)
    cache.hca_entries.fill_(n_h)
    L.decode_prime(cache, up(csa["window"]).contiguous(), up(hca["window"]).contiguous())
    torch.cuda.synchronize()

    full = os.path.join(folder, "csa_prefix_full.snap")
    ent = os.path.join(folder, "csa_prefix_entries.snap")
    res = {}
    res["save_full_s"], _ = _wall(torch, lambda: L.prefix_save(cache, 0, full), reps)
    res["save_entries_s"], _ = _wall(torch, lambda: L.prefix_save(cache, 0, ent, parts=L.CSA_PREFIX_ENTRIES), reps)
    res["bytes_full"], res["bytes_entries"] = os.path.getsize(full), os.path.getsize(ent)

    target = L.DecodeCache(1, 128, 64, 64, 1024, W, n_c + 64, n_h + 64, 1.0 / np.sqrt(192), weights, device=dev)
    last = up(csa["window"]).contiguous(), up(hca["window"]).contiguous()   # raw KV of the last 128 tokens
    res["load_full_s"], pf = _wall(torch, lambda: L.prefix_load(target, 0, full), reps)
    assert pf == CTX
    for k in ("csa_kv", "csa_keys", "csa_key_scales", "hca_kv", "csa_win", "hca_win"):
        assert torch.equal(getattr(target, k), getattr(cache, k)), k

    def load_entries_and_prime():
        p = L.prefix_load(target, 0, ent, parts=L.CSA_PREFIX_ENTRIES)
        L.decode_prime(target, *last)
        return p
    res["load_entries_prime_s"], pf = _wall(torch, load_entries_and_prime, reps)
    assert pf == CTX - 128
    half = CTX // 2
    res["load_half_prefix_s"], pf = _wall(
        torch, lambda: L.prefix_load(target, 0, ent, parts=L.CSA_PREFIX_ENTRIES, prefix_len=half), reps)
    assert pf == half - 128 and int(target.csa_entries[0]) == half // 4

    # what a restore replaces here: both compressors over 2^20 raw BF16 tokens
    raw = torch.randn(1, CTX, 192, device=dev).to(torch.bfloat16)
    kv = torch.empty(1, n_c, 256, dtype=torch.uint8, device=dev)
    keys = torch.empty(1, n_c, 32, dtype=torch.uint8, device=dev)
    scl = torch.empty(1, n_c, 2, dtype=torch.uint8, device=dev)
    kvh = torch.empty(1, n_h, 256, dtype=torch.uint8, device=dev)

    def recompute():
        L.csa_compress(raw, 0, weights["csa_w_gate"], weights["csa_pos_bias"], 0, n_c, kv, w_idx=weights["csa_w_idx"],
                       key_out=keys, key_scales=scl)
        L.hca_compress(raw, 0, weights["hca_w_gate"], weights["hca_pos_bias"], 0, n_h, kvh)
    recompute()
    res["recompute_s"], _ = _wall(torch, recompute, reps)
    for p in (full, ent):
        os.remove(p)
    return res


def write_md(res: dict, out: str, command: str):
    mb = 1e6
    rows = [("prefix_save, entries + rings (full caching)", res["save_full_s"], res["bytes_full"]),
            ("prefix_save, entries only (no SWA caching)", res["save_entries_s"], res["bytes_entries"]),
            ("prefix_load, entries + rings", res["load_full_s"], res["bytes_full"]),
            ("prefix_load, entries + decode_prime of the last 128 tokens", res["load_entries_prime_s"],
             res["bytes_entries"]),
            ("prefix_load, entries of a 2^19-token prefix (file read whole, half copied)", res["load_half_prefix_s"],
             res["bytes_entries"])]
    lines = ["# Prefix reuse, one sequence at 1M context (CSA + HCA layer pair)", "",
             "Command:", "", "```", command, "```", "",
             "Snapshot of one sequence at position 2^20: 262,144 CSA entries (256 B) with MXFP4 keys (34 B) and",
             "8,192 HCA entries; the rings add the window and compressor state. Wall-clock medians (host I/O through",
             "the file system of the snapshot folder, device copies included; the calls synchronise the stream).", "",
             "| operation | ms | file MB | GB/s of file |", "|---|---:|---:|---:|"]
    for name, s, b in rows:
        lines.append(f"| {name} | {s * 1e3:.1f} | {b / mb:.1f} | {b / s / 1e9:.2f} |")
    lines += ["", f"Recomputing the same entries from 2^20 raw BF16 tokens on the GPU (csa_compress with MXFP4 keys +",
              f"hca_compress, the work a restore replaces on this path): {res['recompute_s'] * 1e3:.1f} ms. The model's",
              "own prefill of the prefix (projections that produce the raw KV, every other layer) is outside this path",
              "and is what a restore saves in a deployment.", "", "```", json.dumps(res), "```", ""]
    with open(out, "w") as f:
        f.write("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--dir", default="/tmp")
    ap.add_argument("--reps", type=int, default=5)
    ap.add_argument("--json", help="write the measurements here")
    ap.add_argument("--out", help="markdown summary")
    ap.add_argument("--from-json", help="summarise an earlier --json run instead of measuring")
    a = ap.parse_args()
    js = a.from_json or a.json or "prefix.json"  # the measurement run's JSON, as given on the command line
    cmd = ("cd /tmp && export TMPDIR=/tmp && cd $REPO\n"
           f"python3 -m long_context_compressed_compress_amd.prefix_report --dir {a.dir} --json {js}\n"
           f"python -m long_context_compressed_compress_amd.prefix_report --from-json {js} --out {a.out}")
    if a.from_json:
        res = json.load(open(a.from_json))
    else:
        res = measure(a.dir, a.reps)
        print(json.dumps(res), flush=True)
        if a.json:
            with open(a.json, "w") as f:
                json.dump(res, f)
    if a.out:
        write_md(res, a.out, cmd)


if __name__ == "__main__":
    main()
