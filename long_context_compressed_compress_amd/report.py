"""Per-workload report: every stage of the five workloads timed on the GPU,
with its algorithmic bytes and flops against the chip's peaks.

The workloads (sizes and seeded inputs from ``workloads``):
  1 CSA decode, tiny, float32 end to end;
  2 CSA chunked prefill, one 4096-query chunk against 16384 entries;
  3 CSA decode at 1M context, batch 8;
  4 HCA decode at 1M context, batch 32;
  5 hybrid CSA + HCA layer pair, 131072-token prefill in 32 chunks.

Steps:
  time:      python -m long_context_compressed_compress_amd.report --json T.json
  counters:  for each workload N, two rocprofv3 passes (FETCH_SIZE, then
             WRITE_SIZE) over
               python3 -m long_context_compressed_compress_amd.report --config N --reps 1 --warmup 0 \\
                   --markers --calibrate-copy
             (each stage runs once per call, cfg 5 once per chunk; a float64
             fill before every stage call and after the last marks where each
             call's dispatches begin);
  summary:   python -m long_context_compressed_compress_amd.report --summarize T.json \\
                 --counters DIR --out profiles/NAME.md
             (DIR holds fetch_N.csv / write_N.csv per workload).

Algorithmic bytes count each tensor a stage must read or write once (keys
resident in L2 across the queries of a prefill chunk count once); flops
count 2 per multiply-add of the stage's contractions.  The MFMA fraction is
algorithmic flops / time against the dense peak of the contraction's
operand type; it is the utilisation the arithmetic asks for, not a counter.
"""
from __future__ import annotations

import argparse
import collections
import csv
import json
import math
import os
import sys

import numpy as np

HBM_PEAK_GBS = 8000.0
PEAK_TFLOPS = {"fp4": 10100.0, "bf16": 2500.0, "fp32": 157.3}
DIM = 192
SCALE = 1.0 / math.sqrt(DIM)
MARKER = "FillFunctor<double>"  # kernel name of the marker fill
CONFIG_NAMES = {1: "CSA decode tiny (fp32)", 2: "CSA chunked prefill (4096 x 16384)",
                3: "CSA decode 1M, batch 8", 4: "HCA decode 1M, batch 32",
                5: "hybrid pair prefill, 131072 tokens"}


class Stage:
    def __init__(self, name, fn, nbytes, flops, kind, units=0.0):
        self.name, self.fn, self.bytes, self.flops, self.kind, self.units = name, fn, float(nbytes), float(flops), \
            kind, units


def _n_vis(q_pos, n_entries, m):
    return np.minimum(np.asarray(n_entries, np.int64), (np.asarray(q_pos, np.int64) + 1) // m)


# ---------------------------------------------------------------------------
# Workload set-ups: each returns (stages of one pass, units per pass, unit name)
# ---------------------------------------------------------------------------
class Ctx:
    def __init__(self, torch, L):
        self.torch, self.L = torch, L
        self.dev = torch.device("cuda:0")

    def up(self, a, dtype=None):
        t = self.torch.from_numpy(np.ascontiguousarray(a)).to(self.dev)
        return t if dtype is None else t.to(dtype)

    def packed(self, x_f32):
        flat = self.up(x_f32.reshape(-1, DIM))
        out = self.torch.empty(flat.shape[0], 256, dtype=self.torch.uint8, device=self.dev)
        self.L.kv_pack(flat, out)
        return out.view(*x_f32.shape[:-1], 256)

    def mx(self, x_f32):
        t = self.up(x_f32) if isinstance(x_f32, np.ndarray) else x_f32
        d = t.shape[-1]
        codes = self.torch.empty(*t.shape[:-1], d // 2, dtype=self.torch.uint8, device=self.dev)
        scales = self.torch.empty(*t.shape[:-1], d // 32, dtype=self.torch.uint8, device=self.dev)
        self.L.mxfp4_quantize(t.contiguous(), codes, scales)
        return codes, scales


def cfg1(c: Ctx):
    from long_context_compressed_compress_amd import workloads as WL
    L, torch = c.L, c.torch
    w = WL.csa_decode_tiny()
    p = w.params
    T, HI, DI, HQ, K, W = p["n_q"], p["h_idx"], p["d_idx"], p["n_heads"], p["topk"], p["window"]
    n = p["L"] // 4
    x, wg, pb, wi = c.up(w["x"]), c.up(w["w_gate"]), c.up(w["pos_bias"]), c.up(w["w_idx"])
    kv = torch.empty(1, n, DIM, dtype=torch.float32, device=c.dev)
    key = torch.empty(1, n, DI, dtype=torch.float32, device=c.dev)
    ne, qp = c.up(np.array([n], np.int32)), c.up(p["q_pos"])
    qi, wq, q = c.up(w["q_idx"]), c.up(w["w"]), c.up(w["q"])
    sc = torch.empty(1, T, n, dtype=torch.float32, device=c.dev)
    idx = torch.empty(1, T, K, dtype=torch.int32, device=c.dev)
    out = torch.empty(1, T, HQ, DIM, dtype=torch.float32, device=c.dev)
    nv = _n_vis(p["q_pos"][0], n, 4)
    stages = [
        Stage("csa_compress", lambda: L.csa_compress(x, 0, wg, pb, 0, n, kv, w_idx=wi, key_out=key),
              p["L"] * DIM * 4 + n * (DIM + DI) * 4, p["L"] * 2 * DIM * DIM + n * 2 * DIM * DI, "fp32"),
        Stage("indexer_score (fp32)", lambda: L.indexer_score(qi, wq, key, ne, qp, 4, sc),
              n * DI * 4 + T * HI * (DI + 1) * 4 + T * n * 4, nv.sum() * HI * DI * 2, "fp32"),
        Stage("topk_select", lambda: L.topk_select(sc, ne, qp, 4, K, idx), T * n * 4 + T * K * 4, 0, "hbm"),
        Stage("sparse_window_attn (fp32)",
              lambda: L.sparse_window_attn(q, kv, ne, 4, idx, x, 0, qp, W, SCALE, out),
              T * (K + W) * DIM * 4 + 2 * T * HQ * DIM * 4, T * HQ * (K + W) * DIM * 4, "fp32"),
    ]
    return stages, T, "query rows"


def cfg2(c: Ctx):
    from long_context_compressed_compress_amd import workloads as WL
    L, torch = c.L, c.torch
    w = WL.csa_prefill_chunk()
    p = w.params
    T, N, K, H, W, HI, DI = p["n_q"], p["n_entries"], p["topk"], p["n_heads"], p["window"], p["h_idx"], p["d_idx"]
    entm, winm = c.packed(w["entries"]), c.packed(w["window"])
    kc, ks = c.mx(w["k_idx"])
    qf, wq = c.up(w["q_idx"]), c.up(w["w"])
    qb = c.up(w["q"], torch.bfloat16)
    ne, qp = c.up(np.array([N], np.int32)), c.up(p["q_pos"])
    sc = torch.empty(1, T, N, dtype=torch.bfloat16, device=c.dev)
    idx = torch.empty(1, T, K, dtype=torch.int32, device=c.dev)
    out = torch.empty(1, T, H, DIM, dtype=torch.bfloat16, device=c.dev)
    nv = _n_vis(p["q_pos"][0], N, 4)
    n_win = w["window"].shape[1]
    stages = [
        Stage("indexer_score (MXFP4, float32 q)", lambda: L.indexer_score(qf, wq, kc, ne, qp, 4, sc, k_scales=ks),
              N * (DI // 2 + DI // 32) + T * HI * (DI + 1) * 4 + T * N * 2, nv.sum() * HI * DI * 2, "fp4"),
        Stage("topk_select", lambda: L.topk_select(sc, ne, qp, 4, K, idx), T * N * 2 + T * K * 4, 0, "hbm"),
        Stage("sparse_window_attn",
              lambda: L.sparse_window_attn(qb, entm, ne, 4, idx, winm, p["win_pos0"], qp, W, SCALE, out),
              (N + n_win) * 256 + 2 * T * H * DIM * 2, T * H * (K + W) * DIM * 4, "bf16"),
    ]
    return stages, T, "query rows"


def cfg3(c: Ctx):
    from long_context_compressed_compress_amd import workloads as WL
    L, torch = c.L, c.torch
    w = WL.csa_decode_1m()
    p = w.params
    B, N, K, H, W, HI, DI = p["batch"], p["n_entries"], p["topk"], p["n_heads"], p["window"], p["h_idx"], p["d_idx"]
    t = int(p["q_pos"][0, 0])
    entm = c.packed(w["entries"])
    kc, ks = c.mx(w["k_idx"])
    ring_f = np.empty_like(w["window"])
    ring_f[:, np.arange(t - W + 1, t + 1) % W] = w["window"]
    ringm = c.packed(ring_f)
    qf, wq = c.up(w["q_idx"]), c.up(w["w"])
    qb = c.up(w["q"], torch.bfloat16)
    ne, qp = c.up(np.full(B, N, np.int32)), c.up(p["q_pos"])
    sc = torch.empty(B, 1, N, dtype=torch.bfloat16, device=c.dev)
    idx = torch.empty(B, 1, K, dtype=torch.int32, device=c.dev)
    out = torch.empty(B, 1, H, DIM, dtype=torch.bfloat16, device=c.dev)
    ws = torch.zeros(max(L.topk_workspace_size(B, 1, N, K, L.CSA_BF16), 16), dtype=torch.uint8, device=c.dev)
    stages = [
        Stage("indexer_score (MXFP4, float32 q)", lambda: L.indexer_score(qf, wq, kc, ne, qp, 4, sc, k_scales=ks),
              B * (N * (DI // 2 + DI // 32) + HI * (DI + 1) * 4 + N * 2), B * N * HI * DI * 2, "hbm"),
        Stage("topk_select", lambda: L.topk_select(sc, ne, qp, 4, K, idx, workspace=ws), B * (N * 2 + K * 4), 0,
              "hbm"),
        Stage("sparse_window_attn", lambda: L.sparse_window_attn(qb, entm, ne, 4, idx, ringm, 0, qp, W, SCALE, out),
              B * ((K + W) * 256 + 2 * H * DIM * 2 + K * 4), B * H * (K + W) * DIM * 4, "hbm"),
    ]
    return stages, B, "tokens"


def cfg4(c: Ctx):
    from long_context_compressed_compress_amd import workloads as WL
    L, torch = c.L, c.torch
    w = WL.hca_decode_1m()
    p = w.params
    B, N, H, W = p["batch"], p["n_entries"], p["n_heads"], p["window"]
    t = int(p["q_pos"][0, 0])
    entm = c.packed(w["entries"])
    ring_f = np.empty_like(w["window"])
    ring_f[:, np.arange(t - W + 1, t + 1) % W] = w["window"]
    ringm = c.packed(ring_f)
    qb = c.up(w["q"], torch.bfloat16)
    ne, qp = c.up(np.full(B, N, np.int32)), c.up(p["q_pos"])
    out = torch.empty(B, 1, H, DIM, dtype=torch.bfloat16, device=c.dev)
    stages = [
        Stage("hca_dense_attn", lambda: L.hca_dense_attn(qb, entm, ne, 128, ringm, 0, qp, W, SCALE, out),
              B * ((N + W) * 256 + 2 * H * DIM * 2), B * H * (N + W) * DIM * 4, "hbm"),
    ]
    return stages, B, "tokens"


class Cfg5:
    """The long prefill, chunk by chunk: stages_for(c) after the previous chunks ran."""

    def __init__(self, c: Ctx):
        from long_context_compressed_compress_amd import workloads as WL
        self.c, self.WL = c, WL
        L, torch = c.L, c.torch
        w = self.w = WL.hybrid_prefill_weights()
        p = self.p = w.params
        self.Lt, self.C, self.K, self.H, self.W, self.HI, self.DI = p["L"], p["chunk"], p["topk"], p["n_heads"], \
            p["window"], p["h_idx"], p["d_idx"]
        n_csa, n_hca = self.Lt // 4, self.Lt // 128
        self.raw = torch.empty(1, self.Lt, DIM, dtype=torch.bfloat16, device=c.dev)
        L.kv_pack(c.up(w["x"][0]), self.raw[0])
        self.winm = c.packed(w["x"])
        self.kv = torch.empty(1, n_csa, 256, dtype=torch.uint8, device=c.dev)
        self.kc = torch.empty(1, n_csa, self.DI // 2, dtype=torch.uint8, device=c.dev)
        self.ks = torch.empty(1, n_csa, self.DI // 32, dtype=torch.uint8, device=c.dev)
        self.kvh = torch.empty(1, n_hca, 256, dtype=torch.uint8, device=c.dev)
        self.wts = [c.up(w[k]) for k in ("w_gate", "pos_bias", "w_gate_hca", "pos_bias_hca", "w_idx")]
        self.sc = torch.empty(1, self.C * n_csa, dtype=torch.bfloat16, device=c.dev)
        self.idx = torch.empty(1, self.C, self.K, dtype=torch.int32, device=c.dev)
        self.out = torch.empty(1, self.C, self.H, DIM, dtype=torch.bfloat16, device=c.dev)
        self.outh = torch.empty_like(self.out)

    def stages_for(self, ch: int):
        c, L, torch = self.c, self.c.L, self.c.torch
        C, K, H, W, HI, DI = self.C, self.K, self.H, self.W, self.HI, self.DI
        qd = self.WL.hybrid_prefill_chunk(self.w, ch)
        n, nh = (ch + 1) * C // 4, (ch + 1) * C // 128           # entries once this chunk is compressed
        q_pos = qd["q_pos"]
        qp = c.up(q_pos)
        qf, wq = c.up(qd["q_idx"]), c.up(qd["w"])
        qcb, qhb = c.up(qd["q_csa"], torch.bfloat16), c.up(qd["q_hca"], torch.bfloat16)
        ne, neh = c.up(np.array([n], np.int32)), c.up(np.array([nh], np.int32))
        sc = self.sc[:, : C * n].view(1, C, n)
        kv, kc, ks, kvh = self.kv[:, :n], self.kc[:, :n], self.ks[:, :n], self.kvh[:, :nh]
        wg, pb, wgh, pbh, wi = self.wts
        nv = _n_vis(q_pos[0], n, 4)
        nvh = _n_vis(q_pos[0], nh, 128)
        n_win = np.minimum(q_pos[0] + 1, W)
        return [
            Stage("csa_compress", lambda: L.csa_compress(self.raw, 0, wg, pb, ch * C // 4, C // 4, self.kv, w_idx=wi,
                                                          key_out=self.kc, key_scales=self.ks),
                  (C + 4) * DIM * 2 + C // 4 * (256 + DI // 2 + DI // 32), C * 2 * DIM * DIM + C // 4 * 2 * DIM * DI,
                  "fp32"),
            Stage("hca_compress", lambda: L.hca_compress(self.raw, 0, wgh, pbh, ch * C // 128, C // 128, self.kvh),
                  C * DIM * 2 + C // 128 * 256, C * 2 * DIM * DIM, "fp32"),
            Stage("indexer_score (MXFP4, float32 q)", lambda: L.indexer_score(qf, wq, kc, ne, qp, 4, sc, k_scales=ks),
                  n * (DI // 2 + DI // 32) + C * HI * (DI + 1) * 4 + C * n * 2, nv.sum() * HI * DI * 2, "fp4"),
            Stage("topk_select", lambda: L.topk_select(sc, ne, qp, 4, K, self.idx), C * n * 2 + C * K * 4, 0, "hbm"),
            Stage("sparse_window_attn",
                  lambda: L.sparse_window_attn(qcb, kv, ne, 4, self.idx, self.winm, 0, qp, W, SCALE, self.out),
                  n * 256 + (C + W) * 256 + 2 * C * H * DIM * 2,
                  (np.minimum(nv, K) + n_win).sum() * H * DIM * 4, "bf16"),
            Stage("hca_dense_attn", lambda: L.hca_dense_attn(qhb, kvh, neh, 128, self.winm, 0, qp, W, SCALE, self.outh),
                  nh * 256 + (C + W) * 256 + 2 * C * H * DIM * 2, (nvh + n_win).sum() * H * DIM * 4, "bf16"),
        ]


# ---------------------------------------------------------------------------
# Timing
# ---------------------------------------------------------------------------
def _marker(torch, dev, i):
    if not hasattr(_marker, "t"):
        _marker.t = torch.empty(1, dtype=torch.float64, device=dev)  # created without a fill kernel
    _marker.t.fill_(float(i))


def _time(torch, stages, reps, warmup, markers, acc, dev):
    """Time each stage: `warmup` untimed calls, then `reps` calls between HIP
    events on the current stream; adds to acc[name] = [calls, ms, bytes, flops, kind]."""
    for st in stages:
        for _ in range(warmup):
            st.fn()
        evs = []
        for r in range(reps):
            if markers:
                _marker(torch, dev, r)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            st.fn()
            b.record()
            evs.append((a, b))
        torch.cuda.synchronize()
        ms = sum(a.elapsed_time(b) for a, b in evs)
        e = acc.setdefault(st.name, [0, 0.0, 0.0, 0.0, st.kind])
        e[0] += reps
        e[1] += ms
        e[2] += st.bytes * reps
        e[3] += st.flops * reps


def run(configs, reps, warmup, markers):
    import torch
    from long_context_compressed_compress_amd import libcsa as L
    c = Ctx(torch, L)
    results = {}
    for n in configs:
        print(f"[report] workload {n}: {CONFIG_NAMES[n]}", flush=True)
        acc = collections.OrderedDict()
        if n == 5:
            cf = Cfg5(c)
            torch.cuda.synchronize()
            units = 0
            for ch in range(cf.p["n_chunks"]):
                _time(torch, cf.stages_for(ch), reps, warmup if ch == 0 else 0, markers, acc, c.dev)
                units += cf.C
                if ch % 8 == 7:
                    print(f"[report]   chunk {ch} done", flush=True)
            per_pass, unit = cf.Lt, "tokens"
            passes = reps  # every chunk's stages ran reps times
        else:
            stages, per_pass, unit = {1: cfg1, 2: cfg2, 3: cfg3, 4: cfg4}[n](c)
            torch.cuda.synchronize()
            _time(torch, stages, reps, warmup, markers, acc, c.dev)
            passes = reps
        if markers:
            _marker(torch, c.dev, -1)
        torch.cuda.synchronize()
        total_ms = sum(v[1] for v in acc.values()) / passes
        results[n] = {"name": CONFIG_NAMES[n], "units_per_pass": per_pass, "unit": unit, "pass_ms": total_ms,
                      "stages": [{"stage": k, "calls": v[0], "ms_per_call": v[1] / v[0], "bytes_per_call": v[2] / v[0],
                                  "flops_per_call": v[3] / v[0], "kind": v[4]} for k, v in acc.items()]}
        print(f"[report]   {total_ms:.3f} ms per pass", flush=True)
        torch.cuda.empty_cache()
    return results


# ---------------------------------------------------------------------------
# Counters and summary
# ---------------------------------------------------------------------------
def _dispatches(path, counter):
    rows = collections.OrderedDict()
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            d = int(r["Dispatch_Id"])
            name, val = rows.get(d, (r["Kernel_Name"], 0.0))
            rows[d] = (name, val + float(r["Counter_Value"]))
    return [rows[d] for d in sorted(rows)]


def counter_bytes(fetch_csv, write_csv):
    """Per stage call (segments between marker fills): bytes moved by the
    library's kernels, each counter scaled by its reading of the 1 GiB copy."""
    out = []
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        ds = _dispatches(path, counter)
        copy = [v for n, v in ds if "csa::" not in n and v * 1024 > (1 << 29)]
        if not copy:
            raise SystemExit(f"{path}: no 1 GiB calibration copy found")
        factor = (1 << 30) / (sorted(copy)[len(copy) // 2] * 1024)
        segs, cur, seen = [], None, 0
        for name, v in ds:
            if MARKER in name:
                if cur is not None and seen:  # a segment without a library kernel is no stage call
                    segs.append(cur)
                cur, seen = 0.0, 0
            elif cur is not None and "csa::" in name:
                cur += v * 1024 * factor
                seen += 1
        out.append(segs)
    if len(out[0]) != len(out[1]):
        raise SystemExit("fetch and write runs saw different numbers of stage calls")
    return [f + w for f, w in zip(*out)]


def device_rates(reps=20):
    """Achievable HBM rates on this device, for scale: a streaming read of
    1 GiB and of 75 MB (the decode indexer's footprint) by the probe kernel
    (probe/read_rate.hip), and a 1 GiB device copy (read + write, torch's
    kernel), each timed back to back with events."""
    import ctypes

    import torch
    from . import build as B
    lib = ctypes.CDLL(B.PROBE_OUT)
    lib.read_rate_probe.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                    ctypes.POINTER(ctypes.c_float), ctypes.c_void_p]
    n = 1 << 30
    x = torch.zeros(n, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    grid = 2048
    sink = torch.empty(grid * 256, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    out = {}
    for key, nbytes in (("read_gbs", n), ("read_75mb_gbs", 75 << 20)):
        us = ctypes.c_float()
        rc = lib.read_rate_probe(ctypes.c_void_p(x.data_ptr()), nbytes, ctypes.c_void_p(sink.data_ptr()), grid, reps,
                                 ctypes.byref(us), ctypes.c_void_p(stream))
        if rc != 0:
            raise RuntimeError(f"read_rate_probe returned {rc}")
        out[key] = nbytes / (us.value * 1e-6) / 1e9
    for _ in range(3):
        y.copy_(x)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        y.copy_(x)
    b.record()
    torch.cuda.synchronize()
    out["copy_gbs"] = 2 * n / (a.elapsed_time(b) / reps / 1e3) / 1e9
    return out


def summarize(time_json, counters_dir, out_md, command):
    res = json.load(open(time_json))
    rates = res.pop("rates", None)
    lines = ["# Per-workload report: every stage on MI355X against the chip's peaks", "",
             "Commands (run from the repository root; counter passes per workload N = 1..5):", "", "```", command, "```",
             "", "Algorithmic bytes count each tensor a stage must touch once; flops count 2 per multiply-add.",
             "Peaks: HBM 8000 GB/s; dense MFMA FP4 10.1 PFLOP/s, BF16 2.5 PFLOP/s; FP32 vector 157.3 TFLOP/s.",
             "`counter GB/s` = (FETCH_SIZE + WRITE_SIZE bytes of the stage's kernels, each scaled by its reading of a",
             "1 GiB copy) / the stage's time.", ""]
    if rates:
        lines += [f"Achievable rates measured in the same run: a streaming read reaches {rates['read_gbs']:,.0f} GB/s "
                  f"over 1 GiB ({100 * rates['read_gbs'] / HBM_PEAK_GBS:.0f} % of the peak) and "
                  f"{rates['read_75mb_gbs']:,.0f} GB/s over 75 MB (probe/read_rate.hip); a 1 GiB device copy moves "
                  f"{rates['copy_gbs']:,.0f} GB/s (read + write, torch's kernel).", ""]
    for n in sorted(res, key=int):
        r = res[n]
        ctr = None
        f = os.path.join(counters_dir, f"fetch_{n}.csv") if counters_dir else None
        if f and os.path.exists(f):
            # counter runs call every stage once (workload 5: once per chunk, the
            # stages in order within each chunk), so segment k is stage k mod n
            segs = counter_bytes(f, os.path.join(counters_dir, f"write_{n}.csv"))
            n_st = len(r["stages"])
            if len(segs) % n_st:
                raise SystemExit(f"workload {n}: {len(segs)} stage calls for {n_st} stages")
            ctr = {st["stage"]: float(np.mean(segs[j::n_st])) for j, st in enumerate(r["stages"])}
        rate = r["units_per_pass"] / (r["pass_ms"] / 1e3)
        lines += [f"## {n}. {r['name']}", "",
                  f"One pass: {r['pass_ms']:.3f} ms, {rate:,.0f} {r['unit']}/s.", "",
                  "| stage | us per call | alg. GB/s | % HBM | counter GB/s | TFLOP/s | % of peak (type) |",
                  "|---|---:|---:|---:|---:|---:|---:|"]
        for st in r["stages"]:
            s = st["ms_per_call"] / 1e3
            gbs = st["bytes_per_call"] / s / 1e9
            tf = st["flops_per_call"] / s / 1e12
            kind = st["kind"]
            if kind == "hbm":
                peak_col = f"{100 * gbs / HBM_PEAK_GBS:.1f} (HBM)"
            else:
                peak_col = f"{100 * tf / PEAK_TFLOPS[kind]:.1f} ({kind})"
            cg = "" if ctr is None else f"{ctr[st['stage']] / s / 1e9:,.0f}"
            lines.append(f"| {st['stage']} | {st['ms_per_call'] * 1e3:,.1f} | {gbs:,.0f} | "
                         f"{100 * gbs / HBM_PEAK_GBS:.1f} | {cg} | {tf:,.2f} | {peak_col} |")
        if int(n) == 3:
            ix = [st for st in r["stages"] if st["stage"].startswith(("indexer", "sparse"))]
            b = sum(st["bytes_per_call"] for st in ix)
            t = sum(st["ms_per_call"] for st in ix) / 1e3
            lines += ["", f"Indexer + attention: {b / t / 1e9:,.0f} GB/s algorithmic, "
                          f"{100 * b / t / 1e9 / HBM_PEAK_GBS:.1f} % of HBM peak"
                          + (f", {100 * b / t / 1e9 / rates['read_gbs']:.1f} % of the measured read rate." if rates
                             else ".")]
        lines.append("")
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines))
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--config", type=int, action="append", help="workload number (repeatable; default all)")
    ap.add_argument("--reps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--markers", action="store_true", help="marker fill before every stage call (counter runs)")
    ap.add_argument("--calibrate-copy", action="store_true", help="end with a plain 1 GiB device copy")
    ap.add_argument("--json", help="write the timings here")
    ap.add_argument("--summarize", metavar="TIME_JSON")
    ap.add_argument("--counters", help="folder with fetch_N.csv / write_N.csv")
    ap.add_argument("--out", help="markdown summary path")
    ap.add_argument("--command", default="", help="command text recorded in the summary")
    a = ap.parse_args()
    if a.summarize:
        summarize(a.summarize, a.counters, a.out, a.command)
        return
    res = run(a.config or [1, 2, 3, 4, 5], a.reps, a.warmup, a.markers)
    if not a.markers:
        res["rates"] = device_rates()
        print(json.dumps(res["rates"]))
    if a.calibrate_copy:
        import torch
        x = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        y = torch.empty_like(x)
        y.copy_(x)
        torch.cuda.synchronize()
    if a.json:
        with open(a.json, "w") as fh:
            json.dump(res, fh, indent=1)
    for n, r in res.items():
        if n == "rates":
            continue
        print(json.dumps({"workload": n, "pass_ms": round(r["pass_ms"], 4),
                          "stages": {s["stage"]: round(s["ms_per_call"] * 1e3, 2) for s in r["stages"]}}))


if __name__ == "__main__":
    sys.exit(main())
