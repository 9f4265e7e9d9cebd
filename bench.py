"""Benchmark: CSA + HCA decode at 1M-token context on one MI355X.

One step = one decode token for every sequence of the batch through a CSA
layer and an HCA layer, every step of the path on the GPU:
  append the new token's raw KV (BF16 raw ring, with its gate logits) and
  stored row (FP8/BF16 window ring) for each layer; compress a CSA entry (with
  its MXFP4 indexer key) every 4 steps and an HCA entry every 128 steps;
  Lightning Indexer over all ~262144 CSA entries (the float32 query is
  quantised to MXFP4 inside the scoring kernel); top-1024; sparse + window
  attention (128 query heads); HCA dense + window attention over ~8192 entries.
By default the step is the layers in a model's order over the device-resident
cache: decode_csa_layer, then decode_hca_layer (--order paired: one
decode_step call, both layers' attention in one launch; --path calls: the same
step as the individual calls).
Inputs are synthetic and seeded (long_context_compressed_compress_amd.workloads),
resident in HBM before timing starts.

Prints one JSON line (rank 0).  --gpus above 1 is refused: the benchmark measures
one GPU.  --oracle-report OUT instead times the fp64 oracle on the five
workloads on the host cores (no GPU use) and writes a markdown summary.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "CSA+HCA decode tokens/sec at 1M ctx; indexer+attn HBM GB/s vs peak"
# rocprofv3 byte-counter summary of the dominant kernel on this workload
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "indexer_mxfp4_decode_pair_1m_b8_traffic.md")
# the same counters summed over every kernel of a decode step
STEP_TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "decode_step_1m_b8_traffic.md")
HBM_PEAK_GBS = 8000.0
CTX = 1 << 20
W = 128
D = 192


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--batch", type=int, default=8)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--path", choices=("fused", "calls"), default="fused",
                    help="fused: the decode calls over the device-resident cache; calls: the individual calls")
    ap.add_argument("--order", choices=("sequential", "paired"), default="sequential",
                    help="sequential: the CSA layer's calls, then the HCA layer's (a model's layer order: the HCA "
                         "layer's input is the CSA layer's output); paired: one decode_step call running both "
                         "layers' attention in one launch (two layers whose inputs are ready together)")
    ap.add_argument("--variant", choices=("pro", "flash"), default="pro",
                    help="pro: top-1024; flash: top-512 and a sliding-window-only layer in each step")
    ap.add_argument("--paged", type=int, default=0, metavar="P",
                    help="entries of both layers in pages of P entries behind page tables (a seeded scattered "
                         "assignment); 0 = contiguous per sequence.  Fused path only")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (reference for HBM byte counters)")
    ap.add_argument("--oracle-report", metavar="OUT",
                    help="time the fp64 oracle on the five workloads on the host cores, write a markdown summary "
                         "to OUT and exit (no GPU use)")
    return ap.parse_args()


class DecodePair:
    """A CSA + HCA layer pair's decode cache (entries, keys, rings, positions),
    weights and pre-drawn per-step inputs.  path "fused": the decode calls
    (append, compress-on-boundary, index, select, attend; positions and counts
    on the device), per layer in order ("sequential") or one decode_step for
    both ("paired").  path "calls": the same step as the individual calls, with
    positions and counts computed on the host."""

    def __init__(self, L, torch, batch: int, total_steps: int, pool: int = 32, path: str = "fused",
                 variant: str = "pro", order: str = "sequential", paged: int = 0):
        from long_context_compressed_compress_amd import workloads as WL
        self.L, self.torch, self.path, self.order = L, torch, path, order
        dev = torch.device("cuda:0")
        self.dev = dev
        B = self.B = batch
        self.n0 = CTX // 4
        self.n0h = CTX // 128
        # cache capacity: the context's entries plus those the run appends, in whole 64-entry groups
        self.n_cap = (self.n0 + total_steps // 4 + 2 + 63) // 64 * 64
        self.n_cap_h = (self.n0h + total_steps // 128 + 2 + 63) // 64 * 64
        if paged:   # paged entries: capacities in whole pages
            self.n_cap = (self.n_cap + paged - 1) // paged * paged
            self.n_cap_h = (self.n_cap_h + paged - 1) // paged * paged

        csa = WL.csa_decode_1m(batch_rows=range(B))
        hca = WL.hca_decode_1m(batch_rows=range(B))
        wts = WL.hybrid_prefill_weights()
        self.HI, self.DI, self.HQ, self.K = 64, 64, 128, csa.params["topk"]
        self.variant = variant
        if variant == "flash":  # V4-Flash: top-512, and a pure sliding-window layer in each step
            self.K = 512
        self.scale = 1.0 / math.sqrt(D)

        def up(a):
            return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

        weights = {"csa_w_gate": up(wts["w_gate"]), "csa_pos_bias": up(wts["pos_bias"]),
                   "csa_w_idx": up(wts["w_idx"]), "hca_w_gate": up(wts["w_gate_hca"]),
                   "hca_pos_bias": up(wts["pos_bias_hca"])}
        tables = {}
        if paged:   # a seeded scattered assignment of every sequence's pages
            prng = np.random.default_rng(11)
            for name, cap in (("csa_pages", self.n_cap), ("hca_pages", self.n_cap_h)):
                n = cap // paged
                tables[name] = torch.from_numpy(prng.permutation(B * n).astype(np.int32).reshape(B, n))
        c = self.cache = L.DecodeCache(B, self.HQ, self.HI, self.DI, self.K, W, self.n_cap, self.n_cap_h, self.scale,
                                       weights, win_rows=W, device=dev, page_entries=paged, **tables)

        def seq_rows(name, b):
            """Sequence b's rows of an entry array in logical order (a staging copy when paged)."""
            t = getattr(c, name)
            if not paged:
                return t[b]
            cap = self.n_cap_h if name == "hca_kv" else self.n_cap
            return torch.zeros(cap, t.shape[2], dtype=t.dtype, device=dev)

        def seq_store(name, b, rows):
            if paged:
                tab = (c.hca_pages if name == "hca_kv" else c.csa_pages)[b].long()
                getattr(c, name)[tab] = rows.view(tab.shape[0], paged, -1)
        # the context: CSA entries + MXFP4 indexer keys, HCA entries (stored rows)
        for src_f32, name in ((csa["entries"], "csa_kv"), (hca["entries"], "hca_kv")):
            src = up(src_f32)
            for b in range(B):
                rows = seq_rows(name, b)
                L.kv_pack(src[b], rows[: src_f32.shape[1]])
                seq_store(name, b, rows)
            del src
        kf = up(csa["k_idx"])
        for b in range(B):
            kc, ks = seq_rows("csa_keys", b), seq_rows("csa_key_scales", b)
            L.mxfp4_quantize(kf[b], kc[: self.n0], ks[: self.n0])
            seq_store("csa_keys", b, kc)
            seq_store("csa_key_scales", b, ks)
        del kf
        c.pos.fill_(CTX)
        c.csa_entries.fill_(self.n0)
        c.hca_entries.fill_(self.n0h)

        # per-step inputs: a pool of drawn steps, cycled
        st = WL.decode_stream(pool, B, self.HI, self.DI, self.HQ)
        self.pool = pool
        self.x_csa, self.x_hca = up(st["x_csa"]), up(st["x_hca"])
        self.q_idx, self.w = up(st["q_idx"]), up(st["w"])
        self.q_csa = up(st["q_csa"]).to(torch.bfloat16)
        self.q_hca = up(st["q_hca"]).to(torch.bfloat16)
        self.out = torch.empty(B, self.HQ, D, dtype=torch.bfloat16, device=dev)
        self.out_h = torch.empty(B, self.HQ, D, dtype=torch.bfloat16, device=dev)

        if variant == "flash":
            sw = WL.swa_layer_stream(pool, B, self.HQ, W)
            self.swa_win = torch.empty(B, W, 256, dtype=torch.uint8, device=dev)   # ring: position p in row p mod W
            pos = np.arange(CTX - W, CTX)
            ring_f = np.empty_like(sw["window"])
            ring_f[:, pos % W] = sw["window"]
            src = up(ring_f)
            for b in range(B):
                L.kv_pack(src[b], self.swa_win[b])
            self.x_swa = up(sw["x"])
            self.q_swa = up(sw["q"]).to(torch.bfloat16)
            self.out_swa = torch.empty(B, 1, self.HQ, D, dtype=torch.bfloat16, device=dev)
            self.ws_swa = self._ws(L.attn_workspace_size(B, 1, self.HQ, W, L.CSA_BF16, L.CSA_KV_MIXED))
        if path == "fused":
            # rings: the last 128 context tokens (positions CTX-128 .. CTX-1) of each layer
            L.decode_prime(c, up(csa["window"]), up(hca["window"]))
            self.ws = c.workspace(torch.bfloat16)
        else:
            self.kv, self.kc, self.ks, self.kv_h = c.csa_kv, c.csa_keys, c.csa_key_scales, c.hca_kv
            self.win, self.raw = self._rings(up, csa["window"])
            self.win_h, self.raw_h = self._rings(up, hca["window"])
            self.w_gate, self.pos_bias, self.w_idx = (weights[k] for k in ("csa_w_gate", "csa_pos_bias",
                                                                            "csa_w_idx"))
            self.w_gate_h, self.pos_bias_h = weights["hca_w_gate"], weights["hca_pos_bias"]
            # positions and entry counts of every step (step s decodes position CTX + s)
            t = CTX + np.arange(total_steps, dtype=np.int64)
            self.q_pos = up(np.repeat(t[:, None], B, axis=1)).view(total_steps, B, 1)
            self.n_ent = up(np.repeat(((t + 1) // 4).astype(np.int32)[:, None], B, axis=1))
            self.n_ent_h = up(np.repeat(((t + 1) // 128).astype(np.int32)[:, None], B, axis=1))
            self.scores = torch.empty(B, 1, self.n_cap, dtype=torch.bfloat16, device=dev)
            self.idx = torch.empty(B, 1, self.K, dtype=torch.int32, device=dev)
            self.topk_ws = self._ws(L.topk_workspace_size(B, 1, self.n_cap, self.K, L.CSA_BF16))
            self.attn_ws = self._ws(L.attn_workspace_size(B, 1, self.HQ, self.K + W, L.CSA_BF16, L.CSA_KV_MIXED))
            self.attn_ws_h = self._ws(L.attn_workspace_size(B, 1, self.HQ, self.n_cap_h + W, L.CSA_BF16,
                                                            L.CSA_KV_MIXED))
        torch.cuda.synchronize()

    def _ws(self, n):
        return self.torch.zeros(max(int(n), 16), dtype=self.torch.uint8, device=self.dev)

    def _rings(self, up, window_f32):
        """Window ring (stored rows) and raw ring (BF16) holding positions CTX-128 .. CTX-1."""
        torch, L, B = self.torch, self.L, self.B
        pos = np.arange(CTX - W, CTX)
        ring_f = np.empty_like(window_f32)
        ring_f[:, pos % W] = window_f32
        src = up(ring_f)
        win = torch.empty(B, W, 256, dtype=torch.uint8, device=self.dev)
        raw = torch.empty(B, W, D, dtype=torch.bfloat16, device=self.dev)
        for b in range(B):
            L.kv_pack(src[b], win[b])
            L.kv_pack(src[b], raw[b])
        return win, raw

    def step(self, s: int, ev=None):
        """Decode position CTX + s for every sequence.  `ev` (optional) = pair of
        events recorded around the indexer's scoring kernel."""
        p = s % self.pool
        if self.variant == "flash":
            # the sliding-window layer at the position the step decodes (before decode_step advances it)
            pos = self.cache.pos if self.path == "fused" else self.q_pos[s].view(self.B)
            self.L.kv_append(self.x_swa[p], pos, win_ring=self.swa_win)
            self.L.swa_attn(self.q_swa[p].view(self.B, 1, self.HQ, D), self.swa_win, 0, pos.view(self.B, 1), W,
                            self.scale, self.out_swa, workspace=self.ws_swa)
        if self.path == "fused":
            if self.order == "paired":
                self.L.decode_step(self.cache, self.x_csa[p], self.x_hca[p], self.q_idx[p], self.w[p], self.q_csa[p],
                                   self.q_hca[p], self.out, self.out_h, self.ws, stage_events=ev)
            else:   # the CSA layer of the token, then its HCA layer
                self.L.decode_csa_layer(self.cache, self.x_csa[p], self.q_idx[p], self.w[p], self.q_csa[p], self.out,
                                        self.ws, stage_events=ev)
                self.L.decode_hca_layer(self.cache, self.x_hca[p], self.q_hca[p], self.out_h, self.ws)
            return
        L, B = self.L, self.B
        t = CTX + s
        # append the new token of each layer: raw BF16 ring + stored window ring (one launch per layer)
        pos = self.q_pos[s].view(B)
        L.kv_append(self.x_csa[p], pos, raw_ring=self.raw, win_ring=self.win)
        L.kv_append(self.x_hca[p], pos, raw_ring=self.raw_h, win_ring=self.win_h)
        if (t + 1) % 4 == 0:    # a CSA entry completes: pool tokens t-7 .. t, emit its MXFP4 key
            L.csa_compress(self.raw, 0, self.w_gate, self.pos_bias, (t - 3) // 4, 1, self.kv, w_idx=self.w_idx,
                           key_out=self.kc, key_scales=self.ks)
        if (t + 1) % 128 == 0:  # an HCA entry completes
            L.hca_compress(self.raw_h, 0, self.w_gate_h, self.pos_bias_h, (t - 127) // 128, 1, self.kv_h)
        q_pos, ne, ne_h = self.q_pos[s], self.n_ent[s], self.n_ent_h[s]
        # float32 query, quantized to MXFP4 inside the indexer kernel, which also
        # builds top-k's first histogram; the events bracket that kernel alone
        L.indexer_topk(self.q_idx[p].view(B, 1, self.HI, self.DI), self.w[p].view(B, 1, self.HI), self.kc,
                       ne, q_pos, 4, self.scores, self.K, self.idx, k_scales=self.ks, workspace=self.topk_ws,
                       stage_events=ev)
        L.sparse_window_attn(self.q_csa[p].view(B, 1, self.HQ, D), self.kv, ne, 4, self.idx, self.win, 0, q_pos, W,
                             self.scale, self.out.view(B, 1, self.HQ, D), workspace=self.attn_ws)
        L.hca_dense_attn(self.q_hca[p].view(B, 1, self.HQ, D), self.kv_h, ne_h, 128, self.win_h, 0, q_pos, W,
                         self.scale, self.out_h.view(B, 1, self.HQ, D), workspace=self.attn_ws_h)

    def step_bytes(self, s: int) -> dict:
        """Algorithmic bytes of one step's indexer and attention, every operand
        counted once: per sequence, the CSA layer reads the MXFP4 keys of the
        visible entries (32 B codes + 2 B scales), the float32 indexer query and
        head weights, the selected entry rows and the window rows (256 B each),
        its query and writes its output (BF16, 128 heads x 192); the HCA layer
        reads every visible entry row and the window rows, its query and writes
        its output.  Scores passed from the indexer to top-k are not counted (an
        implementation choice, not an operand of the method)."""
        t = CTX + s
        n_vis, n_vis_h = (t + 1) // 4, (t + 1) // 128
        q_out = 2 * self.HQ * D * 2
        csa = n_vis * 34 + self.HI * self.DI * 4 + self.HI * 4 + (self.K + W) * 256 + q_out
        hca = (n_vis_h + W) * 256 + q_out
        return {"csa": self.B * csa, "hca": self.B * hca}

    def indexer_bytes(self, s: int) -> int:
        """Algorithmic bytes of one indexer launch: MXFP4 keys of the visible
        entries (32 B codes + 2 B scales), the float32 query (quantized in the
        call) and head weights, and the BF16 score row written for every cached
        entry."""
        n_vis = (CTX + s + 1) // 4
        per_seq = n_vis * 34 + self.HI * self.DI * 4 + self.HI * 4 + self.n_cap * 2
        return self.B * per_seq


def cpu_baseline(seconds_target=12.0, variant="pro"):
    """The fp64 oracle on a bounded sample of the same workload: full decode
    steps (CSA indexer over 262144 entries, top-1024 (flash: top-512 and a
    sliding-window-only layer), sparse+window attention, HCA dense+window
    attention over 8192 entries) of single sequences."""
    from long_context_compressed_compress_amd import workloads as WL
    from oracle import csa_oracle as O
    csa = WL.csa_decode_1m(batch_rows=[0])
    hca = WL.hca_decode_1m(batch_rows=[0])
    kc, ks = O.mxfp4_quantize(csa["k_idx"][0])          # stored keys
    rows = O.kv_pack(csa["entries"][0])                 # stored CSA entries
    rows_h = O.kv_pack(hca["entries"][0])
    win = O.kv_pack(csa["window"][0])
    win_h = O.kv_pack(hca["window"][0])
    k = csa.params["topk"] if variant == "pro" else 512
    if variant == "flash":
        sw = WL.swa_layer_stream(1, 1)
        win_s = O.kv_unpack(O.kv_pack(sw["window"][0]))
    t = CTX - 1
    scale = 1.0 / math.sqrt(D)
    n_steps, t0 = 0, time.perf_counter()
    while True:
        qc, qs = O.mxfp4_quantize(csa["q_idx"][0, 0])
        sc = O.indexer_scores(O.mxfp4_dequantize(qc, qs)[None], csa["w"][0], O.mxfp4_dequantize(kc, ks),
                              [rows.shape[0]], True)[0]
        sel = O.topk_select(sc, k)
        ent = np.zeros((rows.shape[0], D))
        ent[sel] = O.kv_unpack(rows[sel])
        q = O.bf16_round(csa["q"][0, 0])
        O.sparse_window_attn(q, ent, sel, rows.shape[0], O.kv_unpack(win), t - W + 1, t, W, scale)
        qh = O.bf16_round(hca["q"][0, 0])
        O.hca_dense_attn(qh, O.kv_unpack(rows_h), rows_h.shape[0], O.kv_unpack(win_h), t - W + 1, t, W, scale)
        if variant == "flash":   # window-only attention: no compressed entries
            O.hca_dense_attn(O.bf16_round(sw["q"][0, 0]), np.zeros((1, D)), 0, win_s, t - W + 1, t, W, scale)
        n_steps += 1
        if time.perf_counter() - t0 >= seconds_target:
            break
    el = time.perf_counter() - t0
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return {"value": n_steps / el, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{n_steps} single-sequence decode steps of the same {variant} CSA+HCA layer step at 1M context "
                      f"(numpy fp64, {el:.1f} s; storage encoding of the caches done once beforehand)"}


def _host():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    try:
        from threadpoolctl import threadpool_info
        blas = max((p.get("num_threads", 0) for p in threadpool_info() if p.get("user_api") == "blas"), default=0)
    except Exception:
        blas = 0
    return model, cores, blas


def oracle_workload_times(log=print):
    """The fp64 oracle on each of the five workloads, on the host cores (the
    CPU-baseline leg, nothing on the GPU).  Every timed region covers the same
    stages as the GPU pass of that workload; the stored form of the inputs
    (mixed rows, MXFP4 keys) is encoded and decoded once beforehand, as the GPU
    receives them stored.  Workloads 1 to 4 run whole; the long prefill runs its
    compressors whole and its per-query stages on 256 rows (8 from each chunk),
    then a least-squares line in the visible-entry count, summed over all
    131072 rows, stands in for the rest (labelled as extrapolated)."""
    from long_context_compressed_compress_amd import workloads as WL
    from oracle import csa_oracle as O
    scale = 1.0 / math.sqrt(D)
    clock = time.perf_counter
    res = []

    def mx(x):
        return O.mxfp4_dequantize(*O.mxfp4_quantize(x))

    # 1. CSA decode tiny: compressor (entries + keys), indexer, top-k, attention, all fp32 data
    w = WL.csa_decode_tiny()
    p = w.params
    n_cap, q_pos = p["L"] // 4, p["q_pos"][0]
    t0 = clock()
    ent = O.csa_compress(w["x"][0], w["w_gate"], w["pos_bias"], 0, n_cap)
    keys = O.csa_compress_key(ent, w["w_idx"])
    nv = O.n_visible(q_pos, n_cap, 4)
    sc = O.indexer_scores(w["q_idx"][0], w["w"][0], keys, nv, False)
    for t in range(p["n_q"]):
        sel = O.topk_select(sc[t], p["topk"])
        O.sparse_window_attn(w["q"][0, t], ent, sel, int(nv[t]), w["x"][0], 0, int(q_pos[t]), p["window"], scale)
    el = clock() - t0
    res.append(("1. CSA decode tiny (16 queries, 1024 entries)", el, p["n_q"] / el, "query rows/s", "whole"))
    log(f"oracle workload 1: {el:.2f} s", flush=True)

    # 2. CSA chunked prefill: 4096 rows over 16384 entries, k = 512
    w = WL.csa_prefill_chunk()
    p = w.params
    kdec = mx(w["k_idx"][0])
    entv = O.kv_round(w["entries"][0])
    winv = O.kv_round(w["window"][0])
    qv = O.bf16_round(w["q"][0])
    q_pos = p["q_pos"][0]
    nv = O.n_visible(q_pos, p["n_entries"], 4)
    t0 = clock()
    for t in range(p["n_q"]):
        s = O.indexer_scores(mx(w["q_idx"][0, t])[None], w["w"][0, t][None], kdec, [nv[t]], True)[0]
        sel = O.topk_select(s, p["topk"])
        O.sparse_window_attn(qv[t], entv, sel, int(nv[t]), winv, p["win_pos0"], int(q_pos[t]), p["window"], scale)
    el = clock() - t0
    res.append(("2. CSA chunked prefill (4096 rows x 16384 entries)", el, p["n_q"] / el, "query rows/s", "whole"))
    log(f"oracle workload 2: {el:.2f} s", flush=True)
    del w, kdec, entv, winv, qv

    # 3. CSA decode at 1M context, batch 8: one step, sequence by sequence
    el = 0.0
    for b in range(8):
        w = WL.csa_decode_1m(batch_rows=[b])
        p = w.params
        kdec = mx(w["k_idx"][0])
        rows = O.kv_pack(w["entries"][0])
        winv = O.kv_round(w["window"][0])
        n, t = p["n_entries"], int(p["q_pos"][0, 0])
        t0 = clock()
        s = O.indexer_scores(mx(w["q_idx"][0, 0])[None], w["w"][0], kdec, [n], True)[0]
        sel = O.topk_select(s, p["topk"])
        entv = np.zeros((n, D))
        entv[sel] = O.kv_unpack(rows[sel])
        O.sparse_window_attn(O.bf16_round(w["q"][0, 0]), entv, sel, n, winv, t - W + 1, t, W, scale)
        el += clock() - t0
        del w, kdec, rows, entv
    res.append(("3. CSA decode 1M, batch 8 (one step)", el, 8 / el, "tokens/s", "whole"))
    log(f"oracle workload 3: {el:.2f} s", flush=True)

    # 4. HCA decode at 1M context, batch 32: one step
    w = WL.hca_decode_1m()
    p = w.params
    n, t = p["n_entries"], int(p["q_pos"][0, 0])
    entv = [O.kv_round(w["entries"][b]) for b in range(32)]
    winv = [O.kv_round(w["window"][b]) for b in range(32)]
    qv = O.bf16_round(w["q"])
    t0 = clock()
    for b in range(32):
        O.hca_dense_attn(qv[b, 0], entv[b], n, winv[b], t - W + 1, t, W, scale)
    el = clock() - t0
    res.append(("4. HCA decode 1M, batch 32 (one step)", el, 32 / el, "tokens/s", "whole"))
    log(f"oracle workload 4: {el:.2f} s", flush=True)
    del w, entv, winv, qv

    # 5. long prefill of a CSA + HCA layer pair, 131072 tokens in 32 chunks
    w = WL.hybrid_prefill_weights()
    p = w.params
    Lt, C, K = p["L"], p["chunk"], p["topk"]
    n_csa, n_hca = Lt // 4, Lt // 128
    xr = O.bf16_round(w["x"][0])
    t0 = clock()
    ent = O.csa_compress(xr, w["w_gate"], w["pos_bias"], 0, n_csa)
    keys = O.csa_compress_key(ent, w["w_idx"])
    enth = O.hca_compress(xr, w["w_gate_hca"], w["pos_bias_hca"], 0, n_hca)
    kc, ks = O.mxfp4_quantize(keys)
    entv, enthv = O.kv_round(ent), O.kv_round(enth)
    el_comp = clock() - t0
    log(f"oracle workload 5 compressors: {el_comp:.2f} s", flush=True)
    kdec = O.mxfp4_dequantize(kc, ks)
    winv = O.kv_round(w["x"][0])
    rng = np.random.default_rng(5)
    nvs, secs = [], []
    for c in range(p["n_chunks"]):
        rows = np.sort(rng.choice(C, 8, replace=False))
        qd = WL.hybrid_prefill_chunk(w, c, q_rows=rows)
        qcv, qhv = O.bf16_round(qd["q_csa"][0]), O.bf16_round(qd["q_hca"][0])
        for i in range(len(rows)):
            tq = int(qd["q_pos"][0, i])
            nv = int(O.n_visible(tq, n_csa, 4))
            t0 = clock()
            s = O.indexer_scores(mx(qd["q_idx"][0, i])[None], qd["w"][0, i][None], kdec, [nv], True)[0]
            sel = O.topk_select(s, K)
            O.sparse_window_attn(qcv[i], entv, sel, nv, winv, 0, tq, W, scale)
            O.hca_dense_attn(qhv[i], enthv, int(O.n_visible(tq, n_hca, 128)), winv, 0, tq, W, scale)
            secs.append(clock() - t0)
            nvs.append(nv)
    a, b = np.polyfit(np.asarray(nvs, np.float64), np.asarray(secs), 1)
    all_nv = O.n_visible(np.arange(Lt), n_csa, 4).astype(np.float64)
    el_rows = float(np.sum(a * all_nv + b))
    el = el_comp + el_rows
    res.append(("5. hybrid pair prefill, 131072 tokens", el, Lt / el, "tokens/s",
                f"extrapolated: compressors timed whole ({el_comp:.1f} s); per-row stages timed on 256 rows "
                f"({sum(secs):.1f} s), fitted as {b * 1e3:.2f} ms + {a * 1e6:.3f} us per visible entry and summed "
                f"over all rows"))
    log(f"oracle workload 5: {el:.1f} s (extrapolated)", flush=True)
    return res


def write_oracle_report(res, out):
    model, cores, blas = _host()
    lines = ["# The fp64 oracle on the five workloads (host CPU)", "",
             "Command:", "", "```", "python bench.py --oracle-report " + os.path.relpath(out, ROOT), "```", "",
             f"Host: {model}; {cores} cores available to the process; BLAS threads {blas or 'unknown'}.",
             "Numpy float64, the oracle as the parity tests use it (not tuned). Each timed region covers the same",
             "stages as the GPU pass of the workload; the stored inputs are encoded and decoded once beforehand.", "",
             "| workload | oracle s | rate | unit | coverage |", "|---|---:|---:|---|---|"]
    for name, s, rate, unit, how in res:
        lines.append(f"| {name} | {s:.2f} | {rate:,.1f} | {unit} | {how} |")
    lines.append("")
    with open(out, "w") as f:
        f.write("\n".join(lines))


def main():
    args = parse()
    if args.oracle_report:
        write_oracle_report(oracle_workload_times(), args.oracle_report)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              f"(the decode path would shard by sequence, with no communication between GPUs)", file=sys.stderr)
        sys.exit(2)
    import torch
    from long_context_compressed_compress_amd import libcsa as L

    # warm-up, the timed steps, then as many steps again with timing events
    # around the indexer's scoring kernel (events in the stream serialise it, so
    # they stay out of the throughput measurement)
    total = args.warmup + 2 * args.steps
    if args.paged and args.path != "fused":
        print("bench.py: --paged applies to the fused path (the decode cache)", file=sys.stderr)
        sys.exit(2)
    pair = DecodePair(L, torch, args.batch, total, path=args.path, variant=args.variant, order=args.order,
                      paged=args.paged)
    for s in range(args.warmup):
        pair.step(s)
    torch.cuda.synchronize()

    t0 = time.perf_counter()
    for i in range(args.steps):
        pair.step(args.warmup + i)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0

    s_ev = args.warmup + args.steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        pair.step(s_ev + i, evs[i])
    torch.cuda.synchronize()
    idx_ms = [a.elapsed_time(b) for a, b in evs]
    idx_avg_s = float(np.mean(idx_ms)) / 1e3
    idx_bytes = float(np.mean([pair.indexer_bytes(s_ev + i) for i in range(args.steps)]))
    achieved = idx_bytes / idx_avg_s / 1e9

    if args.calibrate_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=pair.dev)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()

    from long_context_compressed_compress_amd import traffic as TR
    traffic = TR.load(TRAFFIC_SUMMARY, "indexer_mx_kernel")  # None when absent or the kernel changed since
    step_traffic = TR.load(STEP_TRAFFIC_SUMMARY, "decode_step")
    sb = [pair.step_bytes(args.warmup + i) for i in range(args.steps)]
    step_b = float(np.mean([d["csa"] + d["hca"] for d in sb]))
    step_s = el / args.steps
    step_gbs = step_b / step_s / 1e9
    res = {
        "metric": METRIC,
        "value": args.batch * args.steps / el,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": el / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4+bf16",
        "data": "synthetic",
        "config": {"workload": "csa_hca_pair_decode_1m" if args.variant == "pro" else
                   "csa_hca_swa_decode_1m_flash", "batch": args.batch, "context": CTX,
                   "csa_entries": CTX // 4, "hca_entries": CTX // 128, "topk": pair.K, "window": W,
                   "query_heads": pair.HQ, "indexer_heads": pair.HI, "indexer_dim": pair.DI,
                   "kv_storage": "fp8_e4m3(128)+bf16(64)", "parallelism": "single_gpu", "path": args.path,
                   "layer_order": args.order if args.path == "fused" else "sequential",
                   "entry_layout": f"paged_{args.paged}" if args.paged else "contiguous",
                   "swa_layers": 1 if args.variant == "flash" else 0},
        # the metric's own figure: indexer + attention of both layers over the whole step
        "roofline": {"scope": "decode step: indexer + top-k + attention of the CSA layer and attention of the HCA "
                              "layer (appends and compression included in the time)",
                     "bound": "hbm", "achieved": round(step_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(step_gbs / HBM_PEAK_GBS, 4),
                     "traffic": None if step_traffic is None else int(step_traffic),
                     "bytes_per_step": int(step_b), "us_per_step": round(step_s * 1e6, 2),
                     "timing": "algorithmic bytes of one step over the timed steps' wall time per step",
                     # the dominant kernel of the step
                     "dominant_kernel": {
                         "kernel": "indexer_mx_kernel (MXFP4 Lightning Indexer, the scoring stage of a decode step)",
                         "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBS, 4),
                         "traffic": None if traffic is None else int(traffic),
                         "avg_launch_us": round(idx_avg_s * 1e6, 2), "bytes_per_launch": int(idx_bytes),
                         "timing": f"HIP events around each of {args.steps} launches on the decode stream, in a "
                                   f"pass after the timed steps"}},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(variant=args.variant)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
