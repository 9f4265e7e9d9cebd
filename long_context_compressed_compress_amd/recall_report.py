"""Top-k recall of the MXFP4 Lightning Indexer against the float32 indexer.

The pages give the FP4 indexer's top-k recall on the trained model's data
(gitcode.csdn.net DeepSeek-V4 解读, 核心创新一 §1.4); on the seeded synthetic
workloads there is no printed value to match, so this is a reported figure.

For every query row of a workload, both selections are made on the GPU by the
library: the MXFP4 path (keys and queries quantized to MXFP4, BF16 scores,
indexer_topk) and the float32 path (the same unquantized keys and queries,
float32 scores, indexer_score + topk_select).  recall@k = |both| / k.  (That
the float32 path selects exactly the top-k of the exact scores is what the
GPU parity tests check against the oracle; this report does not use it.)

Usage (on a GPU machine):
  python -m long_context_compressed_compress_amd.recall_report --out profiles/indexer_mxfp4_recall.md
"""
from __future__ import annotations

import argparse
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def _recall(a, b, k):
    out = []
    for x, y in zip(a.reshape(-1, k), b.reshape(-1, k)):
        x, y = x[x >= 0], y[y >= 0]
        out.append(len(np.intersect1d(x, y)) / max(1, min(k, len(y))))
    return np.asarray(out)


def run(L, torch, dev, keys, q, w, q_pos, n_entries, k, want_scores=False):
    """Selections of both paths: keys [B, N, D], q [B, T, H, D] float32 (host)."""
    B, N, D = keys.shape
    T = q.shape[1]

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    kf, qf, wg, qp, ne = up(keys), up(q), up(w), up(q_pos), up(n_entries)
    kc = torch.empty(B, N, D // 2, dtype=torch.uint8, device=dev)
    ks = torch.empty(B, N, D // 32, dtype=torch.uint8, device=dev)
    L.mxfp4_quantize(kf.view(B * N, D), kc.view(B * N, D // 2), ks.view(B * N, D // 32))
    sb = torch.empty(B, T, N, dtype=torch.bfloat16, device=dev)
    i_mx = torch.empty(B, T, k, dtype=torch.int32, device=dev)
    L.indexer_topk(qf, wg, kc, ne, qp, 4, sb, k, i_mx, k_scales=ks)
    del sb
    s32 = torch.empty(B, T, N, dtype=torch.float32, device=dev)
    L.indexer_score(qf, wg, kf, ne, qp, 4, s32)
    i_32 = torch.empty(B, T, k, dtype=torch.int32, device=dev)
    L.topk_select(s32, ne, qp, 4, k, i_32)
    torch.cuda.synchronize()
    if want_scores:
        return i_mx.cpu().numpy(), i_32.cpu().numpy(), s32.cpu().numpy()
    return i_mx.cpu().numpy(), i_32.cpu().numpy()


def planted_keys(keys, q, w, k, strength, seed):
    """Keys with k relevant entries per sequence: each moved by `strength` key
    standard deviations along the sequence's weighted query direction
    u = sum_h w_h q_h / |.|, so their scores stand above the bulk.  A stand-in
    for trained data, where the entries an indexer should find score well
    apart from the rest; the i.i.d. keys have no such gap."""
    rng = np.random.default_rng(seed)
    out = keys.copy()
    for b in range(keys.shape[0]):
        u = (w[b, 0][:, None] * q[b, 0]).sum(0)
        u = (u / np.linalg.norm(u)).astype(np.float32)
        rel = rng.choice(keys.shape[1], size=k, replace=False)
        out[b, rel] += np.float32(strength) * u
    return out


def score_gap(s32, k):
    """(mean of the top k float32 scores - the (2k)-th score) / the bulk's
    standard deviation, per row: how far the selected entries stand out."""
    g = []
    for row in s32.reshape(-1, s32.shape[-1]):
        srt = np.sort(row)[::-1]
        g.append((srt[:k].mean() - srt[2 * k]) / srt[2 * k:].std())
    return np.asarray(g)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", required=True)
    a = ap.parse_args()
    import torch
    from long_context_compressed_compress_amd import libcsa as L
    from long_context_compressed_compress_amd import workloads as WL
    dev = torch.device("cuda:0")
    planted_rows = []
    lines = ["# Top-k recall of the MXFP4 indexer against the float32 indexer", "",
             "Command:", "", "```",
             "python -m long_context_compressed_compress_amd.recall_report --out " + os.path.relpath(a.out, ROOT),
             "```", "",
             "Both selections are the library's, on the GPU, from the same seeded inputs: MXFP4 keys and queries",
             "(BF16 scores, `indexer_topk`) and the unquantized float32 keys and queries (float32 scores,",
             "`indexer_score` + `topk_select`).  recall@k = shared entries / k, per query row.  The pages",
             "report 99.7 % on the",
             "trained model's data; N(0,1) synthetic keys and queries have no printed counterpart.", "",
             "| workload | rows | entries visible | k | recall mean | min | p1 | rows with recall 1 |",
             "|---|---:|---:|---:|---:|---:|---:|---:|"]

    # decode at 1M context: 8 sequences x 262144 entries, k = 1024
    w = WL.csa_decode_1m()
    p = w.params
    B, N, K = p["batch"], p["n_entries"], p["topk"]
    ne = np.full(B, N, np.int32)
    i_mx, i_32 = run(L, torch, dev, w["k_idx"], w["q_idx"], w["w"], p["q_pos"], ne, K)
    r = _recall(i_mx, i_32, K)
    lines.append(f"| CSA decode 1M (B=8) | {len(r)} | {N} | {K} | {r.mean():.4f} | {r.min():.4f} | "
                 f"{np.percentile(r, 1):.4f} | {int((r == 1).sum())} |")
    print(lines[-1], flush=True)
    # the same shape with planted relevant entries
    for strength in (2.0, 4.0, 6.0, 8.0):
        kp = planted_keys(w["k_idx"], w["q_idx"], w["w"], K, strength, seed=1000 + int(strength))
        i_mx, i_32, s32 = run(L, torch, dev, kp, w["q_idx"], w["w"], p["q_pos"], ne, K, want_scores=True)
        r = _recall(i_mx, i_32, K)
        planted_rows.append(f"| {strength:g} | {score_gap(s32, K).mean():.2f} | {r.mean():.4f} | {r.min():.4f} | "
                            f"{int((r == 1).sum())} of {len(r)} |")
        print(planted_rows[-1], flush=True)
        del kp, s32
    del w

    # chunked prefill: 4096 query rows x 16384 entries (15360 .. 16384 visible), k = 512
    w = WL.csa_prefill_chunk()
    p = w.params
    N, K, T = p["n_entries"], p["topk"], p["n_q"]
    i_mx, i_32 = run(L, torch, dev, w["k_idx"], w["q_idx"], w["w"], p["q_pos"], np.array([N], np.int32), K)
    r = _recall(i_mx, i_32, K)
    nv = np.minimum((np.asarray(p["q_pos"][0]) + 1) // 4, N)   # entries whose four tokens are all <= t
    lines.append(f"| CSA chunked prefill | {len(r)} | {int(nv.min())}..{int(nv.max())} | {K} | {r.mean():.4f} | "
                 f"{r.min():.4f} | {np.percentile(r, 1):.4f} | {int((r == 1).sum())} |")
    print(lines[-1], flush=True)
    lines += ["", "## Decode at 1M context with planted relevant entries", "",
              "The decode keys above with k = 1,024 entries per sequence moved `strength` key standard deviations",
              "along the sequence's weighted query direction (seeded choice of entries), as a stand-in for trained",
              "data where the entries to find score apart from the rest.  `gap` = (mean of the top-k float32",
              "scores - the 2k-th score) / the standard deviation of the scores below it, mean over rows.  For the",
              "i.i.d. keys above the gap is small and MXFP4 rounding reorders the tail; as the gap grows the MXFP4",
              "selection converges to the float32 one.", "",
              "| strength | gap | recall mean | min | rows with recall 1 |", "|---:|---:|---:|---:|---:|"]
    lines += planted_rows + [""]
    with open(a.out, "w") as f:
        f.write("\n".join(lines))


if __name__ == "__main__":
    main()
