"""Seeded synthetic workloads for the CSA + HCA compressed-attention path.

This module only draws random numbers: shapes, distributions and seeds of the
five workloads (tiny CSA decode, CSA chunked prefill, CSA decode at 1M context,
HCA decode at 1M context, hybrid-pair prefill) and of the decode stream that
the benchmark replays.  It holds no step of the method (no pooling, scoring,
selection, attention, rounding or encoding), so both the GPU path and the fp64
oracle can take their inputs from here without sharing any arithmetic.

Every tensor is drawn from its own child of
``SeedSequence([0xC5A, workload_id])``; tensors with a batch axis draw each
batch row (and, for the long-prefill queries, each chunk) from a grandchild, so
a test can regenerate a single row without drawing the others.  All floating
tensors come back as C-contiguous ``float32`` arrays.

"N(0, s)" below means a normal draw with standard deviation ``s``;
"U(0, 1)" a uniform draw on [0, 1).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

SEED_ROOT = 0xC5A
DIM = 192  # per-token / per-entry KV width: 128 no-RoPE dims followed by 64 RoPE dims


def _children(workload_id: int, n: int) -> list[np.random.SeedSequence]:
    return np.random.SeedSequence([SEED_ROOT, workload_id]).spawn(n)


def _gen(ss: np.random.SeedSequence) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(ss))


def _normal(ss, shape, std=1.0) -> np.ndarray:
    a = _gen(ss).standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def _uniform(ss, shape) -> np.ndarray:
    return _gen(ss).random(shape, dtype=np.float32)


def _rows(ss: np.random.SeedSequence, n_total: int, rows, shape, std=1.0, dist="normal"):
    """Draw the selected batch rows of a [n_total, *shape] tensor, one grandchild per row."""
    kids = ss.spawn(n_total)
    rows = range(n_total) if rows is None else list(rows)
    draw = _normal if dist == "normal" else (lambda s, sh, std=1.0: _uniform(s, sh))
    return np.stack([draw(kids[r], shape, std) for r in rows]) if len(rows) else np.zeros((0, *shape), np.float32)


@dataclass
class Workload:
    """A named bundle of seeded tensors plus the scalar parameters of one workload."""

    name: str
    params: dict
    tensors: dict = field(default_factory=dict)

    def __getitem__(self, k):
        return self.tensors[k]


# ---------------------------------------------------------------------------
# 1. CSA decode, tiny (fp32 throughout)
# ---------------------------------------------------------------------------
def csa_decode_tiny() -> Workload:
    """Batch 1, 4096 tokens, m=4 -> 1024 entries; 4 indexer heads x dim 32;
    top-k 64; window 128; 8 query heads; last 16 query positions."""
    L, T, HI, DI, HQ = 4096, 16, 4, 32, 8
    c = _children(1, 7)
    w = Workload("csa_decode_tiny", dict(batch=1, L=L, m=4, n_q=T, h_idx=HI, d_idx=DI,
                                          topk=64, window=128, n_heads=HQ,
                                          q_pos=np.arange(L - T, L, dtype=np.int64)[None, :]))
    w.tensors = dict(
        x=_normal(c[0], (1, L, DIM)),                       # raw token KV
        w_gate=_normal(c[1], (DIM, DIM), 0.02),             # gate projection, z = x @ w_gate
        pos_bias=_normal(c[2], (8, DIM), 0.1),              # per-slot, per-channel bias (2m = 8 slots)
        w_idx=_normal(c[3], (DIM, DI), 1.0 / np.sqrt(DIM)),  # entry -> indexer-key projection
        q_idx=_normal(c[4], (1, T, HI, DI)),
        w=_uniform(c[5], (1, T, HI)),
        q=_normal(c[6], (1, T, HQ, DIM)),
    )
    return w


# ---------------------------------------------------------------------------
# 2. CSA chunked prefill: one 4096-query chunk at the end of a 65536-token context
# ---------------------------------------------------------------------------
def csa_prefill_chunk(q_rows=None) -> Workload:
    """Entries are drawn directly (N(0,1)); q rows can be restricted to ``q_rows``."""
    L, T, N, HI, DI, HQ, W = 65536, 4096, 16384, 64, 64, 64, 128
    c = _children(2, 6)
    t0 = L - T
    win_lo = t0 - W + 1  # oldest token any query of the chunk can see in its window
    rows = np.arange(T) if q_rows is None else np.asarray(q_rows)
    kq = c[2].spawn(T)
    kw = c[3].spawn(T)
    kqa = c[4].spawn(T)
    w = Workload("csa_prefill_chunk", dict(batch=1, L=L, m=4, n_q=len(rows), h_idx=HI, d_idx=DI,
                                            topk=512, window=W, n_heads=HQ, n_entries=N,
                                            win_pos0=win_lo, q_rows=rows,
                                            q_pos=(t0 + rows).astype(np.int64)[None, :]))
    w.tensors = dict(
        entries=_normal(c[0], (1, N, DIM)),
        k_idx=_normal(c[1], (1, N, DI)),
        q_idx=np.stack([_normal(kq[r], (HI, DI)) for r in rows])[None],
        w=np.stack([_uniform(kw[r], (HI,)) for r in rows])[None],
        q=np.stack([_normal(kqa[r], (HQ, DIM)) for r in rows])[None],
        window=_normal(c[5], (1, L - win_lo, DIM)),  # raw tokens at positions win_lo .. L-1
    )
    return w


# ---------------------------------------------------------------------------
# 3. CSA decode at 1M context (batch 8) and 4. HCA decode at 1M context (batch 32)
# ---------------------------------------------------------------------------
CTX_1M = 1 << 20


def csa_decode_1m(batch_rows=None, n_entries=CTX_1M // 4) -> Workload:
    """Batch 8, 2^20 tokens pre-compressed to 262144 entries; indexer 64 heads x 64;
    top-k 1024; 128 query heads; window 128.  Query position 2^20 - 1."""
    B, HI, DI, HQ, W = 8, 64, 64, 128, 128
    c = _children(3, 6)
    rows = list(range(B)) if batch_rows is None else list(batch_rows)
    t = CTX_1M - 1
    w = Workload("csa_decode_1m", dict(batch=len(rows), L=CTX_1M, m=4, n_q=1, h_idx=HI, d_idx=DI,
                                        topk=1024, window=W, n_heads=HQ, n_entries=n_entries,
                                        win_pos0=t - W + 1, batch_rows=rows,
                                        q_pos=np.full((len(rows), 1), t, np.int64)))
    w.tensors = dict(
        entries=_rows(c[0], B, rows, (n_entries, DIM)),
        k_idx=_rows(c[1], B, rows, (n_entries, DI)),
        q_idx=_rows(c[2], B, rows, (1, HI, DI)),
        w=_rows(c[3], B, rows, (1, HI), dist="uniform"),
        q=_rows(c[4], B, rows, (1, HQ, DIM)),
        window=_rows(c[5], B, rows, (W, DIM)),  # raw tokens at positions t-127 .. t
    )
    return w


def hca_decode_1m(batch_rows=None, n_entries=CTX_1M // 128) -> Workload:
    """Batch 32, 2^20 tokens compressed with m'=128 to 8192 entries; 128 query heads;
    dense attention plus a 128-token window.  Query position 2^20 - 1."""
    B, HQ, W = 32, 128, 128
    c = _children(4, 3)
    rows = list(range(B)) if batch_rows is None else list(batch_rows)
    t = CTX_1M - 1
    w = Workload("hca_decode_1m", dict(batch=len(rows), L=CTX_1M, m=128, n_q=1, window=W,
                                        n_heads=HQ, n_entries=n_entries, win_pos0=t - W + 1,
                                        batch_rows=rows, q_pos=np.full((len(rows), 1), t, np.int64)))
    w.tensors = dict(
        entries=_rows(c[0], B, rows, (n_entries, DIM)),
        q=_rows(c[1], B, rows, (1, HQ, DIM)),
        window=_rows(c[2], B, rows, (W, DIM)),
    )
    return w


def decode_stream(n_steps: int, batch: int, h_idx=64, d_idx=64, n_heads=128, workload_id=30) -> dict:
    """Per-step fresh inputs for a decode run of a CSA + HCA layer pair: the new token's
    raw KV for each layer, the indexer query and head weights, and both layers' queries."""
    c = _children(workload_id, 6)
    return dict(
        x_csa=_normal(c[0], (n_steps, batch, DIM)),
        x_hca=_normal(c[1], (n_steps, batch, DIM)),
        q_idx=_normal(c[2], (n_steps, batch, h_idx, d_idx)),
        w=_uniform(c[3], (n_steps, batch, h_idx)),
        q_csa=_normal(c[4], (n_steps, batch, n_heads, DIM)),
        q_hca=_normal(c[5], (n_steps, batch, n_heads, DIM)),
    )


def swa_layer_stream(n_steps: int, batch: int, n_heads=128, window=128, workload_id=32) -> dict:
    """A pure sliding-window layer at decode (the V4-Flash variant's first layers):
    its window of raw token KV before the run, then per step the new token's raw KV
    and the layer's queries."""
    c = _children(workload_id, 3)
    return dict(window=_normal(c[0], (batch, window, DIM)),      # positions t0-window .. t0-1
                x=_normal(c[1], (n_steps, batch, DIM)),
                q=_normal(c[2], (n_steps, batch, n_heads, DIM)))


def decode_prefix_raw(batch: int, n_tok=128, workload_id=31) -> dict:
    """Raw KV of the last ``n_tok`` context tokens of each layer before a decode run starts."""
    c = _children(workload_id, 2)
    return dict(csa=_normal(c[0], (batch, n_tok, DIM)), hca=_normal(c[1], (batch, n_tok, DIM)))


# ---------------------------------------------------------------------------
# 5. Hybrid layer pair, long prefill: 131072 tokens in 32 chunks of 4096
# ---------------------------------------------------------------------------
def hybrid_prefill_weights() -> Workload:
    L, HI, DI = 131072, 64, 64
    c = _children(5, 7)
    w = Workload("hybrid_prefill", dict(batch=1, L=L, chunk=4096, n_chunks=32, m=4, m_hca=128,
                                         h_idx=HI, d_idx=DI, topk=1024, window=128, n_heads=128))
    w.tensors = dict(
        x=_normal(c[0], (1, L, DIM)),                 # raw token KV (stored as BF16 by the user)
        w_gate=_normal(c[1], (DIM, DIM), 0.02),
        pos_bias=_normal(c[2], (8, DIM), 0.1),
        w_gate_hca=_normal(c[3], (DIM, DIM), 0.02),
        pos_bias_hca=_normal(c[4], (128, DIM), 0.1),
        w_idx=_normal(c[5], (DIM, DI), 1.0 / np.sqrt(DIM)),
    )
    w._chunk_seed = c[6]
    return w


def hybrid_prefill_chunk(weights: Workload, chunk: int, q_rows=None) -> dict:
    """Per-chunk queries of the long prefill (each chunk and each row seeded on its own)."""
    T, HI, DI, HQ = 4096, 64, 64, 128
    kid = weights._chunk_seed.spawn(32)[chunk].spawn(4)
    rows = np.arange(T) if q_rows is None else np.asarray(q_rows)
    kq, kw, kc, kh = (k.spawn(T) for k in kid)
    return dict(
        q_rows=rows,
        q_pos=(chunk * T + rows).astype(np.int64)[None, :],
        q_idx=np.stack([_normal(kq[r], (HI, DI)) for r in rows])[None],
        w=np.stack([_uniform(kw[r], (HI,)) for r in rows])[None],
        q_csa=np.stack([_normal(kc[r], (HQ, DIM)) for r in rows])[None],
        q_hca=np.stack([_normal(kh[r], (HQ, DIM)) for r in rows])[None],
    )
