"""fp64 CPU oracle of the CSA + HCA compressed-attention hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or link
this module: only the test suite, the smoke check and the benchmark's CPU
baseline leg use it.  It shares no code with the HIP library (no kernels,
headers, tables or helpers); the two meet only in the seeded input generator,
which holds none of the method's arithmetic.

Plain numpy in float64, written for a reader to check against the pages by eye:
no blocking, no fusion, no reordering beyond the definitions below.

Sources (web pages summarising the DeepSeek-V4 technical report; cited by the
page title and the section on that page):
  [TRIPBOT] 「论文解读｜DeepSeek-V4：百万 token 上下文的效率革命」 (blog.tripbot.top)
  [CSDN]    DeepSeek-V4 解读 on gitcode.csdn.net (导读「从论文出发，逐层剖析 CSA / HCA 混合注意力…」)
  [AUSTERY] DeepSeek-V4 technical-report notes on austery.github.io
  [YANBAOKE]「DeepSeek-V4 详细总结」 (研报客, pc.yanbaoke.cn)

What each function follows:
  * kv storage (bf16 RoPE dims + fp8 rest) ........ [CSDN] 核心创新一 §1.4「存储格式混合」
  * MXFP4 block quantisation ........................ [AUSTERY] 全栈工程优化 (FP4/MXFP4 indexer QK path);
                                                      [CSDN] §1.4「LIGHTNING INDEXER 的 FP4 计算」
  * CSA compressor, m=4, overlapped C^a/C^b ........ [TRIPBOT] §3.1 第一步 + Figure 3; [CSDN] §1.1「工程细节」
  * HCA compressor, m'=128 ......................... [TRIPBOT] §3.2; [CSDN] §1.2; [AUSTERY] 架构革新一
  * Lightning Indexer score, BF16 score rounding .... [TRIPBOT] §3.1 第二步; [CSDN] §1.4
  * top-k (k=1024 Pro / 512 Flash) ................. [TRIPBOT] §3.1 第二步; [CSDN] §1.1 关键参数
  * attention over selected entries + window 128,
    learnable sink ................................. [TRIPBOT] §3.3 + Figure 3; [AUSTERY] 架构革新一
  * HCA dense attention ............................. [TRIPBOT] §3.2; [CSDN] §1.2

Readings where the pages leave a step open are stated next to the code that
takes them.

Parity pins: every function here is pinned by tests/test_oracle_pins.py against
closed forms, special cases, library routines or brute force.  What stays a
reading rather than a fact of the pages is said where it is taken (the
entry -> indexer-key projection in ``csa_compress_key`` is one).
"""
from __future__ import annotations

import math

import numpy as np

DIM = 192          # per-entry width: dims [0,128) carry no position, [128,192) are the RoPE dims
DIM_NOPE = 128     # stored as FP8 E4M3
DIM_ROPE = 64      # stored as BF16
ROW_BYTES = 256    # 128 x 1 B + 64 x 2 B
MX_BLOCK = 32      # MXFP4 block length


# =============================================================================
# Number formats
# =============================================================================
def round_to_format(x, mant_bits: int, emin: int, max_finite: float, saturate: bool):
    """Round fp64 values to a binary floating-point format, round-to-nearest-even.

    ``mant_bits`` explicit mantissa bits, ``emin`` the exponent of the smallest
    normal binade (below it the quantum stays fixed: subnormals).  Overflow
    either saturates to ``max_finite`` or becomes inf.  The sign is kept
    (a negative value that rounds to zero gives -0.0).
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, E = np.frexp(a)                      # a = f * 2**E with f in [0.5, 1): leading bit at 2**(E-1)
    e = np.maximum(E - 1, emin)
    quantum = np.ldexp(1.0, e - mant_bits)
    r = np.rint(a / quantum) * quantum      # np.rint rounds half to even
    if saturate:
        r = np.minimum(r, max_finite)
    else:
        r = np.where(r > max_finite, np.inf, r)
    r = np.where(np.isnan(a), np.nan, r)
    return np.copysign(r, x)


# --- BF16: 8 exponent bits, 7 mantissa bits, IEEE-style overflow to inf ---------
BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def bf16_round(x):
    return round_to_format(x, 7, -126, BF16_MAX, saturate=False)


def bf16_encode(x) -> np.ndarray:
    """fp64 -> bf16 bit patterns (uint16), RNE."""
    r = bf16_round(x)
    return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def bf16_decode(bits) -> np.ndarray:
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# --- FP8 E4M3 (OCP "e4m3fn": bias 7, max 448, no infinities), saturating --------
FP8_MAX = 448.0


def fp8_round(x):
    return round_to_format(x, 3, -6, FP8_MAX, saturate=True)


def fp8_encode(x) -> np.ndarray:
    """fp64 -> E4M3 bytes, RNE, magnitudes beyond 448 (and inf) saturate to 448."""
    r = fp8_round(np.nan_to_num(np.asarray(x, np.float64), nan=0.0, posinf=FP8_MAX, neginf=-FP8_MAX))
    a = np.abs(r)
    sign = np.signbit(r).astype(np.uint8) << 7
    _, E = np.frexp(a)
    sub = a < 2.0 ** -6
    exp_field = np.where(sub, 0, E - 1 + 7)
    mant = np.where(sub, a / 2.0 ** -9, (np.ldexp(a, -(E - 1)) - 1.0) * 8.0)
    return (sign | (exp_field.astype(np.uint8) << 3) | np.rint(mant).astype(np.uint8)).astype(np.uint8)


def fp8_decode(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    s = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = b & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return s * mag


# --- E2M1 (FP4) element format: values {0, .5, 1, 1.5, 2, 3, 4, 6}, saturating ---
E2M1_MAX = 6.0


def e2m1_round(x):
    return round_to_format(x, 1, 0, E2M1_MAX, saturate=True)


def e2m1_encode(x) -> np.ndarray:
    """fp64 (already divided by the block scale) -> 4-bit codes; sign kept in bit 3."""
    r = e2m1_round(x)
    a = np.abs(r)
    sign = np.signbit(r).astype(np.uint8) << 3
    _, E = np.frexp(a)
    sub = a < 1.0
    exp_field = np.where(sub, 0, E - 1 + 1)
    mant = np.where(sub, a / 0.5, (np.ldexp(a, -(E - 1)) - 1.0) * 2.0)
    return (sign | (exp_field.astype(np.uint8) << 1) | np.rint(mant).astype(np.uint8)).astype(np.uint8)


def e2m1_decode(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x8, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = c & 0x1
    mag = np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * np.ldexp(1.0, e - 1))
    return s * mag


# =============================================================================
# Storage of KV rows: dims 0..127 as FP8 E4M3, dims 128..191 as BF16
# ([CSDN] 核心创新一 §1.4: RoPE dims kept in BF16, the other dims in FP8).
# Reading: the RoPE dims are the last 64 of the 192; row = 256 bytes,
# bytes [0,128) the FP8 codes in dim order, bytes [128,256) the BF16 values
# little-endian in dim order.
# =============================================================================
def kv_pack(x) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    assert x.shape[-1] == DIM
    lo = fp8_encode(x[..., :DIM_NOPE])
    hi = bf16_encode(x[..., DIM_NOPE:]).astype("<u2").view(np.uint8).reshape(*x.shape[:-1], 2 * DIM_ROPE)
    return np.concatenate([lo, hi], axis=-1)


def kv_unpack(rows) -> np.ndarray:
    rows = np.asarray(rows, dtype=np.uint8)
    assert rows.shape[-1] == ROW_BYTES
    lo = fp8_decode(rows[..., :DIM_NOPE])
    hi = bf16_decode(np.ascontiguousarray(rows[..., DIM_NOPE:]).view("<u2"))
    return np.concatenate([lo, hi], axis=-1)


def kv_round(x) -> np.ndarray:
    """The fp64 value a row takes once stored (pack then unpack)."""
    return kv_unpack(kv_pack(x))


# =============================================================================
# MXFP4: blocks of 32 values along the last axis share one E8M0 scale 2**e and
# each value is an E2M1 code ([AUSTERY] 全栈工程优化: the indexer QK path is MXFP4).
# Reading (the OCP MX v1.0 rule): e = floor(log2(max|v|)) - 2 (2 = the largest
# E2M1 exponent), clamped to [-127, 127]; an all-zero block takes e = -127.
# Scale byte = e + 127.  Codes are packed two per byte, the even element in the
# low nibble.
# =============================================================================
def mxfp4_scale_exp(block_amax) -> np.ndarray:
    amax = np.asarray(block_amax, dtype=np.float64)
    _, E = np.frexp(amax)
    e = np.where(amax > 0, E - 1 - 2, -127)
    return np.clip(e, -127, 127).astype(np.int64)


def mxfp4_quantize(x):
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    assert D % MX_BLOCK == 0
    blocks = x.reshape(*x.shape[:-1], D // MX_BLOCK, MX_BLOCK)
    e = mxfp4_scale_exp(np.abs(blocks).max(axis=-1))
    codes = e2m1_encode(np.ldexp(blocks, -e[..., None])).reshape(*x.shape[:-1], D)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    return packed, (e + 127).astype(np.uint8)


def mxfp4_dequantize(packed, scales) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8)
    codes = np.stack([packed & 0xF, packed >> 4], axis=-1).reshape(*packed.shape[:-1], 2 * packed.shape[-1])
    vals = e2m1_decode(codes)
    e = np.asarray(scales, dtype=np.int64) - 127
    D = vals.shape[-1]
    blocks = vals.reshape(*vals.shape[:-1], D // MX_BLOCK, MX_BLOCK)
    return np.ldexp(blocks, e[..., None]).reshape(vals.shape)


# =============================================================================
# Compressors
# =============================================================================
def gated_pool(tokens, valid, w_gate, bias) -> np.ndarray:
    """Softmax-gated pooling of a window of token KV rows into one entry.

    tokens [S, 192], valid [S] bool, w_gate [192, 192], bias [S, 192].
    Gate logits z[s, c] = sum_d tokens[s, d] * w_gate[d, c] + bias[s, c]; the
    weights are a softmax over the valid slots s, separately for each channel c;
    the entry is the weighted sum of the token rows themselves.
    Readings: the gate is applied per channel, the slot bias is per slot and
    per channel, there is no other gate bias, and the pooled value is the raw
    token KV (no separate value projection).
    """
    tokens = np.asarray(tokens, np.float64)
    z = tokens @ np.asarray(w_gate, np.float64) + np.asarray(bias, np.float64)
    z = np.where(valid[:, None], z, -np.inf)
    z = z - z.max(axis=0, keepdims=True)
    g = np.exp(z)
    alpha = g / g.sum(axis=0, keepdims=True)
    return (alpha * np.where(valid[:, None], tokens, 0.0)).sum(axis=0)


def csa_slot_tokens(i: int, m: int = 4) -> np.ndarray:
    """Token positions read by CSA entry i: slots 0..m-1 are the previous block
    (C^b), slots m..2m-1 the entry's own block (C^a) ([CSDN] §1.1 工程细节).
    Positions below zero do not exist (first entry)."""
    return m * (i - 1) + np.arange(2 * m)


def csa_compress(x, w_gate, pos_bias, entry_begin: int, n_new: int, m: int = 4) -> np.ndarray:
    """CSA entries entry_begin .. entry_begin+n_new-1 of one sequence.

    x [L, 192] raw token KV by absolute position; pos_bias [2m, 192].
    Reading for the first entry (no previous block): its C^b slots are left
    out of the softmax (masked), so a constant sequence still pools to itself.
    """
    x = np.asarray(x, np.float64)
    out = np.empty((n_new, DIM))
    for n, i in enumerate(range(entry_begin, entry_begin + n_new)):
        j = csa_slot_tokens(i, m)
        valid = j >= 0
        out[n] = gated_pool(x[np.maximum(j, 0)], valid, w_gate, pos_bias)
    return out


def hca_compress(x, w_gate, pos_bias, entry_begin: int, n_new: int, m: int = 128) -> np.ndarray:
    """HCA entries: entry i pools tokens m*i .. m*i+m-1, no overlap ([TRIPBOT] §3.2)."""
    x = np.asarray(x, np.float64)
    out = np.empty((n_new, DIM))
    for n, i in enumerate(range(entry_begin, entry_begin + n_new)):
        j = m * i + np.arange(m)
        out[n] = gated_pool(x[j], np.ones(m, bool), w_gate, pos_bias)
    return out


def csa_compress_key(entries, w_idx) -> np.ndarray:
    """Indexer key of each entry: the pooled entry projected to the indexer width.

    Reading: the pages give one lightweight key per compressed block and no
    formula for it; the reading taken here is k_i = C_i @ w_idx, shared by all
    indexer heads, projected from the pooled value C_i itself (not its stored
    FP8/BF16 form).  Pinned by basis-vector rows, a brute-force loop and the
    compressor -> key chain on constant and slot-selected inputs.
    """
    return np.asarray(entries, np.float64) @ np.asarray(w_idx, np.float64)


# =============================================================================
# Visibility (causality)
# =============================================================================
def n_visible(t, n_entries, m: int) -> np.ndarray:
    """Entries visible to a query at position t: entry i covers tokens up to
    m*i+m-1 and is visible iff that is <= t.  Also capped by the entries that
    exist."""
    t = np.asarray(t, np.int64)
    return np.minimum(np.asarray(n_entries, np.int64), (t + 1) // m)


# =============================================================================
# Lightning Indexer ([TRIPBOT] §3.1 第二步: multi-head dot-product scorer over
# all compressed blocks; [CSDN] §1.4: QK in FP4, score from FP32 to BF16)
# =============================================================================
def indexer_scores(q, w, k, n_vis, bf16_scores: bool) -> np.ndarray:
    """I[t, s] = sum_h w[t, h] * max(0, q[t, h, :] . k[s, :]) for s < n_vis[t], else -inf.

    q [T, H, DI], w [T, H], k [N, DI] (already-decoded values, so MXFP4 inputs
    are the dequantised numbers), n_vis [T].  With ``bf16_scores`` the fp64
    score is rounded to BF16 (RNE), the format the pages keep index scores in.
    """
    q = np.asarray(q, np.float64)
    w = np.asarray(w, np.float64)
    k = np.asarray(k, np.float64)
    T = q.shape[0]
    N = k.shape[0]
    out = np.full((T, N), -np.inf)
    for t in range(T):
        nv = int(n_vis[t])
        if nv <= 0:
            continue
        dots = q[t] @ k[:nv].T                       # [H, nv]
        s = w[t] @ np.maximum(dots, 0.0)             # [nv]
        out[t, :nv] = bf16_round(s) if bf16_scores else s
    return out


# =============================================================================
# Top-k ([TRIPBOT] §3.1 第二步: keep the k best-scoring compressed entries)
# =============================================================================
def topk_select(scores_row, k: int) -> np.ndarray:
    """The k visible entries with the largest scores, ties broken toward the
    lower index; -inf marks an invisible entry and is never chosen.

    Returned as the selected indices in ascending index order, padded with -1
    to length k (the set is what attention consumes; ascending order is the
    canonical form the calls exchange).
    """
    s = np.asarray(scores_row, np.float64)
    vis = np.flatnonzero(s > -np.inf)
    order = vis[np.lexsort((vis, -s[vis]))]          # score desc, then index asc
    chosen = np.sort(order[:k])
    out = np.full(k, -1, np.int64)
    out[: len(chosen)] = chosen
    return out


# =============================================================================
# Attention ([TRIPBOT] §3.3 + Figure 3; [TRIPBOT] §3.2 for HCA)
# =============================================================================
def attend(q, keys, scale: float, sink=None):
    """Softmax attention of each head of q [H, 192] over the key rows [n, 192].

    Readings: MQA (all query heads share the one stored row), the value is the
    same stored row as the key (all 192 dims), one joint softmax over every
    key in the set.  The learnable sink adds exp(sink[h]) to head h's
    denominator, so weights may sum to less than 1.  Returns (o [H, 192],
    lse [H]); an empty key set gives o = 0 and lse = -inf.
    """
    q = np.asarray(q, np.float64)
    keys = np.asarray(keys, np.float64)
    H = q.shape[0]
    if keys.shape[0] == 0:
        return np.zeros((H, DIM)), np.full(H, -np.inf)
    logits = scale * (q @ keys.T)                                  # [H, n]
    mx = logits.max(axis=1)
    if sink is not None:
        mx = np.maximum(mx, np.asarray(sink, np.float64))
    p = np.exp(logits - mx[:, None])
    denom = p.sum(axis=1)
    if sink is not None:
        denom = denom + np.exp(np.asarray(sink, np.float64) - mx)
    o = (p @ keys) / denom[:, None]
    with np.errstate(divide="ignore"):
        lse = mx + np.log(p.sum(axis=1))
    return o, lse


def window_positions(t: int, window: int) -> np.ndarray:
    """Sliding-window branch: the most recent ``window`` raw tokens up to and
    including the query's own position ([TRIPBOT] §3.3: window of 128)."""
    return np.arange(max(0, t - window + 1), t + 1)


def sparse_window_attn(q, entries, idx, n_vis: int, tok, tok_pos0: int, t: int, window: int,
                       scale: float, sink=None):
    """CSA attention of one query position.

    q [H, 192]; entries [N, 192] decoded stored entries; idx the selected entry
    indices (entries < 0 or >= n_vis are skipped); tok [P, 192] decoded stored
    raw tokens at positions tok_pos0 .. tok_pos0+P-1.  The key set is the
    selected entries together with the window tokens (no de-duplication).
    """
    idx = np.asarray(idx, np.int64)
    sel = idx[(idx >= 0) & (idx < n_vis)]
    win = window_positions(t, window) - tok_pos0
    assert win.size == 0 or win.min() >= 0, "window tokens not supplied"
    keys = np.concatenate([np.asarray(entries)[sel], np.asarray(tok)[win]], axis=0)
    return attend(q, keys, scale, sink)


def hca_dense_attn(q, entries, n_vis: int, tok, tok_pos0: int, t: int, window: int,
                   scale: float, sink=None):
    """HCA attention of one query position: every visible entry plus the window."""
    win = window_positions(t, window) - tok_pos0
    assert win.size == 0 or win.min() >= 0, "window tokens not supplied"
    keys = np.concatenate([np.asarray(entries)[:n_vis], np.asarray(tok)[win]], axis=0)
    return attend(q, keys, scale, sink)


def default_scale() -> float:
    return 1.0 / math.sqrt(DIM)
