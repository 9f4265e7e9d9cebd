"""Helpers shared by the GPU parity tests: device upload, tolerance rules and
boundary-aware comparisons.  The expected values always come from the oracle."""
from __future__ import annotations

import numpy as np
import torch

from oracle import csa_oracle as O

SCALE = 1.0 / np.sqrt(192.0)


def dev():
    return torch.device("cuda:0")


def up(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a)).to(dev())
    return t if dtype is None else t.to(dtype)


def down(t) -> np.ndarray:
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy()


def bf16_tensor(a_f32: np.ndarray):
    """The caller's BF16 copy of float32 data (a plain RNE cast, input marshalling)."""
    return torch.from_numpy(np.ascontiguousarray(a_f32, dtype=np.float32)).to(torch.bfloat16).to(dev())


def bf16_ulp(x) -> np.ndarray:
    """Spacing of BF16 numbers at |x| (0 for x == 0)."""
    a = np.abs(np.asarray(x, np.float64))
    _, E = np.frexp(a)
    return np.where(a > 0, np.ldexp(1.0, E - 1 - 7), 0.0)


def attn_bound(ref: np.ndarray, out_bf16: bool) -> np.ndarray:
    """Attention acceptance: |err| <= 2e-3 * ||ref||_inf for FP8/BF16 storage, plus
    half a BF16 ulp of the reference when the output itself is BF16."""
    b = 2e-3 * np.abs(ref).max()
    return b + (0.5 * bf16_ulp(ref) if out_bf16 else 0.0)


def assert_attn_close(got, ref, out_bf16, what=""):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    bound = attn_bound(ref, out_bf16)
    err = np.abs(got - ref)
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements beyond bound; max err/||ref|| = "
                           f"{err.max() / np.abs(ref).max():.3e}")
    return float(err.max() / np.abs(ref).max())


def assert_f32_close(got, ref, rel=1e-5, what=""):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    fin = np.isfinite(ref)
    assert (np.isfinite(got) == fin).all(), f"{what}: -inf pattern differs"
    if not fin.any():
        return 0.0
    scale = np.abs(ref[fin]).max()
    err = np.abs(got[fin] - ref[fin]).max()
    assert err <= rel * scale, f"{what}: max err {err:.3e} > {rel:g} * ||ref|| ({scale:.3e})"
    return float(err / scale)


def mixed_mismatches_near_midpoints(got_rows: np.ndarray, ref_vals: np.ndarray, rel=1e-5, abs_frac=2.0 ** -20) -> int:
    """Compare stored 256-byte rows with the storage rounding of fp64 values.
    Bytes must match, except where the fp64 value lies within float32 error of
    the midpoint between the two neighbouring stored values (a float32
    computation may land on either side): within `rel` of the value, or within
    `abs_frac` * max|ref| (float32 sums of O(1) terms err in absolute terms, so
    a result that cancels to near zero keeps that absolute error).  Returns the
    number of such tolerated elements."""
    want_rows = O.kv_pack(ref_vals)
    g = O.kv_unpack(got_rows)
    w = O.kv_unpack(want_rows)
    diff = g != w
    if not diff.any():
        return 0
    mid = 0.5 * (g[diff] + w[diff])
    v = ref_vals[diff]
    near = np.abs(v - mid) <= rel * np.abs(v) + abs_frac * np.abs(ref_vals).max()
    assert near.all(), (f"{int((~near).sum())} stored elements differ away from a rounding midpoint "
                        f"(e.g. value {v[~near][:3]}, got {g[diff][~near][:3]}, want {w[diff][~near][:3]})")
    return int(diff.sum())


E2M1_BOUNDS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])


def mxfp4_mismatches_near_boundaries(codes, scales, ref_vals, rel=1e-5) -> int:
    """MXFP4 of float32-computed values vs the oracle's quantisation of the fp64
    values: equal except for elements whose scaled fp64 value sits within `rel`
    of an E2M1 decision boundary, or blocks whose max magnitude sits within
    `rel` of a power of two (the shared exponent may then differ)."""
    rc, rs = O.mxfp4_quantize(ref_vals)
    D = ref_vals.shape[-1]
    blocks = ref_vals.reshape(-1, D // 32, 32)
    rs2 = rs.reshape(-1, D // 32)
    gs2 = np.asarray(scales).reshape(-1, D // 32)
    amax = np.abs(blocks).max(axis=-1)
    pow2_near = np.abs(amax - np.exp2(np.round(np.log2(np.maximum(amax, 1e-300))))) <= rel * amax
    scale_diff = gs2 != rs2
    assert (pow2_near[scale_diff]).all(), "a block scale differs away from a power-of-two boundary"
    def unpack(p):
        p = np.asarray(p, np.uint8)
        return np.stack([p & 0xF, p >> 4], axis=-1).reshape(*p.shape[:-1], 2 * p.shape[-1])
    gc = unpack(codes).reshape(-1, D // 32, 32)
    rcu = unpack(rc).reshape(-1, D // 32, 32)
    elem_diff = (gc != rcu) & ~scale_diff[..., None]
    if elem_diff.any():
        e = rs2.astype(np.int64) - 127
        sv = np.abs(np.ldexp(blocks, -e[..., None]))[elem_diff]
        # scaled block maxima lie in [4, 8): float32 error is relative to that magnitude
        near = (np.abs(sv[:, None] - E2M1_BOUNDS[None]) <= rel * 8.0).any(axis=1)
        assert near.all(), f"{int((~near).sum())} E2M1 codes differ away from a rounding boundary"
    return int(elem_diff.sum() + 32 * scale_diff.sum())


def topk_unique_part_ok(got_idx, ref_scores, k, ulps=2.0):
    """Top-k of a GPU score row vs the oracle's scores when the two score arrays
    may differ by rounding: every entry scoring clearly above the oracle's k-th
    value must be selected, none clearly below it, and the selection must be a
    valid set (distinct, visible, k or all visible).  Returns recall vs the
    oracle's own top-k."""
    s = np.asarray(ref_scores, np.float64)
    vis = np.flatnonzero(s > -np.inf)
    got = np.asarray(got_idx)
    sel = got[got >= 0]
    assert len(np.unique(sel)) == len(sel), "duplicate indices"
    assert np.isin(sel, vis).all(), "selected an invisible entry"
    assert len(sel) == min(k, len(vis)), "wrong number selected"
    assert (np.diff(sel) > 0).all(), "not in ascending index order"
    ref_sel = O.topk_select(s, k)
    ref_sel = ref_sel[ref_sel >= 0]
    if len(vis) <= k:
        assert np.array_equal(np.sort(sel), np.sort(vis))
        return 1.0
    tau = np.sort(s[vis])[::-1][k - 1]
    margin = ulps * max(bf16_ulp(tau), 1e-30)
    must = vis[s[vis] > tau + margin]
    never = vis[s[vis] < tau - margin]
    assert np.isin(must, sel).all(), "an entry clearly above the k-th score was dropped"
    assert not np.isin(never, sel).any(), "an entry clearly below the k-th score was chosen"
    return float(np.isin(ref_sel, sel).mean())


def assert_is_topk_of(got_idx, scores, k, what=""):
    """The selection is exactly the top-k of `scores` by definition: the min(k,
    visible) visible entries (score > -inf) that come first when ordered by
    score descending, then index ascending, listed in ascending index order and
    padded with -1.  Checked directly (no sort): every selected entry must
    precede every visible entry left out in that order."""
    s = np.asarray(scores, np.float64)
    got = np.asarray(got_idx)
    vis = np.flatnonzero(s > -np.inf)
    n_sel = min(k, len(vis))
    assert got.shape == (k,), f"{what}: shape {got.shape}"
    assert (got[n_sel:] == -1).all(), f"{what}: padding"
    sel = got[:n_sel]
    assert (np.diff(sel) > 0).all(), f"{what}: not strictly ascending"
    assert np.isin(sel, vis).all(), f"{what}: selected an invisible entry"
    out = np.setdiff1d(vis, sel, assume_unique=True)
    if len(out) == 0 or n_sel == 0:
        return
    # the weakest selected entry: lowest score, and among those the highest index
    lo = s[sel].min()
    weakest = sel[s[sel] == lo].max()
    hi = s[out].max()
    strongest_out = out[s[out] == hi].min()
    assert lo > hi or (lo == hi and weakest < strongest_out), (
        f"{what}: entry {strongest_out} (score {hi}) outranks selected entry {weakest} (score {lo})")
