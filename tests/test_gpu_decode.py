"""GPU parity of the decode step over a device-resident cache.

decode_step (append + compress-on-boundary + indexer + top-k + both attentions,
positions and counts on the device) against the same step made of the
individual calls (kv_append, csa_compress with its MXFP4 key, hca_compress,
indexer_topk, sparse_window_attn, hca_dense_attn), each of which has its own
oracle parity tests: outputs, entries, keys, rings, counts and positions equal
bit for bit, with sequences at different positions (first CSA entries with
masked slots, CSA and HCA boundaries at different steps).  The entries the
steps create are also checked against the oracle's compressors directly."""
import math

import numpy as np
import pytest
import torch

from oracle import csa_oracle as O
from tests.gpu_util import dev, down, mixed_mismatches_near_midpoints, mxfp4_mismatches_near_boundaries, up

pytestmark = pytest.mark.gpu


def _weights(rng, DI):
    return {"csa_w_gate": (rng.standard_normal((192, 192)) * 0.02).astype(np.float32),
            "csa_pos_bias": (rng.standard_normal((8, 192)) * 0.1).astype(np.float32),
            "csa_w_idx": (rng.standard_normal((192, DI)) / np.sqrt(192)).astype(np.float32),
            "hca_w_gate": (rng.standard_normal((192, 192)) * 0.02).astype(np.float32),
            "hca_pos_bias": (rng.standard_normal((128, 192)) * 0.1).astype(np.float32)}


@pytest.mark.parametrize("q_bf16", [True, False])
def test_decode_step_equals_the_individual_calls(q_bf16):
    from long_context_compressed_compress_amd import libcsa as L
    rng = np.random.default_rng(40 + q_bf16)
    B, H, HI, DI, K, W = 3, 32 if q_bf16 else 8, 64, 64, 64, 128
    p0 = np.array([125, 509, 3], np.int64)       # HCA boundary at step 2 / step 2; first CSA entry at step 0
    steps = 9
    L_hist = int(p0.max()) + steps
    csa_cap, hca_cap = 160, 8
    scale = 1.0 / math.sqrt(192)
    wts = _weights(rng, DI)
    wd = {k: up(v) for k, v in wts.items()}
    xc = rng.standard_normal((B, L_hist, 192)).astype(np.float32)    # raw KV of the CSA layer, by position
    xh = rng.standard_normal((B, L_hist, 192)).astype(np.float32)    # raw KV of the HCA layer
    xc_b, xh_b = up(xc).to(torch.bfloat16), up(xh).to(torch.bfloat16)
    qdt = torch.bfloat16 if q_bf16 else torch.float32
    q_idx = up(rng.standard_normal((steps, B, HI, DI)).astype(np.float32))
    w = up(rng.random((steps, B, HI)).astype(np.float32))
    q_c = up(rng.standard_normal((steps, B, H, 192)).astype(np.float32)).to(qdt)
    q_h = up(rng.standard_normal((steps, B, H, 192)).astype(np.float32)).to(qdt)

    # ---- the prefix: entries by the prefill compressors, rings by decode_prime
    cache = L.DecodeCache(B, H, HI, DI, K, W, csa_cap, hca_cap, scale, wd, device=dev())
    for b in range(B):
        nc, nh = int(p0[b]) // 4, int(p0[b]) // 128
        if nc:
            L.csa_compress(xc_b[b:b + 1], 0, wd["csa_w_gate"], wd["csa_pos_bias"], 0, nc, cache.csa_kv[b:b + 1],
                           w_idx=wd["csa_w_idx"], key_out=cache.csa_keys[b:b + 1],
                           key_scales=cache.csa_key_scales[b:b + 1])
        if nh:
            L.hca_compress(xh_b[b:b + 1], 0, wd["hca_w_gate"], wd["hca_pos_bias"], 0, nh, cache.hca_kv[b:b + 1])
    cache.pos.copy_(up(p0))
    cache.csa_entries.copy_(up((p0 // 4).astype(np.int32)))
    cache.hca_entries.copy_(up((p0 // 128).astype(np.int32)))
    n_prime = 128
    prime_c = torch.zeros(B, n_prime, 192, dtype=torch.bfloat16, device=dev())
    prime_h = torch.zeros_like(prime_c)
    for b in range(B):
        lo = int(p0[b]) - n_prime
        src = slice(max(lo, 0), int(p0[b]))
        prime_c[b, max(-lo, 0):] = xc_b[b, src]
        prime_h[b, max(-lo, 0):] = xh_b[b, src]
    L.decode_prime(cache, prime_c, prime_h)

    # ---- the same state for the call-by-call path (raw rings of 128 rows)
    kv_c, kc, ks, kv_h = (t.clone() for t in (cache.csa_kv, cache.csa_keys, cache.csa_key_scales, cache.hca_kv))
    win_c, win_h = cache.csa_win.clone(), cache.hca_win.clone()
    raw_c = torch.zeros(B, 128, 192, dtype=torch.bfloat16, device=dev())
    raw_h = torch.zeros_like(raw_c)
    for b in range(B):
        ps = torch.arange(max(int(p0[b]) - 128, 0), int(p0[b]), device=dev())
        raw_c[b, ps % 128] = xc_b[b, ps]
        raw_h[b, ps % 128] = xh_b[b, ps]
    n_c = cache.csa_entries.clone()
    n_h = cache.hca_entries.clone()
    scores = torch.empty(B, 1, csa_cap, dtype=torch.bfloat16, device=dev())
    idx = torch.empty(B, 1, K, dtype=torch.int32, device=dev())
    out_c2 = torch.empty(B, 1, H, 192, dtype=torch.bfloat16, device=dev())
    out_h2 = torch.empty_like(out_c2)

    ws = cache.workspace(qdt)
    out_c = torch.empty(B, H, 192, dtype=torch.bfloat16, device=dev())
    out_h = torch.empty_like(out_c)
    for s in range(steps):
        pos = torch.from_numpy(p0 + s).to(dev())
        xs_c = torch.stack([xc_b[b, int(p0[b]) + s] for b in range(B)])
        xs_h = torch.stack([xh_b[b, int(p0[b]) + s] for b in range(B)])
        print(f"decode step {s} positions {(p0 + s).tolist()} q_bf16={q_bf16}", flush=True)
        L.decode_step(cache, xs_c, xs_h, q_idx[s], w[s], q_c[s], q_h[s], out_c, out_h, ws)
        # call by call
        L.kv_append(xs_c, pos, raw_ring=raw_c, win_ring=win_c)
        L.kv_append(xs_h, pos, raw_ring=raw_h, win_ring=win_h)
        for b in range(B):
            p = int(p0[b]) + s
            if (p + 1) % 4 == 0:
                i = (p + 1) // 4 - 1
                L.csa_compress(raw_c[b:b + 1], 0, wd["csa_w_gate"], wd["csa_pos_bias"], i, 1, kv_c[b:b + 1],
                               w_idx=wd["csa_w_idx"], key_out=kc[b:b + 1], key_scales=ks[b:b + 1])
                n_c[b] = i + 1
            if (p + 1) % 128 == 0:
                i = (p + 1) // 128 - 1
                L.hca_compress(raw_h[b:b + 1], 0, wd["hca_w_gate"], wd["hca_pos_bias"], i, 1, kv_h[b:b + 1])
                n_h[b] = i + 1
        qp = pos.view(B, 1)
        L.indexer_topk(q_idx[s].view(B, 1, HI, DI), w[s].view(B, 1, HI), kc, n_c, qp, 4, scores, K, idx,
                       k_scales=ks)
        L.sparse_window_attn(q_c[s].view(B, 1, H, 192), kv_c, n_c, 4, idx, win_c, 0, qp, W, scale, out_c2)
        L.hca_dense_attn(q_h[s].view(B, 1, H, 192), kv_h, n_h, 128, win_h, 0, qp, W, scale, out_h2)
        assert torch.equal(out_c.view(torch.int16), out_c2.view(B, H, 192).view(torch.int16)), s
        assert torch.equal(out_h.view(torch.int16), out_h2.view(B, H, 192).view(torch.int16)), s

    torch.cuda.synchronize()
    assert torch.equal(cache.pos, torch.from_numpy(p0 + steps).to(dev()))
    assert torch.equal(cache.csa_entries, n_c) and torch.equal(cache.hca_entries, n_h)
    assert torch.equal(cache.csa_kv, kv_c) and torch.equal(cache.hca_kv, kv_h)
    assert torch.equal(cache.csa_keys, kc) and torch.equal(cache.csa_key_scales, ks)
    assert torch.equal(cache.csa_win, win_c) and torch.equal(cache.hca_win, win_h)
    for b in range(B):
        end = int(p0[b]) + steps
        ps = torch.arange(end - 8, end, device=dev())
        assert torch.equal(cache.csa_raw[b, ps % 8], raw_c[b, ps % 128])
        ps = torch.arange(end - 128, end, device=dev())
        assert torch.equal(cache.hca_raw[b, ps % 128], raw_h[b, ps % 128])

    # ---- the entries the steps created, against the oracle's compressors
    got_c, got_kc, got_ks, got_h = down(cache.csa_kv), down(cache.csa_keys), down(cache.csa_key_scales), \
        down(cache.hca_kv)
    raw_vals_c = xc_b.float().cpu().numpy()
    raw_vals_h = xh_b.float().cpu().numpy()
    new_c = new_h = tol_e = tol_k = 0
    for b in range(B):
        i0, i1 = int(p0[b]) // 4, (int(p0[b]) + steps) // 4
        if i1 > i0:
            ref = O.csa_compress(raw_vals_c[b], wts["csa_w_gate"], wts["csa_pos_bias"], i0, i1 - i0)
            tol_e += mixed_mismatches_near_midpoints(got_c[b, i0:i1], ref)
            tol_k += mxfp4_mismatches_near_boundaries(got_kc[b, i0:i1], got_ks[b, i0:i1],
                                                      O.csa_compress_key(ref, wts["csa_w_idx"]))
            new_c += i1 - i0
        h0, h1 = int(p0[b]) // 128, (int(p0[b]) + steps) // 128
        if h1 > h0:
            ref = O.hca_compress(raw_vals_h[b], wts["hca_w_gate"], wts["hca_pos_bias"], h0, h1 - h0)
            tol_e += mixed_mismatches_near_midpoints(got_h[b, h0:h1], ref)
            new_h += h1 - h0
    assert new_c >= 6 and new_h == 2
    assert tol_e <= 0.002 * (new_c + new_h) * 192 and tol_k <= 0.002 * new_c * DI


def test_decode_step_sinks_inactive_sequence_and_capacity():
    """decode_step with learnable sinks on both layers, an inactive sequence
    (pos -1: nothing appended or compressed, its state unchanged, outputs zero)
    and a sequence whose CSA entries reach the cache capacity mid-run (entries
    at or past the capacity are not stored and the count stays at it), against
    the same step made of the individual calls, bit for bit."""
    from long_context_compressed_compress_amd import libcsa as L
    rng = np.random.default_rng(47)
    B, H, HI, DI, K, W = 3, 32, 64, 64, 64, 128
    p0 = np.array([125, -1, 155], np.int64)      # seq 0: HCA boundary at step 2; seq 2: CSA capacity at step 8
    steps = 9
    csa_cap, hca_cap = 40, 2
    L_hist = int(p0.max()) + steps
    scale = 1.0 / math.sqrt(192)
    wts = _weights(rng, DI)
    wts["csa_sink"] = rng.standard_normal(H).astype(np.float32)
    wts["hca_sink"] = rng.standard_normal(H).astype(np.float32)
    wd = {k: up(v) for k, v in wts.items()}
    xc_b = up(rng.standard_normal((B, L_hist, 192)).astype(np.float32)).to(torch.bfloat16)
    xh_b = up(rng.standard_normal((B, L_hist, 192)).astype(np.float32)).to(torch.bfloat16)
    q_idx = up(rng.standard_normal((steps, B, HI, DI)).astype(np.float32))
    w = up(rng.random((steps, B, HI)).astype(np.float32))
    q_c = up(rng.standard_normal((steps, B, H, 192)).astype(np.float32)).to(torch.bfloat16)
    q_h = up(rng.standard_normal((steps, B, H, 192)).astype(np.float32)).to(torch.bfloat16)

    cache = L.DecodeCache(B, H, HI, DI, K, W, csa_cap, hca_cap, scale, wd, device=dev())
    for b in (0, 2):
        nc, nh = int(p0[b]) // 4, int(p0[b]) // 128
        L.csa_compress(xc_b[b:b + 1], 0, wd["csa_w_gate"], wd["csa_pos_bias"], 0, nc, cache.csa_kv[b:b + 1],
                       w_idx=wd["csa_w_idx"], key_out=cache.csa_keys[b:b + 1], key_scales=cache.csa_key_scales[b:b + 1])
        if nh:
            L.hca_compress(xh_b[b:b + 1], 0, wd["hca_w_gate"], wd["hca_pos_bias"], 0, nh, cache.hca_kv[b:b + 1])
    cache.pos.copy_(up(p0))
    cache.csa_entries.copy_(up(np.maximum(p0 // 4, 0).astype(np.int32)))
    cache.hca_entries.copy_(up(np.maximum(p0 // 128, 0).astype(np.int32)))
    prime_c = torch.zeros(B, 128, 192, dtype=torch.bfloat16, device=dev())
    prime_h = torch.zeros_like(prime_c)
    for b in (0, 2):
        lo = int(p0[b]) - 128
        prime_c[b, max(-lo, 0):] = xc_b[b, max(lo, 0):int(p0[b])]
        prime_h[b, max(-lo, 0):] = xh_b[b, max(lo, 0):int(p0[b])]
    L.decode_prime(cache, prime_c, prime_h)                       # sequence 1 (inactive) is skipped

    kv_c, kc, ks, kv_h = (t.clone() for t in (cache.csa_kv, cache.csa_keys, cache.csa_key_scales, cache.hca_kv))
    win_c, win_h = cache.csa_win.clone(), cache.hca_win.clone()
    idle = {k: getattr(cache, k)[1].clone() for k in ("csa_raw", "csa_logits", "hca_raw", "hca_logits", "csa_win",
                                                       "hca_win", "csa_kv", "hca_kv", "csa_keys")}
    raw_c = torch.zeros(B, 128, 192, dtype=torch.bfloat16, device=dev())
    raw_h = torch.zeros_like(raw_c)
    for b in (0, 2):
        ps = torch.arange(max(int(p0[b]) - 128, 0), int(p0[b]), device=dev())
        raw_c[b, ps % 128] = xc_b[b, ps]
        raw_h[b, ps % 128] = xh_b[b, ps]
    n_c, n_h = cache.csa_entries.clone(), cache.hca_entries.clone()
    scores = torch.empty(B, 1, csa_cap, dtype=torch.bfloat16, device=dev())
    idx = torch.empty(B, 1, K, dtype=torch.int32, device=dev())
    out_c2 = torch.empty(B, 1, H, 192, dtype=torch.bfloat16, device=dev())
    out_h2 = torch.empty_like(out_c2)
    ws = cache.workspace(torch.bfloat16)
    out_c = torch.empty(B, H, 192, dtype=torch.bfloat16, device=dev())
    out_h = torch.empty_like(out_c)
    for s in range(steps):
        pv = np.where(p0 >= 0, p0 + s, -1)
        pos = torch.from_numpy(pv).to(dev())
        xs_c = torch.stack([xc_b[b, max(int(pv[b]), 0)] for b in range(B)])
        xs_h = torch.stack([xh_b[b, max(int(pv[b]), 0)] for b in range(B)])
        print(f"decode step {s} positions {pv.tolist()} (sinks, inactive, capacity)", flush=True)
        L.decode_step(cache, xs_c, xs_h, q_idx[s], w[s], q_c[s], q_h[s], out_c, out_h, ws)
        L.kv_append(xs_c, pos, raw_ring=raw_c, win_ring=win_c)
        L.kv_append(xs_h, pos, raw_ring=raw_h, win_ring=win_h)
        for b in (0, 2):
            p = int(pv[b])
            if (p + 1) % 4 == 0:
                i = (p + 1) // 4 - 1
                if i < csa_cap:
                    L.csa_compress(raw_c[b:b + 1], 0, wd["csa_w_gate"], wd["csa_pos_bias"], i, 1, kv_c[b:b + 1],
                                   w_idx=wd["csa_w_idx"], key_out=kc[b:b + 1], key_scales=ks[b:b + 1])
                n_c[b] = min(i + 1, csa_cap)
            if (p + 1) % 128 == 0:
                i = (p + 1) // 128 - 1
                if i < hca_cap:
                    L.hca_compress(raw_h[b:b + 1], 0, wd["hca_w_gate"], wd["hca_pos_bias"], i, 1, kv_h[b:b + 1])
                n_h[b] = min(i + 1, hca_cap)
        qp = pos.view(B, 1)
        L.indexer_topk(q_idx[s].view(B, 1, HI, DI), w[s].view(B, 1, HI), kc, n_c, qp, 4, scores, K, idx,
                       k_scales=ks)
        L.sparse_window_attn(q_c[s].view(B, 1, H, 192), kv_c, n_c, 4, idx, win_c, 0, qp, W, scale, out_c2,
                             sink=wd["csa_sink"])
        L.hca_dense_attn(q_h[s].view(B, 1, H, 192), kv_h, n_h, 128, win_h, 0, qp, W, scale, out_h2,
                         sink=wd["hca_sink"])
        for b in (0, 2):
            assert torch.equal(out_c[b].view(torch.int16), out_c2[b, 0].view(torch.int16)), (s, b)
            assert torch.equal(out_h[b].view(torch.int16), out_h2[b, 0].view(torch.int16)), (s, b)
        assert not out_c[1].float().abs().any() and not out_h[1].float().abs().any(), s
    torch.cuda.synchronize()
    assert cache.pos.tolist() == [int(p0[0]) + steps, -1, int(p0[2]) + steps]
    assert torch.equal(cache.csa_entries, n_c) and torch.equal(cache.hca_entries, n_h)
    assert int(cache.csa_entries[2]) == csa_cap and int(cache.csa_entries[1]) == 0
    for b in (0, 2):
        assert torch.equal(cache.csa_kv[b], kv_c[b]) and torch.equal(cache.hca_kv[b], kv_h[b])
        assert torch.equal(cache.csa_keys[b], kc[b]) and torch.equal(cache.csa_key_scales[b], ks[b])
        assert torch.equal(cache.csa_win[b], win_c[b]) and torch.equal(cache.hca_win[b], win_h[b])
    for k, v in idle.items():
        assert torch.equal(getattr(cache, k)[1], v), k


def _random_cache(L, rng, B, K, csa_cap, hca_cap, pos, n_csa, n_hca, H=32, HI=64, DI=64):
    """A decode cache holding random stored entries, keys and rings (their
    values do not matter here: two caches built from the same draw are
    compared with each other)."""
    wd = {k: up(v) for k, v in _weights(rng, DI).items()}
    c = L.DecodeCache(B, H, HI, DI, K, 128, csa_cap, hca_cap, 1.0 / math.sqrt(192), wd, device=dev())
    ent = up(rng.standard_normal((B * csa_cap, 192)).astype(np.float32))
    L.kv_pack(ent, c.csa_kv.view(B * csa_cap, 256))
    enth = up(rng.standard_normal((B * hca_cap, 192)).astype(np.float32))
    L.kv_pack(enth, c.hca_kv.view(B * hca_cap, 256))
    c.csa_keys.copy_(up(rng.integers(0, 256, (B, csa_cap, DI // 2), dtype=np.uint8)))
    c.csa_key_scales.copy_(up(rng.integers(123, 131, (B, csa_cap, DI // 32), dtype=np.uint8)))
    c.pos.fill_(pos)
    c.csa_entries.fill_(n_csa)
    c.hca_entries.fill_(n_hca)
    L.decode_prime(c, up(rng.standard_normal((B, 128, 192)).astype(np.float32)),
                   up(rng.standard_normal((B, 128, 192)).astype(np.float32)))
    return c


def _run_steps(L, c, rng, ws, n):
    B, H, HI, DI = c.c.batch, c.c.n_heads, c.c.idx_heads, c.c.idx_dim
    outs = []
    for _ in range(n):
        xc = up(rng.standard_normal((B, 192)).astype(np.float32))
        xh = up(rng.standard_normal((B, 192)).astype(np.float32))
        qi = up(rng.standard_normal((B, HI, DI)).astype(np.float32))
        w = up(rng.random((B, HI)).astype(np.float32))
        qc = up(rng.standard_normal((B, H, 192)).astype(np.float32)).to(torch.bfloat16)
        qh = up(rng.standard_normal((B, H, 192)).astype(np.float32)).to(torch.bfloat16)
        oc = torch.empty(B, H, 192, dtype=torch.bfloat16, device=dev())
        oh = torch.empty_like(oc)
        L.decode_step(c, xc, xh, qi, w, qc, qh, oc, oh, ws)
        outs += [oc, oh]
    torch.cuda.synchronize()
    return outs


def test_decode_workspace_serves_caches_of_other_shapes():
    """One zero-filled workspace serves a cache of one shape and then a cache
    of another (batch, capacity, top-k): the second cache's steps give the
    same outputs and state as with a fresh workspace, i.e. the parts that must
    be zero at rest are left at zero at offsets that do not move with the
    shape.  Both shapes take the split top-k path."""
    from long_context_compressed_compress_amd import libcsa as L
    big = _random_cache(L, np.random.default_rng(60), 6, 128, 40000, 64, 4 * 39990 + 1, 39990, 64)
    small = [_random_cache(L, np.random.default_rng(61), 2, 64, 20000, 32, 4 * 16000 + 2, 16000, 32)
             for _ in range(2)]
    n = max(big.workspace_size(), small[0].workspace_size())
    shared = torch.zeros(n, dtype=torch.uint8, device=dev())
    print("decode workspace reuse: the larger cache first", flush=True)
    _run_steps(L, big, np.random.default_rng(62), shared, 5)
    print("decode workspace reuse: the smaller cache, shared and fresh workspace", flush=True)
    a = _run_steps(L, small[0], np.random.default_rng(63), shared, 6)
    b = _run_steps(L, small[1], np.random.default_rng(63), small[1].workspace(), 6)
    for i, (x, y) in enumerate(zip(a, b)):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16)), i
    for k in ("pos", "csa_entries", "hca_entries", "csa_kv", "csa_keys", "csa_key_scales", "hca_kv"):
        assert torch.equal(getattr(small[0], k), getattr(small[1], k)), k


def test_layer_by_layer_calls_equal_decode_step():
    """decode_csa_layer then decode_hca_layer, token after token, give what
    decode_step gives, bit for bit: the outputs of both layers at every step
    (across CSA boundaries every 4 tokens and an HCA boundary), the positions,
    counts, entries, keys and rings; an inactive sequence stays untouched."""
    from long_context_compressed_compress_amd import libcsa as L
    B, p0 = 3, 128 * 500 - 5
    a, b = (_random_cache(L, np.random.default_rng(70), B, 64, 20000, 512, p0, p0 // 4, p0 // 128) for _ in range(2))
    for c in (a, b):
        c.pos[1] = -1
    wa, wb = a.workspace(), b.workspace()
    rng = np.random.default_rng(71)
    H, HI, DI = a.c.n_heads, a.c.idx_heads, a.c.idx_dim
    for s in range(9):
        xc = up(rng.standard_normal((B, 192)).astype(np.float32))
        xh = up(rng.standard_normal((B, 192)).astype(np.float32))
        qi = up(rng.standard_normal((B, HI, DI)).astype(np.float32))
        w = up(rng.random((B, HI)).astype(np.float32))
        qc = up(rng.standard_normal((B, H, 192)).astype(np.float32)).to(torch.bfloat16)
        qh = up(rng.standard_normal((B, H, 192)).astype(np.float32)).to(torch.bfloat16)
        oc1, oh1, oc2, oh2 = (torch.empty(B, H, 192, dtype=torch.bfloat16, device=dev()) for _ in range(4))
        print(f"layer-by-layer decode, step {s}", flush=True)
        L.decode_step(a, xc, xh, qi, w, qc, qh, oc1, oh1, wa)
        L.decode_csa_layer(b, xc, qi, w, qc, oc2, wb)
        L.decode_hca_layer(b, xh, qh, oh2, wb)
        torch.cuda.synchronize()
        assert torch.equal(oc1.view(torch.int16), oc2.view(torch.int16)), s
        assert torch.equal(oh1.view(torch.int16), oh2.view(torch.int16)), s
        assert torch.equal(a.pos, b.pos), s
    assert a.pos.tolist() == [p0 + 9, -1, p0 + 9]
    assert b.hca_entries.tolist() == [p0 // 128 + 1, p0 // 128, p0 // 128 + 1]
    for k in ("pos", "csa_entries", "hca_entries", "csa_raw", "csa_logits", "hca_raw", "hca_logits", "csa_win",
              "hca_win", "csa_kv", "csa_keys", "csa_key_scales", "hca_kv"):
        x, y = getattr(a, k), getattr(b, k)
        assert torch.equal(x.view(torch.uint8) if x.dtype != torch.uint8 else x,
                           y.view(torch.uint8) if y.dtype != torch.uint8 else y), k
