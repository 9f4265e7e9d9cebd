"""The five workloads at full size on the GPU, in the same launch configuration
as the benchmark, checked against the oracle on sampled outputs.

1  CSA decode, tiny, fp32 end to end (compress -> FP32 indexer -> top-k ->
   attention): entries/keys/scores to 1e-5, top-k index sets bit-exact,
   attention to 1e-5.
2  CSA chunked prefill (4096 queries x 16384 entries, MXFP4 indexer, k=512,
   64 heads, BF16 out): sampled query rows.
3  CSA decode at 1M context (8 x 262144 entries, k=1024, 128 heads): sampled
   sequences.
4  HCA decode at 1M context (32 x 8192 entries, 128 heads): every sequence.
5  Hybrid pair, long prefill (131072 BF16 tokens in 32 chunks): both
   compressors over every chunk, then CSA and HCA attention of chunks 0 and 31
   on sampled rows."""
import functools

import numpy as np
import pytest
import torch

from long_context_compressed_compress_amd import workloads as WL
from oracle import csa_oracle as O
from tests.gpu_util import (SCALE, assert_attn_close, assert_f32_close, assert_is_topk_of, bf16_ulp, dev, down,
                            mixed_mismatches_near_midpoints, mxfp4_mismatches_near_boundaries, topk_unique_part_ok,
                            up)

pytestmark = pytest.mark.gpu


def _lib():
    from long_context_compressed_compress_amd import libcsa as L
    return L


def _pack_mixed(x_f32):
    L = _lib()
    flat = x_f32.reshape(-1, 192)
    out = torch.empty(flat.shape[0], 256, dtype=torch.uint8, device=dev())
    L.kv_pack(up(flat) if isinstance(flat, np.ndarray) else flat, out)
    return out.view(*x_f32.shape[:-1], 256)


def _mx(x_f32):
    L = _lib()
    t = up(x_f32) if isinstance(x_f32, np.ndarray) else x_f32
    d = t.shape[-1]
    codes = torch.empty(*t.shape[:-1], d // 2, dtype=torch.uint8, device=dev())
    scales = torch.empty(*t.shape[:-1], d // 32, dtype=torch.uint8, device=dev())
    L.mxfp4_quantize(t.contiguous(), codes, scales)
    return codes, scales


def _mx_ref(x):
    return O.mxfp4_dequantize(*O.mxfp4_quantize(x))


@functools.lru_cache(maxsize=None)
def _decode_1m_ref_keys(b):
    """The oracle's decoded MXFP4 keys of context sequence b (262144 x 64)."""
    return _mx_ref(WL.csa_decode_1m(batch_rows=[b])["k_idx"][0])


# -----------------------------------------------------------------------------
def test_workload1_csa_decode_tiny_fp32_chain():
    L = _lib()
    w = WL.csa_decode_tiny()
    p = w.params
    x, wg, pb, wi = w["x"], w["w_gate"], w["pos_bias"], w["w_idx"]
    n_cap = p["L"] // 4
    kv = torch.empty(1, n_cap, 192, dtype=torch.float32, device=dev())
    key = torch.empty(1, n_cap, p["d_idx"], dtype=torch.float32, device=dev())
    L.csa_compress(up(x), 0, up(wg), up(pb), 0, n_cap, kv, w_idx=up(wi), key_out=key)
    ne = np.array([n_cap], np.int32)
    q_pos = p["q_pos"]
    sc = torch.empty(1, p["n_q"], n_cap, dtype=torch.float32, device=dev())
    L.indexer_score(up(w["q_idx"]), up(w["w"]), key, up(ne), up(q_pos), 4, sc)
    idx = torch.empty(1, p["n_q"], p["topk"], dtype=torch.int32, device=dev())
    L.topk_select(sc, up(ne), up(q_pos), 4, p["topk"], idx)
    out = torch.empty(1, p["n_q"], p["n_heads"], 192, dtype=torch.float32, device=dev())
    L.sparse_window_attn(up(w["q"]), kv, up(ne), 4, idx, up(x), 0, up(q_pos), p["window"], SCALE, out)

    ent = O.csa_compress(x[0], wg, pb, 0, n_cap)
    assert_f32_close(down(kv)[0], ent, 1e-5, "entries")
    keys = O.csa_compress_key(ent, wi)
    assert_f32_close(down(key)[0], keys, 1e-5, "keys")
    nv = O.n_visible(q_pos[0], n_cap, 4)
    ref_sc = O.indexer_scores(w["q_idx"][0], w["w"][0], keys, nv, False)
    assert_f32_close(down(sc)[0], ref_sc, 1e-5, "scores")
    gi, go = down(idx)[0], down(out)[0]
    for t in range(p["n_q"]):
        ref_idx = O.topk_select(ref_sc[t], p["topk"])
        assert np.array_equal(gi[t], ref_idx), f"top-k set differs at query {t}"
        o, _ = O.sparse_window_attn(w["q"][0, t], ent, ref_idx, int(nv[t]), x[0], 0, int(q_pos[0, t]), p["window"],
                                    SCALE)
        assert_f32_close(go[t], o, 1e-5, "attention")


# -----------------------------------------------------------------------------
def test_workload2_csa_prefill_chunk():
    L = _lib()
    w = WL.csa_prefill_chunk()
    p = w.params
    T, N, K, H, W = p["n_q"], p["n_entries"], p["topk"], p["n_heads"], p["window"]
    entm = _pack_mixed(w["entries"])
    kc, ks = _mx(w["k_idx"])
    qc, qs = _mx(w["q_idx"])
    qb = up(w["q"]).to(torch.bfloat16)
    winm = _pack_mixed(w["window"])
    win_base = p["win_pos0"]
    q_pos, ne = p["q_pos"], np.array([N], np.int32)
    sc = torch.empty(1, T, N, dtype=torch.bfloat16, device=dev())
    L.indexer_score(qc, up(w["w"]), kc, up(ne), up(q_pos), 4, sc, q_scales=qs, k_scales=ks)
    idx = torch.empty(1, T, K, dtype=torch.int32, device=dev())
    L.topk_select(sc, up(ne), up(q_pos), 4, K, idx)
    out = torch.empty(1, T, H, 192, dtype=torch.bfloat16, device=dev())
    L.sparse_window_attn(qb, entm, up(ne), 4, idx, winm, win_base, up(q_pos), W, SCALE, out)
    gsc, gi, go = down(sc)[0], down(idx)[0], down(out)[0]

    rng = np.random.default_rng(200)
    rows = np.unique(np.r_[0, 1, 2047, 2048, T - 1, rng.integers(0, T, 11)])
    kdec = _mx_ref(w["k_idx"][0])
    entv = O.kv_round(w["entries"][0])
    winv = O.kv_round(w["window"][0])
    qv = qb.double().cpu().numpy()[0]
    nv = O.n_visible(q_pos[0], N, 4)
    ref_rows, ref_idx = [], []
    same_sets = 0
    for t in rows:
        ref = O.indexer_scores(_mx_ref(w["q_idx"][0, t])[None], w["w"][0, t][None], kdec, [nv[t]], True)[0]
        fin = np.isfinite(ref)
        assert (np.isfinite(gsc[t]) == fin).all()
        assert (np.abs(gsc[t][fin] - ref[fin]) <= bf16_ulp(ref[fin]) + 1e-30).all()
        topk_unique_part_ok(gi[t], ref, K)
        ri = O.topk_select(ref, K)
        ref_rows.append(ref)
        ref_idx.append(ri)
        if np.array_equal(gi[t], ri):
            same_sets += 1
            o, _ = O.sparse_window_attn(qv[t], entv, ri, int(nv[t]), winv, win_base, int(q_pos[0, t]), W, SCALE)
            assert_attn_close(go[t], o, True, f"prefill row {t}")
    # top-k kernel on the oracle's own score rows: bit-exact
    s_ref = torch.from_numpy(np.stack(ref_rows).astype(np.float32)).to(torch.bfloat16).to(dev())[None]
    idx2 = torch.empty(1, len(rows), K, dtype=torch.int32, device=dev())
    L.topk_select(s_ref, up(ne), up(q_pos[:, rows].copy()), 4, K, idx2)
    assert np.array_equal(down(idx2)[0], np.stack(ref_idx))
    # attention kernel on the oracle's selections: within tolerance
    out2 = torch.empty(1, len(rows), H, 192, dtype=torch.bfloat16, device=dev())
    L.sparse_window_attn(qb[:, rows].contiguous(), entm, up(ne), 4, up(np.stack(ref_idx)[None].astype(np.int32)), winm,
                         win_base, up(q_pos[:, rows].copy()), W, SCALE, out2)
    g2 = down(out2)[0]
    for n, t in enumerate(rows):
        o, _ = O.sparse_window_attn(qv[t], entv, ref_idx[n], int(nv[t]), winv, win_base, int(q_pos[0, t]), W, SCALE)
        assert_attn_close(g2[n], o, True, f"prefill row {t} (oracle selection)")
    print(f"workload 2: {same_sets}/{len(rows)} sampled rows select the oracle's exact set")


# -----------------------------------------------------------------------------
def test_workload3_csa_decode_1m():
    L = _lib()
    w = WL.csa_decode_1m()
    p = w.params
    B, N, K, H, W = p["batch"], p["n_entries"], p["topk"], p["n_heads"], p["window"]
    t = int(p["q_pos"][0, 0])
    entm = _pack_mixed(w["entries"])
    kc, ks = _mx(w["k_idx"])
    qc, qs = _mx(w["q_idx"])
    qb = up(w["q"]).to(torch.bfloat16)
    ring_f = np.empty_like(w["window"])
    pos = np.arange(t - W + 1, t + 1)
    ring_f[:, pos % W] = w["window"]
    ringm = _pack_mixed(ring_f)
    q_pos, ne = p["q_pos"], np.full(B, N, np.int32)
    sc = torch.empty(B, 1, N, dtype=torch.bfloat16, device=dev())
    L.indexer_score(qc, up(w["w"]), kc, up(ne), up(q_pos), 4, sc, q_scales=qs, k_scales=ks)
    idx = torch.empty(B, 1, K, dtype=torch.int32, device=dev())
    L.topk_select(sc, up(ne), up(q_pos), 4, K, idx)
    out = torch.empty(B, 1, H, 192, dtype=torch.bfloat16, device=dev())
    L.sparse_window_attn(qb, entm, up(ne), 4, idx, ringm, 0, up(q_pos), W, SCALE, out)
    gsc, gi, go = down(sc), down(idx), down(out)
    qv = qb.double().cpu().numpy()
    recalls = []
    for b in range(B):
        print(f"workload 3: sequence {b}", flush=True)
        ref = O.indexer_scores(_mx_ref(w["q_idx"][b, 0])[None], w["w"][b], _decode_1m_ref_keys(b), [N], True)[0]
        assert (np.abs(gsc[b, 0] - ref) <= bf16_ulp(ref) + 1e-30).all()
        assert_is_topk_of(gi[b, 0], gsc[b, 0], K, f"seq {b}")
        recalls.append(topk_unique_part_ok(gi[b, 0], ref, K))
        ri = O.topk_select(ref, K)
        sel = np.union1d(ri, gi[b, 0])
        entv = np.zeros((N, 192))
        entv[sel] = O.kv_round(w["entries"][b][sel])
        winv = O.kv_round(w["window"][b])
        o, _ = O.sparse_window_attn(qv[b, 0], entv, ri, N, winv, t - W + 1, t, W, SCALE)
        if np.array_equal(ri, gi[b, 0]):
            assert_attn_close(go[b, 0], o, True, f"decode seq {b}")
        # attention kernel on the oracle's selection
        o2 = torch.empty(1, 1, H, 192, dtype=torch.bfloat16, device=dev())
        L.sparse_window_attn(qb[b:b + 1].contiguous(), entm[b:b + 1], up(ne[:1]), 4, up(ri[None, None].astype(np.int32)),
                             ringm[b:b + 1], 0, up(q_pos[b:b + 1]), W, SCALE, o2)
        assert_attn_close(down(o2)[0, 0], o, True, f"decode seq {b} (oracle selection)")
    print(f"workload 3: recall vs the oracle's BF16-score selection {recalls}")


# -----------------------------------------------------------------------------
def test_workload4_hca_decode_1m():
    L = _lib()
    w = WL.hca_decode_1m()
    p = w.params
    B, N, H, W = p["batch"], p["n_entries"], p["n_heads"], p["window"]
    t = int(p["q_pos"][0, 0])
    entm = _pack_mixed(w["entries"])
    qb = up(w["q"]).to(torch.bfloat16)
    ring_f = np.empty_like(w["window"])
    pos = np.arange(t - W + 1, t + 1)
    ring_f[:, pos % W] = w["window"]
    ringm = _pack_mixed(ring_f)
    out = torch.empty(B, 1, H, 192, dtype=torch.bfloat16, device=dev())
    L.hca_dense_attn(qb, entm, up(np.full(B, N, np.int32)), 128, ringm, 0, up(p["q_pos"]), W, SCALE, out)
    go = down(out)
    qv = qb.double().cpu().numpy()
    for b in range(B):  # every sequence
        o, _ = O.hca_dense_attn(qv[b, 0], O.kv_round(w["entries"][b]), N, O.kv_round(w["window"][b]), t - W + 1, t,
                                W, SCALE)
        assert_attn_close(go[b, 0], o, True, f"hca seq {b}")


# -----------------------------------------------------------------------------
def test_workload5_hybrid_prefill():
    L = _lib()
    w = WL.hybrid_prefill_weights()
    p = w.params
    Lt, C, K, H, W, DI = p["L"], p["chunk"], p["topk"], p["n_heads"], p["window"], p["d_idx"]
    n_csa, n_hca = Lt // 4, Lt // 128
    x = w["x"]
    raw = torch.empty(1, Lt, 192, dtype=torch.bfloat16, device=dev())
    L.kv_pack(up(x[0]), raw[0])                                     # raw BF16 token KV
    winm = _pack_mixed(x)                                            # stored raw tokens (window rows)
    kv = torch.empty(1, n_csa, 256, dtype=torch.uint8, device=dev())
    kc = torch.empty(1, n_csa, DI // 2, dtype=torch.uint8, device=dev())
    ks = torch.empty(1, n_csa, DI // 32, dtype=torch.uint8, device=dev())
    kvh = torch.empty(1, n_hca, 256, dtype=torch.uint8, device=dev())
    wg, pb, wgh, pbh, wi = (up(w[k]) for k in ("w_gate", "pos_bias", "w_gate_hca", "pos_bias_hca", "w_idx"))
    for c in range(p["n_chunks"]):
        L.csa_compress(raw, 0, wg, pb, c * C // 4, C // 4, kv, w_idx=wi, key_out=kc, key_scales=ks)
        L.hca_compress(raw, 0, wgh, pbh, c * C // 128, C // 128, kvh)
    g_kv, g_kc, g_ks, g_kvh = down(kv)[0], down(kc)[0], down(ks)[0], down(kvh)[0]

    xr = O.bf16_round(x[0])                                          # the BF16 raw tokens, as numbers
    ent = O.csa_compress(xr, w["w_gate"], w["pos_bias"], 0, n_csa)
    keys = O.csa_compress_key(ent, w["w_idx"])
    enth = O.hca_compress(xr, w["w_gate_hca"], w["pos_bias_hca"], 0, n_hca)
    tol = mixed_mismatches_near_midpoints(g_kv, ent)
    tol += mixed_mismatches_near_midpoints(g_kvh, enth)
    tolk = mxfp4_mismatches_near_boundaries(g_kc, g_ks, keys)
    assert tol <= 1e-3 * (n_csa + n_hca) * 192 and tolk <= 1e-3 * n_csa * DI
    print(f"workload 5: stored-entry elements at a rounding midpoint {tol}, key codes at a boundary {tolk}")

    entv, enthv, winv = O.kv_round(ent), O.kv_round(enth), O.kv_round(x[0])
    rkc, rks = O.mxfp4_quantize(keys)
    kdec = O.mxfp4_dequantize(rkc, rks)
    # entries whose stored key has the oracle's bytes (all but those counted at a rounding boundary above)
    key_same = (g_kc == rkc).all(axis=1) & (g_ks == rks).all(axis=1)
    assert (~key_same).sum() <= tolk
    ne, neh = np.array([n_csa], np.int32), np.array([n_hca], np.int32)
    rng = np.random.default_rng(500)
    for c in (0, 31):
        rows = np.unique(np.r_[0, 1, 127, 128, C - 1, rng.integers(0, C, 5)])
        qd = WL.hybrid_prefill_chunk(w, c)
        q_pos = qd["q_pos"]
        qc, qs = _mx(qd["q_idx"])
        sc = torch.empty(1, C, n_csa, dtype=torch.bfloat16, device=dev())
        L.indexer_score(qc, up(qd["w"]), kc, up(ne), up(q_pos), 4, sc, q_scales=qs, k_scales=ks)
        idx = torch.empty(1, C, K, dtype=torch.int32, device=dev())
        L.topk_select(sc, up(ne), up(q_pos), 4, K, idx)
        qcb = up(qd["q_csa"]).to(torch.bfloat16)
        qhb = up(qd["q_hca"]).to(torch.bfloat16)
        out = torch.empty(1, C, H, 192, dtype=torch.bfloat16, device=dev())
        L.sparse_window_attn(qcb, kv, up(ne), 4, idx, winm, 0, up(q_pos), W, SCALE, out)
        outh = torch.empty(1, C, H, 192, dtype=torch.bfloat16, device=dev())
        L.hca_dense_attn(qhb, kvh, up(neh), 128, winm, 0, up(q_pos), W, SCALE, outh)
        gsc, gi, go, goh = down(sc)[0], down(idx)[0], down(out)[0], down(outh)[0]
        qcv, qhv = qcb.double().cpu().numpy()[0], qhb.double().cpu().numpy()[0]
        ref_rows, ref_out = [], []
        for t in rows:
            tq = int(q_pos[0, t])
            nv = int(O.n_visible(tq, n_csa, 4))
            ref = O.indexer_scores(_mx_ref(qd["q_idx"][0, t])[None], qd["w"][0, t][None], kdec, [nv], True)[0]
            fin = np.isfinite(ref)
            assert (np.isfinite(gsc[t]) == fin).all()
            # every entry whose stored key has the oracle's bytes scores within one BF16 ulp (a key code
            # computed in float32 may sit on the other side of a rounding boundary: counted above)
            chk = fin & key_same
            assert (np.abs(gsc[t][chk] - ref[chk]) <= bf16_ulp(ref[chk]) + 1e-30).all(), f"chunk {c} row {t}"
            assert_is_topk_of(gi[t], gsc[t], K, f"chunk {c} row {t}")
            ri = O.topk_select(ref, K)
            ref_rows.append(ri)
            o, _ = O.sparse_window_attn(qcv[t], entv, ri, nv, winv, 0, tq, W, SCALE)
            ref_out.append(o)
            if np.array_equal(ri, gi[t]):
                assert_attn_close(go[t], o, True, f"CSA chunk {c} row {t}")
            oh, _ = O.hca_dense_attn(qhv[t], enthv, int(O.n_visible(tq, n_hca, 128)), winv, 0, tq, W, SCALE)
            assert_attn_close(goh[t], oh, True, f"HCA chunk {c} row {t}")
        # the attention kernel on the oracle's selection of every sampled row
        out2 = torch.empty(1, len(rows), H, 192, dtype=torch.bfloat16, device=dev())
        L.sparse_window_attn(qcb[:, rows].contiguous(), kv, up(ne), 4, up(np.stack(ref_rows)[None].astype(np.int32)),
                             winm, 0, up(q_pos[:, rows].copy()), W, SCALE, out2)
        g2 = down(out2)[0]
        for n, t in enumerate(rows):
            assert_attn_close(g2[n], ref_out[n], True, f"CSA chunk {c} row {t} (oracle selection)")


# -----------------------------------------------------------------------------
@pytest.mark.parametrize("variant", ["pro", "flash"])
def test_decode_step_1m_as_benchmarked(variant):
    """Four decode steps of the benchmark's layers at full size (8 sequences
    from position 2^20 over 262144 CSA entries and 8192 HCA entries, 128 query
    heads; pro: top-1024; flash: top-512 plus a sliding-window-only layer),
    built and launched exactly as the benchmark does.  After every step the
    fused step equals the call-by-call step bit for bit (outputs, positions,
    entry counts); the fourth step completes CSA entry 262144, whose stored row
    and MXFP4 key are checked against the oracle's compression of the same raw
    tokens.  On the first step the call-by-call scores, selection and outputs
    are checked against the oracle on every sequence:
    scores within one BF16 ulp of the oracle's MXFP4 indexer, the selection
    exactly the top-k of those BF16 scores and valid against the oracle's own,
    and every attention output within the attention bound."""
    import bench
    L = _lib()
    B, W, D, t = 8, bench.W, bench.D, bench.CTX
    fused = bench.DecodePair(L, torch, B, 4, path="fused", variant=variant)
    calls = bench.DecodePair(L, torch, B, 4, path="calls", variant=variant)
    K, HQ = fused.K, fused.HQ
    assert K == (512 if variant == "flash" else 1024)
    st = WL.decode_stream(calls.pool, B, calls.HI, calls.DI, HQ)
    seqs = range(B)
    for step in range(4):
        print(f"{variant} decode step {step} at 1M", flush=True)
        fused.step(step)
        calls.step(step)
        torch.cuda.synchronize()
        assert torch.equal(fused.out.view(torch.int16), calls.out.view(torch.int16)), f"step {step}"
        assert torch.equal(fused.out_h.view(torch.int16), calls.out_h.view(torch.int16)), f"step {step}"
        if variant == "flash":
            assert torch.equal(fused.out_swa.view(torch.int16), calls.out_swa.view(torch.int16)), f"step {step}"
        p_next = t + step + 1
        assert torch.equal(fused.cache.pos.cpu(), torch.full((B,), p_next, dtype=torch.int64))
        assert torch.equal(fused.cache.csa_entries.cpu(), torch.full((B,), p_next // 4, dtype=torch.int32))
        assert torch.equal(fused.cache.hca_entries.cpu(), torch.full((B,), p_next // 128, dtype=torch.int32))
        if step == 0:
            _check_decode_step0(calls, st, seqs, variant, K, HQ, B, W, D, t)

    # the fourth step (position 2^20 + 3) completed CSA entry 262144 = tokens 2^20-4 .. 2^20+3:
    # the last four context tokens and the four step tokens, pooled from their BF16 raw values
    i_new = t // 4
    g_kv = down(fused.cache.csa_kv)[:, i_new]
    g_kc = down(fused.cache.csa_keys)[:, i_new]
    g_ks = down(fused.cache.csa_key_scales)[:, i_new]
    assert np.array_equal(g_kv, down(calls.kv)[:, i_new])
    assert np.array_equal(g_kc, down(calls.kc)[:, i_new]) and np.array_equal(g_ks, down(calls.ks)[:, i_new])
    wts = WL.hybrid_prefill_weights()
    csa_all = WL.csa_decode_1m(batch_rows=range(B))
    ents, keys = [], []
    for b in range(B):
        toks = O.bf16_round(np.concatenate([csa_all["window"][b][-4:], st["x_csa"][:4, b]]))
        ent = O.gated_pool(toks, np.ones(8, bool), wts["w_gate"], wts["pos_bias"])
        ents.append(ent)
        keys.append(O.csa_compress_key(ent[None], wts["w_idx"])[0])
    tol = mixed_mismatches_near_midpoints(g_kv, np.stack(ents))
    tolk = mxfp4_mismatches_near_boundaries(g_kc, g_ks, np.stack(keys))
    print(f"  appended entry: stored elements at a rounding midpoint {tol}, key codes at a boundary {tolk}")


def _check_decode_step0(calls, st, seqs, variant, K, HQ, B, W, D, t):
    gsc, gi, go, goh = down(calls.scores), down(calls.idx), down(calls.out), down(calls.out_h)
    N, Nh = (t + 1) // 4, (t + 1) // 128
    for b in seqs:
        print(f"  oracle check, sequence {b}", flush=True)
        csa = WL.csa_decode_1m(batch_rows=[b])
        hca = WL.hca_decode_1m(batch_rows=[b])
        ref = O.indexer_scores(_mx_ref(st["q_idx"][0, b])[None], st["w"][0, b][None], _decode_1m_ref_keys(b),
                               [N], True)[0]
        assert (np.abs(gsc[b, 0, :N] - ref) <= bf16_ulp(ref) + 1e-30).all()
        assert_is_topk_of(gi[b, 0], gsc[b, 0, :N], K, f"seq {b}")
        recall = topk_unique_part_ok(gi[b, 0], ref, K)
        # window tokens t-127 .. t: the last 127 context tokens and the step's own
        win = O.kv_round(np.concatenate([csa["window"][0][1:], st["x_csa"][0, b][None]]))
        win_h = O.kv_round(np.concatenate([hca["window"][0][1:], st["x_hca"][0, b][None]]))
        sel = gi[b, 0][gi[b, 0] >= 0]
        entv = np.zeros((N, D))
        entv[sel] = O.kv_round(csa["entries"][0][sel])
        o, _ = O.sparse_window_attn(O.bf16_round(st["q_csa"][0, b]), entv, sel, N, win, t - W + 1, t, W, SCALE)
        assert_attn_close(go[b], o, True, f"{variant} CSA seq {b}")
        oh, _ = O.hca_dense_attn(O.bf16_round(st["q_hca"][0, b]), O.kv_round(hca["entries"][0]), Nh, win_h,
                                 t - W + 1, t, W, SCALE)
        assert_attn_close(goh[b], oh, True, f"{variant} HCA seq {b}")
        if variant == "flash":
            sw = WL.swa_layer_stream(calls.pool, B, HQ, W)
            win_s = O.kv_round(np.concatenate([sw["window"][b][1:], sw["x"][0, b][None]]))
            os_, _ = O.hca_dense_attn(O.bf16_round(sw["q"][0, b]), np.zeros((1, D)), 0, win_s, t - W + 1, t, W,
                                      SCALE)
            assert_attn_close(down(calls.out_swa)[b, 0], os_, True, f"SWA seq {b}")
        print(f"  recall vs the oracle's own top-{K}: {recall:.4f}", flush=True)
