"""GPU parity of the Lightning Indexer and of top-k selection.

* FP32 indexer: scores to 1e-5 relative; on exact-arithmetic inputs bit-exact,
  and the top-k index sets bit-exact.
* MXFP4 indexer: on exact-arithmetic inputs (E2M1-grid values with a +-4/+-6 in
  every block, dyadic head weights) the BF16 scores equal BF16(oracle) bit for
  bit; on N(0,1) inputs every score is within one BF16 ulp of BF16(oracle).
* top-k: on identical score arrays the selection is bit-exact (ties to the
  lower index, -inf never chosen, -1 padding)."""
import numpy as np
import pytest
import torch

from oracle import csa_oracle as O
from tests.gpu_util import assert_f32_close, assert_is_topk_of, bf16_ulp, dev, down, topk_unique_part_ok, up

pytestmark = pytest.mark.gpu
GRID = np.array([0.5, 1, 1.5, 2, 3, 4, 6, -0.5, -1, -1.5, -2, -3, -4, -6], np.float32)


def _exact_inputs(rng, B, T, H, D, N):
    q = rng.choice(GRID, (B, T, H, D))
    k = rng.choice(GRID, (B, N, D))
    for blk in range(D // 32):
        q[..., 32 * blk + 3] = 6.0
        k[..., 32 * blk + 7] = -4.0
    w = (rng.integers(0, 16, (B, T, H)) / 8.0).astype(np.float32)
    return q.astype(np.float32), w, k.astype(np.float32)


def _mx(a):
    codes, scales = O.mxfp4_quantize(a)
    return codes, scales


def test_indexer_f32_random_and_causal():
    from long_context_compressed_compress_amd import libcsa as L
    rng = np.random.default_rng(20)
    B, T, H, D, N = 2, 16, 4, 32, 1100
    q, w = rng.standard_normal((B, T, H, D)).astype(np.float32), rng.random((B, T, H)).astype(np.float32)
    k = rng.standard_normal((B, N, D)).astype(np.float32)
    q_pos = rng.integers(0, 4 * N + 50, (B, T)).astype(np.int64)
    q_pos[0, :3] = [0, 3, 4 * 17 + 2]
    ne = np.array([N, 900], np.int32)
    sc = torch.empty(B, T, N, dtype=torch.float32, device=dev())
    L.indexer_score(up(q), up(w), up(k), up(ne), up(q_pos), 4, sc)
    got = down(sc)
    for b in range(B):
        ref = O.indexer_scores(q[b], w[b], k[b], O.n_visible(q_pos[b], ne[b], 4), False)
        assert_f32_close(got[b], ref, 1e-5, "fp32 scores")


def test_indexer_f32_exact_inputs_bit_exact_with_topk():
    from long_context_compressed_compress_amd import libcsa as L
    rng = np.random.default_rng(21)
    B, T, H, D, N, K = 1, 16, 4, 32, 1024, 64
    q, w, k = _exact_inputs(rng, B, T, H, D, N)
    q_pos = np.arange(4096 - T, 4096, dtype=np.int64)[None]
    ne = np.array([N], np.int32)
    sc = torch.empty(B, T, N, dtype=torch.float32, device=dev())
    L.indexer_score(up(q), up(w), up(k), up(ne), up(q_pos), 4, sc)
    idx = torch.empty(B, T, K, dtype=torch.int32, device=dev())
    L.topk_select(sc, up(ne), up(q_pos), 4, K, idx)
    ref = O.indexer_scores(q[0], w[0], k[0], O.n_visible(q_pos[0], N, 4), False)
    assert np.array_equal(down(sc)[0], ref)
    gi = down(idx)[0]
    for t in range(T):
        assert np.array_equal(gi[t], O.topk_select(ref[t], K))


@pytest.mark.parametrize("H,D", [(64, 64), (32, 128), (128, 64), (96, 256)])
def test_indexer_mxfp4_exact_inputs_bit_exact(H, D):
    from long_context_compressed_compress_amd import libcsa as L
    rng = np.random.default_rng(22 + H + D)
    B, T, N, K = 2, 3, 777, 100
    q, w, k = _exact_inputs(rng, B, T, H, D, N)
    qc, qs = _mx(q)
    kc, ks = _mx(k)
    q_pos = np.array([[4 * N + 3, 4 * 300 + 3, 4 * 300 + 2], [2, 4 * N, 4 * 500 + 7]], np.int64)
    ne = np.array([N, N - 5], np.int32)
    sc = torch.empty(B, T, N, dtype=torch.bfloat16, device=dev())
    L.indexer_score(up(qc), up(w), up(kc), up(ne), up(q_pos), 4, sc, q_scales=up(qs), k_scales=up(ks))
    idx = torch.empty(B, T, K, dtype=torch.int32, device=dev())
    L.topk_select(sc, up(ne), up(q_pos), 4, K, idx)
    got, gi = down(sc), down(idx)
    for b in range(B):
        ref = O.indexer_scores(q[b], w[b], k[b], O.n_visible(q_pos[b], ne[b], 4), True)
        assert np.array_equal(got[b], ref)
        for t in range(T):
            assert np.array_equal(gi[b, t], O.topk_select(ref[t], K))


def test_indexer_mxfp4_random_within_one_bf16_ulp():
    from long_context_compressed_compress_amd import libcsa as L
    rng = np.random.default_rng(23)
    B, T, H, D, N = 2, 4, 64, 64, 5000
    qf = rng.standard_normal((B, T, H, D)).astype(np.float32)
    kf = rng.standard_normal((B, N, D)).astype(np.float32)
    w = rng.random((B, T, H)).astype(np.float32)
    w[1, 0] -= 0.5                                   # signed head weights are allowed
    qc, qs = _mx(qf)
    kc, ks = _mx(kf)
    q_pos = np.array([[4 * N - 1, 4 * N + 10, 4 * 1234 + 2, 10], [4 * N - 1, 4 * 2000 + 3, 77, 4 * N - 1]], np.int64)
    ne = np.array([N, N], np.int32)
    sc = torch.empty(B, T, N, dtype=torch.bfloat16, device=dev())
    L.indexer_score(up(qc), up(w), up(kc), up(ne), up(q_pos), 4, sc, q_scales=up(qs), k_scales=up(ks))
    got = down(sc)
    exact = 0
    for b in range(B):
        ref = O.indexer_scores(O.mxfp4_dequantize(qc[b], qs[b]), w[b], O.mxfp4_dequantize(kc[b], ks[b]),
                               O.n_visible(q_pos[b], ne[b], 4), True)
        fin = np.isfinite(ref)
        assert (np.isfinite(got[b]) == fin).all()
        err = np.abs(got[b][fin] - ref[fin])
        assert (err <= bf16_ulp(ref[fin]) + 1e-30).all()
        exact += int((err == 0).sum())
    print(f"MXFP4 scores equal to BF16(oracle): {exact} of {int(np.isfinite(got).sum())}")


def test_indexer_float32_query_quantized_inside_the_call():
    """q given as float32 with MXFP4 keys: the call quantizes q itself.  Parity:
    every score within one BF16 ulp of BF16(oracle on the oracle's MXFP4 of q);
    consistency: bit-identical to mxfp4_quantize followed by the MXFP4 call."""
    from long_context_compressed_compress_amd import libcsa as L
    rng = np.random.default_rng(29)
    B, T, H, D, N = 2, 3, 64, 64, 3000
    qf = rng.standard_normal((B, T, H, D)).astype(np.float32)
    qf[0, 0, 5] *= 1e-30                                  # tiny block scales
    qf[1, 2, 7] = 0.0                                     # an all-zero head (scale -127)
    qf[0, 1, 9, :32] = 7.0                                # saturating codes
    kf = rng.standard_normal((B, N, D)).astype(np.float32)
    w = rng.random((B, T, H)).astype(np.float32)
    kc, ks = _mx(kf)
    q_pos = np.array([[4 * N - 1, 4 * 1000 + 1, 4 * N + 7], [4 * N - 1, 6, 4 * 2500]], np.int64)
    ne = np.array([N, N - 100], np.int32)
    fused = torch.empty(B, T, N, dtype=torch.bfloat16, device=dev())
    L.indexer_score(up(qf), up(w), up(kc), up(ne), up(q_pos), 4, fused, k_scales=up(ks))
    qc_g = torch.empty(B, T, H, D // 2, dtype=torch.uint8, device=dev())
    qs_g = torch.empty(B, T, H, D // 32, dtype=torch.uint8, device=dev())
    L.mxfp4_quantize(up(qf), qc_g, qs_g)
    two = torch.empty_like(fused)
    L.indexer_score(qc_g, up(w), up(kc), up(ne), up(q_pos), 4, two, q_scales=qs_g, k_scales=up(ks))
    assert torch.equal(fused.view(torch.int16), two.view(torch.int16))
    got = down(fused)
    qc, qs = _mx(qf)
    for b in range(B):
        ref = O.indexer_scores(O.mxfp4_dequantize(qc[b], qs[b]), w[b], O.mxfp4_dequantize(kc[b], ks[b]),
                               O.n_visible(q_pos[b], ne[b], 4), True)
        fin = np.isfinite(ref)
        assert (np.isfinite(got[b]) == fin).all()
        assert (np.abs(got[b][fin] - ref[fin]) <= bf16_ulp(ref[fin]) + 1e-30).all()


def _topk_check(scores_np, dtype, n_entries, q_pos, k, ratio=4):
    from long_context_compressed_compress_amd import libcsa as L
    B, T, N = scores_np.shape
    st = up(scores_np.astype(np.float32), dtype if dtype == torch.float32 else None)
    if dtype == torch.bfloat16:
        st = st.to(torch.bfloat16)
    vals = st.float().cpu().numpy().astype(np.float64) if dtype == torch.bfloat16 else scores_np.astype(np.float64)
    idx = torch.full((B, T, k), 12345, dtype=torch.int32, device=dev())
    L.topk_select(st, up(n_entries), up(q_pos), ratio, k, idx)
    gi = down(idx)
    for b in range(B):
        nv = O.n_visible(q_pos[b], n_entries[b], ratio)
        for t in range(T):
            row = vals[b, t].copy()
            row[int(nv[t]):] = -np.inf
            want = O.topk_select(row, k)
            assert np.array_equal(gi[b, t], want), (b, t)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_topk_ties_inf_and_short_rows(dtype):
    rng = np.random.default_rng(24)
    B, T, N = 3, 6, 3000
    s = np.round(rng.standard_normal((B, T, N)), 1)        # heavy ties
    s[0, 0, ::7] = -np.inf                                  # -inf never chosen
    s[0, 1] = 0.0
    s[0, 1, 100:200] = -0.0                                 # -0 ties with +0
    s[1, 2, :] = 5.0                                        # all equal: lowest indices
    s[2, 3, 50:60] = 1e30 if dtype == torch.float32 else 3e38
    q_pos = np.tile(np.array([4 * N - 1, 4 * N - 1, 4 * 40 + 3, 3, 2, 4 * 2000]), (B, 1)).astype(np.int64)
    ne = np.array([N, N - 1000, N], np.int32)
    for k in (1, 37, 512, 2999, 3500):
        _topk_check(s, dtype, ne, q_pos, k)


@pytest.mark.parametrize("n_cap", [1, 5, 15, 16, 17, 31, 4097])
def test_topk_capacities_around_the_16_key_piece(n_cap):
    """Row capacities below, at and just above the 16 keys of a thread's
    piece (and one past a 4,096-key round): short rows read element by
    element, the straddling piece too; bit-exact against the oracle."""
    rng = np.random.default_rng(25 + n_cap)
    B, T = 2, 3
    s = np.round(rng.standard_normal((B, T, n_cap)), 1)
    q_pos = np.tile(np.array([4 * n_cap - 1, 4 * (n_cap // 2) + 3, 2]), (B, 1)).astype(np.int64)
    ne = np.array([n_cap, max(n_cap - 1, 0)], np.int32)
    for k in sorted({1, 3, n_cap, n_cap + 2}):
        _topk_check(s, torch.bfloat16, ne, q_pos, k)


def test_topk_split_path_edges():
    """Few long BF16 rows go through the multi-work-group path: ties, -inf, -0,
    short visibility, k above the visible count, nothing visible; and the same
    workspace reused across calls of different shapes."""
    rng = np.random.default_rng(28)
    B, T, N = 3, 2, 40000
    s = np.round(rng.standard_normal((B, T, N)) * 3, 0).astype(np.float32)   # ~20 distinct values
    s[0, 0, ::3] = -np.inf
    s[0, 1, 5000:9000] = 7.0
    s[1, 0, 1000:] = -0.0
    s[1, 0, :1000] = 0.0
    q_pos = np.array([[4 * N - 1, 4 * N - 1], [4 * N - 1, 4 * 700 + 1], [2, 4 * 30000 + 3]], np.int64)
    ne = np.array([N, N, N - 77], np.int32)
    for k in (1, 512, 1024, 1500, 5000):
        _topk_check(s, torch.bfloat16, ne, q_pos, k)
    from long_context_compressed_compress_amd import libcsa as L
    ws = torch.zeros(L.topk_workspace_size(8, 1, 262144, 1024, L.CSA_BF16), dtype=torch.uint8, device=dev())
    assert ws.numel() > 0
    for n_cap, k in ((262144, 1024), (50001, 64), (262144, 1024)):     # 50001: rows not 16-byte aligned
        sc = up((rng.standard_normal((2, 1, n_cap)) * 20).astype(np.float32)).to(torch.bfloat16)
        qp = np.full((2, 1), 4 * n_cap, np.int64)
        nn = np.array([n_cap, n_cap // 2], np.int32)
        idx = torch.empty(2, 1, k, dtype=torch.int32, device=dev())
        L.topk_select(sc, up(nn), up(qp), 4, k, idx, workspace=ws)
        vals = sc.float().cpu().numpy().astype(np.float64)
        gi = down(idx)
        for b in range(2):
            row = vals[b, 0].copy()
            row[int(nn[b]):] = -np.inf
            assert np.array_equal(gi[b, 0], O.topk_select(row, k))


def test_topk_split_path_rows_per_xcd():
    """The split path's passes 2-3 place row r's chunks on XCD r mod 8: 21 rows
    give XCDs two or three rows each (and padding work-groups on the XCDs with
    two); every row bit-exact, with its own visible count."""
    rng = np.random.default_rng(33)
    B, T, N = 7, 3, 20000
    s = np.round(rng.standard_normal((B, T, N)) * 5, 0).astype(np.float32)   # heavy ties
    s[2, 1, ::4] = -np.inf
    q_pos = (4 * N - 1 - 4 * 137 * np.arange(B * T, dtype=np.int64)).reshape(B, T)
    ne = np.full(B, N, np.int32)
    ne[5] = N - 3001
    for k in (256, 2048):
        _topk_check(s, torch.bfloat16, ne, q_pos, k)


def test_topk_prefill_shape_bit_exact():
    """4096 queries x 16384 BF16 scores, k = 512, causal visibility (chunked prefill)."""
    rng = np.random.default_rng(25)
    T, N, k = 4096, 16384, 512
    s = (rng.standard_normal((1, T, N)) * 30 + 100).astype(np.float32)
    q_pos = np.arange(61440, 65536, dtype=np.int64)[None]
    ne = np.array([N], np.int32)
    from long_context_compressed_compress_amd import libcsa as L
    st = up(s).to(torch.bfloat16)
    vals = st.float().cpu().numpy().astype(np.float64)
    idx = torch.empty(1, T, k, dtype=torch.int32, device=dev())
    L.topk_select(st, up(ne), up(q_pos), 4, k, idx)
    gi = down(idx)
    nv = O.n_visible(q_pos[0], N, 4)
    for t in list(range(0, T, 97)) + [T - 1]:
        row = vals[0, t].copy()
        row[int(nv[t]):] = -np.inf
        assert np.array_equal(gi[0, t], O.topk_select(row, k)), t


def test_topk_decode_shape_bit_exact():
    """8 sequences x 262144 BF16 scores, k = 1024 (decode at 1M context)."""
    rng = np.random.default_rng(26)
    B, N, k = 8, 262144, 1024
    s = (rng.standard_normal((B, 1, N)) * 40 + 100).astype(np.float32)
    q_pos = np.full((B, 1), 4 * N - 1, np.int64)
    ne = np.array([N] * B, np.int32)
    from long_context_compressed_compress_amd import libcsa as L
    st = up(s).to(torch.bfloat16)
    vals = st.float().cpu().numpy().astype(np.float64)
    idx = torch.empty(B, 1, k, dtype=torch.int32, device=dev())
    L.topk_select(st, up(ne), up(q_pos), 4, k, idx)
    gi = down(idx)
    for b in range(B):
        assert np.array_equal(gi[b, 0], O.topk_select(vals[b, 0], k)), b


def test_topk_of_gpu_mxfp4_scores_vs_oracle_scores():
    """The chain indexer -> top-k on the GPU against the oracle's own chain: the
    unique part of the selection agrees (entries clearly above/below the k-th
    score), and recall against the FP32 indexer's selection is reported."""
    from long_context_compressed_compress_amd import libcsa as L
    rng = np.random.default_rng(27)
    B, H, D, N, k = 2, 64, 64, 20000, 512
    qf = rng.standard_normal((B, 1, H, D)).astype(np.float32)
    kf = rng.standard_normal((B, N, D)).astype(np.float32)
    w = rng.random((B, 1, H)).astype(np.float32)
    qc, qs = _mx(qf)
    kc, ks = _mx(kf)
    q_pos = np.full((B, 1), 4 * N - 1, np.int64)
    ne = np.array([N, N], np.int32)
    sc = torch.empty(B, 1, N, dtype=torch.bfloat16, device=dev())
    L.indexer_score(up(qc), up(w), up(kc), up(ne), up(q_pos), 4, sc, q_scales=up(qs), k_scales=up(ks))
    idx = torch.empty(B, 1, k, dtype=torch.int32, device=dev())
    L.topk_select(sc, up(ne), up(q_pos), 4, k, idx)
    gi = down(idx)
    recalls = []
    for b in range(B):
        ref = O.indexer_scores(O.mxfp4_dequantize(qc[b], qs[b]), w[b], O.mxfp4_dequantize(kc[b], ks[b]), [N], True)
        topk_unique_part_ok(gi[b, 0], ref[0], k)
        fp32_sel = O.topk_select(O.indexer_scores(qf[b], w[b], kf[b], [N], False)[0], k)
        recalls.append(np.isin(fp32_sel, gi[b, 0]).mean())
    print(f"recall@{k} of the MXFP4 indexer vs the unquantised indexer: {np.round(recalls, 4).tolist()}")


def _random_mx_keys(rng, B, N, D):
    """Random MXFP4 keys: any code byte, block scales 2^-4 .. 2^3."""
    kc = rng.integers(0, 256, (B, N, D // 2), dtype=np.uint8)
    ks = rng.integers(123, 131, (B, N, D // 32), dtype=np.uint8)
    return kc, ks


def test_indexer_topk_equals_the_two_calls():
    """indexer_topk gives the scores of indexer_score and the selection of
    topk_select on those scores, bit for bit, at decode shape (few long rows,
    where the indexer also builds top-k's first histogram) and at a prefill
    shape; one workspace serves every call, so the zero-at-rest contract is
    exercised across both top-k paths and both callers.  The selection is also
    checked to be the top-k of the returned scores by definition."""
    from long_context_compressed_compress_amd import libcsa as L
    rng = np.random.default_rng(30)
    H, D = 64, 64
    ws = torch.zeros(L.topk_workspace_size(8, 1, 262144, 1024, L.CSA_BF16), dtype=torch.uint8, device=dev())
    cases = [
        # (B, T, N, k, q_pos, n_entries, q as float32)
        (8, 1, 262144, 1024, [4 * 262144 - 1] * 7 + [4 * 100000 + 2], [262144] * 7 + [200000], True),
        (3, 1, 40000, 512, [4 * 40000 - 1, 4 * 300 + 3, 2], [40000, 40000, 40000], False),  # short + empty rows
        (1, 64, 5000, 256, list(range(4 * 5000 - 64, 4 * 5000)), [5000], True),          # per-row path
        (2, 1, 50001, 64, [4 * 50001, 4 * 50001], [50001, 25000], False),                 # ragged n_cap
        (8, 1, 262144, 1024, [4 * 262144 - 1] * 8, [262144] * 8, True),
    ]
    for B, T, N, k, qp, ne, qf32 in cases:
        print(f"indexer_topk case B={B} T={T} N={N} k={k} q_f32={qf32}", flush=True)
        kc, ks = _random_mx_keys(rng, B, N, D)
        qf = rng.standard_normal((B, T, H, D)).astype(np.float32)
        w = rng.random((B, T, H)).astype(np.float32)
        q_pos = np.array(qp, np.int64).reshape(B, T)
        ne = np.array(ne, np.int32)
        kc_g, ks_g, w_g, ne_g, qp_g = up(kc), up(ks), up(w), up(ne), up(q_pos)
        if qf32:
            qa, qsa = up(qf), None
        else:
            qc, qs = _mx(qf)
            qa, qsa = up(qc), up(qs)
        s1 = torch.empty(B, T, N, dtype=torch.bfloat16, device=dev())
        i1 = torch.full((B, T, k), 7777, dtype=torch.int32, device=dev())
        ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        L.indexer_topk(qa, w_g, kc_g, ne_g, qp_g, 4, s1, k, i1, q_scales=qsa, k_scales=ks_g, workspace=ws,
                       stage_events=ev if qf32 else None)
        if qf32:
            torch.cuda.synchronize()
            assert ev[0].elapsed_time(ev[1]) > 0.0    # the events bracket the scoring kernel
        s2 = torch.empty_like(s1)
        i2 = torch.full_like(i1, 8888)
        L.indexer_score(qa, w_g, kc_g, ne_g, qp_g, 4, s2, q_scales=qsa, k_scales=ks_g)
        L.topk_select(s2, ne_g, qp_g, 4, k, i2, workspace=ws)
        assert torch.equal(s1.view(torch.int16), s2.view(torch.int16))
        assert torch.equal(i1, i2)
        vals = s1.float().cpu().numpy().astype(np.float64)
        gi = down(i1)
        for b in range(B):
            nv = O.n_visible(q_pos[b], ne[b], 4)
            for t in sorted({0, T - 1}):
                row = vals[b, t].copy()
                row[int(nv[t]):] = -np.inf
                assert_is_topk_of(gi[b, t], row, k, f"B={B} T={T} N={N} b={b} t={t}")
    # the zero-at-rest part is zero again: of the split path's per-row totals
    # (128 rows x 512 words at the start of the workspace) the first-pass half,
    # which calls accumulate into (the second half is cleared inside each call)
    assert not ws[:128 * 512 * 4].view(torch.int32).view(128, 512)[:, :256].any()


def test_topk_split_path_several_rounds():
    """Rows longer than 2^20 entries: each work-group of the split path takes
    several 4096-key rounds (the per-round counts, ties carried across rounds
    and chunks).  Heavy ties, -inf, a short visible prefix; bit-exact."""
    from long_context_compressed_compress_amd import libcsa as L
    rng = np.random.default_rng(31)
    n_cap = 1_500_000
    s = np.round(rng.standard_normal((2, 1, n_cap)) * 4, 0).astype(np.float32)   # ~30 distinct values
    s[0, 0, ::5] = -np.inf
    s[1, 0, 700_000:] = 9.0                                                      # ties past the visible end
    q_pos = np.array([[4 * n_cap + 3], [4 * 1_000_003 + 1]], np.int64)
    ne = np.array([n_cap, n_cap], np.int32)
    sc = up(s).to(torch.bfloat16)
    vals = sc.float().cpu().numpy().astype(np.float64)
    ws = torch.zeros(L.topk_workspace_size(2, 1, n_cap, 2048, L.CSA_BF16), dtype=torch.uint8, device=dev())
    for k in (1024, 2048):
        print(f"top-k split path, several rounds: n_cap={n_cap} k={k}", flush=True)
        idx = torch.empty(2, 1, k, dtype=torch.int32, device=dev())
        L.topk_select(sc, up(ne), up(q_pos), 4, k, idx, workspace=ws)
        gi = down(idx)
        for b in range(2):
            nv = int(O.n_visible(q_pos[b, 0], ne[b], 4))
            row = vals[b, 0].copy()
            row[nv:] = -np.inf
            assert np.array_equal(gi[b, 0], O.topk_select(row, k)), (b, k)


def test_indexer_topk_batch_invariance():
    """Scores and selections of a sequence do not depend on the batch it runs
    in: the decode shape (MXFP4 keys, float32 query quantized in the call, the
    indexer building top-k's first pass) over 8 sequences, and each sequence
    alone, give the same bits; so does a prefill-shaped call of 64 query rows
    against the same rows taken 4 and 1 at a time.  Run twice: the same bits."""
    from long_context_compressed_compress_amd import libcsa as L
    rng = np.random.default_rng(32)
    H, D, B, N, k = 64, 64, 8, 262144, 1024
    kc, ks = _random_mx_keys(rng, B, N, D)
    qf = rng.standard_normal((B, 1, H, D)).astype(np.float32)
    w = rng.random((B, 1, H)).astype(np.float32)
    q_pos = np.array([4 * N - 1] * 5 + [4 * 1000 + 3, 4 * 200000 + 1, 2], np.int64).reshape(B, 1)
    ne = np.array([N] * 8, np.int32)
    ws = torch.zeros(L.topk_workspace_size(B, 1, N, k, L.CSA_BF16), dtype=torch.uint8, device=dev())
    kc_g, ks_g, q_g, w_g, ne_g, qp_g = up(kc), up(ks), up(qf), up(w), up(ne), up(q_pos)

    def run(sl):
        s = torch.empty(sl.stop - sl.start, 1, N, dtype=torch.bfloat16, device=dev())
        i = torch.empty(sl.stop - sl.start, 1, k, dtype=torch.int32, device=dev())
        L.indexer_topk(q_g[sl].contiguous(), w_g[sl].contiguous(), kc_g[sl].contiguous(), ne_g[sl].contiguous(),
                       qp_g[sl].contiguous(), 4, s, k, i, k_scales=ks_g[sl].contiguous(), workspace=ws)
        return s, i

    s_all, i_all = run(slice(0, B))
    s_again, i_again = run(slice(0, B))
    assert torch.equal(s_all.view(torch.int16), s_again.view(torch.int16)) and torch.equal(i_all, i_again)
    for b in range(B):
        print(f"indexer_topk batch invariance: sequence {b} alone", flush=True)
        s1, i1 = run(slice(b, b + 1))
        assert torch.equal(s1.view(torch.int16), s_all[b:b + 1].view(torch.int16)), b
        assert torch.equal(i1, i_all[b:b + 1]), b

    # prefill shape: 64 query rows of one sequence, whole and in groups
    T, N2, k2 = 64, 16384, 512
    kc2, ks2 = _random_mx_keys(rng, 1, N2, D)
    q2 = rng.standard_normal((1, T, H, D)).astype(np.float32)
    w2 = rng.random((1, T, H)).astype(np.float32)
    qp2 = (4 * N2 - T + np.arange(T, dtype=np.int64))[None]
    ne2 = up(np.array([N2], np.int32))
    kc2_g, ks2_g = up(kc2), up(ks2)

    def run2(lo, hi):
        s = torch.empty(1, hi - lo, N2, dtype=torch.bfloat16, device=dev())
        i = torch.empty(1, hi - lo, k2, dtype=torch.int32, device=dev())
        L.indexer_topk(up(q2[:, lo:hi]), up(w2[:, lo:hi]), kc2_g, ne2, up(qp2[:, lo:hi]), 4, s, k2, i,
                       k_scales=ks2_g, workspace=ws)
        return s, i

    s_all, i_all = run2(0, T)
    for g in (4, 1):
        for lo in range(0, T, 16):
            s1, i1 = run2(lo, lo + g)
            assert torch.equal(s1.view(torch.int16), s_all[:, lo:lo + g].view(torch.int16)), (g, lo)
            assert torch.equal(i1, i_all[:, lo:lo + g]), (g, lo)
