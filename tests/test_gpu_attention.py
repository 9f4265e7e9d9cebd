"""GPU parity of sparse_window_attn (CSA) and hca_dense_attn (HCA).

FP32 path (float32 rows and queries): max|err| <= 1e-5 * ||ref||_inf.
Matrix-core path (BF16 queries, FP8/BF16 mixed rows): max|err| <= 2e-3 *
||ref||_inf, plus half a BF16 ulp of the reference for BF16 outputs.
Also: k >= visible entries equals dense attention (GPU vs GPU), the sink,
lse, -1 padding, early positions, window-only, ring wrap, determinism and batch
invariance (bitwise), causality (bitwise)."""
import numpy as np
import pytest
import torch

from oracle import csa_oracle as O
from tests.gpu_util import SCALE, assert_attn_close, assert_f32_close, bf16_tensor, dev, down, up

pytestmark = pytest.mark.gpu


def _mixed(x_f32):
    """Stored mixed rows of float32 data, packed by the GPU kernel (its bit-exactness
    with the oracle's encoder is tested separately) and the oracle's decoded values."""
    from long_context_compressed_compress_amd import libcsa as L
    flat = np.ascontiguousarray(x_f32.reshape(-1, 192))
    out = torch.empty(flat.shape[0], 256, dtype=torch.uint8, device=dev())
    L.kv_pack(up(flat), out)
    return out.view(*x_f32.shape[:-1], 256), O.kv_round(x_f32)


def _sparse_ref(q, ent, idx, ne, win_vals, win_pos0, q_pos, W, sink=None, ratio=4):
    B, T = q.shape[:2]
    out = np.zeros(q.shape)
    lse = np.zeros(q.shape[:3])
    for b in range(B):
        for t in range(T):
            nv = int(O.n_visible(q_pos[b, t], ne[b], ratio))
            out[b, t], lse[b, t] = O.sparse_window_attn(q[b, t], ent[b], idx[b, t], nv, win_vals[b], win_pos0,
                                                        int(q_pos[b, t]), W, SCALE, sink)
    return out, lse


def _dense_ref(q, ent, ne, win_vals, win_pos0, q_pos, W, sink=None, ratio=128):
    B, T = q.shape[:2]
    out = np.zeros(q.shape)
    lse = np.zeros(q.shape[:3])
    for b in range(B):
        for t in range(T):
            nv = int(O.n_visible(q_pos[b, t], ne[b], ratio))
            out[b, t], lse[b, t] = O.hca_dense_attn(q[b, t], ent[b], nv, win_vals[b], win_pos0, int(q_pos[b, t]), W,
                                                    SCALE, sink)
    return out, lse


def test_fp32_path_sparse_and_dense_with_sink_and_lse():
    from long_context_compressed_compress_amd import libcsa as L
    rng = np.random.default_rng(30)
    B, T, H, N, K, W = 2, 16, 8, 1024, 64, 128
    q = rng.standard_normal((B, T, H, 192)).astype(np.float32)
    ent = rng.standard_normal((B, N, 192)).astype(np.float32)
    tok = rng.standard_normal((B, 4096, 192)).astype(np.float32)
    q_pos = np.stack([np.arange(4080, 4096), np.r_[np.arange(0, 8), np.arange(4000, 4008)]]).astype(np.int64)
    ne = np.array([N, 700], np.int32)
    idx = np.stack([[np.sort(rng.choice(N, K, replace=False)) for _ in range(T)] for _ in range(B)]).astype(np.int32)
    idx[0, 0, -5:] = -1
    idx[1, 3, :10] = 1023                                # beyond n_entries of sequence 1: skipped
    sink = rng.standard_normal(H).astype(np.float32)
    for s_ in (None, sink):
        out = torch.empty(B, T, H, 192, dtype=torch.float32, device=dev())
        lse = torch.empty(B, T, H, dtype=torch.float32, device=dev())
        L.sparse_window_attn(up(q), up(ent), up(ne), 4, up(idx), up(tok), 0, up(q_pos), W, SCALE, out,
                             sink=None if s_ is None else up(s_), lse=lse)
        ref, rlse = _sparse_ref(q, ent, idx, ne, tok, 0, q_pos, W, s_)
        assert_f32_close(down(out), ref, 1e-5, "fp32 sparse")
        assert np.abs(down(lse) - rlse).max() <= 1e-5 * np.abs(rlse).max()
        out2 = torch.empty(B, T, H, 192, dtype=torch.float32, device=dev())
        L.hca_dense_attn(up(q), up(ent[:, :40].copy()), up(np.array([40, 20], np.int32)), 128, up(tok), 0,
                         up(q_pos), W, SCALE, out2, sink=None if s_ is None else up(s_))
        ref2, _ = _dense_ref(q, ent[:, :40], np.array([40, 20]), tok, 0, q_pos, W, s_)
        assert_f32_close(down(out2), ref2, 1e-5, "fp32 dense")


@pytest.mark.parametrize("H,B,T,K,out_dtype", [(64, 1, 7, 512, torch.bfloat16), (128, 2, 1, 1024, torch.bfloat16),
                                                 (128, 3, 2, 100, torch.float32), (32, 2, 3, 64, torch.float32),
                                                 (96, 1, 1, 0, torch.float32)])
def test_mfma_sparse(H, B, T, K, out_dtype):
    from long_context_compressed_compress_amd import libcsa as L
    rng = np.random.default_rng(31 + H + K)
    N, W, P = 3000, 128, 13000
    qf = rng.standard_normal((B, T, H, 192)).astype(np.float32)
    qb = bf16_tensor(qf)
    qv = qb.double().cpu().numpy()
    entm, entv = _mixed(rng.standard_normal((B, N, 192)).astype(np.float32))
    winm, winv = _mixed(rng.standard_normal((B, P, 192)).astype(np.float32))
    q_pos = rng.integers(4 * N - 200, P, (B, T)).astype(np.int64)
    q_pos[0, 0] = 57                                      # early: partial window, few entries
    ne = np.array([N - 13 * b for b in range(B)], np.int32)
    idx = np.stack([[np.sort(rng.choice(N, K, replace=False)) for _ in range(T)] for _ in range(B)])
    idx = idx.reshape(B, T, K).astype(np.int32)
    if K:
        idx[0, 0, :3] = -1
    out = torch.empty(B, T, H, 192, dtype=out_dtype, device=dev())
    lse = torch.empty(B, T, H, dtype=torch.float32, device=dev())
    L.sparse_window_attn(qb, entm, up(ne), 4, up(idx), winm, 0, up(q_pos), W, SCALE, out, lse=lse)
    ref, rlse = _sparse_ref(qv, entv, idx, ne, winv, 0, q_pos, W)
    assert_attn_close(down(out), ref, out_dtype == torch.bfloat16, f"sparse H={H} K={K}")
    assert np.abs(down(lse) - rlse).max() <= 2e-3 * np.abs(rlse).max()


@pytest.mark.parametrize("H,B,n_cap,out_dtype", [(128, 4, 8192, torch.bfloat16), (64, 2, 1000, torch.float32)])
def test_mfma_dense_decode(H, B, n_cap, out_dtype):
    from long_context_compressed_compress_amd import libcsa as L
    rng = np.random.default_rng(32 + H)
    W = 128
    t = 128 * n_cap + 300
    qb = bf16_tensor(rng.standard_normal((B, 1, H, 192)).astype(np.float32))
    entm, entv = _mixed(rng.standard_normal((B, n_cap, 192)).astype(np.float32))
    # window ring of 128 rows: position p in row p % 128
    tokf = rng.standard_normal((B, W, 192)).astype(np.float32)      # positions t-127 .. t
    pos = np.arange(t - W + 1, t + 1)
    ring_f = np.empty_like(tokf)
    ring_f[:, pos % W] = tokf
    ringm, _ = _mixed(ring_f)
    tokv = O.kv_round(tokf)
    q_pos = np.full((B, 1), t, np.int64)
    ne = np.array([n_cap] * B, np.int32)
    sink = np.linspace(-1, 2, H).astype(np.float32)
    out = torch.empty(B, 1, H, 192, dtype=out_dtype, device=dev())
    L.hca_dense_attn(qb, entm, up(ne), 128, ringm, 0, up(q_pos), W, SCALE, out, sink=up(sink))
    ref, _ = _dense_ref(qb.double().cpu().numpy(), entv, ne, tokv, t - W + 1, q_pos, W, sink)
    assert_attn_close(down(out), ref, out_dtype == torch.bfloat16, "dense decode")


def test_topk_covering_everything_equals_dense_on_gpu():
    """k >= visible entries: the CSA kernel over every entry equals the HCA kernel
    over the same entries (both on the GPU, same storage).  With the same key
    list (selection = 0..n_vis-1) the two are bitwise equal; with -1 padding in
    the selection the blocking of the list shifts, and they agree to the
    attention tolerance."""
    from long_context_compressed_compress_amd import libcsa as L
    rng = np.random.default_rng(33)
    B, T, H, N = 2, 3, 128, 600
    qb = bf16_tensor(rng.standard_normal((B, T, H, 192)).astype(np.float32))
    entm, _ = _mixed(rng.standard_normal((B, N, 192)).astype(np.float32))
    winm, _ = _mixed(rng.standard_normal((B, 4000, 192)).astype(np.float32))
    q_pos = np.array([[2400, 3000, 3999], [2398, 2600, 3001]], np.int64)
    ne = np.array([N, N], np.int32)
    o2 = torch.empty(B, T, H, 192, dtype=torch.float32, device=dev())
    L.hca_dense_attn(qb, entm, up(ne), 4, winm, 0, up(q_pos), 128, SCALE, o2)
    dense = down(o2)
    o1 = torch.empty_like(o2)
    idx = np.tile(np.arange(N, dtype=np.int32), (B, T, 1))
    idx[1, 0, 599] = -1                                   # query at 2398 sees 599 entries only
    L.sparse_window_attn(qb, entm, up(ne), 4, up(idx), winm, 0, up(q_pos), 128, SCALE, o1)
    same = down(o1)
    assert np.array_equal(same[0], dense[0])
    assert np.array_equal(same[1, 1:], dense[1, 1:])
    assert_attn_close(same[1, 0], dense[1, 0], False, "trailing -1")
    idx_pad = np.concatenate([idx, np.full((B, T, 24), -1, np.int32)], axis=2)
    L.sparse_window_attn(qb, entm, up(ne), 4, up(idx_pad), winm, 0, up(q_pos), 128, SCALE, o1)
    assert_attn_close(down(o1), dense, False, "padded selection")


def test_determinism_batch_invariance_and_causality():
    from long_context_compressed_compress_amd import libcsa as L
    rng = np.random.default_rng(34)
    B, H, N, K = 8, 128, 20000, 1024
    t = 4 * N - 1
    qb = bf16_tensor(rng.standard_normal((B, 1, H, 192)).astype(np.float32))
    entm, _ = _mixed(rng.standard_normal((B, N + 64, 192)).astype(np.float32))
    winm, _ = _mixed(rng.standard_normal((B, 128, 192)).astype(np.float32))
    idx = np.stack([np.sort(rng.choice(N, K, replace=False)) for _ in range(B)])[:, None].astype(np.int32)
    q_pos = np.full((B, 1), t, np.int64)
    ne = np.array([N] * B, np.int32)

    def run(qq, ee, ii, ww, pp, nn):
        o = torch.empty(qq.shape[0], 1, H, 192, dtype=torch.bfloat16, device=dev())
        L.sparse_window_attn(qq, ee, up(nn), 4, up(ii), ww, 0, up(pp), 128, SCALE, o)
        return down(o)

    full = run(qb, entm, idx, winm, q_pos, ne)
    assert np.array_equal(full, run(qb, entm, idx, winm, q_pos, ne))                     # run twice
    one = run(qb[3:4].contiguous(), entm[3:4].contiguous(), idx[3:4], winm[3:4].contiguous(), q_pos[3:4], ne[3:4])
    assert np.array_equal(full[3:4], one)                                                 # alone vs in a batch
    # entries past n_vis (not yet complete) and index values past them change nothing
    ent2 = entm.clone()
    ent2[:, N:] = 0x7E
    idx2 = idx.copy()
    idx2[:, 0, :8] = N + np.arange(8)
    assert np.array_equal(np.sort(idx2[:, 0, 8:], axis=1), idx2[:, 0, 8:])
    a = run(qb, ent2, idx2, winm, q_pos, ne)
    b = run(qb, entm, np.concatenate([np.full((B, 1, 8), -1, np.int32), idx[:, :, 8:]], axis=2), winm, q_pos, ne)
    assert np.array_equal(a, b)
    # HCA: entries not yet visible to the query do not matter
    o1 = torch.empty(B, 1, H, 192, dtype=torch.bfloat16, device=dev())
    o2 = torch.empty_like(o1)
    tq = np.full((B, 1), 128 * 100 + 5, np.int64)                 # 100 HCA entries visible
    L.hca_dense_attn(qb, entm, up(np.array([N] * B, np.int32)), 128, winm, 0, up(tq), 128, SCALE, o1)
    L.hca_dense_attn(qb, ent2, up(np.array([N] * B, np.int32)), 128, winm, 0, up(tq), 128, SCALE, o2)
    ent3 = entm.clone()
    ent3[:, 100:] = 0x55
    o3 = torch.empty_like(o1)
    L.hca_dense_attn(qb, ent3, up(np.array([N] * B, np.int32)), 128, winm, 0, up(tq), 128, SCALE, o3)
    assert torch.equal(o1, o2) and torch.equal(o1, o3)


def test_window_only_and_empty_key_sets():
    from long_context_compressed_compress_amd import libcsa as L
    rng = np.random.default_rng(35)
    B, H = 2, 64
    qb = bf16_tensor(rng.standard_normal((B, 2, H, 192)).astype(np.float32))
    winm, winv = _mixed(rng.standard_normal((B, 300, 192)).astype(np.float32))
    entm, entv = _mixed(rng.standard_normal((B, 8, 192)).astype(np.float32))
    q_pos = np.array([[0, 299], [5, 130]], np.int64)
    ne = np.array([8, 8], np.int32)
    out = torch.empty(B, 2, H, 192, dtype=torch.float32, device=dev())
    L.sparse_window_attn(qb, entm, up(ne), 4, up(np.zeros((B, 2, 0), np.int32)), winm, 0, up(q_pos), 128, SCALE, out)
    ref, _ = _sparse_ref(qb.double().cpu().numpy(), entv, np.zeros((B, 2, 0), np.int64), ne, winv, 0, q_pos, 128)
    assert_attn_close(down(out), ref, False, "window only")
    # no window and no visible entry: output 0, lse -inf
    lse = torch.empty(B, 2, H, dtype=torch.float32, device=dev())
    L.hca_dense_attn(qb, entm, up(ne), 128, winm, 0, up(q_pos), 0, SCALE, out, lse=lse)
    g = down(out)
    assert not g[0, 0].any() and not g[1, 0].any()
    assert np.isneginf(down(lse)[:, 0]).all()


@pytest.mark.parametrize("fp32", [False, True])
def test_swa_attn_window_only_layer(fp32):
    """swa_attn (the pure sliding-window layers) against the oracle's window-only
    attention (no entry visible): rows over a wrapped ring, rows at the start of a
    sequence (t < W), a sink and lse; and bitwise equal to hca_dense_attn over
    zero entries."""
    from long_context_compressed_compress_amd import libcsa as L
    rng = np.random.default_rng(37 + fp32)
    B, T, H, W, R = 4, 3, 8 if fp32 else 128, 128, 256     # the ring holds every query's window
    q_pos = np.array([[5, 6, 7], [127, 128, 129], [1000, 1001, 1002], [0, 1, 130]], np.int64)
    tok = rng.standard_normal((B, 1200, 192)).astype(np.float32)     # raw token KV by position
    ring = np.zeros((B, R, 192), np.float32)
    for b in range(B):
        hi = int(q_pos[b].max())
        for p in range(max(0, hi - R + 1), hi + 1):
            ring[b, p % R] = tok[b, p]
    sink = rng.standard_normal(H).astype(np.float32)
    if fp32:
        q = rng.standard_normal((B, T, H, 192)).astype(np.float32)
        qg, wing, ringv, out_dtype = up(q), up(ring), ring.astype(np.float64), torch.float32
        qv = q.astype(np.float64)
    else:
        qg = bf16_tensor(rng.standard_normal((B, T, H, 192)).astype(np.float32))
        wing, ringv = _mixed(ring)
        qv, out_dtype = qg.double().cpu().numpy(), torch.bfloat16
    out = torch.empty(B, T, H, 192, dtype=out_dtype, device=dev())
    lse = torch.empty(B, T, H, dtype=torch.float32, device=dev())
    L.swa_attn(qg, wing, 0, up(q_pos), W, SCALE, out, sink=up(sink), lse=lse)
    go, gl = down(out), down(lse)
    refs = {}
    for b in range(B):
        hi = int(q_pos[b].max())
        lo_held = max(0, hi - R + 1)
        vals = np.zeros((hi + 1, 192))
        for p in range(lo_held, hi + 1):
            vals[p] = ringv[b, p % R]
        for t in range(T):
            tq = int(q_pos[b, t])
            assert tq - W + 1 >= lo_held or tq - W + 1 < 0
            ref, ref_lse = O.hca_dense_attn(qv[b, t], np.zeros((1, 192)), 0, vals[lo_held:], lo_held, tq, W, SCALE,
                                            sink)
            refs[b, t] = ref
            if fp32:
                assert_f32_close(go[b, t], ref, 1e-5, f"swa fp32 {b},{t}")
            else:
                assert_attn_close(go[b, t], ref, True, f"swa {b},{t}")
            fin = np.isfinite(ref_lse)
            assert np.allclose(gl[b, t][fin], ref_lse[fin], rtol=1e-4, atol=1e-4)
    # the same computation through hca_dense_attn with no entries.  The float32
    # path is bitwise equal; on the matrix cores the entry capacity (1 here) adds
    # a key block to the longest list, which changes the split plan (5 blocks are
    # cut in two, 4 are not), so the two agree to the attention tolerance.
    out2 = torch.empty_like(out)
    ent = torch.zeros(B, 1, 192 if fp32 else 256, dtype=torch.float32 if fp32 else torch.uint8, device=dev())
    L.hca_dense_attn(qg, ent, up(np.zeros(B, np.int32)), 128, wing, 0, up(q_pos), W, SCALE, out2, sink=up(sink))
    if fp32:
        assert torch.equal(out, out2)
    else:
        g2 = down(out2)
        for (b, t), ref in refs.items():
            assert_attn_close(g2[b, t], ref, True, f"hca_dense_attn without entries {b},{t}")


def test_mfma_value_range_documented_clamp():
    """The matrix-core path uses the stored row exactly in the logits but as
    FP16 in P.V, so a BF16 (RoPE-dim) value beyond +-65504 acts as +-65504 in
    the output, as the header states.  With one key (a selected entry, no
    window) every head's output is that row (the oracle's single-key case):
    the GPU gives the row in every dim inside FP16's range and +-65504 in the
    dims beyond it (to float32 rounding); the float32 path gives the row itself."""
    from long_context_compressed_compress_amd import libcsa as L
    rng = np.random.default_rng(36)
    H = 64
    row = rng.standard_normal((1, 4, 192)).astype(np.float32)
    row[0, 2, 130] = 1.0e5     # BF16 99840
    row[0, 2, 177] = -3.0e5    # BF16 -299008
    row[0, 2, 150] = 60000.0   # inside FP16's range: exact (BF16 59904)
    entm, entv = _mixed(row)
    qb = bf16_tensor(rng.standard_normal((1, 1, H, 192)).astype(np.float32) * 0.01)
    q_pos = np.array([[100]], np.int64)
    ne = np.array([4], np.int32)
    idx = np.array([[[2]]], np.int32)
    ref, _ = _sparse_ref(qb.double().cpu().numpy(), entv, idx.astype(np.int64), ne, np.zeros((1, 1, 192)), 0, q_pos, 0)
    assert np.allclose(ref[0, 0], entv[0, 2][None], rtol=1e-15, atol=0)   # one key: the output is the row
    win = torch.zeros(1, 1, 256, dtype=torch.uint8, device=dev())
    out = torch.empty(1, 1, H, 192, dtype=torch.float32, device=dev())
    L.sparse_window_attn(qb, entm, up(ne), 4, up(idx), win, 0, up(q_pos), 0, SCALE, out)
    g = down(out)[0, 0]
    want = np.clip(ref[0, 0], -65504.0, 65504.0)
    tiny = np.abs(want) < 2.0 ** -14       # FP16 subnormals: quantum 2^-24, rounded toward zero
    want = np.where(tiny, np.trunc(want * 2.0 ** 24) * 2.0 ** -24, want)
    assert want[:, 130].max() == 65504.0 and want[:, 177].min() == -65504.0 and want[0, 150] == 59904.0
    # p = 1 up to the float32 rounding of the scaled logit (|logit| ~ 300 here: half an ulp is 1.5e-5 in
    # the exponent), so the row to 3e-5 relative
    assert (np.abs(g - want) <= 3e-5 * np.abs(want)).all()
    # the float32 path keeps the row's full range
    ent32 = up(entv.astype(np.float32))
    out32 = torch.empty(1, 1, H, 192, dtype=torch.float32, device=dev())
    L.sparse_window_attn(up(qb.float().cpu().numpy()), ent32, up(ne), 4, up(idx),
                         torch.zeros(1, 1, 192, dtype=torch.float32, device=dev()), 0, up(q_pos), 0, SCALE, out32)
    assert_f32_close(down(out32)[0, 0], ref[0, 0], 1e-6, "float32 path, one key")
