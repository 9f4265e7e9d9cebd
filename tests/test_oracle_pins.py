"""Pins of the fp64 oracle against facts fixed outside it: the pages' numbers
(tests/golden), closed forms, special cases that reduce to library routines
(torch casts, scaled_dot_product_attention, np.mean), invariants and brute force
on tiny inputs.  Each test is chosen so that a plausible slip in the oracle
(dropped term, wrong sign or index, transposed operand, wrong softmax axis,
wrong slot -> token mapping, off-by-one in causality or the window) fails it.
CPU only."""
import json
import math
import os

import numpy as np
import pytest
import torch
from hypothesis import given, settings
from hypothesis import strategies as st

from oracle import csa_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_facts.json")


@pytest.fixture(scope="module")
def facts():
    with open(GOLDEN) as f:
        return json.load(f)


def _rng(seed):
    return np.random.default_rng(seed)


# =============================================================================
# Entry counts (the pages' own numbers)
# =============================================================================
def test_entry_counts_match_pages(facts):
    m, mh = facts["csa_ratio"]["value"], facts["hca_ratio"]["value"]
    big = 1 << 40
    # one million tokens -> 250 thousand CSA entries, about 7800 HCA entries
    t = 10 ** 6 - 1
    assert O.n_visible(t, big, m) == facts["csa_entries_at_1e6_tokens"]["value"]
    nh = int(O.n_visible(t, big, mh))
    approx = facts["hca_entries_at_1e6_tokens_approx"]
    assert abs(nh - approx["value"]) <= approx["approx_rel"] * approx["value"]
    assert nh == 7812
    # the configs' 1M = 2**20 tokens
    assert O.n_visible((1 << 20) - 1, big, 4) == 262144
    assert O.n_visible((1 << 20) - 1, big, 128) == 8192


def test_worked_example_grouping(facts):
    ex = facts["worked_example_grouping"]
    m = facts["csa_ratio"]["value"]
    assert O.n_visible(ex["tokens"] - 1, 1 << 30, m) == ex["entries"]
    # an entry becomes visible exactly when its own last token has arrived
    for i in range(5):
        assert O.n_visible(m * i + m - 1, 1 << 30, m) == i + 1
        assert O.n_visible(m * i + m - 2, 1 << 30, m) == i
    # capped by the entries that exist
    assert O.n_visible(10 ** 6, 17, 4) == 17


def test_csa_window_covers_previous_and_current_block(facts):
    m = facts["csa_ratio"]["value"]
    assert len(O.csa_slot_tokens(5, m)) == facts["csa_window_tokens_per_entry"]["value"]
    assert list(O.csa_slot_tokens(1, m)) == list(range(0, 8))
    assert list(O.csa_slot_tokens(3, m)) == list(range(8, 16))


# =============================================================================
# Number formats
# =============================================================================
def _all_finite_f32(n, seed):
    bits = _rng(seed).integers(0, 2 ** 32, n, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    return x[np.isfinite(x)]


def test_bf16_encoder_matches_torch_cast():
    x = np.concatenate([_all_finite_f32(200000, 1),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.3895314e38, -3.4e38], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.bf16_encode(x), ref)
    # decode is exact
    assert np.array_equal(O.bf16_decode(ref), torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).double().numpy())


def test_fp8_encoder_matches_torch_cast_after_clamp():
    x = np.concatenate([_all_finite_f32(200000, 2), (_rng(3).standard_normal(50000) * 100).astype(np.float32),
                        np.array([448.0, 463.9, 464.0, 1e30, -1e30, 2 ** -10, 2 ** -9 * 1.5, 0.0], np.float32)])
    ref = torch.from_numpy(np.clip(x, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = O.fp8_encode(x)
    # torch keeps the sign of values that round to zero; so do we
    assert np.array_equal(ours, ref)
    assert np.array_equal(O.fp8_decode(ref), torch.from_numpy(ref).view(torch.float8_e4m3fn).double().numpy(),
                          equal_nan=True)


def test_fp8_table_textbook_values():
    # E4M3: 1.0 = exponent field 7, 448 = 0x7E, smallest subnormal 2^-9 = 0x01
    assert O.fp8_encode(np.array([1.0, 448.0, 2.0 ** -9, -2.0]))[:4].tolist() == [0x38, 0x7E, 0x01, 0xC0]


def test_kv_row_layout(facts):
    x = np.zeros(O.DIM)
    x[0], x[1], x[127], x[128], x[191] = 1.0, -2.0, 448.0, 1.0, -3.0
    row = O.kv_pack(x)
    assert row.shape == (facts["mixed_row_bytes"]["value"],)
    assert row[0] == 0x38 and row[1] == 0xC0 and row[127] == 0x7E
    assert row[128] == 0x80 and row[129] == 0x3F          # bf16 1.0 = 0x3F80, little-endian
    assert row[254] == 0x40 and row[255] == 0xC0          # bf16 -3.0 = 0xC040
    assert 2 * O.DIM == facts["mixed_row_bytes"]["bf16_row_bytes"]
    y = _rng(4).standard_normal((64, O.DIM)).astype(np.float32)
    dec = O.kv_unpack(O.kv_pack(y))
    t = torch.from_numpy(y)
    ref = np.concatenate([t[:, :128].to(torch.float8_e4m3fn).double().numpy(),
                          t[:, 128:].to(torch.bfloat16).double().numpy()], axis=1)
    assert np.array_equal(dec, ref)


E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_code_table():
    vals = O.e2m1_decode(np.arange(16))
    assert vals[:8].tolist() == E2M1_TABLE
    assert (vals[8:] == -np.array(E2M1_TABLE)).all() and np.signbit(vals[8])


def _e2m1_brute(v):
    """Nearest E2M1 value by exhaustive search; ties go to the code with mantissa bit 0."""
    cands = [(abs(abs(v) - g), c & 1, g) for c, g in enumerate(E2M1_TABLE)]
    if abs(v) >= 6.0:
        return math.copysign(6.0, v)
    d = min(c[0] for c in cands)
    best = sorted([c for c in cands if c[0] == d], key=lambda c: c[1])[0]
    return math.copysign(best[2], v)


def test_e2m1_rounding_brute_force():
    r = _rng(5)
    v = np.concatenate([r.uniform(-8, 8, 20000), np.arange(-32, 33) / 4.0])  # includes every midpoint
    ours = O.e2m1_round(v)
    brute = np.array([_e2m1_brute(x) for x in v])
    assert np.array_equal(ours, brute)


def test_e2m1_midpoints_round_to_even():
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, 100.0])
    assert O.e2m1_round(mids).tolist() == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6.0, 6.0]


def test_mxfp4_scale_rule_and_zero_block():
    for e in [-20, -3, 0, 1, 5, 40]:
        for amax in [4.0, 5.9, 6.0, 7.99]:
            x = np.zeros(32)
            x[7] = -amax * 2.0 ** e
            _, s = O.mxfp4_quantize(x)
            assert int(s[0]) - 127 == e
    codes, s = O.mxfp4_quantize(np.zeros(64))
    assert s.tolist() == [0, 0] and not codes.any()


def test_mxfp4_exhaustive_roundtrip():
    """Every (scale, code) pattern whose block holds a magnitude-4 or -6 element
    decodes and re-encodes to itself."""
    r = _rng(6)
    for sbyte in range(1, 255):
        codes = r.integers(0, 16, 64).astype(np.uint8)
        codes[r.integers(0, 32)] = 6 + (sbyte & 1)          # 4.0 or 6.0 in block 0
        codes[32 + r.integers(0, 32)] = 14 + (sbyte & 1)    # -4.0 or -6.0 in block 1
        packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
        scales = np.array([sbyte, 254 - sbyte + 1], np.uint8)
        x = O.mxfp4_dequantize(packed, scales)
        p2, s2 = O.mxfp4_quantize(x)
        assert np.array_equal(s2, scales)
        assert np.array_equal(p2, packed)


def test_mxfp4_nibble_order():
    x = np.zeros(32)
    x[0], x[1], x[31] = 6.0, -1.0, 0.5     # scale exponent 0
    p, s = O.mxfp4_quantize(x)
    assert s[0] == 127
    assert p[0] == (0x7 | (0xA << 4))       # even element in the low nibble
    assert p[15] == (0x1 << 4)


def test_fp4_to_fp8_lossless(facts):
    """E2M1 values times any block scale that keeps them in E4M3's range are
    exactly representable in E4M3."""
    assert facts["fp4_to_fp8_lossless"]["value"]
    for e in range(-8, 7):
        v = np.array(E2M1_TABLE[1:]) * 2.0 ** e
        assert np.array_equal(O.fp8_round(v), v)
        assert np.array_equal(O.fp8_decode(O.fp8_encode(v)), v)


# =============================================================================
# Compressors
# =============================================================================
def _gates(seed, slots):
    r = _rng(seed)
    return r.normal(0, 0.02, (O.DIM, O.DIM)), r.normal(0, 0.1, (slots, O.DIM))


def test_constant_input_pools_to_itself():
    v = _rng(7).standard_normal(O.DIM)
    x = np.tile(v, (64, 1))
    wg, b = _gates(8, 8)
    c = O.csa_compress(x, wg, b, 0, 16)
    assert np.allclose(c, v, rtol=4 * np.finfo(float).eps, atol=0)
    x = np.tile(v, (512, 1))
    wg, b = _gates(9, 128)
    c = O.hca_compress(x, wg, b, 0, 4)
    assert np.allclose(c, v, rtol=8 * np.finfo(float).eps, atol=0)


def test_zero_gates_give_plain_mean():
    x = _rng(10).standard_normal((40, O.DIM))
    c = O.csa_compress(x, np.zeros((O.DIM, O.DIM)), np.zeros((8, O.DIM)), 0, 10)
    assert np.allclose(c[0], x[0:4].mean(axis=0), atol=1e-14)      # first entry: its own block only
    for i in range(1, 10):
        assert np.allclose(c[i], x[4 * i - 4:4 * i + 4].mean(axis=0), atol=1e-14)
    x = _rng(11).standard_normal((384, O.DIM))
    c = O.hca_compress(x, np.zeros((O.DIM, O.DIM)), np.zeros((128, O.DIM)), 0, 3)
    for i in range(3):
        assert np.allclose(c[i], x[128 * i:128 * i + 128].mean(axis=0), atol=1e-14)


def test_slot_bias_selects_slot_token():
    """A huge bias on slot s makes entry i equal to token 4(i-1)+s: slots 0..3
    read the previous block (C^b), slots 4..7 the entry's own block (C^a)."""
    x = _rng(12).standard_normal((48, O.DIM))
    wg, _ = _gates(13, 8)
    for s in range(8):
        b = np.zeros((8, O.DIM))
        b[s] = 1e4
        c = O.csa_compress(x, wg, b, 1, 10)
        for n, i in enumerate(range(1, 11)):
            assert np.array_equal(c[n], x[4 * (i - 1) + s])
    # on entry 0 the previous-block slots do not exist: bias there is ignored
    b = np.zeros((8, O.DIM))
    b[1] = 1e4
    c0 = O.csa_compress(x, np.zeros((O.DIM, O.DIM)), b, 0, 1)
    assert np.allclose(c0[0], x[0:4].mean(axis=0), atol=1e-14)


def test_gate_softmax_is_per_channel():
    """Channel c selects slot c % 8 (bias per slot AND per channel): entry i,
    channel c equals token 4(i-1) + c%8 at channel c."""
    x = _rng(14).standard_normal((48, O.DIM))
    b = np.zeros((8, O.DIM))
    for c in range(O.DIM):
        b[c % 8, c] = 1e4
    out = O.csa_compress(x, np.zeros((O.DIM, O.DIM)), b, 2, 5)
    for n, i in enumerate(range(2, 7)):
        for c in range(O.DIM):
            assert out[n, c] == x[4 * (i - 1) + c % 8, c]
    bh = np.zeros((128, O.DIM))
    for c in range(O.DIM):
        bh[(5 * c) % 128, c] = 1e4
    xh = _rng(15).standard_normal((256, O.DIM))
    outh = O.hca_compress(xh, np.zeros((O.DIM, O.DIM)), bh, 1, 1)
    for c in range(O.DIM):
        assert outh[0, c] == xh[128 + (5 * c) % 128, c]


def test_gate_projection_orientation():
    """z = x @ W_g: a single large W_g[d0, c0] makes channel c0 pick the token
    with the largest x[d0]; every other channel stays the plain mean."""
    d0, c0 = 17, 150
    x = _rng(16).standard_normal((48, O.DIM))
    wg = np.zeros((O.DIM, O.DIM))
    wg[d0, c0] = 1e4
    out = O.csa_compress(x, wg, np.zeros((8, O.DIM)), 3, 4)
    for n, i in enumerate(range(3, 7)):
        toks = x[4 * (i - 1):4 * i + 4]
        j = np.argmax(toks[:, d0])
        assert out[n, c0] == toks[j, c0]
        others = [c for c in range(O.DIM) if c != c0]
        assert np.allclose(out[n, others], toks[:, others].mean(axis=0), atol=1e-14)


def test_gated_pool_two_slot_closed_form():
    """Two tokens, zero W_g, bias difference b per channel: weight of slot 1 is
    the logistic function of b (textbook two-way softmax)."""
    x = _rng(17).standard_normal((8, O.DIM))
    b = np.zeros((8, O.DIM))
    diff = np.linspace(-5, 5, O.DIM)
    b[5] = diff                      # entry 0 has valid slots 4..7 = tokens 0..3
    b[6] = -1e4
    b[7] = -1e4
    out = O.csa_compress(x, np.zeros((O.DIM, O.DIM)), b, 0, 1)[0]
    sig = 1.0 / (1.0 + np.exp(-diff))
    assert np.allclose(out, (1 - sig) * x[0] + sig * x[1], atol=1e-12)


# =============================================================================
# Indexer key of an entry (the reading k_i = C_i @ W_kI, one key shared by all
# indexer heads)
# =============================================================================
def test_indexer_key_basis_rows():
    """Basis-vector entries pick out rows of the projection: e_c @ W = W[c].
    A square, non-symmetric W (D_I = 192) catches a transposed operand, which
    would return column c instead."""
    r = _rng(30)
    for di in (192, 64):
        w = r.standard_normal((O.DIM, di))
        keys = O.csa_compress_key(np.eye(O.DIM), w)
        assert keys.shape == (O.DIM, di)
        assert np.array_equal(keys, w)
    w = r.standard_normal((O.DIM, O.DIM))
    assert not np.allclose(w, w.T)
    assert not np.allclose(O.csa_compress_key(np.eye(O.DIM), w), w.T)


def test_indexer_key_brute_force_loop():
    """k[i, t] = sum_c C[i, c] * W[c, t], written as a double loop over (i, t)
    with an explicit sum over c."""
    r = _rng(31)
    ent = r.standard_normal((5, O.DIM))
    w = r.standard_normal((O.DIM, 32))
    got = O.csa_compress_key(ent, w)
    for i in range(5):
        for t in range(32):
            acc = 0.0
            for c in range(O.DIM):
                acc += ent[i, c] * w[c, t]
            assert math.isclose(got[i, t], acc, rel_tol=1e-12, abs_tol=1e-12)
    # linear in the entry: the key of a combination is the combination of keys
    a, b = 0.375, -2.5
    assert np.allclose(O.csa_compress_key(a * ent[0] + b * ent[1], w),
                       a * got[0] + b * got[1], rtol=1e-13, atol=1e-13)


def test_indexer_key_projects_the_pooled_entry():
    """Compressor -> key chain: the key comes from the pooled value itself, not
    from its stored FP8/BF16 form.  Constant tokens pool to themselves, so every
    entry's key is v @ W exactly; v is chosen off the FP8 grid (1.1 is not an
    E4M3 value), so projecting the stored row would give a different key."""
    v = np.full(O.DIM, 1.1)
    v[O.DIM_NOPE:] = -0.3
    assert not np.array_equal(O.kv_round(v), v)
    x = np.tile(v, (40, 1))
    wg, b = _gates(32, 8)
    w = _rng(33).standard_normal((O.DIM, 64))
    ent = O.csa_compress(x, wg, b, 0, 10)
    keys = O.csa_compress_key(ent, w)
    want = v @ w
    stored = O.kv_round(v) @ w
    assert np.allclose(keys, want[None], rtol=1e-12, atol=1e-12)
    assert np.abs(want - stored).max() > 1e-2
    # a huge slot bias selects one token per entry, so its key is that token's projection
    x = _rng(34).standard_normal((48, O.DIM))
    for s in (2, 6):
        bias = np.zeros((8, O.DIM))
        bias[s] = 1e4
        ent = O.csa_compress(x, wg, bias, 1, 10)
        keys = O.csa_compress_key(ent, w)
        for n, i in enumerate(range(1, 11)):
            assert np.allclose(keys[n], x[4 * (i - 1) + s] @ w, rtol=1e-12, atol=1e-12)


# =============================================================================
# Indexer
# =============================================================================
def test_indexer_basis_closed_form():
    H, DI, N = 3, 8, 8
    q = np.zeros((1, H, DI))
    q[0, 0, 2], q[0, 1, 5], q[0, 2, 2] = 1.0, 2.0, -1.0
    w = np.array([[0.5, 0.25, 4.0]])
    k = np.eye(N, DI)
    s = O.indexer_scores(q, w, k, [N], bf16_scores=False)[0]
    # entry 2: head0 dot 1 (x0.5), head2 dot -1 -> ReLU 0; entry 5: head1 dot 2 (x0.25)
    expect = np.zeros(N)
    expect[2], expect[5] = 0.5, 0.5
    assert np.array_equal(s, expect)


def test_indexer_relu_drops_negative_heads():
    r = _rng(18)
    k = r.standard_normal((5, 16))
    q = np.stack([k[3], -k[3]])[None]            # head 0 aligned, head 1 anti-aligned with entry 3
    w = np.array([[0.7, 0.9]])
    s = O.indexer_scores(q, w, k, [5], False)[0]
    assert np.isclose(s[3], 0.7 * k[3] @ k[3], rtol=1e-15)
    # every entry, written out: head 0 keeps its dot only when positive, head 1
    # only when negative (its query is the negated row)
    for j in range(5):
        d = float(k[3] @ k[j])
        assert np.isclose(s[j], 0.7 * max(d, 0.0) + 0.9 * max(-d, 0.0), rtol=1e-14, atol=0)
    # ReLU(d) + ReLU(-d) = |d|
    q2 = np.stack([k[0], -k[0]])[None]
    s2 = O.indexer_scores(q2, np.array([[1.0, 1.0]]), k, [5], False)[0]
    assert np.allclose(s2, np.abs(k @ k[0]), rtol=1e-14)


def test_indexer_invariances():
    r = _rng(19)
    T, H, DI, N = 3, 4, 32, 50
    q, w, k = r.standard_normal((T, H, DI)), r.uniform(0, 1, (T, H)), r.standard_normal((N, DI))
    nv = [50, 50, 50]
    s = O.indexer_scores(q, w, k, nv, False)
    assert np.allclose(O.indexer_scores(q, 3.0 * w, k, nv, False), 3.0 * s, rtol=1e-14)      # linear in w
    assert np.allclose(O.indexer_scores(q, w, 2.5 * k, nv, False), 2.5 * s, rtol=1e-14)      # pos. homogeneous in k
    assert np.allclose(O.indexer_scores(-q, w, -k, nv, False), s, rtol=1e-14)
    perm = r.permutation(H)
    assert np.allclose(O.indexer_scores(q[:, perm], w[:, perm], k, nv, False), s, rtol=1e-14)
    # a brute-force triple loop on one row
    t = 1
    brute = [sum(w[t, h] * max(0.0, sum(q[t, h, d] * k[n, d] for d in range(DI))) for h in range(H)) for n in range(N)]
    assert np.allclose(s[t], brute, rtol=1e-13)


def test_indexer_causality_and_bf16_rounding():
    r = _rng(20)
    q, w, k = r.standard_normal((2, 4, 32)), r.uniform(0, 1, (2, 4)), r.standard_normal((40, 32))
    n_vis = O.n_visible(np.array([4 * 10 + 3, 4 * 10 + 2]), 40, 4)
    assert n_vis.tolist() == [11, 10]
    s = O.indexer_scores(q, w, k, n_vis, False)
    assert np.isfinite(s[0, :11]).all() and (s[0, 11:] == -np.inf).all()
    assert np.isfinite(s[1, :10]).all() and (s[1, 10:] == -np.inf).all()
    sb = O.indexer_scores(q, w, k, n_vis, True)
    ref = torch.from_numpy(s[0, :11].astype(np.float32)).to(torch.bfloat16).double().numpy()
    # rounding fp64 directly and rounding its fp32 image agree except in double-rounding corner cases
    assert np.array_equal(sb[0, :11], ref)


def test_indexer_mxfp4_exact_inputs():
    """Inputs on the E2M1 grid with a +-4 or +-6 in every 32-block quantise
    losslessly; dyadic w then keeps every product and sum exact, so the fp64
    score equals the integer-arithmetic result bit for bit."""
    r = _rng(21)
    grid = np.array(E2M1_TABLE[1:] + [-g for g in E2M1_TABLE[1:]])
    q = r.choice(grid, (2, 4, 64))
    k = r.choice(grid, (30, 64))
    q[..., 0] = 6.0
    q[..., 32] = -4.0
    k[:, 5] = 4.0
    k[:, 40] = -6.0
    w = r.integers(0, 16, (2, 4)) / 8.0
    for arr in (q, k):
        p, s = O.mxfp4_quantize(arr)
        assert np.array_equal(O.mxfp4_dequantize(p, s), arr)
    s = O.indexer_scores(q, w, k, [30, 30], False)
    qi, ki, wi = (q * 2).astype(np.int64), (k * 2).astype(np.int64), (w * 8).astype(np.int64)
    exact = np.einsum("th,thn->tn", wi, np.maximum(np.einsum("thd,nd->thn", qi, ki), 0))
    assert np.array_equal(s, exact / 32.0)


# =============================================================================
# Top-k
# =============================================================================
def _topk_brute(s, k):
    """Rank by counting: entry i is selected iff fewer than k visible entries
    beat it (higher score, or equal score and lower index)."""
    n = len(s)
    sel = []
    for i in range(n):
        if s[i] == -np.inf:
            continue
        beats = sum(1 for j in range(n) if s[j] > -np.inf and (s[j] > s[i] or (s[j] == s[i] and j < i)))
        if beats < k:
            sel.append(i)
    return sel + [-1] * (k - len(sel))


def test_topk_ties_and_edges():
    s = np.array([1.0, 3.0, 3.0, 2.0, 3.0, -np.inf, 3.0, 0.5])
    assert O.topk_select(s, 3).tolist() == [1, 2, 4]            # four-way tie at 3.0 -> lowest indices
    assert O.topk_select(s, 5).tolist() == [1, 2, 3, 4, 6]
    assert O.topk_select(s, 10).tolist() == [0, 1, 2, 3, 4, 6, 7, -1, -1, -1]
    assert O.topk_select(np.full(6, -np.inf), 4).tolist() == [-1] * 4
    assert O.topk_select(np.array([]), 2).tolist() == [-1, -1]


@settings(max_examples=300, deadline=None)
@given(st.lists(st.sampled_from([-np.inf, -1.0, 0.0, 0.5, 1.0, 2.0, 7.0]), min_size=0, max_size=40),
       st.integers(min_value=1, max_value=45))
def test_topk_matches_rank_counting(vals, k):
    s = np.array(vals, dtype=np.float64)
    assert O.topk_select(s, k).tolist() == _topk_brute(s, k)


def test_topk_random_against_rank_counting():
    r = _rng(22)
    for _ in range(20):
        n = int(r.integers(1, 200))
        s = np.round(r.standard_normal(n), 1)       # many exact ties
        s[r.random(n) < 0.1] = -np.inf
        k = int(r.integers(1, 80))
        assert O.topk_select(s, k).tolist() == _topk_brute(s, k)


# =============================================================================
# Attention
# =============================================================================
def _sdpa(q, keys, scale):
    qt = torch.from_numpy(q)[None, :, None, :]               # [1, H, 1, D]
    kt = torch.from_numpy(keys)[None, None].expand(1, q.shape[0], -1, -1).contiguous()
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, kt, scale=scale)[0, :, 0].numpy()


def test_topk_covering_all_entries_is_dense_attention():
    """k >= visible entries: CSA = dense softmax attention over every visible
    entry plus the window (library SDPA in float64), and = the HCA routine."""
    r = _rng(23)
    H, N = 8, 20
    entries = r.standard_normal((N, O.DIM))
    tok = r.standard_normal((300, O.DIM))
    q = r.standard_normal((H, O.DIM))
    t = 4 * N + 7                                  # all 20 entries (plus more) complete -> n_vis capped at N
    nv = int(O.n_visible(t, N, 4))
    idx = O.topk_select(r.standard_normal(N), 64)  # 64 >= 20: every entry selected
    o, _ = O.sparse_window_attn(q, entries, idx, nv, tok, 0, t, 128, O.default_scale())
    keys = np.concatenate([entries, tok[max(0, t - 127):t + 1]])
    assert np.allclose(o, _sdpa(q, keys, O.default_scale()), rtol=1e-12, atol=1e-14)
    o2, _ = O.hca_dense_attn(q, entries, nv, tok, 0, t, 128, O.default_scale())
    assert np.allclose(o, o2, rtol=1e-13, atol=1e-15)


def test_attention_special_cases():
    r = _rng(24)
    H = 4
    q = r.standard_normal((H, O.DIM))
    row = r.standard_normal((1, O.DIM))
    o, lse = O.attend(q, row, 0.3)
    assert np.allclose(o, np.tile(row, (H, 1)), rtol=1e-15)          # one key -> that row
    o, _ = O.attend(q, np.tile(row, (9, 1)), 0.3)
    assert np.allclose(o, np.tile(row, (H, 1)), rtol=1e-14)          # equal keys -> that row
    keys = r.standard_normal((30, O.DIM))
    o0, lse0 = O.attend(q, keys, 0.1)
    o1, _ = O.attend(q, keys, 0.1, sink=np.full(H, -np.inf))
    assert np.allclose(o0, o1, rtol=1e-15)                           # sink -inf -> no sink
    o2, _ = O.attend(q, keys, 0.1, sink=np.full(H, 800.0))
    assert np.abs(o2).max() < 1e-300                                  # huge sink -> output -> 0
    # q = 0: uniform weights; with a sink the weights sum to n / (n + e^sink)
    sink = np.array([0.0, 1.0, -2.0, 3.0])
    o3, _ = O.attend(np.zeros((H, O.DIM)), keys, 0.1, sink=sink)
    expect = (30 / (30 + np.exp(sink)))[:, None] * keys.mean(axis=0)[None]
    assert np.allclose(o3, expect, rtol=1e-13)
    assert np.allclose(lse0, np.log(np.exp(0.1 * q @ keys.T).sum(axis=1)), rtol=1e-13)
    o4, lse4 = O.attend(q, np.zeros((0, O.DIM)), 0.1)
    assert not o4.any() and (lse4 == -np.inf).all()


def test_attention_is_a_set_function_of_topk():
    r = _rng(25)
    entries = r.standard_normal((100, O.DIM))
    tok = r.standard_normal((600, O.DIM))
    q = r.standard_normal((4, O.DIM))
    idx = r.choice(100, 16, replace=False)
    o1, _ = O.sparse_window_attn(q, entries, idx, 100, tok, 0, 500, 128, 0.07)
    o2, _ = O.sparse_window_attn(q, entries, r.permutation(idx), 100, tok, 0, 500, 128, 0.07)
    assert np.allclose(o1, o2, rtol=1e-13)
    # -1 padding and out-of-range indices are skipped
    o3, _ = O.sparse_window_attn(q, entries, np.concatenate([idx, [-1, -1, 100, 5000]]), 100, tok, 0, 500, 128, 0.07)
    assert np.allclose(o1, o3, rtol=1e-13)


def test_window_extent_and_causality():
    """The window is tokens t-127..t inclusive; later tokens and not-yet-visible
    entries do not affect the output."""
    r = _rng(26)
    entries = r.standard_normal((200, O.DIM))
    tok = r.standard_normal((800, O.DIM))
    q = r.standard_normal((4, O.DIM))
    t = 601
    nv = int(O.n_visible(t, 200, 4))
    assert nv == 150
    idx = np.arange(0, 150, 3)
    base, _ = O.sparse_window_attn(q, entries, idx, nv, tok, 0, t, 128, 0.07)
    for pos, changes in [(t - 128, False), (t - 127, True), (t, True), (t + 1, False)]:
        tok2 = tok.copy()
        tok2[pos] += 1.0
        o, _ = O.sparse_window_attn(q, entries, idx, nv, tok2, 0, t, 128, 0.07)
        assert (not np.allclose(o, base, rtol=0, atol=0)) == changes, pos
    ent2 = entries.copy()
    ent2[150:] = 1e3
    o, _ = O.sparse_window_attn(q, ent2, np.arange(0, 200, 3), nv, tok, 0, t, 128, 0.07)
    o_ref, _ = O.sparse_window_attn(q, entries, np.arange(0, 150, 3), nv, tok, 0, t, 128, 0.07)
    assert np.array_equal(o, o_ref)
    o, _ = O.hca_dense_attn(q, ent2, nv, tok, 0, t, 128, 0.07)
    o_ref, _ = O.hca_dense_attn(q, entries, nv, tok, 0, t, 128, 0.07)
    assert np.array_equal(o, o_ref)
    # early positions: the window starts at token 0
    assert O.window_positions(5, 128).tolist() == list(range(6))
