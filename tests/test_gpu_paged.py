"""GPU checks of the paged decode cache: entries of both layers (with the CSA
MXFP4 keys) in pools of fixed-size pages behind per-sequence page tables.

A paged cache holding the same entries as a contiguous one, on a scattered
page assignment with pages no sequence uses, gives bit for bit the same
outputs, positions, counts, entries and keys over decode steps that cross page
boundaries, CSA and HCA compression boundaries, through decode_step and the
per-layer calls, on the matrix-core and float32 attention paths, and on the
1M-context decode shape.  decode_fork shares a sequence's full pages with
another, which then decodes exactly as an unshared copy would, while the
shared pages stay untouched.  Snapshots of paged and contiguous caches are
byte-identical files and load into either layout."""
import math

import numpy as np
import pytest
import torch

from tests.gpu_util import dev, up

pytestmark = pytest.mark.gpu


def _weights(rng, DI):
    return {"csa_w_gate": up((rng.standard_normal((192, 192)) * 0.02).astype(np.float32)),
            "csa_pos_bias": up((rng.standard_normal((8, 192)) * 0.1).astype(np.float32)),
            "csa_w_idx": up((rng.standard_normal((192, DI)) / np.sqrt(192)).astype(np.float32)),
            "hca_w_gate": up((rng.standard_normal((192, 192)) * 0.02).astype(np.float32)),
            "hca_pos_bias": up((rng.standard_normal((128, 192)) * 0.1).astype(np.float32))}


def _contiguous(L, rng, B, H, K, csa_cap, hca_cap, pos, DI=64):
    """A contiguous cache with random stored entries, keys and rings; counts
    from the positions (negative position: an inactive sequence)."""
    pos = np.asarray(pos, np.int64)
    c = L.DecodeCache(B, H, 64, DI, K, 128, csa_cap, hca_cap, 1.0 / math.sqrt(192), _weights(rng, DI), device=dev())
    L.kv_pack(up(rng.standard_normal((B * csa_cap, 192)).astype(np.float32)), c.csa_kv.view(B * csa_cap, 256))
    L.kv_pack(up(rng.standard_normal((B * hca_cap, 192)).astype(np.float32)), c.hca_kv.view(B * hca_cap, 256))
    c.csa_keys.copy_(up(rng.integers(0, 256, (B, csa_cap, DI // 2), dtype=np.uint8)))
    c.csa_key_scales.copy_(up(rng.integers(123, 131, (B, csa_cap, DI // 32), dtype=np.uint8)))
    c.pos.copy_(up(pos))
    c.csa_entries.copy_(up(np.clip(pos // 4, 0, csa_cap).astype(np.int32)))
    c.hca_entries.copy_(up(np.clip(pos // 128, 0, hca_cap).astype(np.int32)))
    L.decode_prime(c, up(rng.standard_normal((B, 128, 192)).astype(np.float32)),
                   up(rng.standard_normal((B, 128, 192)).astype(np.float32)))
    return c


def _tables(rng, B, n_pages, spare):
    """A scattered assignment of B x n_pages logical pages to a pool with
    `spare` pages no sequence uses."""
    perm = rng.permutation(B * n_pages + spare)[:B * n_pages]
    return torch.from_numpy(perm.astype(np.int32).reshape(B, n_pages))


def _paged_copy(L, rng, c, P, spare=5):
    """A paged cache with the same state as contiguous cache c (garbage in the
    pages no sequence uses)."""
    B, cc, hc = c.c.batch, c.c.csa_cap, c.c.hca_cap
    tc, th = _tables(rng, B, cc // P, spare), _tables(rng, B, hc // P, spare)
    p = L.DecodeCache(B, c.c.n_heads, c.c.idx_heads, c.c.idx_dim, c.c.topk, c.c.window, cc, hc, c.c.scale, c.weights,
                      device=dev(), page_entries=P, csa_pool_pages=B * (cc // P) + spare,
                      hca_pool_pages=B * (hc // P) + spare, csa_pages=tc, hca_pages=th)
    for name in ("csa_kv", "csa_keys", "csa_key_scales", "hca_kv"):
        pool = getattr(p, name)
        pool.copy_(up(rng.integers(0, 256, tuple(pool.shape), dtype=np.uint8)))
        tab = (p.hca_pages if name == "hca_kv" else p.csa_pages).long()
        src = getattr(c, name)
        pool[tab.view(-1)] = src.view(B * tab.shape[1], P, -1)
    for name in ("pos", "csa_entries", "hca_entries", "csa_raw", "csa_logits", "hca_raw", "hca_logits", "csa_win",
                 "hca_win"):
        getattr(p, name).copy_(getattr(c, name))
    return p


def _logical(p, name):
    """The entry array of a paged cache in logical order [B, cap, row]."""
    tab = (p.hca_pages if name == "hca_kv" else p.csa_pages).long()
    pool = getattr(p, name)
    return pool[tab.view(-1)].view(tab.shape[0], tab.shape[1] * pool.shape[1], -1)


def _inputs(rng, B, H, qdt, HI=64, DI=64):
    f = lambda *s: up(rng.standard_normal(s).astype(np.float32))  # noqa: E731
    return dict(xc=f(B, 192), xh=f(B, 192), qi=f(B, HI, DI), w=up(rng.random((B, HI)).astype(np.float32)),
                qc=f(B, H, 192).to(qdt), qh=f(B, H, 192).to(qdt))


def _step(L, c, x, ws, by_layer=False):
    B, H = c.c.batch, c.c.n_heads
    oc = torch.empty(B, H, 192, dtype=torch.bfloat16, device=dev())
    oh = torch.empty_like(oc)
    if by_layer:
        L.decode_csa_layer(c, x["xc"], x["qi"], x["w"], x["qc"], oc, ws)
        L.decode_hca_layer(c, x["xh"], x["qh"], oh, ws)
    else:
        L.decode_step(c, x["xc"], x["xh"], x["qi"], x["w"], x["qc"], x["qh"], oc, oh, ws)
    return oc, oh


def _same_state(c, p, what):
    for name in ("pos", "csa_entries", "hca_entries", "csa_raw", "csa_logits", "hca_raw", "hca_logits", "csa_win",
                 "hca_win"):
        assert torch.equal(getattr(c, name), getattr(p, name)), (what, name)
    for name in ("csa_kv", "csa_keys", "csa_key_scales", "hca_kv"):
        assert torch.equal(getattr(c, name), _logical(p, name)), (what, name)


def _bits(t):
    return t.view(torch.int16)


@pytest.mark.parametrize("P,csa_cap,hca_cap,pos,K,qdt", [
    # page and compression boundaries in the first steps: CSA count 1023 -> 1024 (a new 32-entry page), HCA count
    # 31 -> 32 (also a new page); a sequence at its first entries; the float32 attention path on 8 heads
    (32, 2048, 64, [4093, 4093 - 40, 130], 64, torch.bfloat16),
    (32, 2048, 64, [4093, 515, 6], 48, torch.float32),
    # split top-k path (long rows), 256-entry pages, an inactive sequence
    (256, 40960, 256, [4 * 40704 - 5, 4 * 256 * 60 - 3, -1, 128 * 255 - 2], 512, torch.bfloat16),
])
def test_paged_decode_equals_contiguous(P, csa_cap, hca_cap, pos, K, qdt):
    from long_context_compressed_compress_amd import libcsa as L
    rng = np.random.default_rng(70 + P + K)
    B = len(pos)
    H = 8 if qdt == torch.float32 else 32
    c = _contiguous(L, rng, B, H, K, csa_cap, hca_cap, pos)
    p = _paged_copy(L, rng, c, P)
    _same_state(c, p, "initial")
    wc, wp = c.workspace(qdt), p.workspace(qdt)
    for s in range(10):
        x = _inputs(rng, B, H, qdt)
        print(f"paged decode P={P} step {s} by_layer={s % 3 == 2}", flush=True)
        a = _step(L, c, x, wc)
        b = _step(L, p, x, wp, by_layer=s % 3 == 2)
        torch.cuda.synchronize()
        assert torch.equal(_bits(a[0]), _bits(b[0])), ("csa", s)
        assert torch.equal(_bits(a[1]), _bits(b[1])), ("hca", s)
    _same_state(c, p, "after the steps")


def test_fork_shares_full_pages_and_decodes_like_a_copy():
    """decode_fork 0 -> 1 and 2 -> 3 on a paged cache against a contiguous
    cache whose sequences 1 and 3 are copies of 0 and 2: the four sequences
    then decode with different inputs, bit for bit alike in both caches; the
    forked sequences' tables name the source's full pages, and those pages
    never change."""
    from long_context_compressed_compress_amd import libcsa as L
    rng = np.random.default_rng(80)
    P, csa_cap, hca_cap, K, H = 32, 2048, 64, 64, 32
    pos = [4 * 1000 + 1, 9, 4093 - 8, 300]      # CSA counts 1000 (partial page) and 1021; HCA 31 (partial)
    c = _contiguous(L, rng, 4, H, K, csa_cap, hca_cap, pos)
    p = _paged_copy(L, rng, c, P)
    for src, dst in ((0, 1), (2, 3)):
        L.decode_fork(p, src, dst)
        # the copy: state, and the entries below the counts (rows past them stay dst's, as in dst's own pages)
        nc, nh = int(c.csa_entries[src]), int(c.hca_entries[src])
        for name in ("pos", "csa_entries", "hca_entries", "csa_raw", "csa_logits", "hca_raw", "hca_logits", "csa_win",
                     "hca_win"):
            getattr(c, name)[dst].copy_(getattr(c, name)[src])
        for name in ("csa_kv", "csa_keys", "csa_key_scales"):
            getattr(c, name)[dst, :nc].copy_(getattr(c, name)[src, :nc])
        c.hca_kv[dst, :nh].copy_(c.hca_kv[src, :nh])
    torch.cuda.synchronize()
    _same_state(c, p, "after the forks")
    shared = {}
    for src, dst in ((0, 1), (2, 3)):
        nc, nh = int(c.csa_entries[src]) // P, int(c.hca_entries[src]) // P
        assert torch.equal(p.csa_pages[dst, :nc], p.csa_pages[src, :nc])
        assert torch.equal(p.hca_pages[dst, :nh], p.hca_pages[src, :nh])
        assert p.csa_pages[dst, nc] != p.csa_pages[src, nc]        # the partly filled page is dst's own
        shared[src] = ([p.csa_kv[i].clone() for i in p.csa_pages[src, :nc].tolist()],
                       [p.csa_keys[i].clone() for i in p.csa_pages[src, :nc].tolist()],
                       [p.hca_kv[i].clone() for i in p.hca_pages[src, :nh].tolist()], nc, nh)
    wc, wp = c.workspace(), p.workspace()
    for s in range(12):
        x = _inputs(rng, 4, H, torch.bfloat16)
        print(f"forked decode step {s}", flush=True)
        a = _step(L, c, x, wc)
        b = _step(L, p, x, wp)
        torch.cuda.synchronize()
        assert torch.equal(_bits(a[0]), _bits(b[0])), ("csa", s)
        assert torch.equal(_bits(a[1]), _bits(b[1])), ("hca", s)
    _same_state(c, p, "after the steps")
    for src, (kv, keys, hkv, nc, nh) in shared.items():
        for j, i in enumerate(p.csa_pages[src, :nc].tolist()):
            assert torch.equal(p.csa_kv[i], kv[j]) and torch.equal(p.csa_keys[i], keys[j])
        for j, i in enumerate(p.hca_pages[src, :nh].tolist()):
            assert torch.equal(p.hca_kv[i], hkv[j])


def test_paged_snapshots(tmp_path):
    """prefix_save of a sequence gives the same file from a paged and from a
    contiguous cache; the file loads into either layout (a shorter prefix too)
    with the same entries and state."""
    from long_context_compressed_compress_amd import libcsa as L
    rng = np.random.default_rng(90)
    P = 64
    c = _contiguous(L, rng, 3, 32, 64, 4096, 128, [4 * 2000 + 3, 130, 4 * 1500])
    p = _paged_copy(L, rng, c, P)
    for seq in range(3):
        L.prefix_save(c, seq, str(tmp_path / f"c{seq}.snap"))
        L.prefix_save(p, seq, str(tmp_path / f"p{seq}.snap"))
        assert (tmp_path / f"c{seq}.snap").read_bytes() == (tmp_path / f"p{seq}.snap").read_bytes(), seq
    # sequence 0's snapshot into sequence 2 of both caches, full and shorter prefixes
    for plen in (-1, 4 * 1200 + 1):
        parts = L.CSA_PREFIX_ENTRIES | (L.CSA_PREFIX_RINGS if plen < 0 else 0)
        a = L.prefix_load(c, 2, str(tmp_path / "p0.snap"), parts, plen)
        b = L.prefix_load(p, 2, str(tmp_path / "c0.snap"), parts, plen)
        assert a == b
        _same_state(c, p, f"prefix {plen}")
    # a table naming a page outside the pool is refused before anything is written
    before = [t.clone() for t in (p.csa_kv, p.pos)]
    p.csa_pages[1, 0] = p.c.csa_pool_pages
    with pytest.raises(L.CsaError) as ex:
        L.prefix_load(p, 1, str(tmp_path / "c0.snap"), L.CSA_PREFIX_ENTRIES)
    assert ex.value.status == L.CSA_ERR_RANGE
    assert torch.equal(before[0], p.csa_kv) and torch.equal(before[1], p.pos)


def test_paged_decode_1m_context():
    """The 1M-context decode shape (batch 8, 262,144 CSA entries, top-1024,
    128 heads) paged in 256-entry pages: 4 steps bit for bit equal to the
    contiguous cache, a CSA entry completing on the way."""
    from long_context_compressed_compress_amd import libcsa as L
    rng = np.random.default_rng(95)
    B, P = 8, 256
    csa_cap, hca_cap = 262144 + 256, 8192 + 256
    pos = [(1 << 20) - 2] * 6 + [(1 << 20) - 4 * 3000 - 1, 4 * 100 + 1]
    c = _contiguous(L, rng, B, 128, 1024, csa_cap, hca_cap, pos)
    p = _paged_copy(L, rng, c, P, spare=17)
    wc, wp = c.workspace(), p.workspace()
    for s in range(4):
        x = _inputs(rng, B, 128, torch.bfloat16)
        print(f"paged decode 1M step {s}", flush=True)
        a = _step(L, c, x, wc)
        b = _step(L, p, x, wp)
        torch.cuda.synchronize()
        assert torch.equal(_bits(a[0]), _bits(b[0])), ("csa", s)
        assert torch.equal(_bits(a[1]), _bits(b[1])), ("hca", s)
    _same_state(c, p, "after the steps")
