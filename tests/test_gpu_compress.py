"""GPU parity of the CSA and HCA compressors with the oracle: float32 output to
1e-5 relative, stored formats byte-exact except at float32-vs-fp64 rounding
midpoints, indexer keys likewise."""
import numpy as np
import pytest
import torch

from oracle import csa_oracle as O
from tests.gpu_util import (assert_f32_close, bf16_tensor, dev, down, mixed_mismatches_near_midpoints,
                            mxfp4_mismatches_near_boundaries, up)

pytestmark = pytest.mark.gpu


def _weights(seed, slots, d_idx=32):
    r = np.random.default_rng(seed)
    return ((r.standard_normal((192, 192)) * 0.02).astype(np.float32),
            (r.standard_normal((slots, 192)) * 0.1).astype(np.float32),
            (r.standard_normal((192, d_idx)) / np.sqrt(192)).astype(np.float32))


def test_csa_compress_f32_entries_and_keys_batch():
    from long_context_compressed_compress_amd import libcsa as L
    rng = np.random.default_rng(10)
    B, T, n_cap = 3, 203, 60
    x = rng.standard_normal((B, T, 192)).astype(np.float32)
    wg, pb, wi = _weights(11, 8)
    kv = torch.zeros(B, n_cap, 192, dtype=torch.float32, device=dev())
    key = torch.zeros(B, n_cap, 32, dtype=torch.float32, device=dev())
    L.csa_compress(up(x), 0, up(wg), up(pb), 0, 50, kv, w_idx=up(wi), key_out=key)   # 50 entries: 7 blocks of 8
    got, gk = down(kv), down(key)
    for b in range(B):
        ref = O.csa_compress(x[b], wg, pb, 0, 50)
        assert_f32_close(got[b, :50], ref, 1e-5, "entries")
        assert_f32_close(gk[b, :50], O.csa_compress_key(ref, wi), 1e-5, "keys")
    assert not got[:, 50:].any() and not gk[:, 50:].any()      # nothing written past the request


def test_csa_compress_mixed_and_mxfp4_keys_from_bf16_ring():
    """Decode-style: raw tokens in a 128-row ring (wrapped), one entry at a time and a
    batch of entries, BF16 raw input, mixed storage, MXFP4 indexer keys."""
    from long_context_compressed_compress_amd import libcsa as L
    rng = np.random.default_rng(12)
    B, R, n_cap, DI = 4, 128, 400, 64
    wg, pb, wi = _weights(13, 8, DI)
    t_end = 1000                         # tokens 0..999 exist; ring holds 872..999
    xs = rng.standard_normal((B, t_end, 192)).astype(np.float32)
    xb = bf16_tensor(xs)                 # the caller's BF16 raw KV
    xb_vals = xb.float().cpu().numpy()
    ring = torch.empty(B, R, 192, dtype=torch.bfloat16, device=dev())
    pos = torch.arange(t_end - R, t_end, device=dev())
    ring[:, pos % R] = xb[:, pos]
    kv = torch.zeros(B, n_cap, 256, dtype=torch.uint8, device=dev())
    kc = torch.zeros(B, n_cap, DI // 2, dtype=torch.uint8, device=dev())
    ks = torch.zeros(B, n_cap, DI // 32, dtype=torch.uint8, device=dev())
    # entries 219..249 read tokens 872..999 (entry i reads 4i-4 .. 4i+3)
    L.csa_compress(ring, 0, up(wg), up(pb), 219, 31, kv, w_idx=up(wi), key_out=kc, key_scales=ks)
    got, gkc, gks = down(kv), down(kc), down(ks)
    tol_e = tol_k = 0
    for b in range(B):
        ref = O.csa_compress(xb_vals[b], wg, pb, 219, 31)
        tol_e += mixed_mismatches_near_midpoints(got[b, 219:250], ref)
        tol_k += mxfp4_mismatches_near_boundaries(gkc[b, 219:250], gks[b, 219:250], O.csa_compress_key(ref, wi))
    assert tol_e <= 0.002 * B * 31 * 192 and tol_k <= 0.002 * B * 31 * DI
    assert not got[:, :219].any() and not got[:, 250:].any()


def test_csa_compress_first_entries_and_constant_input():
    from long_context_compressed_compress_amd import libcsa as L
    v = np.random.default_rng(14).standard_normal(192).astype(np.float32)
    x = np.tile(v, (1, 64, 1))
    wg, pb, _ = _weights(15, 8)
    kv = torch.zeros(1, 16, 192, dtype=torch.float32, device=dev())
    L.csa_compress(up(x), 0, up(wg), up(pb), 0, 16, kv)
    assert np.allclose(down(kv)[0], v[None], rtol=2e-6, atol=0)      # constant input pools to itself
    x2 = np.random.default_rng(16).standard_normal((1, 64, 192)).astype(np.float32)
    L.csa_compress(up(x2), 0, up(np.zeros((192, 192), np.float32)), up(np.zeros((8, 192), np.float32)), 0, 3, kv)
    g = down(kv)[0]
    assert np.allclose(g[0], x2[0, 0:4].mean(0), rtol=1e-6, atol=1e-6)   # entry 0: its own block only
    assert np.allclose(g[2], x2[0, 4:12].mean(0), rtol=1e-6, atol=1e-6)


def test_hca_compress_f32_and_mixed():
    from long_context_compressed_compress_amd import libcsa as L
    rng = np.random.default_rng(17)
    B, T = 2, 128 * 6
    x = rng.standard_normal((B, T, 192)).astype(np.float32)
    wg, pb, _ = _weights(18, 128)
    kv = torch.zeros(B, 8, 192, dtype=torch.float32, device=dev())
    L.hca_compress(up(x), 0, up(wg), up(pb), 1, 5, kv)
    got = down(kv)
    for b in range(B):
        assert_f32_close(got[b, 1:6], O.hca_compress(x[b], wg, pb, 1, 5), 1e-5, "hca entries")
    assert not got[:, 0].any() and not got[:, 6:].any()
    # BF16 raw tokens in a contiguous buffer that starts at position 256, mixed storage
    xb = bf16_tensor(x)
    kvm = torch.zeros(B, 8, 256, dtype=torch.uint8, device=dev())
    L.hca_compress(xb[:, 256:].contiguous(), 256, up(wg), up(pb), 2, 4, kvm)
    xv = xb.float().cpu().numpy()
    gm = down(kvm)
    n_tol = sum(mixed_mismatches_near_midpoints(gm[b, 2:6], O.hca_compress(xv[b], wg, pb, 2, 4)) for b in range(B))
    assert n_tol <= 0.002 * B * 4 * 192
    v = rng.standard_normal(192).astype(np.float32)
    kvc = torch.zeros(1, 2, 192, dtype=torch.float32, device=dev())
    L.hca_compress(up(np.tile(v, (1, 256, 1))), 0, up(wg), up(pb), 0, 2, kvc)
    assert np.allclose(down(kvc)[0], v[None], rtol=2e-6, atol=0)


def test_compressors_read_unaligned_rings_like_aligned_ones():
    """A ring whose base is not 16-byte aligned goes through the element-wise
    loads, an aligned one through the 16-byte pieces: same bytes either way
    (BF16 and float32 rings, the one-entry and eight-entry CSA paths, HCA)."""
    from long_context_compressed_compress_amd import libcsa as L
    rng = np.random.default_rng(19)
    B, T = 2, 512
    x = rng.standard_normal((B, T, 192)).astype(np.float32)
    wg, pb, wi = _weights(20, 8, 64)
    _, pbh, _ = _weights(21, 128)
    for dt in (torch.bfloat16, torch.float32):
        src = torch.from_numpy(x).to(device=dev(), dtype=dt)
        flat = torch.zeros(B * T * 192 + 1, dtype=dt, device=dev())
        flat[1:] = src.reshape(-1)
        shifted = flat[1:].view(B, T, 192)               # base 2 or 4 bytes past an aligned address
        assert shifted.data_ptr() % 16 != 0 and src.data_ptr() % 16 == 0
        for first, n in ((0, 9), (40, 3), (5, 100)):     # eight-entry blocks and one-entry blocks
            outs = []
            for ring in (src, shifted):
                kv = torch.zeros(B, 128, 192, dtype=torch.float32, device=dev())
                key = torch.zeros(B, 128, 64, dtype=torch.float32, device=dev())
                L.csa_compress(ring, 0, up(wg), up(pb), first, n, kv, w_idx=up(wi), key_out=key)
                outs.append((down(kv), down(key)))
            assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
        outs = []
        for ring in (src, shifted):
            kv = torch.zeros(B, 4, 256, dtype=torch.uint8, device=dev())
            L.hca_compress(ring, 0, up(wg), up(pbh), 0, 4, kv)
            outs.append(down(kv))
        assert np.array_equal(outs[0], outs[1])
        kv = torch.zeros(B, 4, 192, dtype=torch.float32, device=dev())
        L.hca_compress(src, 0, up(wg), up(pbh), 0, 4, kv)
        for b in range(B):
            ref = O.hca_compress(src[b].float().cpu().numpy(), wg, pbh, 0, 4)
            assert_f32_close(down(kv)[b], ref, 1e-5, "hca entries")
