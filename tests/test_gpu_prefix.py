"""GPU tests of prefix reuse (prefix_save / prefix_load): a sequence restored
from a snapshot, with the window state taken from the file or recomputed from
the raw tokens, is the same cache as one built directly at that position — the
state arrays are equal bit for bit, and so are the outputs of the decode steps
that follow (across CSA and HCA compression boundaries) — and those outputs
match the oracle's attention over the oracle's own compression of the same
raw tokens.  Full caching, no SWA
caching, a shorter shared prefix, and a periodic checkpoint plus a later
entries-only snapshot are covered."""
import functools
import math

import numpy as np
import pytest
import torch

from oracle import csa_oracle as O
from tests.gpu_util import assert_attn_close, dev, down, up

pytestmark = pytest.mark.gpu

B, H, HI, DI, K, W = 2, 32, 64, 64, 64, 128
CSA_CAP, HCA_CAP = 128, 4
N_HIST = 300          # raw tokens of the subject sequence
SCALE = 1.0 / math.sqrt(192)


@pytest.fixture(scope="module")
def env():
    from long_context_compressed_compress_amd import libcsa as L
    rng = np.random.default_rng(77)
    wts = {"csa_w_gate": rng.standard_normal((192, 192)) * 0.02, "csa_pos_bias": rng.standard_normal((8, 192)) * 0.1,
           "csa_w_idx": rng.standard_normal((192, DI)) / np.sqrt(192),
           "hca_w_gate": rng.standard_normal((192, 192)) * 0.02, "hca_pos_bias": rng.standard_normal((128, 192)) * 0.1}
    wd = {k: up(v.astype(np.float32)) for k, v in wts.items()}
    xc = up(rng.standard_normal((1, N_HIST, 192)).astype(np.float32)).to(torch.bfloat16)   # raw KV by position
    xh = up(rng.standard_normal((1, N_HIST, 192)).astype(np.float32)).to(torch.bfloat16)
    q_idx = up(rng.standard_normal((N_HIST, HI, DI)).astype(np.float32))                   # decode inputs by position
    w = up(rng.random((N_HIST, HI)).astype(np.float32))
    q_c = up(rng.standard_normal((N_HIST, H, 192)).astype(np.float32)).to(torch.bfloat16)
    q_h = up(rng.standard_normal((N_HIST, H, 192)).astype(np.float32)).to(torch.bfloat16)
    e = dict(L=L, wd=wd, wts={k: v.astype(np.float32).astype(np.float64) for k, v in wts.items()}, xc=xc, xh=xh,
             q_idx=q_idx, w=w, q_c=q_c, q_h=q_h, id=len(_ENV))
    _ENV.append(e)
    return e


_ENV = []


def _cache(e):
    c = e["L"].DecodeCache(B, H, HI, DI, K, W, CSA_CAP, HCA_CAP, SCALE, e["wd"], device=dev())
    c.pos.fill_(-1)        # every sequence inactive until filled or loaded
    return c


def _fill(e, cache, b, p):
    """Sequence b of the cache at position p, built directly: entries by the
    prefill compressors, rings by decode_prime over the last 128 tokens."""
    L, wd = e["L"], e["wd"]
    v = cache.seq_view(b)
    nc, nh = p // 4, p // 128
    if nc:
        L.csa_compress(e["xc"], 0, wd["csa_w_gate"], wd["csa_pos_bias"], 0, nc, v.csa_kv, w_idx=wd["csa_w_idx"],
                       key_out=v.csa_keys, key_scales=v.csa_key_scales)
    if nh:
        L.hca_compress(e["xh"], 0, wd["hca_w_gate"], wd["hca_pos_bias"], 0, nh, v.hca_kv)
    v.pos.fill_(p)
    v.csa_entries.fill_(nc)
    v.hca_entries.fill_(nh)
    _prime(e, cache, b, max(0, p - 128), p)


def _prime(e, cache, b, lo, hi):
    if hi > lo:
        e["L"].decode_prime(cache.seq_view(b), e["xc"][:, lo:hi].contiguous(), e["xh"][:, lo:hi].contiguous())


def _steps(e, cache, b, p, n):
    """n decode steps of sequence b from position p (the other sequence
    inactive); returns the outputs of each step."""
    L = e["L"]
    ws = cache.workspace(torch.bfloat16)
    outs = []
    for s in range(n):
        t = p + s

        def row(x):
            z = torch.zeros((B,) + tuple(x.shape[1:]), dtype=x.dtype, device=x.device)
            z[b] = x[t]
            return z
        oc = torch.empty(B, H, 192, dtype=torch.bfloat16, device=dev())
        oh = torch.empty_like(oc)
        L.decode_step(cache, row(e["xc"][0]), row(e["xh"][0]), row(e["q_idx"]), row(e["w"]), row(e["q_c"]),
                      row(e["q_h"]), oc, oh, ws)
        outs.append((oc[b].clone(), oh[b].clone()))
    torch.cuda.synchronize()
    return outs


@functools.lru_cache(maxsize=None)
def _oracle_layers(env_id):
    """The oracle's view of the subject sequence: BF16 raw tokens of both
    layers as numbers, every CSA and HCA entry they compress into (fp64), and
    the stored (decoded) forms of entries and tokens."""
    e = _ENV[env_id]
    xc = e["xc"].double().cpu().numpy()[0]
    xh = e["xh"].double().cpu().numpy()[0]
    wts = e["wts"]
    ent = O.csa_compress(xc, wts["csa_w_gate"], wts["csa_pos_bias"], 0, N_HIST // 4)
    enth = O.hca_compress(xh, wts["hca_w_gate"], wts["hca_pos_bias"], 0, N_HIST // 128)
    return dict(ent=O.kv_round(ent), enth=O.kv_round(enth), winc=O.kv_round(xc), winh=O.kv_round(xh))


def _assert_oracle_steps(e, outs, p):
    """Outputs of decode steps at positions p, p+1, .. against the oracle:
    the CSA layer selects every visible entry (at most K = 64 exist here), so
    its output is attention over all of them plus the window; the HCA layer
    attends to every visible entry plus the window."""
    ref = _oracle_layers(e["id"])
    assert (p + len(outs)) // 4 <= K
    for s, (oc, oh) in enumerate(outs):
        t = p + s
        n, nh = (t + 1) // 4, (t + 1) // 128
        qc = O.bf16_round(e["q_c"][t].float().cpu().numpy())
        qh = O.bf16_round(e["q_h"][t].float().cpu().numpy())
        o, _ = O.sparse_window_attn(qc, ref["ent"], np.arange(n), n, ref["winc"], 0, t, W, SCALE)
        assert_attn_close(down(oc), o, True, f"CSA output at position {t}")
        o, _ = O.hca_dense_attn(qh, ref["enth"], nh, ref["winh"], 0, t, W, SCALE)
        assert_attn_close(down(oh), o, True, f"HCA output at position {t}")


def _same_state(a, ba, c, bc):
    """Sequence ba of cache a and sequence bc of cache c hold the same state."""
    assert int(a.pos[ba]) == int(c.pos[bc])
    nc, nh = int(a.csa_entries[ba]), int(a.hca_entries[ba])
    assert (nc, nh) == (int(c.csa_entries[bc]), int(c.hca_entries[bc]))
    for k, n in (("csa_kv", nc), ("csa_keys", nc), ("csa_key_scales", nc), ("hca_kv", nh)):
        assert torch.equal(getattr(a, k)[ba, :n], getattr(c, k)[bc, :n]), k
    p = int(a.pos[ba])
    for k, rows in (("csa_raw", 8), ("csa_logits", 8), ("hca_raw", 128), ("hca_logits", 128), ("csa_win", W),
                    ("hca_win", W)):
        r = torch.arange(max(0, p - rows), p, device=dev()) % rows     # rows holding positions < p
        x, y = getattr(a, k)[ba, r], getattr(c, k)[bc, r]
        assert torch.equal(x.view(torch.uint8) if x.dtype != torch.uint8 else x,
                           y.view(torch.uint8) if y.dtype != torch.uint8 else y), k


def _same_steps(o1, o2):
    for s, ((a1, b1), (a2, b2)) in enumerate(zip(o1, o2)):
        assert torch.equal(a1.view(torch.int16), a2.view(torch.int16)), f"CSA output, step {s}"
        assert torch.equal(b1.view(torch.int16), b2.view(torch.int16)), f"HCA output, step {s}"


def test_full_caching_resumes_exactly(env, tmp_path):
    L = env["L"]
    a = _cache(env)
    _fill(env, a, 0, 248)
    _steps(env, a, 0, 248, 3)                       # a at 251 (its entries include decode-made ones)
    path = str(tmp_path / "full.snap")
    L.prefix_save(a, 0, path)                       # entries + rings
    c = _cache(env)
    print("prefix: full caching, restore into sequence 1", flush=True)
    assert L.prefix_load(c, 1, path) == 251         # nothing to recompute
    _same_state(a, 0, c, 1)
    # 251 .. 258: CSA entries complete at 251 and 255, an HCA entry at 255
    restored = _steps(env, c, 1, 251, 8)
    _same_steps(_steps(env, a, 0, 251, 8), restored)
    _same_state(a, 0, c, 1)
    # and the restored sequence's outputs against the oracle's attention over
    # the oracle's own entries of the same raw tokens
    _assert_oracle_steps(env, restored, 251)


def test_no_swa_caching_recomputes_the_window(env, tmp_path):
    L = env["L"]
    a = _cache(env)
    _fill(env, a, 1, 248)
    _steps(env, a, 1, 248, 3)
    path = str(tmp_path / "entries.snap")
    L.prefix_save(a, 1, path, parts=L.CSA_PREFIX_ENTRIES)
    c = _cache(env)
    print("prefix: entries only, window recomputed", flush=True)
    start = L.prefix_load(c, 0, path, parts=L.CSA_PREFIX_ENTRIES)
    assert start == 251 - 128
    _prime(env, c, 0, start, 251)
    _same_state(a, 1, c, 0)
    restored = _steps(env, c, 0, 251, 8)
    _same_steps(_steps(env, a, 1, 251, 8), restored)
    _assert_oracle_steps(env, restored, 251)


def test_shorter_shared_prefix(env, tmp_path):
    """A snapshot at 251 serves a prompt that shares only its first 201 tokens."""
    L = env["L"]
    a = _cache(env)
    _fill(env, a, 0, 248)
    _steps(env, a, 0, 248, 3)
    path = str(tmp_path / "long.snap")
    L.prefix_save(a, 0, path)
    c = _cache(env)
    print("prefix: 201 tokens of a 251-token snapshot", flush=True)
    start = L.prefix_load(c, 0, path, parts=L.CSA_PREFIX_ENTRIES, prefix_len=201)
    assert start == 201 - 128 and int(c.csa_entries[0]) == 50 and int(c.hca_entries[0]) == 1
    _prime(env, c, 0, start, 201)
    d = _cache(env)
    _fill(env, d, 0, 201)
    _same_state(d, 0, c, 0)
    _same_steps(_steps(env, d, 0, 201, 6), _steps(env, c, 0, 201, 6))


def test_periodic_checkpoint(env, tmp_path):
    """Rings from a checkpoint at 230, entries from a snapshot at 251, prefix 240:
    only tokens 230 .. 239 are recomputed."""
    L = env["L"]
    a = _cache(env)
    _fill(env, a, 0, 226)
    _steps(env, a, 0, 226, 4)
    ck = str(tmp_path / "ck230.snap")
    L.prefix_save(a, 0, ck)                                  # checkpoint: entries + rings at 230
    _steps(env, a, 0, 230, 21)
    later = str(tmp_path / "e251.snap")
    L.prefix_save(a, 0, later, parts=L.CSA_PREFIX_ENTRIES)   # entries only at 251
    c = _cache(env)
    print("prefix: checkpoint 230 + entries 251 -> prefix 240", flush=True)
    L.prefix_load(c, 1, later, parts=L.CSA_PREFIX_ENTRIES, prefix_len=240)
    with pytest.raises(L.CsaError) as ex:                    # the later snapshot holds no rings
        L.prefix_load(c, 1, later, parts=L.CSA_PREFIX_RINGS, prefix_len=240)
    assert ex.value.status == L.CSA_ERR_FORMAT
    with pytest.raises(L.CsaError) as ex:                    # sequence 0 is inactive: nothing to save
        L.prefix_save(c, 0, str(tmp_path / "x.snap"))
    assert ex.value.status == L.CSA_ERR_RANGE
    start = L.prefix_load(c, 1, ck, parts=L.CSA_PREFIX_RINGS, prefix_len=240)
    assert start == 230
    _prime(env, c, 1, start, 240)
    d = _cache(env)
    _fill(env, d, 0, 240)
    _same_state(d, 0, c, 1)
    restored = _steps(env, c, 1, 240, 6)
    _same_steps(_steps(env, d, 0, 240, 6), restored)
    _assert_oracle_steps(env, restored, 240)
