"""CPU-only checks of the C-ABI boundary: the library builds and loads, exports
every function include/libcsa.h declares, and rejects bad arguments with the
documented status codes before touching the GPU (no compute call is made)."""
import ctypes
import os
import re
import struct

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libcsa.h")
LIB = os.path.join(ROOT, "long_context_compressed_compress_amd", "_native", "libcsa.so")

OK, NULL, SHAPE, DTYPE, ALIGN, RANGE, WORKSPACE, UNSUP, HIP = range(9)
F32, BF16, MIXED, MXFP4 = range(4)
P = ctypes.c_void_p
FAKE = P(0x10000)       # 16-byte aligned, never dereferenced: validation fails before any use
FAKE_MIS = P(0x10004)   # misaligned


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from long_context_compressed_compress_amd.build import build
        build(verbose=False)
    from long_context_compressed_compress_amd import libcsa
    return libcsa._lib


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?(?:int|size_t|char\s*\*|const char\s*\*)\s*\*?\s*(\w+)\s*\(",
                                 text, flags=re.M)))


def test_header_declares_the_path_calls():
    names = declared_functions()
    for n in ["csa_compress", "hca_compress", "indexer_score", "topk_select", "indexer_topk", "decode_step", "swa_attn",
              "decode_prime", "decode_workspace_size", "sparse_window_attn",
              "hca_dense_attn", "kv_pack", "mxfp4_quantize", "topk_workspace_size", "attn_workspace_size",
              "csa_status_string", "csa_last_hip_error", "prefix_save", "prefix_load"]:
        assert n in names, n


def test_library_exports_every_declared_symbol(lib):
    for n in declared_functions():
        assert hasattr(lib, n), f"libcsa.so does not export {n}"


def test_status_strings(lib):
    lib.csa_status_string.restype = ctypes.c_char_p
    for s in range(11):
        assert lib.csa_status_string(s).decode().startswith("CSA_")
    assert b"unknown" in lib.csa_status_string(99)
    assert lib.csa_last_hip_error() == 0


def test_kv_pack_validation(lib):
    f = lib.kv_pack
    assert f(FAKE, 7, 4, 192, FAKE, MIXED, 256, None) == DTYPE
    assert f(FAKE, F32, 4, 192, FAKE, MXFP4, 256, None) == DTYPE
    assert f(FAKE, F32, -1, 192, FAKE, MIXED, 256, None) == SHAPE
    assert f(None, F32, 0, 192, None, MIXED, 256, None) == OK           # nothing to do
    assert f(None, F32, 4, 192, FAKE, MIXED, 256, None) == NULL
    assert f(FAKE, F32, 4, 100, FAKE, MIXED, 256, None) == SHAPE        # row stride below 192
    assert f(FAKE, F32, 4, 192, FAKE, MIXED, 128, None) == SHAPE
    assert f(FAKE_MIS, F32, 4, 192, FAKE, MIXED, 256, None) == ALIGN
    assert f(FAKE, BF16, 4, 196, FAKE, MIXED, 256, None) == ALIGN       # 392-byte stride


def test_kv_append_validation(lib):
    f = lib.kv_append
    i64 = ctypes.c_int64

    def call(x=FAKE, xd=F32, b=8, pos=FAKE, raw=FAKE, rd=BF16, rr=128, win=FAKE, wd=MIXED, wr=128):
        return f(x, xd, b, pos, raw, rd, i64(rr), i64(0), win, wd, i64(wr), i64(0), None)
    assert call(xd=MIXED) == DTYPE                      # the new token arrives as float
    assert call(rd=MIXED) == DTYPE                      # raw tokens stay float for the compressors
    assert call(wd=MXFP4) == DTYPE
    assert call(b=-1) == SHAPE
    assert call(rr=0) == SHAPE
    assert call(wr=0) == SHAPE
    assert call(raw=None, win=None) == OK               # nothing to write
    assert call(b=0) == OK
    assert call(pos=None) == NULL
    assert call(x=None) == NULL
    assert call(win=FAKE_MIS) == ALIGN


def test_mxfp4_quantize_validation(lib):
    f = lib.mxfp4_quantize
    assert f(FAKE, 4, 48, FAKE, FAKE, None) == SHAPE
    assert f(FAKE, 4, 0, FAKE, FAKE, None) == SHAPE
    assert f(None, 4, 64, FAKE, FAKE, None) == NULL
    assert f(FAKE, 4, 64, FAKE_MIS, FAKE, None) == ALIGN
    assert f(None, 0, 64, None, None, None) == OK


def _compress(lib, **kw):
    a = dict(x=FAKE, xd=F32, batch=1, raw_rows=64, raw_base=0, wg=FAKE, pb=FAKE, e0=1, n=4, kv=FAKE, kvd=MIXED,
             n_cap=16, wi=None, di=0, ko=None, ks=None, kd=F32)
    a.update(kw)
    return lib.csa_compress(a["x"], a["xd"], a["batch"], ctypes.c_int64(a["raw_rows"]), ctypes.c_int64(a["raw_base"]),
                            a["wg"], a["pb"], ctypes.c_int64(a["e0"]), a["n"], a["kv"], a["kvd"],
                            ctypes.c_int64(a["n_cap"]), a["wi"], a["di"], a["ko"], a["ks"], a["kd"], None)


def test_csa_compress_validation(lib):
    assert _compress(lib, xd=MIXED) == DTYPE
    assert _compress(lib, kvd=MXFP4) == DTYPE
    assert _compress(lib, n=-1) == SHAPE
    assert _compress(lib, e0=14, n=4) == RANGE                     # 18 entries > n_cap 16
    assert _compress(lib, raw_base=4) == RANGE                     # entry 1 needs token 0
    assert _compress(lib, e0=2, n=4, raw_base=4, raw_rows=19) == RANGE   # tokens 4..23 need 20 rows
    assert _compress(lib, e0=0, n=8, raw_rows=31) == RANGE         # tokens 0..31 do not fit 31 rows
    assert _compress(lib, x=None) == NULL
    assert _compress(lib, wi=FAKE, di=48, ko=FAKE, ks=FAKE, kd=MXFP4) == SHAPE
    assert _compress(lib, wi=FAKE, di=64, ko=FAKE, ks=None, kd=MXFP4) == NULL
    assert _compress(lib, wi=FAKE, di=64, ko=FAKE_MIS, ks=FAKE, kd=MXFP4) == ALIGN
    assert _compress(lib, wi=FAKE, di=64, ko=FAKE, ks=FAKE, kd=BF16) == DTYPE
    assert _compress(lib, n=0, x=None) == OK


def test_hca_compress_validation(lib):
    f = lib.hca_compress
    i64 = ctypes.c_int64
    assert f(FAKE, F32, 1, i64(255), i64(0), FAKE, FAKE, i64(0), 2, FAKE, MIXED, i64(2), None) == RANGE
    assert f(FAKE, F32, 1, i64(256), i64(1), FAKE, FAKE, i64(0), 2, FAKE, MIXED, i64(2), None) == RANGE
    assert f(FAKE, F32, 1, i64(256), i64(0), FAKE, FAKE, i64(1), 2, FAKE, MIXED, i64(2), None) == RANGE
    assert f(FAKE, 5, 1, i64(256), i64(0), FAKE, FAKE, i64(0), 2, FAKE, MIXED, i64(2), None) == DTYPE
    assert f(FAKE, F32, 1, i64(256), i64(0), None, FAKE, i64(0), 2, FAKE, MIXED, i64(2), None) == NULL


def _index(lib, **kw):
    a = dict(q=FAKE, qs=FAKE, qd=MXFP4, w=FAKE, k=FAKE, ks=FAKE, kd=MXFP4, batch=8, n_q=1, h=64, d=64, n_cap=1024,
             ne=FAKE, qp=FAKE, ratio=4, sc=FAKE, sd=BF16)
    a.update(kw)
    return lib.indexer_score(a["q"], a["qs"], a["qd"], a["w"], a["k"], a["ks"], a["kd"], a["batch"], a["n_q"], a["h"],
                             a["d"], ctypes.c_int64(a["n_cap"]), a["ne"], a["qp"], a["ratio"], a["sc"], a["sd"], None)


def test_indexer_validation(lib):
    assert _index(lib, sd=F32) == DTYPE                 # MXFP4 scores are BF16
    assert _index(lib, qd=F32, kd=F32, sd=BF16) == DTYPE
    assert _index(lib, qd=F32, sd=F32) == DTYPE          # float32 q with MXFP4 keys still scores in BF16
    assert _index(lib, qd=F32, qs=None, ks=None) == NULL  # ... and needs the key scales (q scales unused)
    assert _index(lib, qd=F32, qs=None, q=FAKE_MIS) == ALIGN
    assert _index(lib, qd=F32, h=48) == UNSUP
    assert _index(lib, qd=MXFP4, kd=F32) == DTYPE
    assert _index(lib, h=48) == UNSUP
    assert _index(lib, d=96) == UNSUP
    assert _index(lib, h=256) == UNSUP
    assert _index(lib, ratio=0) == SHAPE
    assert _index(lib, qs=None) == NULL
    assert _index(lib, q=FAKE_MIS) == ALIGN
    assert _index(lib, qd=F32, kd=F32, sd=F32, h=128, d=256) == UNSUP   # too large for the fp32 path's LDS
    assert _index(lib, batch=0) == OK


def test_topk_validation(lib):
    f = lib.topk_select
    i64 = ctypes.c_int64
    lib.topk_workspace_size.restype = ctypes.c_size_t
    assert f(FAKE, MIXED, 1, 1, i64(10), FAKE, FAKE, 4, 4, FAKE, None, 0, None) == DTYPE
    assert f(FAKE, BF16, 1, 1, i64(10), FAKE, FAKE, 4, 0, FAKE, None, 0, None) == SHAPE
    assert f(FAKE, BF16, 1, 1, i64(10), FAKE, FAKE, 0, 4, FAKE, None, 0, None) == SHAPE
    assert f(FAKE, BF16, 1, 1, i64(10), None, FAKE, 4, 4, FAKE, None, 0, None) == NULL
    assert f(FAKE, BF16, 0, 1, i64(10), None, None, 4, 4, None, None, 0, None) == OK
    need = lib.topk_workspace_size(8, 1, i64(262144), 1024, BF16)
    if need:
        assert f(FAKE, BF16, 8, 1, i64(262144), FAKE, FAKE, 4, 1024, FAKE, None, 0, None) == WORKSPACE


def test_indexer_topk_validation(lib):
    """The fused call checks the arguments of both calls it stands for."""
    i64 = ctypes.c_int64
    lib.topk_workspace_size.restype = ctypes.c_size_t
    need = lib.topk_workspace_size(8, 1, i64(262144), 1024, BF16)

    def call(**kw):
        a = dict(q=FAKE, qs=FAKE, qd=MXFP4, w=FAKE, k=FAKE, ks=FAKE, kd=MXFP4, batch=8, n_q=1, h=64, d=64,
                 n_cap=262144, ne=FAKE, qp=FAKE, ratio=4, sc=FAKE, sd=BF16, topk=1024, idx=FAKE, ws=FAKE, wsb=need,
                 ev=None)
        a.update(kw)
        return lib.indexer_topk(a["q"], a["qs"], a["qd"], a["w"], a["k"], a["ks"], a["kd"], a["batch"], a["n_q"],
                                a["h"], a["d"], i64(a["n_cap"]), a["ne"], a["qp"], a["ratio"], a["sc"], a["sd"],
                                a["topk"], a["idx"], a["ws"], ctypes.c_size_t(a["wsb"]), a["ev"], None)
    assert call(sd=F32) == DTYPE              # as indexer_score: MXFP4 keys score in BF16
    assert call(h=48) == UNSUP
    assert call(qs=None) == NULL
    assert call(q=FAKE_MIS) == ALIGN
    assert call(topk=0) == SHAPE              # as topk_select
    assert call(idx=None) == NULL
    assert need > 0 and call(ws=None, wsb=0) == WORKSPACE
    assert call(wsb=need - 16) == WORKSPACE
    assert call(ws=FAKE_MIS) == ALIGN
    assert call(batch=0, q=None, idx=None) == OK
    assert call(qd=F32, kd=F32, sd=F32, n_cap=0, ws=None, wsb=0, idx=None) == NULL   # rows still need idx_out
    assert call(ev=(P * 2)(FAKE, None)) == NULL    # the stage events come as a pair


def test_attention_validation_and_workspace(lib):
    i64 = ctypes.c_int64
    f = lib.sparse_window_attn
    lib.attn_workspace_size.restype = ctypes.c_size_t
    ws = lib.attn_workspace_size(8, 1, 128, i64(1152), BF16, MIXED)
    assert ws > 0 and ws % (128 * (192 * 2 + 8) * 8) == 0             # decode splits the key list: FP16 O/l + fp32 (m, l)
    assert lib.attn_workspace_size(1, 4096, 64, i64(640), BF16, MIXED) == 0   # many queries: no split
    assert lib.attn_workspace_size(1, 16, 8, i64(192), F32, F32) == 0

    def call(**kw):
        a = dict(q=FAKE, qd=BF16, b=8, t=1, h=128, kv=FAKE, kvd=MIXED, n_cap=1000, ne=FAKE, ratio=4, idx=FAKE, k=1024,
                 win=FAKE, wr=128, wb=0, qp=FAKE, W=128, scale=0.07, sink=None, out=FAKE, od=BF16, lse=None, ws=FAKE,
                 wsb=ws)
        a.update(kw)
        return f(a["q"], a["qd"], a["b"], a["t"], a["h"], a["kv"], a["kvd"], i64(a["n_cap"]), a["ne"], a["ratio"],
                 a["idx"], a["k"], a["win"], i64(a["wr"]), i64(a["wb"]), a["qp"], a["W"], ctypes.c_float(a["scale"]),
                 a["sink"], a["out"], a["od"], a["lse"], a["ws"], ctypes.c_size_t(a["wsb"]), None)
    assert call(ws=None, wsb=0) == WORKSPACE
    assert call(wsb=ws - 16) == WORKSPACE
    assert call(qd=MIXED) == DTYPE
    assert call(od=MIXED) == DTYPE
    assert call(wr=100) == RANGE                  # ring smaller than the window
    assert call(idx=None) == NULL
    assert call(win=None) == NULL
    assert call(q=FAKE_MIS) == ALIGN
    assert call(h=0) == SHAPE
    assert call(k=-1) == SHAPE
    assert call(scale=0.0) == RANGE               # the scale must be finite and positive
    assert call(scale=-0.07) == RANGE
    assert call(scale=float("inf")) == RANGE
    assert call(scale=float("nan")) == RANGE
    assert call(b=0) == OK


def test_decode_cache_struct_layout_matches_header(tmp_path):
    """The ctypes mirror of csa_decode_cache has the C compiler's size and offsets."""
    import shutil
    import subprocess
    from long_context_compressed_compress_amd import libcsa as L
    if shutil.which("gcc") is None:
        pytest.skip("no C compiler")
    names = [f[0] for f in L._DecodeCacheC._fields_]
    src = tmp_path / "layout.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "libcsa.h"\nint main(void) {\n'
                   '  printf("%zu\\n", sizeof(csa_decode_cache));\n' +
                   "".join(f'  printf("%zu\\n", offsetof(csa_decode_cache, {n}));\n' for n in names) +
                   "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)], check=True)
    got = [int(v) for v in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()]
    assert got[0] == ctypes.sizeof(L._DecodeCacheC)
    assert got[1:] == [getattr(L._DecodeCacheC, n).offset for n in names]


def _decode_cache(**kw):
    from long_context_compressed_compress_amd import libcsa as L
    c = L._DecodeCacheC(8, 128, 64, 64, 1024, 128, 128, 262208, 8256, 0.072)
    for n, t in L._DecodeCacheC._fields_[10:]:
        if t is ctypes.c_void_p:
            setattr(c, n, 0x10000)
    c.csa_sink = c.hca_sink = None
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_decode_validation(lib):
    """decode_step / decode_prime check the cache description and arguments first."""
    from long_context_compressed_compress_amd import libcsa as L
    L_ = L._lib

    def step(c, **kw):
        a = dict(x=FAKE, xd=BF16, q=FAKE, w=FAKE, qd=BF16, out=FAKE, od=BF16, ws=P(0x100000),
                 wsb=L_.decode_workspace_size(ctypes.byref(c), BF16), ev=None)
        a.update(kw)
        return L_.decode_step(ctypes.byref(c), a["x"], a["x"], a["xd"], a["q"], a["w"], a["q"], a["q"], a["qd"],
                              a["out"], a["out"], a["od"], a["ws"], a["wsb"], a["ev"], None)
    c = _decode_cache()
    need = L_.decode_workspace_size(ctypes.byref(c), BF16)
    assert need > 8 * 262208 * 2                         # holds the score rows
    assert L_.decode_workspace_size(None, BF16) == 0
    assert step(c, ws=None) == WORKSPACE
    assert step(c, wsb=need - 1) == WORKSPACE
    assert step(c, ws=P(0x100010)) == ALIGN              # 256-byte alignment
    assert step(c, xd=MIXED) == DTYPE
    assert step(c, out=None) == NULL
    assert step(c, q=FAKE_MIS) == ALIGN
    assert step(c, ev=(P * 2)(FAKE, None)) == NULL
    assert step(_decode_cache(idx_heads=48)) == UNSUP
    assert step(_decode_cache(idx_dim=96)) == UNSUP
    assert step(_decode_cache(window=200)) == SHAPE      # window larger than its ring
    assert step(_decode_cache(batch=0)) == SHAPE
    assert step(_decode_cache(scale=0.0)) == RANGE
    assert step(_decode_cache(hca_logits=None)) == NULL
    assert step(_decode_cache(csa_kv=0x10008)) == ALIGN
    assert L_.decode_prime(ctypes.byref(c), FAKE, FAKE, BF16, 0, None) == SHAPE
    assert L_.decode_prime(ctypes.byref(c), FAKE, None, BF16, 4, None) == NULL
    assert L_.decode_prime(ctypes.byref(c), FAKE, FAKE, MIXED, 4, None) == DTYPE


def test_paged_cache_validation(lib):
    """The paged layout's description is checked before any launch: a page of a
    power of two >= 32 entries dividing both capacities, pools of at least one
    page and fewer than 2^31 rows, both page tables given; decode_fork needs a
    paged cache and sequences in range."""
    from long_context_compressed_compress_amd import libcsa as L
    L_ = L._lib

    def paged(**kw):
        a = dict(csa_cap=262144, hca_cap=8192, page_entries=256, csa_pool_pages=8192, hca_pool_pages=256)
        a.update(kw)
        return _decode_cache(**a)

    def size(c):
        return L_.decode_workspace_size(ctypes.byref(c), BF16)

    def fork(c, src=0, dst=1):
        return L_.decode_fork(ctypes.byref(c), src, dst, None)
    assert size(paged()) > 0
    for bad in (dict(page_entries=16), dict(page_entries=96), dict(page_entries=-256), dict(csa_cap=262144 + 128),
                dict(hca_cap=8192 + 128), dict(csa_pool_pages=0), dict(hca_pool_pages=0),
                dict(page_entries=1 << 20, csa_cap=1 << 20, hca_cap=1 << 20, csa_pool_pages=2048)):
        assert size(paged(**bad)) == 0, bad
        assert fork(paged(**bad)) == SHAPE, bad
    assert fork(paged(csa_pages=None)) == NULL
    assert fork(paged(hca_pages=None)) == NULL
    assert size(_decode_cache(csa_pages=None, hca_pages=None)) > 0     # contiguous: the tables are not used
    assert fork(_decode_cache()) == UNSUP
    assert fork(paged(), 0, 8) == SHAPE
    assert fork(paged(), -1, 0) == SHAPE
    assert fork(paged(), 3, 3) == OK                                    # a sequence forked onto itself: nothing to do


def test_swa_attn_validation(lib):
    i64 = ctypes.c_int64
    f = lib.swa_attn

    def call(**kw):
        a = dict(q=FAKE, qd=BF16, b=8, t=1, h=128, win=FAKE, wd=MIXED, wr=128, wb=0, qp=FAKE, W=128, scale=0.07,
                 sink=None, out=FAKE, od=BF16, lse=None, ws=None, wsb=0)
        a.update(kw)
        return f(a["q"], a["qd"], a["b"], a["t"], a["h"], a["win"], a["wd"], i64(a["wr"]), i64(a["wb"]), a["qp"],
                 a["W"], ctypes.c_float(a["scale"]), a["sink"], a["out"], a["od"], a["lse"], a["ws"],
                 ctypes.c_size_t(a["wsb"]), None)
    assert call(scale=0.0) == RANGE
    assert call(W=0) == SHAPE
    assert call(win=None) == NULL
    assert call(qp=None) == NULL
    assert call(wr=100) == RANGE              # ring smaller than the window
    assert call(q=FAKE_MIS) == ALIGN
    assert call(qd=MIXED) == DTYPE
    assert call(b=0) == OK


# --- prefix snapshots: every check of the file happens before the cache is touched
_IO, _FORMAT = 9, 10
_HDR = "<8sIIqqqqii10Q"   # magic, version, parts, pos, csa_count, hca_count, win_rows, idx_dim, row_bytes, 10 sums
# ... then a checksum of those 136 bytes (format version 2)


def _snapshot_sum(data: bytes) -> int:
    """The file format's 64-bit section checksum (word-wise multiply-rotate)."""
    M = (1 << 64) - 1
    n = len(data)
    h = 0x9E3779B97F4A7C15 ^ n
    i = 0
    while i + 8 <= n:
        w = int.from_bytes(data[i:i + 8], "little")
        h = ((h ^ ((w * 0xBF58476D1CE4E5B9) & M)) * 0x94D049BB133111EB) & M
        h = ((h << 29) | (h >> 35)) & M
        i += 8
    w = int.from_bytes(data[i:] + bytes(8 - (n - i)), "little")
    h = ((h ^ ((w * 0xBF58476D1CE4E5B9) & M) ^ (n - i)) * 0x94D049BB133111EB) & M
    return h ^ (h >> 31)


def _snapshot(path, pos=1000, nc=250, nh=7, parts=1, idx_dim=64, win_rows=128, magic=b"CSAPFX01", version=2,
              bad_sum=False, bad_head=False, trailing=b"", sections=None, head_sum=True):
    kb, sb = idx_dim // 2, idx_dim // 32
    sizes = [nc * 256, nc * kb, nc * sb, nh * 256, 8 * 192 * 2, 8 * 192 * 4, 128 * 192 * 2, 128 * 192 * 4,
             win_rows * 256, win_rows * 256]
    data = list(sections) if sections is not None else []
    if sections is None:
        for k, n in enumerate(sizes):
            held = (parts & 1) if k < 4 else (parts & 2)
            data.append(bytes((k * 7 + i) & 255 for i in range(n)) if held else b"")
    sums = [_snapshot_sum(d) if d else 0 for d in data]
    if bad_sum:
        sums[0] ^= 1
    hdr = struct.pack(_HDR, magic, version, parts, pos, nc, nh, win_rows, idx_dim, 256, *sums)
    assert len(hdr) == 136
    if head_sum:
        hdr += struct.pack("<Q", _snapshot_sum(hdr) ^ int(bad_head))
    with open(path, "wb") as f:
        f.write(hdr + b"".join(data) + trailing)
    return str(path)


def test_prefix_snapshot_validation(lib, tmp_path):
    """prefix_save / prefix_load: argument checks, then the file's header, sizes,
    parts, prefix length, capacities and checksums, all before any copy."""
    i64 = ctypes.c_int64
    c = _decode_cache()
    pf = i64(-7)

    def load(path, parts=1, prefix=-1, cache=c, seq=0):
        return lib.prefix_load(ctypes.byref(cache), seq, str(path).encode(), parts, i64(prefix), ctypes.byref(pf),
                               None)
    good = _snapshot(tmp_path / "good.snap")
    assert lib.prefix_save(ctypes.byref(c), 0, None, 1, None) == NULL
    assert lib.prefix_save(ctypes.byref(c), 8, b"x", 1, None) == SHAPE          # seq out of range
    assert lib.prefix_save(ctypes.byref(c), 0, b"x", 0, None) == SHAPE          # no part
    assert lib.prefix_save(ctypes.byref(c), 0, b"x", 4, None) == SHAPE          # unknown part
    assert lib.prefix_save(ctypes.byref(_decode_cache(idx_dim=96)), 0, b"x", 1, None) == UNSUP
    assert load(good, parts=3 << 1) == SHAPE
    assert load(good, seq=-1) == SHAPE
    assert load(tmp_path / "missing.snap") == _IO
    with open(tmp_path / "short.snap", "wb") as f:
        f.write(b"CSAPFX01" + bytes(10))
    assert load(tmp_path / "short.snap") == _FORMAT                             # truncated header
    assert load(_snapshot(tmp_path / "m.snap", magic=b"CSAPFX02")) == _FORMAT
    assert load(_snapshot(tmp_path / "v.snap", version=3)) == _FORMAT
    assert load(_snapshot(tmp_path / "v1.snap", version=1, head_sum=False)) == _FORMAT   # the older header
    assert load(_snapshot(tmp_path / "hs.snap", bad_head=True)) == _FORMAT     # damaged header checksum
    assert load(good, parts=2) == _FORMAT                                      # rings not in the file
    assert load(_snapshot(tmp_path / "d.snap", idx_dim=128)) == _FORMAT        # key width of another cache
    assert load(_snapshot(tmp_path / "w.snap", parts=3, win_rows=64), parts=3, prefix=1000) == _FORMAT
    assert load(_snapshot(tmp_path / "c.snap", nc=251)) == _FORMAT             # more CSA entries than 1000 tokens make
    assert load(_snapshot(tmp_path / "h.snap", nh=8)) == _FORMAT
    assert load(_snapshot(tmp_path / "n.snap", pos=-1, nc=0, nh=0)) == _FORMAT
    big = _snapshot(tmp_path / "big.snap", pos=1 << 40, nc=1 << 36, nh=0, sections=[b""] * 10)
    assert load(big) == _FORMAT                                                 # sizes beyond the file
    assert load(good, prefix=1001) == RANGE                                     # prefix longer than the snapshot
    assert load(good, prefix=-2) == RANGE
    assert load(_snapshot(tmp_path / "r.snap", parts=3), parts=3, prefix=999) == RANGE   # rings hold token 999
    assert load(good, cache=_decode_cache(csa_cap=200)) == RANGE                # entries over the capacity
    small = _snapshot(tmp_path / "small.snap", pos=40, nc=10, nh=0, bad_sum=True)  # entries-only file shorter
    assert load(small) == _FORMAT and os.path.getsize(small) < 128 * 256        # than a window: the checksum,
    # not the absent window rows, decides (rows past the file size are only checked for files with rings)
    assert load(_snapshot(tmp_path / "wr.snap", pos=40, nc=10, nh=0, parts=3, win_rows=1 << 20,
                          sections=[b""] * 10), parts=3, prefix=40) == _FORMAT
    assert load(_snapshot(tmp_path / "s.snap", bad_sum=True)) == _FORMAT       # damaged section
    assert load(_snapshot(tmp_path / "t.snap", trailing=b"\0")) == _FORMAT     # trailing bytes
    trunc = tmp_path / "tr.snap"
    with open(good, "rb") as f, open(trunc, "wb") as g:
        g.write(f.read()[:-1])
    assert load(trunc) == _FORMAT                                               # last section cut short
    assert pf.value == -7                                                       # nothing reported on failure


def test_decode_layer_calls_validation(lib):
    """decode_csa_layer / decode_hca_layer: the checks of decode_step, before any launch."""
    from long_context_compressed_compress_amd import libcsa as L
    L_ = L._lib
    c = _decode_cache()
    need = L_.decode_workspace_size(ctypes.byref(c), BF16)

    def csa(c, **kw):
        a = dict(x=FAKE, xd=BF16, qi=FAKE, w=FAKE, q=FAKE, qd=BF16, out=FAKE, od=BF16, ws=P(0x100000), wsb=need, ev=None)
        a.update(kw)
        return L_.decode_csa_layer(ctypes.byref(c), a["x"], a["xd"], a["qi"], a["w"], a["q"], a["qd"], a["out"],
                                   a["od"], a["ws"], a["wsb"], a["ev"], None)

    def hca(c, **kw):
        a = dict(x=FAKE, xd=BF16, q=FAKE, qd=BF16, out=FAKE, od=BF16, ws=P(0x100000), wsb=need)
        a.update(kw)
        return L_.decode_hca_layer(ctypes.byref(c), a["x"], a["xd"], a["q"], a["qd"], a["out"], a["od"], a["ws"],
                                   a["wsb"], None)
    for call in (csa, hca):
        assert call(c, ws=None) == WORKSPACE
        assert call(c, wsb=need - 1) == WORKSPACE
        assert call(c, ws=P(0x100010)) == ALIGN
        assert call(c, xd=MIXED) == DTYPE
        assert call(c, od=MIXED) == DTYPE
        assert call(c, out=None) == NULL
        assert call(c, x=None) == NULL
        assert call(c, q=FAKE_MIS) == ALIGN
        assert call(_decode_cache(batch=0)) == SHAPE
        assert call(_decode_cache(idx_dim=96)) == UNSUP
        assert call(_decode_cache(hca_kv=None)) == NULL
    assert csa(c, qi=None) == NULL
    assert csa(c, ev=(P * 2)(FAKE, None)) == NULL
