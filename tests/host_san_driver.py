"""Child process of test_host_sanitizer.py: drives the sanitizer build of the
library's host code (argument checks and snapshot files) on the CPU.  "Device"
arrays are host numpy buffers here (the build's stand-in copies with memcpy).
Exits non-zero on any failed expectation; AddressSanitizer/UBSan abort the
process on any memory or undefined-behaviour error.

usage: python host_san_driver.py LIB TMPDIR"""
import ctypes
import os
import sys

import numpy as np

LIB, TMP = sys.argv[1], sys.argv[2]
lib = ctypes.CDLL(LIB)
_i32, _i64, _f32, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
OK, NULL, SHAPE, RANGE, HIP, IO, FORMAT = 0, 1, 2, 5, 8, 9, 10
ENTRIES, RINGS = 1, 2

FIELDS = [("batch", _i32), ("n_heads", _i32), ("idx_heads", _i32), ("idx_dim", _i32), ("topk", _i32),
          ("window", _i32), ("win_rows", _i64), ("csa_cap", _i64), ("hca_cap", _i64), ("scale", _f32)] + \
         [(n, _vp) for n in ("csa_w_gate", "csa_pos_bias", "csa_w_idx", "hca_w_gate", "hca_pos_bias", "csa_sink",
                             "hca_sink", "pos", "csa_entries", "hca_entries", "csa_raw", "csa_logits", "hca_raw",
                             "hca_logits", "csa_win", "hca_win", "csa_kv", "csa_keys", "csa_key_scales", "hca_kv")] + \
         [("page_entries", _i32), ("csa_pool_pages", _i32), ("hca_pool_pages", _i32), ("csa_pages", _vp),
          ("hca_pages", _vp)]


class Cache(ctypes.Structure):
    _fields_ = FIELDS


def check(cond, what):
    if not cond:
        print("FAILED:", what, flush=True)
        sys.exit(1)


for st in range(-2, 13):
    s = ctypes.CDLL(LIB).csa_status_string
    s.restype = ctypes.c_char_p
    check(len(s(st)) > 0, f"status string {st}")


def make_cache(rng, B=2, csa_cap=96, hca_cap=6, idx_dim=64, win_rows=128):
    """A cache whose arrays are host buffers filled with random bytes."""
    arrays = {
        "pos": np.zeros(B, np.int64), "csa_entries": np.zeros(B, np.int32), "hca_entries": np.zeros(B, np.int32),
        "csa_raw": rng.integers(0, 256, (B, 8, 192 * 2), dtype=np.uint8),
        "csa_logits": rng.integers(0, 256, (B, 8, 192 * 4), dtype=np.uint8),
        "hca_raw": rng.integers(0, 256, (B, 128, 192 * 2), dtype=np.uint8),
        "hca_logits": rng.integers(0, 256, (B, 128, 192 * 4), dtype=np.uint8),
        "csa_win": rng.integers(0, 256, (B, win_rows, 256), dtype=np.uint8),
        "hca_win": rng.integers(0, 256, (B, win_rows, 256), dtype=np.uint8),
        "csa_kv": rng.integers(0, 256, (B, csa_cap, 256), dtype=np.uint8),
        "csa_keys": rng.integers(0, 256, (B, csa_cap, idx_dim // 2), dtype=np.uint8),
        "csa_key_scales": rng.integers(0, 256, (B, csa_cap, idx_dim // 32), dtype=np.uint8),
        "hca_kv": rng.integers(0, 256, (B, hca_cap, 256), dtype=np.uint8),
    }
    w = {k: np.zeros(shape, np.float32) for k, shape in (("csa_w_gate", (192, 192)), ("csa_pos_bias", (8, 192)),
                                                          ("csa_w_idx", (192, idx_dim)), ("hca_w_gate", (192, 192)),
                                                          ("hca_pos_bias", (128, 192)))}
    c = Cache(B, 32, 64, idx_dim, 16, 128, win_rows, csa_cap, hca_cap, 0.07)
    for k, a in list(arrays.items()) + list(w.items()):
        setattr(c, k, a.ctypes.data)
    return c, arrays, w


save, load = lib.prefix_save, lib.prefix_load
save.argtypes = [ctypes.POINTER(Cache), _i32, ctypes.c_char_p, _i32, _vp]
load.argtypes = [ctypes.POINTER(Cache), _i32, ctypes.c_char_p, _i32, _i64, ctypes.POINTER(_i64), _vp]
save.restype = load.restype = ctypes.c_int

rng = np.random.default_rng(5)
a, A, keep_a = make_cache(rng)
A["pos"][:] = [301, 380]
A["csa_entries"][:] = [301 // 4, 380 // 4]
A["hca_entries"][:] = [301 // 128, 380 // 128]
path = os.path.join(TMP, "seq1.snap").encode()
check(save(ctypes.byref(a), 1, path, ENTRIES | RINGS, None) == OK, "save")
b, Bq, keep_b = make_cache(np.random.default_rng(6))
pf = _i64(0)
check(load(ctypes.byref(b), 0, path, ENTRIES | RINGS, -1, ctypes.byref(pf), None) == OK, "load")
check(pf.value == 380 and Bq["pos"][0] == 380, "restored position")
n, nh = 380 // 4, 380 // 128
for k, rows in (("csa_kv", n), ("csa_keys", n), ("csa_key_scales", n), ("hca_kv", nh)):
    check(np.array_equal(Bq[k][0, :rows], A[k][1, :rows]), f"restored {k}")
for k in ("csa_raw", "csa_logits", "hca_raw", "hca_logits", "csa_win", "hca_win"):
    check(np.array_equal(Bq[k][0], A[k][1]), f"restored {k}")
# a shorter prefix from the same file, entries only
check(load(ctypes.byref(b), 1, path, ENTRIES, 200, ctypes.byref(pf), None) == OK and pf.value == 200 - 128,
      "shorter prefix")
check(Bq["csa_entries"][1] == 50 and Bq["hca_entries"][1] == 1, "shorter prefix counts")

# damaged files: every truncation point of the header and some of the body, every header byte flipped,
# bytes flipped in each section; none may load, none may touch memory it should not
data = open(path, "rb").read()
bad = os.path.join(TMP, "bad.snap").encode()
cuts = list(range(0, 200)) + list(range(200, len(data), max(1, len(data) // 97)))
for cut in cuts:
    open(bad, "wb").write(data[:cut])
    st = load(ctypes.byref(b), 0, bad, ENTRIES | RINGS, -1, ctypes.byref(pf), None)
    check(st in (FORMAT, IO), f"truncated at {cut}: status {st}")
for i in range(144):
    d = bytearray(data)
    d[i] ^= 0x5A
    open(bad, "wb").write(bytes(d))
    st = load(ctypes.byref(b), 0, bad, ENTRIES | RINGS, -1, ctypes.byref(pf), None)
    check(st in (FORMAT, RANGE, IO), f"header byte {i} flipped: status {st}")
for off in range(144, len(data), max(1, (len(data) - 144) // 211)):
    d = bytearray(data)
    d[off] ^= 0x01
    open(bad, "wb").write(bytes(d))
    st = load(ctypes.byref(b), 0, bad, ENTRIES | RINGS, -1, ctypes.byref(pf), None)
    check(st == FORMAT, f"body byte {off} flipped: status {st}")
open(bad, "wb").write(data + b"x")
check(load(ctypes.byref(b), 0, bad, ENTRIES | RINGS, -1, ctypes.byref(pf), None) == FORMAT, "trailing byte")
check(load(ctypes.byref(b), 0, os.path.join(TMP, "missing.snap").encode(), ENTRIES, -1, ctypes.byref(pf), None) == IO,
      "missing file")
# a cache that cannot hold the file's entries, a different key width, arguments out of range
small, S, keep_s = make_cache(np.random.default_rng(7), csa_cap=40)
check(load(ctypes.byref(small), 0, path, ENTRIES, -1, ctypes.byref(pf), None) == RANGE, "capacity")
other, O_, keep_o = make_cache(np.random.default_rng(8), idx_dim=128)
check(load(ctypes.byref(other), 0, path, ENTRIES, -1, ctypes.byref(pf), None) == FORMAT, "key width")
check(load(ctypes.byref(b), 2, path, ENTRIES, -1, ctypes.byref(pf), None) == SHAPE, "sequence index")
check(load(ctypes.byref(b), 0, path, 0, -1, ctypes.byref(pf), None) == SHAPE, "no parts")
check(load(ctypes.byref(b), 0, path, ENTRIES, 381, ctypes.byref(pf), None) == RANGE, "prefix beyond the file")
check(load(None, 0, path, ENTRIES, -1, ctypes.byref(pf), None) == NULL, "null cache")
check(save(ctypes.byref(a), 0, None, ENTRIES, None) == NULL, "null path")
check(save(ctypes.byref(a), 0, os.path.join(TMP, "no", "dir.snap").encode(), ENTRIES, None) == IO, "unwritable path")

# argument checks of the decode calls (kernels are not launched in this build: a valid call reports CSA_ERR_HIP)
ds = lib.decode_step
ds.argtypes = [ctypes.POINTER(Cache), _vp, _vp, _i32, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _i32, _vp, ctypes.c_size_t,
               _vp, _vp]
wsz = lib.decode_workspace_size
wsz.argtypes = [ctypes.POINTER(Cache), _i32]
wsz.restype = ctypes.c_size_t
need = wsz(ctypes.byref(a), 1)
check(need > 0, "workspace size")
ws = np.zeros(need + 256, np.uint8)
wp = (ws.ctypes.data + 255) // 256 * 256
x = np.zeros((2, 192), np.float32)
q = np.zeros((2, 64, 64), np.float32)
for bad_ws in (0, need - 1):
    check(ds(ctypes.byref(a), x.ctypes.data, x.ctypes.data, 0, q.ctypes.data, q.ctypes.data, q.ctypes.data,
             q.ctypes.data, 0, q.ctypes.data, q.ctypes.data, 0, wp, bad_ws, None, None) == 6, "decode workspace")
check(ds(ctypes.byref(a), x.ctypes.data, x.ctypes.data, 0, q.ctypes.data, q.ctypes.data, q.ctypes.data,
         q.ctypes.data, 0, q.ctypes.data, q.ctypes.data, 0, wp, need, None, None) == HIP, "decode step reaches a launch")
print("host sanitizer driver: ok", flush=True)
