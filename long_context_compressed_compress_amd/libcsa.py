"""Thin Python binding of libcsa (the C-ABI in include/libcsa.h).

Argument marshalling only: every function passes torch tensors' device
pointers, sizes and dtype codes to the C function of the same name, on torch's
current stream, and raises CsaError on a non-zero status.  No step of the CSA /
HCA path runs here.  PyTorch supplies device memory and the stream.

The shared library is loaded from this package directory (built by
``python -m long_context_compressed_compress_amd.build``); importing this
module fails loudly if it is missing.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_native", "libcsa.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "libcsa.h")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"libcsa.so not built at {LIB_PATH}; run python -m long_context_compressed_compress_amd.build")
_lib = ctypes.CDLL(LIB_PATH)

# status codes / dtypes (include/libcsa.h)
CSA_OK, CSA_ERR_NULL, CSA_ERR_SHAPE, CSA_ERR_DTYPE, CSA_ERR_ALIGN = 0, 1, 2, 3, 4
CSA_ERR_RANGE, CSA_ERR_WORKSPACE, CSA_ERR_UNSUPPORTED, CSA_ERR_HIP = 5, 6, 7, 8
CSA_ERR_IO, CSA_ERR_FORMAT = 9, 10
CSA_PREFIX_ENTRIES, CSA_PREFIX_RINGS = 1, 2
CSA_F32, CSA_BF16, CSA_KV_MIXED, CSA_MXFP4 = 0, 1, 2, 3
DIM = 192
ROW_BYTES = {CSA_F32: 768, CSA_BF16: 384, CSA_KV_MIXED: 256}

_vp, _i32, _i64, _f32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_SIGS = {
    "csa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "csa_last_hip_error": (ctypes.c_int, []),
    "kv_pack": (ctypes.c_int, [_vp, _i32, _i64, _i64, _vp, _i32, _i64, _vp]),
    "kv_append": (ctypes.c_int, [_vp, _i32, _i32, _vp, _vp, _i32, _i64, _i64, _vp, _i32, _i64, _i64, _vp]),
    "mxfp4_quantize": (ctypes.c_int, [_vp, _i64, _i32, _vp, _vp, _vp]),
    "csa_compress": (ctypes.c_int, [_vp, _i32, _i32, _i64, _i64, _vp, _vp, _i64, _i32, _vp, _i32, _i64,
                                    _vp, _i32, _vp, _vp, _i32, _vp]),
    "hca_compress": (ctypes.c_int, [_vp, _i32, _i32, _i64, _i64, _vp, _vp, _i64, _i32, _vp, _i32, _i64, _vp]),
    "indexer_score": (ctypes.c_int, [_vp, _vp, _i32, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i64,
                                     _vp, _vp, _i32, _vp, _i32, _vp]),
    "topk_workspace_size": (_sz, [_i32, _i32, _i64, _i32, _i32]),
    "topk_select": (ctypes.c_int, [_vp, _i32, _i32, _i32, _i64, _vp, _vp, _i32, _i32, _vp, _vp, _sz, _vp]),
    "indexer_topk": (ctypes.c_int, [_vp, _vp, _i32, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i64,
                                    _vp, _vp, _i32, _vp, _i32, _i32, _vp, _vp, _sz, _vp, _vp]),
    "attn_workspace_size": (_sz, [_i32, _i32, _i32, _i64, _i32, _i32]),
    "sparse_window_attn": (ctypes.c_int, [_vp, _i32, _i32, _i32, _i32, _vp, _i32, _i64, _vp, _i32, _vp, _i32,
                                          _vp, _i64, _i64, _vp, _i32, _f32, _vp, _vp, _i32, _vp, _vp, _sz, _vp]),
    "hca_dense_attn": (ctypes.c_int, [_vp, _i32, _i32, _i32, _i32, _vp, _i32, _i64, _vp, _i32, _vp, _i64, _i64,
                                      _vp, _i32, _f32, _vp, _vp, _i32, _vp, _vp, _sz, _vp]),
    "swa_attn": (ctypes.c_int, [_vp, _i32, _i32, _i32, _i32, _vp, _i32, _i64, _i64, _vp, _i32, _f32, _vp, _vp, _i32,
                                _vp, _vp, _sz, _vp]),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


class CsaError(RuntimeError):
    def __init__(self, status: int, call: str):
        msg = _lib.csa_status_string(status).decode()
        if status == CSA_ERR_HIP:
            msg += f" (hipError {_lib.csa_last_hip_error()})"
        super().__init__(f"{call}: {msg}")
        self.status = status


def _check(status: int, call: str) -> None:
    if status != CSA_OK:
        raise CsaError(status, call)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is not None:
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _float_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return CSA_F32
    if t.dtype == torch.bfloat16:
        return CSA_BF16
    raise TypeError(f"expected float32 or bfloat16, got {t.dtype}")


def _row_code(t: torch.Tensor) -> int:
    """Storage format of a tensor of KV rows: float32/bfloat16 [..., 192] or uint8 [..., 256] (mixed)."""
    if t.dtype == torch.uint8:
        if t.shape[-1] != 256:
            raise ValueError("mixed KV rows are uint8 [..., 256]")
        return CSA_KV_MIXED
    if t.shape[-1] != DIM:
        raise ValueError("KV rows have 192 values")
    return _float_code(t)


def status_string(status: int) -> str:
    return _lib.csa_status_string(status).decode()


# ---------------------------------------------------------------------------
def kv_pack(x: torch.Tensor, out: torch.Tensor, stream=None) -> torch.Tensor:
    """x [n, 192] float32/bfloat16 rows (any row stride) -> out [n, ...] rows in out's format."""
    n = x.shape[0]
    _check(_lib.kv_pack(_ptr(x), _float_code(x), n, x.stride(0), _ptr(out), _row_code(out),
                        out.stride(0) * out.element_size(), _stream(stream)), "kv_pack")
    return out


def kv_append(x, pos, raw_ring=None, raw_base=0, win_ring=None, win_base=0, stream=None):
    """x [B, 192] float32/bfloat16; pos [B] int64 (device); raw_ring [B, rows, 192] float32/bfloat16
    and/or win_ring [B, rows, 192 | 256 bytes]: row (pos - base) mod rows of each ring receives x[b]."""
    B = x.shape[0]
    rd = 0 if raw_ring is None else _float_code(raw_ring)
    wd = 0 if win_ring is None else _row_code(win_ring)
    _check(_lib.kv_append(_ptr(x), _float_code(x), B, _ptr(pos), _ptr(raw_ring), rd,
                          0 if raw_ring is None else raw_ring.shape[1], raw_base, _ptr(win_ring), wd,
                          0 if win_ring is None else win_ring.shape[1], win_base, _stream(stream)), "kv_append")


def mxfp4_quantize(x: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor, stream=None):
    d = x.shape[-1]
    _check(_lib.mxfp4_quantize(_ptr(x), x.numel() // d, d, _ptr(codes), _ptr(scales), _stream(stream)),
           "mxfp4_quantize")
    return codes, scales


def csa_compress(x_raw, raw_base, w_gate, pos_bias, entry_begin, n_new, kv_out, w_idx=None, key_out=None,
                 key_scales=None, stream=None):
    """x_raw [B, raw_rows, 192] ring; kv_out [B, n_cap, row]; key_out float32 [B, n_cap, d_idx] or
    uint8 codes [B, n_cap, d_idx/2] (with key_scales) for MXFP4 keys."""
    B, raw_rows = x_raw.shape[0], x_raw.shape[1]
    d_idx, key_dtype = 0, CSA_F32
    if w_idx is not None:
        d_idx = w_idx.shape[1]
        key_dtype = CSA_F32 if key_out.dtype == torch.float32 else CSA_MXFP4
    _check(_lib.csa_compress(_ptr(x_raw), _float_code(x_raw), B, raw_rows, raw_base, _ptr(w_gate), _ptr(pos_bias),
                             entry_begin, n_new, _ptr(kv_out), _row_code(kv_out), kv_out.shape[1], _ptr(w_idx),
                             d_idx, _ptr(key_out), _ptr(key_scales), key_dtype, _stream(stream)), "csa_compress")
    return kv_out


def hca_compress(x_raw, raw_base, w_gate, pos_bias, entry_begin, n_new, kv_out, stream=None):
    B, raw_rows = x_raw.shape[0], x_raw.shape[1]
    _check(_lib.hca_compress(_ptr(x_raw), _float_code(x_raw), B, raw_rows, raw_base, _ptr(w_gate), _ptr(pos_bias),
                             entry_begin, n_new, _ptr(kv_out), _row_code(kv_out), kv_out.shape[1], _stream(stream)),
           "hca_compress")
    return kv_out


def _indexer_args(q, k, scores):
    B, T, H = q.shape[0], q.shape[1], q.shape[2]
    if q.dtype == torch.uint8:
        qd = kd = CSA_MXFP4
        D = q.shape[3] * 2
    elif k.dtype == torch.uint8:
        qd, kd = CSA_F32, CSA_MXFP4
        D = q.shape[3]
    else:
        qd = kd = CSA_F32
        D = q.shape[3]
    sd = CSA_BF16 if scores.dtype == torch.bfloat16 else CSA_F32
    return B, T, H, D, qd, kd, sd, scores.shape[2]


def indexer_score(q, w, k, n_entries, q_pos, ratio, scores, q_scales=None, k_scales=None, n_heads=None,
                  d_idx=None, stream=None):
    """FP32 path: q float32 [B, T, H, D], k float32 [B, n_cap, D], scores float32 [B, T, n_cap].
    MXFP4 path: q uint8 codes [B, T, H, D/2] + q_scales, k uint8 codes [B, n_cap, D/2] + k_scales,
    scores bfloat16 [B, T, n_cap].  With MXFP4 keys (k uint8) and q float32, q is quantized to
    MXFP4 inside the call."""
    B, T, H, D, qd, kd, sd, n_cap = _indexer_args(q, k, scores)
    _check(_lib.indexer_score(_ptr(q), _ptr(q_scales), qd, _ptr(w), _ptr(k), _ptr(k_scales), kd, B, T, H, D, n_cap,
                              _ptr(n_entries), _ptr(q_pos), ratio, _ptr(scores), sd, _stream(stream)), "indexer_score")
    return scores


def indexer_topk(q, w, k, n_entries, q_pos, ratio, scores, topk, idx_out, q_scales=None, k_scales=None,
                 workspace=None, stage_events=None, stream=None):
    """indexer_score into `scores`, then topk_select of `topk` entries into idx_out [B, T, topk].
    stage_events: optional pair of torch.cuda.Event recorded around the scoring kernel."""
    B, T, H, D, qd, kd, sd, n_cap = _indexer_args(q, k, scores)
    need = topk_workspace_size(B, T, n_cap, topk, sd)
    if workspace is None and need > 0:  # must start zero-filled; calls leave it zero-filled
        workspace = torch.zeros(need, dtype=torch.uint8, device=scores.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    evs = None
    if stage_events is not None:
        for e in stage_events:
            if e.cuda_event == 0:   # torch creates the HIP event at its first record
                e.record()
        evs = (ctypes.c_void_p * 2)(*[ctypes.c_void_p(e.cuda_event) for e in stage_events])
    _check(_lib.indexer_topk(_ptr(q), _ptr(q_scales), qd, _ptr(w), _ptr(k), _ptr(k_scales), kd, B, T, H, D, n_cap,
                             _ptr(n_entries), _ptr(q_pos), ratio, _ptr(scores), sd, topk, _ptr(idx_out),
                             _ptr(workspace), ws_bytes, evs, _stream(stream)), "indexer_topk")
    return idx_out


def topk_workspace_size(batch, n_q, n_cap, k, score_dtype):
    return _lib.topk_workspace_size(batch, n_q, n_cap, k, score_dtype)


def topk_select(scores, n_entries, q_pos, ratio, k, idx_out, workspace=None, stream=None):
    B, T, n_cap = scores.shape
    sd = CSA_BF16 if scores.dtype == torch.bfloat16 else CSA_F32
    need = topk_workspace_size(B, T, n_cap, k, sd)
    if workspace is None and need > 0:  # must start zero-filled; calls leave it zero-filled
        workspace = torch.zeros(need, dtype=torch.uint8, device=scores.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.topk_select(_ptr(scores), sd, B, T, n_cap, _ptr(n_entries), _ptr(q_pos), ratio, k, _ptr(idx_out),
                            _ptr(workspace), ws_bytes, _stream(stream)), "topk_select")
    return idx_out


def attn_workspace_size(batch, n_q, n_heads, max_keys, q_dtype, kv_dtype):
    return _lib.attn_workspace_size(batch, n_q, n_heads, max_keys, q_dtype, kv_dtype)


def _attn_ws(q, kv, max_keys, workspace):
    B, T, H = q.shape[0], q.shape[1], q.shape[2]
    need = attn_workspace_size(B, T, H, max_keys, _float_code(q), _row_code(kv))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    return workspace, (0 if workspace is None else workspace.numel() * workspace.element_size())


def sparse_window_attn(q, kv, n_entries, ratio, idx, win, win_base, q_pos, window, scale, out, sink=None,
                       lse=None, workspace=None, stream=None):
    """q [B, T, H, 192]; kv [B, n_cap, row]; idx int32 [B, T, k]; win [B, win_rows, row] ring;
    out [B, T, H, 192] float32/bfloat16; lse float32 [B, T, H] or None."""
    B, T, H = q.shape[0], q.shape[1], q.shape[2]
    k = idx.shape[2]
    workspace, ws_bytes = _attn_ws(q, kv, k + window, workspace)
    _check(_lib.sparse_window_attn(_ptr(q), _float_code(q), B, T, H, _ptr(kv), _row_code(kv), kv.shape[1],
                                   _ptr(n_entries), ratio, _ptr(idx), k, _ptr(win), win.shape[1], win_base,
                                   _ptr(q_pos), window, scale, _ptr(sink), _ptr(out), _float_code(out), _ptr(lse),
                                   _ptr(workspace), ws_bytes, _stream(stream)), "sparse_window_attn")
    return out


def hca_dense_attn(q, kv, n_entries, ratio, win, win_base, q_pos, window, scale, out, sink=None, lse=None,
                   workspace=None, stream=None):
    B, T, H = q.shape[0], q.shape[1], q.shape[2]
    workspace, ws_bytes = _attn_ws(q, kv, kv.shape[1] + window, workspace)
    _check(_lib.hca_dense_attn(_ptr(q), _float_code(q), B, T, H, _ptr(kv), _row_code(kv), kv.shape[1],
                               _ptr(n_entries), ratio, _ptr(win), win.shape[1], win_base, _ptr(q_pos), window, scale,
                               _ptr(sink), _ptr(out), _float_code(out), _ptr(lse), _ptr(workspace), ws_bytes,
                               _stream(stream)), "hca_dense_attn")
    return out


def swa_attn(q, win, win_base, q_pos, window, scale, out, sink=None, lse=None, workspace=None, stream=None):
    """Sliding-window-only attention: q [B, T, H, 192]; win [B, win_rows, row] ring; out [B, T, H, 192]."""
    B, T, H = q.shape[0], q.shape[1], q.shape[2]
    workspace, ws_bytes = _attn_ws(q, win, window, workspace)
    _check(_lib.swa_attn(_ptr(q), _float_code(q), B, T, H, _ptr(win), _row_code(win), win.shape[1], win_base,
                         _ptr(q_pos), window, scale, _ptr(sink), _ptr(out), _float_code(out), _ptr(lse),
                         _ptr(workspace), ws_bytes, _stream(stream)), "swa_attn")
    return out


# ---------------------------------------------------------------------------
# Decode over a device-resident cache (decode_prime / decode_step)
# ---------------------------------------------------------------------------
class _DecodeCacheC(ctypes.Structure):
    """Field-for-field mirror of csa_decode_cache."""
    _fields_ = [("batch", _i32), ("n_heads", _i32), ("idx_heads", _i32), ("idx_dim", _i32), ("topk", _i32),
                ("window", _i32), ("win_rows", _i64), ("csa_cap", _i64), ("hca_cap", _i64), ("scale", _f32)] + \
               [(n, _vp) for n in ("csa_w_gate", "csa_pos_bias", "csa_w_idx", "hca_w_gate", "hca_pos_bias",
                                   "csa_sink", "hca_sink", "pos", "csa_entries", "hca_entries", "csa_raw",
                                   "csa_logits", "hca_raw", "hca_logits", "csa_win", "hca_win", "csa_kv", "csa_keys",
                                   "csa_key_scales", "hca_kv")] + \
               [("page_entries", _i32), ("csa_pool_pages", _i32), ("hca_pool_pages", _i32), ("csa_pages", _vp),
                ("hca_pages", _vp)]


_lib.decode_workspace_size.restype = _sz
_lib.decode_workspace_size.argtypes = [ctypes.POINTER(_DecodeCacheC), _i32]
_lib.decode_prime.restype = ctypes.c_int
_lib.decode_prime.argtypes = [ctypes.POINTER(_DecodeCacheC), _vp, _vp, _i32, _i32, _vp]
_lib.decode_step.restype = ctypes.c_int
_lib.decode_step.argtypes = [ctypes.POINTER(_DecodeCacheC), _vp, _vp, _i32, _vp, _vp, _vp, _vp, _i32, _vp, _vp,
                             _i32, _vp, _sz, _vp, _vp]

_lib.prefix_save.restype = ctypes.c_int
_lib.prefix_save.argtypes = [ctypes.POINTER(_DecodeCacheC), _i32, ctypes.c_char_p, _i32, _vp]
_lib.prefix_load.restype = ctypes.c_int
_lib.prefix_load.argtypes = [ctypes.POINTER(_DecodeCacheC), _i32, ctypes.c_char_p, _i32, _i64,
                             ctypes.POINTER(_i64), _vp]

_STATE = ("pos", "csa_entries", "hca_entries", "csa_raw", "csa_logits", "hca_raw", "hca_logits", "csa_win", "hca_win",
          "csa_kv", "csa_keys", "csa_key_scales", "hca_kv")
_POOLS = ("csa_kv", "csa_keys", "csa_key_scales", "hca_kv")
_lib.decode_fork.restype = ctypes.c_int
_lib.decode_fork.argtypes = [ctypes.POINTER(_DecodeCacheC), _i32, _i32, _vp]


class DecodeCache:
    """The device arrays of one CSA + HCA layer pair's decode cache (the layout
    of csa_decode_cache), allocated on `device` and owned by this object.

    weights: dict of float32 device tensors csa_w_gate [192,192], csa_pos_bias
    [8,192], csa_w_idx [192, idx_dim], hca_w_gate [192,192], hca_pos_bias
    [128,192], optional csa_sink / hca_sink [n_heads].  Every state array
    starts at zero; set pos, the entry counts, entries and keys (a prefill)
    and call decode_prime for the rings before the first step.

    page_entries = P > 0 gives the paged layout: csa_kv [csa_pool_pages, P,
    256], csa_keys / csa_key_scales [csa_pool_pages, P, ...], hca_kv
    [hca_pool_pages, P, 256], and the page tables csa_pages [B, csa_cap/P],
    hca_pages [B, hca_cap/P] (int32 device tensors, copied; by default
    sequence b's logical page i is physical page b * (cap/P) + i and each
    pool has exactly the pages the tables name)."""

    def __init__(self, batch, n_heads, idx_heads, idx_dim, topk, window, csa_cap, hca_cap, scale, weights,
                 win_rows=None, device="cuda", page_entries=0, csa_pool_pages=None, hca_pool_pages=None,
                 csa_pages=None, hca_pages=None):
        B, u8 = batch, torch.uint8
        win_rows = window if win_rows is None else win_rows
        z = lambda *shape, dtype=u8: torch.zeros(*shape, dtype=dtype, device=device)  # noqa: E731
        self.pos = z(B, dtype=torch.int64)
        self.csa_entries, self.hca_entries = z(B, dtype=torch.int32), z(B, dtype=torch.int32)
        self.csa_raw, self.csa_logits = z(B, 8, 192, dtype=torch.bfloat16), z(B, 8, 192, dtype=torch.float32)
        self.hca_raw, self.hca_logits = z(B, 128, 192, dtype=torch.bfloat16), z(B, 128, 192, dtype=torch.float32)
        self.csa_win, self.hca_win = z(B, win_rows, 256), z(B, win_rows, 256)
        P = int(page_entries)
        self.paged = P > 0
        if self.paged:
            tc, th = csa_cap // P, hca_cap // P
            csa_pool_pages = B * tc if csa_pool_pages is None else csa_pool_pages
            hca_pool_pages = B * th if hca_pool_pages is None else hca_pool_pages
            self.csa_pages = (torch.arange(B * tc, dtype=torch.int32, device=device).view(B, tc) if csa_pages is None
                              else csa_pages.to(device=device, dtype=torch.int32).clone().contiguous())
            self.hca_pages = (torch.arange(B * th, dtype=torch.int32, device=device).view(B, th) if hca_pages is None
                              else hca_pages.to(device=device, dtype=torch.int32).clone().contiguous())
            self.csa_kv = z(csa_pool_pages, P, 256)
            self.csa_keys, self.csa_key_scales = z(csa_pool_pages, P, idx_dim // 2), z(csa_pool_pages, P, idx_dim // 32)
            self.hca_kv = z(hca_pool_pages, P, 256)
        else:
            self.csa_kv = z(B, csa_cap, 256)
            self.csa_keys, self.csa_key_scales = z(B, csa_cap, idx_dim // 2), z(B, csa_cap, idx_dim // 32)
            self.hca_kv = z(B, hca_cap, 256)
        self.weights = dict(weights)
        for k in ("csa_w_gate", "csa_pos_bias", "csa_w_idx", "hca_w_gate", "hca_pos_bias"):
            t = self.weights[k]
            assert t.dtype == torch.float32 and t.is_contiguous(), k
        self.c = _DecodeCacheC(batch, n_heads, idx_heads, idx_dim, topk, window, win_rows, csa_cap, hca_cap,
                               float(scale))
        for k in ("csa_w_gate", "csa_pos_bias", "csa_w_idx", "hca_w_gate", "hca_pos_bias", "csa_sink", "hca_sink"):
            t = self.weights.get(k)
            setattr(self.c, k, None if t is None else t.data_ptr())
        for k in _STATE:
            setattr(self.c, k, getattr(self, k).data_ptr())
        if self.paged:
            self.c.page_entries, self.c.csa_pool_pages, self.c.hca_pool_pages = P, csa_pool_pages, hca_pool_pages
            self.c.csa_pages, self.c.hca_pages = self.csa_pages.data_ptr(), self.hca_pages.data_ptr()

    def seq_view(self, b: int) -> "DecodeCache":
        """Sequence b alone: a batch-1 cache over the same memory (e.g. to
        decode_prime one sequence after prefix_load)."""
        if not 0 <= b < self.c.batch:
            raise IndexError(b)
        v = DecodeCache.__new__(DecodeCache)
        v.paged = self.paged
        for k in _STATE:   # the page pools are shared by every sequence: not sliced
            t = getattr(self, k)
            setattr(v, k, t if (self.paged and k in _POOLS) else t[b:b + 1])
        if self.paged:
            v.csa_pages, v.hca_pages = self.csa_pages[b:b + 1], self.hca_pages[b:b + 1]
        v.weights = self.weights
        v.c = _DecodeCacheC()
        ctypes.memmove(ctypes.byref(v.c), ctypes.byref(self.c), ctypes.sizeof(_DecodeCacheC))
        v.c.batch = 1
        for k in _STATE:
            setattr(v.c, k, getattr(v, k).data_ptr())
        if self.paged:
            v.c.csa_pages, v.c.hca_pages = v.csa_pages.data_ptr(), v.hca_pages.data_ptr()
        return v

    def workspace_size(self, q_dtype=torch.bfloat16) -> int:
        return int(_lib.decode_workspace_size(ctypes.byref(self.c), _float_code_dtype(q_dtype)))

    def workspace(self, q_dtype=torch.bfloat16) -> torch.Tensor:
        """A zero-filled workspace for decode_step (zero-filled once; steps keep
        the part that must start at zero at zero)."""
        n = self.workspace_size(q_dtype)
        if n == 0:
            raise CsaError(CSA_ERR_SHAPE, "decode_workspace_size")
        return torch.zeros(n, dtype=torch.uint8, device=self.pos.device)


def _float_code_dtype(dt) -> int:
    return {torch.float32: CSA_F32, torch.bfloat16: CSA_BF16}[dt]


def decode_prime(cache: DecodeCache, x_csa, x_hca, stream=None):
    """x_csa / x_hca [B, n_tok, 192] float32 or bfloat16: the tokens before pos."""
    c = cache.c
    for x in (x_csa, x_hca):
        if x.dim() != 3 or x.shape[0] != c.batch or x.shape[2] != 192 or not x.is_contiguous():
            raise ValueError(f"decode_prime: raw KV must be a contiguous [{c.batch}, n_tok, 192] tensor")
    assert x_csa.dtype == x_hca.dtype and x_csa.shape == x_hca.shape
    _check(_lib.decode_prime(ctypes.byref(cache.c), _ptr(x_csa), _ptr(x_hca), _float_code(x_csa), x_csa.shape[1],
                             _stream(stream)), "decode_prime")


def decode_fork(cache: DecodeCache, src: int, dst: int, stream=None):
    """Sequence dst takes sequence src's state, sharing src's full entry pages
    (paged caches; dst's page for a partly filled last page must be its own)."""
    _check(_lib.decode_fork(ctypes.byref(cache.c), src, dst, _stream(stream)), "decode_fork")


def prefix_save(cache: DecodeCache, seq: int, path: str, parts=CSA_PREFIX_ENTRIES | CSA_PREFIX_RINGS, stream=None):
    """Write sequence `seq` of the cache (at its current position) to `path`."""
    _check(_lib.prefix_save(ctypes.byref(cache.c), seq, os.fsencode(path), parts, _stream(stream)), "prefix_save")


def prefix_load(cache: DecodeCache, seq: int, path: str, parts=CSA_PREFIX_ENTRIES | CSA_PREFIX_RINGS,
                prefix_len: int = -1, stream=None) -> int:
    """Restore a snapshot into sequence `seq` for a prefix of `prefix_len` tokens
    (-1: the snapshot's own length).  Returns the first position whose raw KV
    the caller must still write with decode_prime on cache.seq_view(seq)."""
    pf = _i64(0)
    _check(_lib.prefix_load(ctypes.byref(cache.c), seq, os.fsencode(path), parts, prefix_len, ctypes.byref(pf),
                            _stream(stream)), "prefix_load")
    return int(pf.value)


def decode_step(cache: DecodeCache, x_csa, x_hca, q_idx, w, q_csa, q_hca, out_csa, out_hca, workspace,
                stage_events=None, stream=None):
    """One decode token per sequence.  x_* [B, 192]; q_idx float32 [B, idx_heads, idx_dim];
    w float32 [B, idx_heads]; q_* [B, n_heads, 192]; out_* [B, n_heads, 192]."""
    assert x_csa.dtype == x_hca.dtype and q_csa.dtype == q_hca.dtype and out_csa.dtype == out_hca.dtype
    c = cache.c
    want = {"x_csa": (x_csa, (c.batch, 192)), "x_hca": (x_hca, (c.batch, 192)),
            "q_idx": (q_idx, (c.batch, c.idx_heads, c.idx_dim)), "w": (w, (c.batch, c.idx_heads)),
            "q_csa": (q_csa, (c.batch, c.n_heads, 192)), "q_hca": (q_hca, (c.batch, c.n_heads, 192)),
            "out_csa": (out_csa, (c.batch, c.n_heads, 192)), "out_hca": (out_hca, (c.batch, c.n_heads, 192))}
    for name, (t, shape) in want.items():
        if tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError(f"decode_step: {name} must be a contiguous {list(shape)} tensor, got {list(t.shape)}")
    if q_idx.dtype != torch.float32 or w.dtype != torch.float32:
        raise ValueError("decode_step: q_idx and w are float32")
    evs = None
    if stage_events is not None:
        for e in stage_events:
            if e.cuda_event == 0:   # torch creates the HIP event at its first record
                e.record()
        evs = (ctypes.c_void_p * 2)(*[ctypes.c_void_p(e.cuda_event) for e in stage_events])
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(_lib.decode_step(ctypes.byref(cache.c), _ptr(x_csa), _ptr(x_hca), _float_code(x_csa), _ptr(q_idx), _ptr(w),
                            _ptr(q_csa), _ptr(q_hca), _float_code(q_csa), _ptr(out_csa), _ptr(out_hca),
                            _float_code(out_csa), _ptr(workspace), ws_bytes, evs, _stream(stream)), "decode_step")


_lib.decode_csa_layer.restype = ctypes.c_int
_lib.decode_csa_layer.argtypes = [ctypes.POINTER(_DecodeCacheC), _vp, _i32, _vp, _vp, _vp, _i32, _vp, _i32, _vp, _sz,
                                  _vp, _vp]
_lib.decode_hca_layer.restype = ctypes.c_int
_lib.decode_hca_layer.argtypes = [ctypes.POINTER(_DecodeCacheC), _vp, _i32, _vp, _i32, _vp, _i32, _vp, _sz, _vp]


def _stage_events(stage_events):
    if stage_events is None:
        return None
    for e in stage_events:
        if e.cuda_event == 0:   # torch creates the HIP event at its first record
            e.record()
    return (ctypes.c_void_p * 2)(*[ctypes.c_void_p(e.cuda_event) for e in stage_events])


def decode_csa_layer(cache: DecodeCache, x_csa, q_idx, w, q_csa, out_csa, workspace, stage_events=None, stream=None):
    """The CSA layer of one decode token (pos unchanged).  x_csa [B, 192]; q_idx float32
    [B, idx_heads, idx_dim]; w float32 [B, idx_heads]; q_csa / out_csa [B, n_heads, 192]."""
    c = cache.c
    want = {"x_csa": (x_csa, (c.batch, 192)), "q_idx": (q_idx, (c.batch, c.idx_heads, c.idx_dim)),
            "w": (w, (c.batch, c.idx_heads)), "q_csa": (q_csa, (c.batch, c.n_heads, 192)),
            "out_csa": (out_csa, (c.batch, c.n_heads, 192))}
    for name, (t, shape) in want.items():
        if tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError(f"decode_csa_layer: {name} must be a contiguous {list(shape)} tensor, got {list(t.shape)}")
    if q_idx.dtype != torch.float32 or w.dtype != torch.float32:
        raise ValueError("decode_csa_layer: q_idx and w are float32")
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(_lib.decode_csa_layer(ctypes.byref(cache.c), _ptr(x_csa), _float_code(x_csa), _ptr(q_idx), _ptr(w),
                                 _ptr(q_csa), _float_code(q_csa), _ptr(out_csa), _float_code(out_csa), _ptr(workspace),
                                 ws_bytes, _stage_events(stage_events), _stream(stream)), "decode_csa_layer")


def decode_hca_layer(cache: DecodeCache, x_hca, q_hca, out_hca, workspace, stream=None):
    """The HCA layer of one decode token, then pos += 1.  x_hca [B, 192]; q_hca / out_hca [B, n_heads, 192]."""
    c = cache.c
    want = {"x_hca": (x_hca, (c.batch, 192)), "q_hca": (q_hca, (c.batch, c.n_heads, 192)),
            "out_hca": (out_hca, (c.batch, c.n_heads, 192))}
    for name, (t, shape) in want.items():
        if tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError(f"decode_hca_layer: {name} must be a contiguous {list(shape)} tensor, got {list(t.shape)}")
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(_lib.decode_hca_layer(ctypes.byref(cache.c), _ptr(x_hca), _float_code(x_hca), _ptr(q_hca),
                                 _float_code(q_hca), _ptr(out_hca), _float_code(out_hca), _ptr(workspace), ws_bytes,
                                 _stream(stream)), "decode_hca_layer")


_lib.topk_select_noalloc.restype = ctypes.c_int
_lib.topk_select_noalloc.argtypes = [_vp, _i32, _i32, _i32, _i64, _vp, _vp, _i32, _i32, _vp, _vp]
TOPK_NOALLOC_MAX_BYTES = 4 << 20


def topk_select_noalloc(scores, n_entries, q_pos, ratio, k, idx_out, stream=None):
    """topk_select with the library's own fixed scratch array as its workspace
    (no allocation; calls on one GPU must not overlap).  Arguments as topk_select."""
    B, T, N = scores.shape
    _check(_lib.topk_select_noalloc(_ptr(scores), _float_code(scores), B, T, N, _ptr(n_entries), _ptr(q_pos), ratio,
                                    k, _ptr(idx_out), _stream(stream)), "topk_select_noalloc")
    return idx_out
