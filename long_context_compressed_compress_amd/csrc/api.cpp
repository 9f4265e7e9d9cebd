// C-ABI of libcsa: host-side validation, then the internal launchers.
// Every check runs before anything is enqueued; no exception crosses the ABI.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/libcsa.h"
#include "common.h"

namespace {

thread_local int g_last_hip_error = 0;

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool raw_dtype_ok(int d) { return d == CSA_F32 || d == CSA_BF16; }
inline bool row_dtype_ok(int d) { return d == CSA_F32 || d == CSA_BF16 || d == CSA_KV_MIXED; }
constexpr int64_t kMaxGridYZ = 65535;

inline int hip_status(hipError_t e) {
  if (e == hipSuccess) return CSA_OK;
  g_last_hip_error = (int)e;
  return CSA_ERR_HIP;
}

// Softmax scale: finite and positive (the kernels fold it into the exponent
// after taking the maximum of the unscaled logits).
bool scale_ok(float scale) { return scale > 0.0f && scale <= 3.4028234663852886e38f; }

// Shared checks of the attention calls. list_len = longest key list of a query.
int check_attention(const void* q, int32_t q_dtype, int32_t batch, int32_t n_q, int32_t n_heads, const void* kv,
                    int32_t kv_dtype, int64_t n_cap, const int32_t* n_entries, int32_t ratio, const void* win,
                    int64_t win_rows, int64_t win_base, const int64_t* q_pos, int32_t window, void* out,
                    int32_t out_dtype, void* workspace, size_t ws_bytes, int64_t list_len) {
  if (batch < 0 || n_q < 0 || n_heads < 1 || n_cap < 0 || window < 0 || ratio < 1 || win_rows < 0)
    return CSA_ERR_SHAPE;
  if (batch > kMaxGridYZ || n_q > kMaxGridYZ) return CSA_ERR_SHAPE;
  // the kernels index a key list and a ring with 32-bit integers
  if (list_len > 0x7fffffffLL || win_rows > (1LL << 30)) return CSA_ERR_SHAPE;
  if (!raw_dtype_ok(q_dtype) || !row_dtype_ok(kv_dtype) || !raw_dtype_ok(out_dtype)) return CSA_ERR_DTYPE;
  if ((int64_t)batch * n_q == 0) return CSA_OK;
  if (!q || !n_entries || !q_pos || !out) return CSA_ERR_NULL;
  if (n_cap > 0 && !kv) return CSA_ERR_NULL;
  if (window > 0) {
    if (!win) return CSA_ERR_NULL;
    if (win_rows < window) return CSA_ERR_RANGE;
  }
  if (!aligned16(q) || !aligned16(out) || (kv && !aligned16(kv)) || (win && !aligned16(win))) return CSA_ERR_ALIGN;
  const size_t need = csa::attn_ws_bytes(batch, n_q, n_heads, list_len, q_dtype, kv_dtype);
  if (need > 0 && (!workspace || ws_bytes < need)) return CSA_ERR_WORKSPACE;
  if (workspace && !aligned16(workspace)) return CSA_ERR_ALIGN;
  (void)win_base;
  return CSA_OK;
}

}  // namespace

extern "C" {

const char* csa_status_string(int status) {
  switch (status) {
    case CSA_OK: return "CSA_OK";
    case CSA_ERR_NULL: return "CSA_ERR_NULL: a required pointer is NULL";
    case CSA_ERR_SHAPE: return "CSA_ERR_SHAPE: a size is out of range or inconsistent";
    case CSA_ERR_DTYPE: return "CSA_ERR_DTYPE: unsupported dtype or dtype combination";
    case CSA_ERR_ALIGN: return "CSA_ERR_ALIGN: pointer or stride not 16-byte aligned";
    case CSA_ERR_RANGE: return "CSA_ERR_RANGE: requested tokens/entries lie outside the supplied buffers";
    case CSA_ERR_WORKSPACE: return "CSA_ERR_WORKSPACE: workspace missing or too small";
    case CSA_ERR_UNSUPPORTED: return "CSA_ERR_UNSUPPORTED: shape not implemented by this library";
    case CSA_ERR_HIP: return "CSA_ERR_HIP: the HIP runtime reported an error";
    case CSA_ERR_IO: return "CSA_ERR_IO: a snapshot file could not be opened, read or written";
    case CSA_ERR_FORMAT: return "CSA_ERR_FORMAT: not a snapshot file, truncated, damaged, or not fitting the cache";
    default: return "unknown libcsa status";
  }
}

int csa_last_hip_error(void) { return g_last_hip_error; }

int kv_pack(const void* x, int32_t x_dtype, int64_t n_rows, int64_t x_row_stride, void* out, int32_t out_dtype,
            int64_t out_row_stride, void* stream) {
  if (!raw_dtype_ok(x_dtype) || !row_dtype_ok(out_dtype)) return CSA_ERR_DTYPE;
  if (n_rows < 0) return CSA_ERR_SHAPE;
  if (n_rows == 0) return CSA_OK;
  if (!x || !out) return CSA_ERR_NULL;
  if (x_row_stride < csa::DIM || out_row_stride < csa::row_bytes(out_dtype)) return CSA_ERR_SHAPE;
  const int64_t xsb = x_row_stride * (x_dtype == CSA_F32 ? 4 : 2);
  if (!aligned16(x) || !aligned16(out) || (xsb & 15) || (out_row_stride & 15)) return CSA_ERR_ALIGN;
  return hip_status(csa::launch_kv_pack(x, x_dtype, n_rows, x_row_stride, out, out_dtype, out_row_stride,
                                        (hipStream_t)stream));
}

int kv_append(const void* x, int32_t x_dtype, int32_t batch, const int64_t* pos, void* raw_ring, int32_t raw_dtype,
              int64_t raw_rows, int64_t raw_base, void* win_ring, int32_t win_dtype, int64_t win_rows,
              int64_t win_base, void* stream) {
  if (!raw_dtype_ok(x_dtype)) return CSA_ERR_DTYPE;
  if (raw_ring && !raw_dtype_ok(raw_dtype)) return CSA_ERR_DTYPE;
  if (win_ring && !row_dtype_ok(win_dtype)) return CSA_ERR_DTYPE;
  if (batch < 0 || (raw_ring && raw_rows < 1) || (win_ring && win_rows < 1)) return CSA_ERR_SHAPE;
  if (batch == 0 || (!raw_ring && !win_ring)) return CSA_OK;
  if (!x || !pos) return CSA_ERR_NULL;
  if (!aligned16(x) || (raw_ring && !aligned16(raw_ring)) || (win_ring && !aligned16(win_ring))) return CSA_ERR_ALIGN;
  return hip_status(csa::launch_kv_append(x, x_dtype, batch, pos, raw_ring, raw_dtype, raw_rows, raw_base, win_ring,
                                          win_dtype, win_rows, win_base, (hipStream_t)stream));
}

int mxfp4_quantize(const float* x, int64_t n_rows, int32_t d, uint8_t* codes, uint8_t* scales, void* stream) {
  if (n_rows < 0 || d <= 0 || d % CSA_MX_BLOCK) return CSA_ERR_SHAPE;
  if (n_rows == 0) return CSA_OK;
  if (!x || !codes || !scales) return CSA_ERR_NULL;
  if (!aligned16(x) || !aligned16(codes)) return CSA_ERR_ALIGN;
  return hip_status(csa::launch_mxfp4_quantize(x, n_rows, d, codes, scales, (hipStream_t)stream));
}

int csa_compress(const void* x_raw, int32_t x_dtype, int32_t batch, int64_t raw_rows, int64_t raw_base,
                 const float* w_gate, const float* pos_bias, int64_t entry_begin, int32_t n_new, void* kv_out,
                 int32_t kv_dtype, int64_t n_cap, const float* w_idx, int32_t d_idx, void* key_out,
                 uint8_t* key_scales, int32_t key_dtype, void* stream) {
  if (!raw_dtype_ok(x_dtype) || !row_dtype_ok(kv_dtype)) return CSA_ERR_DTYPE;
  if (batch < 0 || batch > kMaxGridYZ || raw_rows < 1 || n_new < 0 || entry_begin < 0 || n_cap < 0)
    return CSA_ERR_SHAPE;
  if (w_idx) {
    if (key_dtype != CSA_F32 && key_dtype != CSA_MXFP4) return CSA_ERR_DTYPE;
    if (d_idx < 4 || d_idx > 256 || d_idx % 4 || (key_dtype == CSA_MXFP4 && d_idx % CSA_MX_BLOCK))
      return CSA_ERR_SHAPE;
  }
  if (entry_begin + n_new > n_cap) return CSA_ERR_RANGE;
  if (batch == 0 || n_new == 0) return CSA_OK;
  if (!x_raw || !w_gate || !pos_bias || !kv_out) return CSA_ERR_NULL;
  if (w_idx && (!key_out || (key_dtype == CSA_MXFP4 && !key_scales))) return CSA_ERR_NULL;
  if (!aligned16(w_gate) || (w_idx && !aligned16(w_idx))) return CSA_ERR_ALIGN;
  if (w_idx && key_dtype == CSA_MXFP4 && !aligned16(key_out)) return CSA_ERR_ALIGN;
  const int64_t j_lo = entry_begin > 0 ? 4 * (entry_begin - 1) : 0;
  const int64_t j_hi = 4 * (entry_begin + n_new) - 1;
  if (j_lo < raw_base || j_hi - j_lo + 1 > raw_rows) return CSA_ERR_RANGE;
  return hip_status(csa::launch_csa_compress(x_raw, x_dtype, batch, raw_rows, raw_base, w_gate, pos_bias,
                                             entry_begin, n_new, kv_out, kv_dtype, n_cap, w_idx, d_idx, key_out,
                                             key_scales, key_dtype, (hipStream_t)stream));
}

int hca_compress(const void* x_raw, int32_t x_dtype, int32_t batch, int64_t raw_rows, int64_t raw_base,
                 const float* w_gate, const float* pos_bias, int64_t entry_begin, int32_t n_new, void* kv_out,
                 int32_t kv_dtype, int64_t n_cap, void* stream) {
  if (!raw_dtype_ok(x_dtype) || !row_dtype_ok(kv_dtype)) return CSA_ERR_DTYPE;
  if (batch < 0 || batch > kMaxGridYZ || raw_rows < 1 || n_new < 0 || entry_begin < 0 || n_cap < 0)
    return CSA_ERR_SHAPE;
  if ((int64_t)n_new * 6 > 0x7fffffffLL) return CSA_ERR_SHAPE;
  if (entry_begin + n_new > n_cap) return CSA_ERR_RANGE;
  if (batch == 0 || n_new == 0) return CSA_OK;
  if (!x_raw || !w_gate || !pos_bias || !kv_out) return CSA_ERR_NULL;
  const int64_t j_lo = 128 * entry_begin;
  const int64_t j_hi = 128 * (entry_begin + n_new) - 1;
  if (j_lo < raw_base || j_hi - j_lo + 1 > raw_rows) return CSA_ERR_RANGE;
  return hip_status(csa::launch_hca_compress(x_raw, x_dtype, batch, raw_rows, raw_base, w_gate, pos_bias,
                                             entry_begin, n_new, kv_out, kv_dtype, n_cap, (hipStream_t)stream));
}

namespace {
// Validation of indexer_score's arguments; *mx / *q_f32 say which path runs.
int check_indexer(const void* q, const uint8_t* q_scales, int32_t q_dtype, const float* w, const void* k,
                  const uint8_t* k_scales, int32_t k_dtype, int32_t batch, int32_t n_q, int32_t n_heads,
                  int32_t d_idx, int64_t n_cap, const int32_t* n_entries, const int64_t* q_pos, int32_t ratio,
                  void* scores, int32_t score_dtype, bool* mx_out, bool* q_f32_out) {
  const bool f32 = q_dtype == CSA_F32 && k_dtype == CSA_F32 && score_dtype == CSA_F32;
  // MXFP4 keys: q as MXFP4 codes + scales, or as float32 quantized inside the call
  const bool mx = (q_dtype == CSA_MXFP4 || q_dtype == CSA_F32) && k_dtype == CSA_MXFP4 && score_dtype == CSA_BF16;
  const bool q_f32 = q_dtype == CSA_F32;
  *mx_out = mx;
  *q_f32_out = q_f32;
  if (!f32 && !mx) return CSA_ERR_DTYPE;
  if (batch < 0 || n_q < 0 || n_heads < 1 || d_idx < 1 || n_cap < 0 || ratio < 1) return CSA_ERR_SHAPE;
  if (batch > kMaxGridYZ || n_q > kMaxGridYZ) return CSA_ERR_SHAPE;
  if (f32 && (int64_t)n_heads * (d_idx + 1) > 16384) return CSA_ERR_UNSUPPORTED;
  if (mx) {
    if (d_idx % 64 || (n_heads % 32)) return CSA_ERR_UNSUPPORTED;
    if (n_heads > 128 || (d_idx != 64 && d_idx != 128 && d_idx != 256)) return CSA_ERR_UNSUPPORTED;
    if ((int64_t)batch * n_q > kMaxGridYZ) return CSA_ERR_SHAPE;
  }
  if ((int64_t)batch * n_q == 0 || n_cap == 0) return CSA_OK;
  if (!q || !w || !k || !n_entries || !q_pos || !scores) return CSA_ERR_NULL;
  if (mx && ((!q_f32 && !q_scales) || !k_scales)) return CSA_ERR_NULL;
  if (mx && (!aligned16(q) || !aligned16(k))) return CSA_ERR_ALIGN;
  return CSA_OK;
}

int check_topk(const void* scores, int32_t score_dtype, int32_t batch, int32_t n_q, int64_t n_cap,
               const int32_t* n_entries, const int64_t* q_pos, int32_t ratio, int32_t k, int32_t* idx_out,
               void* workspace, size_t ws_bytes) {
  if (score_dtype != CSA_BF16 && score_dtype != CSA_F32) return CSA_ERR_DTYPE;
  if (batch < 0 || n_q < 0 || n_cap < 0 || k < 1 || ratio < 1) return CSA_ERR_SHAPE;
  if (batch > kMaxGridYZ || n_q > 0x7fffffff) return CSA_ERR_SHAPE;
  if ((int64_t)batch * n_q == 0) return CSA_OK;
  if (!n_entries || !q_pos || !idx_out || (n_cap > 0 && !scores)) return CSA_ERR_NULL;
  const size_t need = csa::topk_ws_bytes(batch, n_q, n_cap, k, score_dtype);
  if (need > 0 && (!workspace || ws_bytes < need)) return CSA_ERR_WORKSPACE;
  if (workspace && !aligned16(workspace)) return CSA_ERR_ALIGN;
  return CSA_OK;
}
}  // namespace

int indexer_score(const void* q, const uint8_t* q_scales, int32_t q_dtype, const float* w, const void* k,
                  const uint8_t* k_scales, int32_t k_dtype, int32_t batch, int32_t n_q, int32_t n_heads,
                  int32_t d_idx, int64_t n_cap, const int32_t* n_entries, const int64_t* q_pos, int32_t ratio,
                  void* scores, int32_t score_dtype, void* stream) {
  bool mx, q_f32;
  const int st = check_indexer(q, q_scales, q_dtype, w, k, k_scales, k_dtype, batch, n_q, n_heads, d_idx, n_cap,
                               n_entries, q_pos, ratio, scores, score_dtype, &mx, &q_f32);
  if (st != CSA_OK || (int64_t)batch * n_q == 0 || n_cap == 0) return st;
  hipError_t e;
  if (!mx)
    e = csa::launch_indexer_f32((const float*)q, w, (const float*)k, batch, n_q, n_heads, d_idx, n_cap, n_entries,
                                q_pos, ratio, (float*)scores, (hipStream_t)stream);
  else
    e = csa::launch_indexer_mxfp4(q, q_f32, q_scales, w, (const uint8_t*)k, k_scales, batch, n_q, n_heads,
                                  d_idx, n_cap, n_entries, q_pos, ratio, (uint16_t*)scores, (hipStream_t)stream);
  return hip_status(e);
}

size_t topk_workspace_size(int32_t batch, int32_t n_q, int64_t n_cap, int32_t k, int32_t score_dtype) {
  if (batch < 0 || n_q < 0 || n_cap < 0 || k < 1) return 0;
  return csa::topk_ws_bytes(batch, n_q, n_cap, k, score_dtype);
}

int topk_select(const void* scores, int32_t score_dtype, int32_t batch, int32_t n_q, int64_t n_cap,
                const int32_t* n_entries, const int64_t* q_pos, int32_t ratio, int32_t k, int32_t* idx_out,
                void* workspace, size_t ws_bytes, void* stream) {
  const int st = check_topk(scores, score_dtype, batch, n_q, n_cap, n_entries, q_pos, ratio, k, idx_out, workspace,
                            ws_bytes);
  if (st != CSA_OK || (int64_t)batch * n_q == 0) return st;
  return hip_status(csa::launch_topk(scores, score_dtype, batch, n_q, n_cap, n_entries, q_pos, ratio, k, idx_out,
                                     workspace, (hipStream_t)stream));
}

int indexer_topk(const void* q, const uint8_t* q_scales, int32_t q_dtype, const float* w, const void* k,
                 const uint8_t* k_scales, int32_t k_dtype, int32_t batch, int32_t n_q, int32_t n_heads,
                 int32_t d_idx, int64_t n_cap, const int32_t* n_entries, const int64_t* q_pos, int32_t ratio,
                 void* scores, int32_t score_dtype, int32_t topk, int32_t* idx_out, void* workspace,
                 size_t ws_bytes, void* const* stage_events, void* stream) {
  bool mx, q_f32;
  int st = check_indexer(q, q_scales, q_dtype, w, k, k_scales, k_dtype, batch, n_q, n_heads, d_idx, n_cap,
                         n_entries, q_pos, ratio, scores, score_dtype, &mx, &q_f32);
  if (st != CSA_OK) return st;
  st = check_topk(scores, score_dtype, batch, n_q, n_cap, n_entries, q_pos, ratio, topk, idx_out, workspace,
                  ws_bytes);
  if (st != CSA_OK || (int64_t)batch * n_q == 0) return st;
  const hipStream_t s = (hipStream_t)stream;
  const int64_t rows = (int64_t)batch * n_q;
  hipError_t e = hipSuccess;
  bool pass1_done = false;
  if (stage_events && (!stage_events[0] || !stage_events[1])) return CSA_ERR_NULL;
  hipEvent_t ev0 = stage_events ? (hipEvent_t)stage_events[0] : nullptr;
  hipEvent_t ev1 = stage_events ? (hipEvent_t)stage_events[1] : nullptr;
  if (n_cap > 0) {
    if (!mx) {  // no dispatch-recorded events on this path: the pair brackets the launch
      if (ev0 && (e = hipEventRecord(ev0, s)) != hipSuccess) return hip_status(e);
      e = csa::launch_indexer_f32((const float*)q, w, (const float*)k, batch, n_q, n_heads, d_idx, n_cap, n_entries,
                                  q_pos, ratio, (float*)scores, s);
      if (e == hipSuccess && ev1) e = hipEventRecord(ev1, s);
      ev0 = ev1 = nullptr;
    } else {
      uint32_t* hist = nullptr;
      int row_words = 0;
      if (csa::topk_uses_split(rows, n_cap, score_dtype)) {  // pass 1 of top-k rides on the indexer
        hist = csa::topk_split_totals(workspace, &row_words);
        pass1_done = true;
      }
      e = csa::launch_indexer_mxfp4(q, q_f32, q_scales, w, (const uint8_t*)k, k_scales, batch, n_q, n_heads, d_idx,
                                    n_cap, n_entries, q_pos, ratio, (uint16_t*)scores, s, hist, row_words, ev0, ev1);
      ev0 = ev1 = nullptr;  // recorded by the launch
    }
    if (e != hipSuccess) return hip_status(e);
  }
  // nothing to score (no entries): the pair is recorded with nothing between
  if (ev0 && (e = hipEventRecord(ev0, s)) != hipSuccess) return hip_status(e);
  if (ev1 && (e = hipEventRecord(ev1, s)) != hipSuccess) return hip_status(e);
  return hip_status(csa::launch_topk(scores, score_dtype, batch, n_q, n_cap, n_entries, q_pos, ratio, topk, idx_out,
                                     workspace, s, pass1_done));
}

size_t attn_workspace_size(int32_t batch, int32_t n_q, int32_t n_heads, int64_t max_keys, int32_t q_dtype,
                           int32_t kv_dtype) {
  if (batch < 0 || n_q < 0 || n_heads < 1 || max_keys < 0) return 0;
  return csa::attn_ws_bytes(batch, n_q, n_heads, max_keys, q_dtype, kv_dtype);
}

int sparse_window_attn(const void* q, int32_t q_dtype, int32_t batch, int32_t n_q, int32_t n_heads, const void* kv,
                       int32_t kv_dtype, int64_t n_cap, const int32_t* n_entries, int32_t ratio, const int32_t* idx,
                       int32_t k, const void* win, int64_t win_rows, int64_t win_base, const int64_t* q_pos,
                       int32_t window, float scale, const float* sink, void* out, int32_t out_dtype, float* lse_out,
                       void* workspace, size_t ws_bytes, void* stream) {
  if (k < 0) return CSA_ERR_SHAPE;
  if (!scale_ok(scale)) return CSA_ERR_RANGE;
  const int st = check_attention(q, q_dtype, batch, n_q, n_heads, kv, kv_dtype, n_cap, n_entries, ratio, win,
                                 win_rows, win_base, q_pos, window, out, out_dtype, workspace, ws_bytes,
                                 (int64_t)k + window);
  if (st != CSA_OK || (int64_t)batch * n_q == 0) return st;
  if (k > 0 && !idx) return CSA_ERR_NULL;
  csa::AttnArgs a{q, q_dtype, batch, n_q, n_heads, kv, kv_dtype, n_cap, n_entries, ratio, idx, k,
                  win, win_rows, win_base, q_pos, window, scale, sink, out, out_dtype, lse_out, workspace};
  if (k == 0) {  // an empty selection: the window alone (dense over zero entries)
    a.idx = nullptr;
    a.n_cap = 0;
  }
  return hip_status(csa::launch_attention(a, (int64_t)k + window, (hipStream_t)stream));
}

int hca_dense_attn(const void* q, int32_t q_dtype, int32_t batch, int32_t n_q, int32_t n_heads, const void* kv,
                   int32_t kv_dtype, int64_t n_cap, const int32_t* n_entries, int32_t ratio, const void* win,
                   int64_t win_rows, int64_t win_base, const int64_t* q_pos, int32_t window, float scale,
                   const float* sink, void* out, int32_t out_dtype, float* lse_out, void* workspace, size_t ws_bytes,
                   void* stream) {
  if (!scale_ok(scale)) return CSA_ERR_RANGE;
  const int st = check_attention(q, q_dtype, batch, n_q, n_heads, kv, kv_dtype, n_cap, n_entries, ratio, win,
                                 win_rows, win_base, q_pos, window, out, out_dtype, workspace, ws_bytes,
                                 n_cap + window);
  if (st != CSA_OK || (int64_t)batch * n_q == 0) return st;
  csa::AttnArgs a{q, q_dtype, batch, n_q, n_heads, kv, kv_dtype, n_cap, n_entries, ratio, nullptr, 0,
                  win, win_rows, win_base, q_pos, window, scale, sink, out, out_dtype, lse_out, workspace};
  return hip_status(csa::launch_attention(a, n_cap + window, (hipStream_t)stream));
}

int swa_attn(const void* q, int32_t q_dtype, int32_t batch, int32_t n_q, int32_t n_heads, const void* win,
             int32_t win_dtype, int64_t win_rows, int64_t win_base, const int64_t* q_pos, int32_t window,
             float scale, const float* sink, void* out, int32_t out_dtype, float* lse_out, void* workspace,
             size_t ws_bytes, void* stream) {
  if (!scale_ok(scale)) return CSA_ERR_RANGE;
  if (window < 1) return CSA_ERR_SHAPE;
  // the shared checks, with no entries (n_entries is then never read)
  static const int32_t kNone = 0;
  const int st = check_attention(q, q_dtype, batch, n_q, n_heads, nullptr, win_dtype, 0, &kNone, 1, win, win_rows,
                                 win_base, q_pos, window, out, out_dtype, workspace, ws_bytes, window);
  if (st != CSA_OK || (int64_t)batch * n_q == 0) return st;
  csa::AttnArgs a{q, q_dtype, batch, n_q, n_heads, nullptr, win_dtype, 0, nullptr, 1, nullptr, 0,
                  win, win_rows, win_base, q_pos, window, scale, sink, out, out_dtype, lse_out, workspace};
  return hip_status(csa::launch_attention(a, window, (hipStream_t)stream));
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Decode over a device-resident cache
// ---------------------------------------------------------------------------
namespace {

inline size_t round256(size_t n) { return (n + 255) & ~(size_t)255; }

// Workspace slices of one decode step, in order: the append kernel's arrival
// counters (room for the largest batch) and the top-k workspace, whose first
// part holds the per-row histogram totals; those two are the parts that are
// zero at rest, and both sit at offsets that do not depend on the cache's
// shape, so a workspace can serve caches of other shapes.  Then the decoded
// positions, the indexer query, scores, selection, and the attention partials
// of the CSA layer and of the HCA layer (the two run in one launch).
constexpr size_t kArriveBytes = 65536 * 4;  // one int32 per sequence, batch <= 65535
struct DecodeWs {
  size_t arrive, topk, qpos, qcodes, qscales, scores, idx, attn, attn_h, total;
};

DecodeWs decode_ws(const csa_decode_cache& c, int q_dtype) {
  DecodeWs w;
  w.arrive = 0;
  w.topk = kArriveBytes;
  size_t off = w.topk + round256(csa::topk_ws_bytes(c.batch, 1, c.csa_cap, c.topk, CSA_BF16));
  w.qpos = off;
  off += round256((size_t)c.batch * 8);
  w.qcodes = off;  // the step's indexer query in MXFP4 (quantized by the append kernel)
  off += round256((size_t)c.batch * c.idx_heads * c.idx_dim / 2);
  w.qscales = off;
  off += round256((size_t)c.batch * c.idx_heads * c.idx_dim / 32);
  w.scores = off;
  off += round256((size_t)c.batch * c.csa_cap * 2);
  w.idx = off;
  off += round256((size_t)c.batch * c.topk * 4);
  w.attn = off;
  const size_t a1 = csa::attn_ws_bytes(c.batch, 1, c.n_heads, (int64_t)c.topk + c.window, q_dtype, CSA_KV_MIXED);
  const size_t a2 = csa::attn_ws_bytes(c.batch, 1, c.n_heads, c.hca_cap + c.window, q_dtype, CSA_KV_MIXED);
  off += round256(a1);
  w.attn_h = off;
  off += round256(a2);
  w.total = off;
  return w;
}

int check_decode_cache(const csa_decode_cache* c) {
  if (!c) return CSA_ERR_NULL;
  if (c->batch < 1 || c->batch > kMaxGridYZ || c->n_heads < 1 || c->topk < 1 || c->window < 0 ||
      c->win_rows < 1 || c->window > c->win_rows || c->csa_cap < 1 || c->hca_cap < 1 || c->csa_cap > 0x7fffffff ||
      c->hca_cap > 0x7fffffff)
    return CSA_ERR_SHAPE;
  if (c->idx_heads < 32 || c->idx_heads % 32 || c->idx_heads > 128) return CSA_ERR_UNSUPPORTED;
  if (c->idx_dim != 64 && c->idx_dim != 128 && c->idx_dim != 256) return CSA_ERR_UNSUPPORTED;
  if (!scale_ok(c->scale)) return CSA_ERR_RANGE;
  if (!c->csa_w_gate || !c->csa_pos_bias || !c->csa_w_idx || !c->hca_w_gate || !c->hca_pos_bias || !c->pos ||
      !c->csa_entries || !c->hca_entries || !c->csa_raw || !c->csa_logits || !c->hca_raw || !c->hca_logits ||
      !c->csa_win || !c->hca_win || !c->csa_kv || !c->csa_keys || !c->csa_key_scales || !c->hca_kv)
    return CSA_ERR_NULL;
  if (!aligned16(c->csa_win) || !aligned16(c->hca_win) || !aligned16(c->csa_kv) || !aligned16(c->csa_keys) ||
      !aligned16(c->hca_kv))
    return CSA_ERR_ALIGN;
  if (c->page_entries != 0) {  // paged entries: pages of a power of two >= 32 entries dividing both capacities
    const int64_t P = c->page_entries;
    if (P < 32 || (P & (P - 1)) || c->csa_cap % P || c->hca_cap % P || c->csa_pool_pages < 1 ||
        c->hca_pool_pages < 1 || (int64_t)c->csa_pool_pages * P > 0x7fffffffLL ||
        (int64_t)c->hca_pool_pages * P > 0x7fffffffLL)
      return CSA_ERR_SHAPE;
    if (!c->csa_pages || !c->hca_pages) return CSA_ERR_NULL;
  }
  return CSA_OK;
}

// The checks every decode call makes, in the order the codes take precedence
// (the cache, the dtypes, the caller's own pointer checks `args_st`, the
// workspace), and the workspace's slices as pointers.
struct DecodeCall {
  DecodeWs L;
  uint8_t* ws;
  int64_t* q_pos;
  int32_t* arrive;
  uint8_t *q_codes, *q_scales;
};
int decode_call(const csa_decode_cache* cache, int32_t x_dtype, int32_t q_dtype, int32_t out_dtype, int args_st,
                void* workspace, size_t ws_bytes, DecodeCall& d) {
  const int st = check_decode_cache(cache);
  if (st != CSA_OK) return st;
  if (!raw_dtype_ok(x_dtype) || !raw_dtype_ok(q_dtype) || !raw_dtype_ok(out_dtype)) return CSA_ERR_DTYPE;
  if (args_st != CSA_OK) return args_st;
  d.L = decode_ws(*cache, q_dtype);
  if (!workspace || ws_bytes < d.L.total) return CSA_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return CSA_ERR_ALIGN;
  d.ws = static_cast<uint8_t*>(workspace);
  d.q_pos = reinterpret_cast<int64_t*>(d.ws + d.L.qpos);
  d.arrive = reinterpret_cast<int32_t*>(d.ws + d.L.arrive);
  d.q_codes = d.ws + d.L.qcodes;
  d.q_scales = d.ws + d.L.qscales;
  return CSA_OK;
}

// The CSA layer's index and select: the indexer over the cache's MXFP4 keys
// (with top-k's first pass when the split path applies), then top-k.
hipError_t decode_select(const csa_decode_cache& c, const DecodeCall& d, const float* w, void* const* stage_events,
                         hipStream_t s) {
  void* topk_ws = d.ws + d.L.topk;
  uint16_t* scores = reinterpret_cast<uint16_t*>(d.ws + d.L.scores);
  uint32_t* hist = nullptr;
  int row_words = 0;
  const bool split = csa::topk_uses_split(c.batch, c.csa_cap, CSA_BF16);
  if (split) hist = csa::topk_split_totals(topk_ws, &row_words);
  hipError_t e = csa::launch_indexer_mxfp4(d.q_codes, false, d.q_scales, w, c.csa_keys, c.csa_key_scales, c.batch, 1,
                                           c.idx_heads, c.idx_dim, c.csa_cap, c.csa_entries, d.q_pos, 4, scores, s,
                                           hist, row_words, stage_events ? (hipEvent_t)stage_events[0] : nullptr,
                                           stage_events ? (hipEvent_t)stage_events[1] : nullptr,
                                           csa::csa_entry_pages(c));
  if (e != hipSuccess) return e;
  return csa::launch_topk(scores, CSA_BF16, c.batch, 1, c.csa_cap, c.csa_entries, d.q_pos, 4, c.topk,
                          reinterpret_cast<int32_t*>(d.ws + d.L.idx), topk_ws, s, split);
}

// Each layer's attention over the cache: CSA over the selection + window,
// HCA over every visible entry + window, partials in the layer's own slice.
csa::AttnArgs csa_layer_attn(const csa_decode_cache& c, const DecodeCall& d, const void* q, int q_dtype, void* out,
                             int out_dtype) {
  return csa::AttnArgs{q, q_dtype, c.batch, 1, c.n_heads, c.csa_kv, CSA_KV_MIXED, c.csa_cap, c.csa_entries, 4,
                       reinterpret_cast<const int32_t*>(d.ws + d.L.idx), c.topk, c.csa_win, c.win_rows, 0, d.q_pos,
                       c.window, c.scale, c.csa_sink, out, out_dtype, nullptr, d.ws + d.L.attn,
                       csa::csa_entry_pages(c)};
}
csa::AttnArgs hca_layer_attn(const csa_decode_cache& c, const DecodeCall& d, const void* q, int q_dtype, void* out,
                             int out_dtype) {
  return csa::AttnArgs{q, q_dtype, c.batch, 1, c.n_heads, c.hca_kv, CSA_KV_MIXED, c.hca_cap, c.hca_entries, 128,
                       nullptr, 0, c.hca_win, c.win_rows, 0, d.q_pos, c.window, c.scale, c.hca_sink, out, out_dtype,
                       nullptr, d.ws + d.L.attn_h, csa::hca_entry_pages(c)};
}

}  // namespace

extern "C" {

size_t decode_workspace_size(const csa_decode_cache* cache, int32_t q_dtype) {
  if (check_decode_cache(cache) != CSA_OK || !raw_dtype_ok(q_dtype)) return 0;
  return decode_ws(*cache, q_dtype).total;
}

int decode_prime(const csa_decode_cache* cache, const void* x_csa, const void* x_hca, int32_t x_dtype,
                 int32_t n_tok, void* stream) {
  const int st = check_decode_cache(cache);
  if (st != CSA_OK) return st;
  if (!raw_dtype_ok(x_dtype)) return CSA_ERR_DTYPE;
  if (n_tok < 1 || n_tok > kMaxGridYZ) return CSA_ERR_SHAPE;
  if (!x_csa || !x_hca) return CSA_ERR_NULL;
  return hip_status(csa::launch_decode_prime(*cache, x_csa, x_hca, x_dtype, n_tok, (hipStream_t)stream));
}

int decode_step(const csa_decode_cache* cache, const void* x_csa, const void* x_hca, int32_t x_dtype,
                const float* q_idx, const float* w, const void* q_csa, const void* q_hca, int32_t q_dtype,
                void* out_csa, void* out_hca, int32_t out_dtype, void* workspace, size_t ws_bytes,
                void* const* stage_events, void* stream) {
  int args_st = CSA_OK;
  if (!x_csa || !x_hca || !q_idx || !w || !q_csa || !q_hca || !out_csa || !out_hca) args_st = CSA_ERR_NULL;
  else if (!aligned16(q_idx) || !aligned16(q_csa) || !aligned16(q_hca) || !aligned16(out_csa) || !aligned16(out_hca))
    args_st = CSA_ERR_ALIGN;
  else if (stage_events && (!stage_events[0] || !stage_events[1])) args_st = CSA_ERR_NULL;
  DecodeCall d;
  const int st = decode_call(cache, x_dtype, q_dtype, out_dtype, args_st, workspace, ws_bytes, d);
  if (st != CSA_OK) return st;
  const hipStream_t s = (hipStream_t)stream;
  // 1-2. append both layers, compress on boundaries, advance pos (q_pos = the decoded positions)
  hipError_t e = csa::launch_decode_append(*cache, x_csa, x_hca, x_dtype, d.q_pos, d.arrive, q_idx, d.q_codes,
                                           d.q_scales, s);
  // 3. indexer (query quantized by the append kernel) with top-k's first pass when it applies, then top-k
  if (e == hipSuccess) e = decode_select(*cache, d, w, stage_events, s);
  if (e != hipSuccess) return hip_status(e);
  // 4. attention of both layers, in one launch
  const csa::AttnArgs a = csa_layer_attn(*cache, d, q_csa, q_dtype, out_csa, out_dtype);
  const csa::AttnArgs h = hca_layer_attn(*cache, d, q_hca, q_dtype, out_hca, out_dtype);
  return hip_status(csa::launch_attention_pair(a, (int64_t)cache->topk + cache->window, h,
                                               cache->hca_cap + cache->window, s));
}

int decode_csa_layer(const csa_decode_cache* cache, const void* x_csa, int32_t x_dtype, const float* q_idx,
                     const float* w, const void* q_csa, int32_t q_dtype, void* out_csa, int32_t out_dtype,
                     void* workspace, size_t ws_bytes, void* const* stage_events, void* stream) {
  int args_st = CSA_OK;
  if (!x_csa || !q_idx || !w || !q_csa || !out_csa) args_st = CSA_ERR_NULL;
  else if (!aligned16(q_idx) || !aligned16(q_csa) || !aligned16(out_csa)) args_st = CSA_ERR_ALIGN;
  else if (stage_events && (!stage_events[0] || !stage_events[1])) args_st = CSA_ERR_NULL;
  DecodeCall d;
  const int st = decode_call(cache, x_dtype, q_dtype, out_dtype, args_st, workspace, ws_bytes, d);
  if (st != CSA_OK) return st;
  const hipStream_t s = (hipStream_t)stream;
  // append + compress the CSA layer (pos unchanged: the HCA layer of the token advances it)
  hipError_t e = csa::launch_decode_append(*cache, x_csa, nullptr, x_dtype, d.q_pos, d.arrive, q_idx, d.q_codes,
                                           d.q_scales, s, 1, false);
  if (e == hipSuccess) e = decode_select(*cache, d, w, stage_events, s);
  if (e != hipSuccess) return hip_status(e);
  const csa::AttnArgs a = csa_layer_attn(*cache, d, q_csa, q_dtype, out_csa, out_dtype);
  return hip_status(csa::launch_attention(a, (int64_t)cache->topk + cache->window, s));
}

int decode_hca_layer(const csa_decode_cache* cache, const void* x_hca, int32_t x_dtype, const void* q_hca,
                     int32_t q_dtype, void* out_hca, int32_t out_dtype, void* workspace, size_t ws_bytes,
                     void* stream) {
  int args_st = CSA_OK;
  if (!x_hca || !q_hca || !out_hca) args_st = CSA_ERR_NULL;
  else if (!aligned16(q_hca) || !aligned16(out_hca)) args_st = CSA_ERR_ALIGN;
  DecodeCall d;
  const int st = decode_call(cache, x_dtype, q_dtype, out_dtype, args_st, workspace, ws_bytes, d);
  if (st != CSA_OK) return st;
  const hipStream_t s = (hipStream_t)stream;
  // append + compress the HCA layer, record the decoded positions, advance pos
  hipError_t e = csa::launch_decode_append(*cache, nullptr, x_hca, x_dtype, d.q_pos, d.arrive, nullptr, nullptr,
                                           nullptr, s, 2, true);
  if (e != hipSuccess) return hip_status(e);
  const csa::AttnArgs h = hca_layer_attn(*cache, d, q_hca, q_dtype, out_hca, out_dtype);
  return hip_status(csa::launch_attention(h, cache->hca_cap + cache->window, s));
}

int decode_fork(const csa_decode_cache* cache, int32_t src, int32_t dst, void* stream) {
  const int st = check_decode_cache(cache);
  if (st != CSA_OK) return st;
  if (src < 0 || src >= cache->batch || dst < 0 || dst >= cache->batch) return CSA_ERR_SHAPE;
  if (cache->page_entries == 0) return CSA_ERR_UNSUPPORTED;
  if (src == dst) return CSA_OK;
  return hip_status(csa::launch_decode_fork(*cache, src, dst, (hipStream_t)stream));
}

}  // extern "C"

// Shared with the snapshot calls (prefix.cpp): the cache check and the
// recording of HIP errors for csa_last_hip_error.
namespace csa {
int abi_decode_cache_status(const csa_decode_cache* c) { return check_decode_cache(c); }
int abi_hip_status(hipError_t e) { return hip_status(e); }
}  // namespace csa
