// Device helpers and internal launcher declarations shared by the libcsa
// kernels (gfx950 / CDNA4, wave64).  Number formats follow the storage rules
// of the DeepSeek-V4 pages: KV rows keep the RoPE dims in BF16 and the other
// dims in FP8 (gitcode.csdn.net DeepSeek-V4 解读, 核心创新一 §1.4); indexer QK
// operands are MXFP4 (austery.github.io DeepSeek-V4 notes, 全栈工程优化).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/libcsa.h"

namespace csa {

constexpr int DIM = 192;
constexpr int DIM_NOPE = 128;
constexpr int DIM_ROPE = 64;
constexpr int ROW_BYTES = 256;
constexpr int MXB = 32;  // MXFP4 block length

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v8s __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// BF16 <-> FP32
// ---------------------------------------------------------------------------
// float32 -> BF16 bits, round to nearest, ties to even (overflow to inf, float32
// denormals rounded like any other value); a NaN stays a quiet NaN with its
// sign.  This is gfx950's v_cvt_pk_bf16_f32 (a plain cast), which for every
// non-NaN input gives exactly the rounding the storage formats define.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
// Two values, packed low / high (one v_cvt_pk_bf16_f32).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32x2_to_bf16x2_rne(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// ---------------------------------------------------------------------------
// FP8 E4M3 (OCP e4m3fn: bias 7, max 448, no inf), RNE, saturating
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t f32_to_fp8_sat(float f) {
  const uint32_t sign = (__float_as_uint(f) >> 24) & 0x80u;
  const float a = fabsf(f);
  if (a != a) return sign | 0x7fu;
  if (a >= 448.0f) return sign | 0x7eu;  // saturate (includes inf)
  uint32_t code;
  if (a < 0.015625f) {  // below 2^-6: fixed quantum 2^-9 (subnormals; 8 = smallest normal)
    code = (uint32_t)rintf(a * 512.0f);
  } else {
    const int e = (int)((__float_as_uint(a) >> 23) & 0xffu) - 127;          // floor(log2 a)
    const float scaled = a * __uint_as_float((uint32_t)(127 + 3 - e) << 23);  // a / 2^(e-3), in [8,16)
    const uint32_t q = (uint32_t)rintf(scaled);                              // 8..16 (16 carries)
    code = ((uint32_t)(e + 7) << 3) + (q - 8u);
    if (code > 0x7eu) code = 0x7eu;
  }
  return sign | code;
}

// FP8 E4M3 byte -> BF16 bits (exact: every E4M3 value has <= 4 significant bits)
__device__ __forceinline__ uint32_t fp8_to_bf16(uint32_t b) {
  const uint32_t s = (b & 0x80u) << 8;
  const uint32_t em = b & 0x7fu;
  uint32_t mag;
  if (em >= 8u) {
    mag = (em << 4) + (120u << 7);  // exponent field e+120, mantissa bits shifted into place
  } else {
    mag = __float_as_uint((float)em * 0.001953125f) >> 16;  // m * 2^-9, exact
  }
  return s | mag;
}
__device__ __forceinline__ float fp8_to_f32(uint32_t b) { return bf16_to_f32(fp8_to_bf16(b)); }

// FP8 E4M3 byte -> FP16 bits (exact: E4M3's range 2^-9 .. 448 lies inside FP16's normal range)
__device__ __forceinline__ uint32_t fp8_to_f16(uint32_t b) {
  const uint32_t s = (b & 0x80u) << 8;
  const uint32_t em = b & 0x7fu;
  uint32_t mag;
  if (em >= 8u) {
    mag = (em << 7) + (8u << 10);  // exponent field e+8, mantissa bits shifted into place
  } else {
    mag = __builtin_bit_cast(uint16_t, (_Float16)((float)em * 0.001953125f));  // m * 2^-9, exact
  }
  return s | mag;
}

// BF16 bits -> FP16 bits, round to nearest even, clamped to +-65504 (FP16's largest finite)
__device__ __forceinline__ uint32_t bf16_to_f16_sat(uint32_t b) {
  const float f = fminf(fmaxf(bf16_to_f32(b), -65504.0f), 65504.0f);
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// ---------------------------------------------------------------------------
// MXFP4 (E2M1 elements, E8M0 block scale), OCP MX v1.0 scale rule
// ---------------------------------------------------------------------------
// Shared exponent of a block from its max magnitude: floor(log2 amax) - 2, clamped.
__device__ __forceinline__ int mx_scale_exp(float amax) {
  if (!(amax > 0.0f)) return -127;
  int e = ilogbf(amax) - 2;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}
// E2M1 code (sign in bit 3) of a value already divided by the block scale: RNE, saturating.
// The magnitude code counts the rounding boundaries at or below |v|: a tie at
// 0.25, 1.25, 2.5 or 5 rounds down to the even code, at 0.75, 1.75 or 3.5 up.
// Written as 7 minus the boundaries above |v| (branch-free; NaN gives 7).
__device__ __forceinline__ uint32_t e2m1_code(float v) {
  const float a = fabsf(v);
  const uint32_t above = (uint32_t)(a <= 0.25f) + (uint32_t)(a < 0.75f) + (uint32_t)(a <= 1.25f) +
                         (uint32_t)(a < 1.75f) + (uint32_t)(a <= 2.5f) + (uint32_t)(a < 3.5f) + (uint32_t)(a <= 5.0f);
  return ((__float_as_uint(v) >> 28) & 0x8u) | (7u - above);
}

// ---------------------------------------------------------------------------
// Wave helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// n_vis(b,t) = min(n_entries[b], (t+1)/m, n_cap), never negative
__device__ __forceinline__ int64_t visible_entries(int64_t n_entries, int64_t t, int ratio, int64_t n_cap) {
  // (t+1)/ratio; a power-of-two ratio (m = 4, m' = 128) shifts instead of a
  // 64-bit division (a long sequence); t < 0 is handled below either way
  int64_t v = (ratio & (ratio - 1)) == 0 ? (t + 1) >> __builtin_ctz((unsigned)ratio) : (t + 1) / ratio;
  if (t < 0) v = 0;
  if (v > n_entries) v = n_entries;
  if (v > n_cap) v = n_cap;
  return v < 0 ? 0 : v;
}

// ---------------------------------------------------------------------------
// Top-k keys (shared by the indexer, which can histogram its scores, and top-k)
// ---------------------------------------------------------------------------
constexpr uint32_t INVALID = 0xffffffffu;  // marker for -inf (never selected)

__device__ __forceinline__ uint32_t bf16_key(uint32_t u) {
  if (u == 0xff80u) return INVALID;  // -inf
  if ((u & 0x7fffu) == 0) u = 0;      // -0 ties with +0
  return (u & 0x8000u) ? (~u & 0xffffu) : (u | 0x8000u);
}

// Work-group histogram of 256 bins kept as HREP copies, word hist[bin*HREP + c]
// for lanes with lane % HREP == c: decode scores crowd into a few bins, and
// the copies spread a wave's atomics on one bin over HREP banks.
constexpr int HREP = 16;
__device__ __forceinline__ void rep_clear(uint32_t* hist, int tid) {
#pragma unroll
  for (int c = 0; c < HREP; ++c) hist[tid * HREP + c] = 0u;
}
__device__ __forceinline__ void rep_add(uint32_t* hist, uint32_t bin, int tid) {
  atomicAdd(&hist[bin * HREP + (tid & (HREP - 1))], 1u);
}
__device__ __forceinline__ uint32_t rep_total(const uint32_t* hist, int bin) {
  uint32_t t = 0;
#pragma unroll
  for (int c = 0; c < HREP; ++c) t += hist[bin * HREP + ((c + bin) & (HREP - 1))];  // rotated: fewer conflicts
  return t;
}

// Write channel c of a KV row in the storage format (float32, BF16, or the
// mixed row: FP8 E4M3 for dims 0..127, BF16 for 128..191).
__device__ __forceinline__ void store_entry_channel(uint8_t* row, int kv_dtype, int c, float v) {
  if (kv_dtype == CSA_F32) {
    reinterpret_cast<float*>(row)[c] = v;
  } else if (kv_dtype == CSA_BF16) {
    reinterpret_cast<uint16_t*>(row)[c] = (uint16_t)f32_to_bf16_rne(v);
  } else if (c < DIM_NOPE) {
    row[c] = (uint8_t)f32_to_fp8_sat(v);
  } else {
    reinterpret_cast<uint16_t*>(row + DIM_NOPE)[c - DIM_NOPE] = (uint16_t)f32_to_bf16_rne(v);
  }
}

// Row of position p in a ring of `rows` rows based at `base`; -1 if p < base.
__device__ __forceinline__ int64_t ring_row(int64_t p, int64_t base, int64_t rows) {
  const int64_t rel = p - base;
  return rel < 0 ? -1 : rel % rows;
}

__host__ __device__ __forceinline__ int row_bytes(int dtype) {
  return dtype == CSA_F32 ? 4 * DIM : dtype == CSA_BF16 ? 2 * DIM : ROW_BYTES;
}

// Where the entries of a decode cache live: contiguous per sequence (pages
// null; entry e of sequence b is row b * cap + e) or paged (entry e of
// sequence b is row e mod 2^shift of physical page pages[b][e >> shift]; the
// page id is clamped into the pool, so a bad table cannot address outside it).
struct EntryPages {
  const int32_t* pages;  // [batch, cap >> shift] or null
  int shift;
  int pool_pages;
  __host__ __device__ __forceinline__ bool paged() const { return pages != nullptr; }
};
__device__ __forceinline__ int64_t entry_row(const EntryPages& m, int64_t cap, int b, int64_t e) {
  if (!m.pages) return (int64_t)b * cap + e;
  int pg = m.pages[(int64_t)b * (cap >> m.shift) + (e >> m.shift)];
  pg = pg < 0 ? 0 : (pg >= m.pool_pages ? m.pool_pages - 1 : pg);
  return ((int64_t)pg << m.shift) | (e & ((1 << m.shift) - 1));
}
__host__ __device__ inline EntryPages csa_entry_pages(const csa_decode_cache& c) {
  EntryPages m{nullptr, 0, 0};
  if (c.page_entries > 0) m = EntryPages{c.csa_pages, 31 - __builtin_clz((unsigned)c.page_entries), c.csa_pool_pages};
  return m;
}
__host__ __device__ inline EntryPages hca_entry_pages(const csa_decode_cache& c) {
  EntryPages m{nullptr, 0, 0};
  if (c.page_entries > 0) m = EntryPages{c.hca_pages, 31 - __builtin_clz((unsigned)c.page_entries), c.hca_pool_pages};
  return m;
}

// ---------------------------------------------------------------------------
// Internal launchers (arguments already validated by the C-ABI layer)
// ---------------------------------------------------------------------------
hipError_t launch_kv_pack(const void* x, int x_dtype, int64_t n_rows, int64_t x_stride, void* out,
                          int out_dtype, int64_t out_stride, hipStream_t s);
hipError_t launch_kv_append(const void* x, int x_dtype, int batch, const int64_t* pos, void* raw_ring, int raw_dtype,
                            int64_t raw_rows, int64_t raw_base, void* win_ring, int win_dtype, int64_t win_rows,
                            int64_t win_base, hipStream_t s);
hipError_t launch_mxfp4_quantize(const float* x, int64_t n_rows, int d, uint8_t* codes, uint8_t* scales,
                                 hipStream_t s);
hipError_t launch_csa_compress(const void* x, int x_dtype, int batch, int64_t raw_rows, int64_t raw_base,
                               const float* w_gate, const float* pos_bias, int64_t entry_begin, int n_new,
                               void* kv_out, int kv_dtype, int64_t n_cap, const float* w_idx, int d_idx,
                               void* key_out, uint8_t* key_scales, int key_dtype, hipStream_t s);
hipError_t launch_hca_compress(const void* x, int x_dtype, int batch, int64_t raw_rows, int64_t raw_base,
                               const float* w_gate, const float* pos_bias, int64_t entry_begin, int n_new,
                               void* kv_out, int kv_dtype, int64_t n_cap, hipStream_t s);
hipError_t launch_indexer_f32(const float* q, const float* w, const float* k, int batch, int n_q, int n_heads,
                              int d_idx, int64_t n_cap, const int32_t* n_entries, const int64_t* q_pos, int ratio,
                              float* scores, hipStream_t s);
hipError_t launch_indexer_mxfp4(const void* q, bool q_f32, const uint8_t* q_scales, const float* w, const uint8_t* k,
                                const uint8_t* k_scales, int batch, int n_q, int n_heads, int d_idx, int64_t n_cap,
                                const int32_t* n_entries, const int64_t* q_pos, int ratio, uint16_t* scores,
                                hipStream_t s, uint32_t* hist = nullptr, int hist_row_words = 0,
                                hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr,
                                EntryPages pages = EntryPages{nullptr, 0, 0});
size_t topk_ws_bytes(int batch, int n_q, int64_t n_cap, int k, int score_dtype);
hipError_t launch_topk(const void* scores, int score_dtype, int batch, int n_q, int64_t n_cap,
                       const int32_t* n_entries, const int64_t* q_pos, int ratio, int k, int32_t* idx_out, void* ws,
                       hipStream_t s, bool pass1_done = false);
// Split (decode) top-k: whether it applies, and its per-row totals in the
// workspace: row r's high-byte totals at base + r * row_words, the low-byte
// totals 256 words further.  Zero at rest.
bool topk_uses_split(int64_t rows, int64_t n_cap, int score_dtype);
uint32_t* topk_split_totals(void* ws, int* row_words);

// layers: bit 0 the CSA layer (with the indexer query), bit 1 the HCA layer;
// advance: pos[b] moves to the next position once every work-group has read it.
hipError_t launch_decode_append(const csa_decode_cache& c, const void* x_csa, const void* x_hca, int x_dtype,
                                int64_t* q_pos, int32_t* arrive, const float* q_idx, uint8_t* q_codes,
                                uint8_t* q_scales, hipStream_t s, int layers = 3, bool advance = true);
hipError_t launch_decode_prime(const csa_decode_cache& c, const void* x_csa, const void* x_hca, int x_dtype,
                               int n_tok, hipStream_t s);
hipError_t launch_decode_fork(const csa_decode_cache& c, int src, int dst, hipStream_t s);

struct AttnArgs {
  const void* q;
  int q_dtype;
  int batch, n_q, n_heads;
  const void* kv;
  int kv_dtype;
  int64_t n_cap;
  const int32_t* n_entries;
  int ratio;
  const int32_t* idx;  // NULL -> dense (every visible entry)
  int k;
  const void* win;
  int64_t win_rows, win_base;
  const int64_t* q_pos;
  int window;
  float scale;
  const float* sink;
  void* out;
  int out_dtype;
  float* lse;
  void* ws;
  EntryPages pages;  // paged entries (kv is then the page pool), or pages null
};
size_t attn_ws_bytes(int batch, int n_q, int n_heads, int64_t max_keys, int q_dtype, int kv_dtype);
hipError_t launch_attention(const AttnArgs& a, int64_t max_keys, hipStream_t s);
// Two problems (same head count) in one launch and one merge; their workspaces
// (a0.ws, a1.ws) must not overlap.  Results equal launch_attention's.
hipError_t launch_attention_pair(const AttnArgs& a0, int64_t max_keys0, const AttnArgs& a1, int64_t max_keys1,
                                 hipStream_t s);

}  // namespace csa
