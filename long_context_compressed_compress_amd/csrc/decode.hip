// Decode over a device-resident cache: append + compress-on-boundary for a CSA
// layer and an HCA layer in one launch.
//   Append ([TRIPBOT] §3.3: the window of the last raw tokens; [CSDN]
//   核心创新一 §1.4: stored rows FP8 + BF16).
//   Compression ([TRIPBOT] §3.1 第一步 + Figure 3, §3.2; [CSDN] 核心创新一 §1.1):
//   entry = per-channel softmax over the block's slots of (x.W_gate + bias[slot])
//   weighting the slots' raw KV.  A token's gate logits do not depend on the
//   slot, so they are computed once, when the token arrives, and kept in a ring
//   next to its raw KV; a boundary step only pools.
// The arithmetic (order of every sum, float32 throughout) is the one of the
// prefill compressors, so a decoded entry has the same bits as csa_compress /
// hca_compress would give on the same raw tokens.
#include "../../include/libcsa.h"
#include "common.h"

namespace csa {

namespace {

constexpr int CSA_RING = 8;    // CSA entry i reads tokens 4i-4 .. 4i+3
constexpr int HCA_RING = 128;  // HCA entry i reads tokens 128i .. 128i+127
constexpr int DEC_THREADS = 2 * DIM;  // threads [0,192): CSA layer, [192,384): HCA layer
constexpr int MAX_DIDX = 256;

__device__ __forceinline__ float load_x(const void* x, int x_dtype, int64_t i) {
  return x_dtype == CSA_F32 ? reinterpret_cast<const float*>(x)[i]
                            : bf16_to_f32(reinterpret_cast<const uint16_t*>(x)[i]);
}

// Channel c of token p: BF16 raw KV into the raw ring and its gate logit
// x.W_gate[:, c] (d ascending, from the BF16 value) into the logit ring when
// `to_ring`, stored row into the window ring when `to_win`.  xs = this layer's
// LDS row, filled here; `sync` = a work-group barrier between filling and
// reading it, reached by every thread.
template <typename Sync>
__device__ __forceinline__ float append_channel(const csa_decode_cache& C, int layer, int b, int c, int64_t p,
                                                float xv, bool to_ring, bool to_win, float* xs, const float* wcol,
                                                Sync sync) {
  const int rr = layer ? HCA_RING : CSA_RING;
  uint16_t* raw = layer ? C.hca_raw : C.csa_raw;
  float* lg = layer ? C.hca_logits : C.csa_logits;
  uint8_t* win = layer ? C.hca_win : C.csa_win;
  const uint32_t xb = f32_to_bf16_rne(xv);
  const int64_t rrow = (int64_t)b * rr + p % rr;
  if (to_ring) raw[rrow * DIM + c] = (uint16_t)xb;
  if (to_win)
    store_entry_channel(win + ((int64_t)b * C.win_rows + p % C.win_rows) * CSA_MIXED_ROW_BYTES, CSA_KV_MIXED, c,
                        xv);
  xs[c] = bf16_to_f32(xb);
  sync();
  float g = 0.0f;
  if (to_ring) {
#pragma unroll
    for (int d = 0; d < DIM; ++d) g = fmaf(xs[d], wcol[d], g);
    lg[rrow * DIM + c] = g;
  }
  return g;
}

// Column c of a layer's gate weights, W_gate[:, c], into registers: 192
// independent loads in flight at once (it does not depend on the position).
__device__ __forceinline__ void load_wcol(const csa_decode_cache& C, int layer, int c, float (&wcol)[DIM]) {
  const float* wg = layer ? C.hca_w_gate : C.csa_w_gate;
#pragma unroll
  for (int d = 0; d < DIM; ++d) wcol[d] = wg[d * DIM + c];
}

}  // namespace

// A layer's channels in waves of 64 over APPEND_GROUPS work-groups: a step
// reads 2 x 192 gate-weight columns (192 loads per channel), and one loading
// wave per work-group spreads those loads over six compute units instead of two.
constexpr int APPEND_GROUPS = DIM / 64;

// grid (B, G * n_layers + (CSA ? 1 : 0)), block 192, sequence b.  The layers
// run are those of `layers` (bit 0: CSA, bit 1: HCA); blockIdx.y = y: the
// first G values of y are the first layer's channel waves, the next G the
// second's, and with the CSA layer the last y quantizes the step's indexer
// query to MXFP4.  Thread c stands for channel c;
// in a layer's work-group g only wave g (channels 64g .. 64g+63) writes the
// rings, computes gate logits and pools, the other waves stage the token's row
// in LDS for the dot products.  When a CSA entry completes, the CSA work-group
// 0 takes every channel (the key projection needs the whole entry) and the
// other CSA work-groups only report arrival.  Every layer work-group of a
// sequence reads pos[b] first; with `advance`, the last to arrive (per-sequence
// arrival counter, zero at rest) advances pos[b], after all have read it.
// The first layer's work-group 0 records the decoded position in q_pos[b].
__global__ void __launch_bounds__(DIM) decode_append_kernel(csa_decode_cache C, const void* __restrict__ x_csa,
                                                            const void* __restrict__ x_hca, int x_dtype,
                                                            int64_t* __restrict__ q_pos, int32_t* __restrict__ arrive,
                                                            const float* __restrict__ q_idx, uint8_t* __restrict__ q_codes,
                                                            uint8_t* __restrict__ q_scales, int layers, int advance) {
  __shared__ float xs[DIM];
  __shared__ float cs[DIM];         // pooled CSA entry (float32) for the key projection
  __shared__ float kq[MAX_DIDX];    // its projected key
  __shared__ uint8_t codes[MAX_DIDX];  // its E2M1 codes, one per byte
  const int b = blockIdx.x;
  const int y = blockIdx.y;  // uniform
  const int c = threadIdx.x;
  const int n_layers = (layers & 1) + (layers >> 1);
  if (y == APPEND_GROUPS * n_layers) {  // (only launched with the CSA layer)
    // this step's indexer query, [idx_heads][idx_dim] float32, to MXFP4 once per
    // sequence (the rule of mxfp4_quantize: block k = values 32k .. 32k+31);
    // it needs neither the position nor the rings
    const int nb = C.idx_heads * C.idx_dim / MXB;
    const float* qr = q_idx + (int64_t)b * C.idx_heads * C.idx_dim;
    for (int k = c; k < nb; k += DIM) {
      float v[MXB];
#pragma unroll
      for (int u = 0; u < MXB / 4; ++u) {
        const float4 f = reinterpret_cast<const float4*>(qr + k * MXB)[u];
        v[4 * u] = f.x, v[4 * u + 1] = f.y, v[4 * u + 2] = f.z, v[4 * u + 3] = f.w;
      }
      float amax = 0.0f;
#pragma unroll
      for (int u = 0; u < MXB; ++u) amax = fmaxf(amax, fabsf(v[u]));
      const int ex = mx_scale_exp(amax);
      uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
      for (int u = 0; u < MXB; ++u) w[u / 8] |= e2m1_code(ldexpf(v[u], -ex)) << (4 * (u % 8));
      reinterpret_cast<uint4*>(q_codes + (int64_t)b * nb * (MXB / 2))[k] = make_uint4(w[0], w[1], w[2], w[3]);
      q_scales[(int64_t)b * nb + k] = (uint8_t)(ex + 127);
    }
    return;
  }
  const int slot = y >= APPEND_GROUPS ? 1 : 0;     // first or second layer of the launch
  const int layer = layers == 2 ? 1 : slot;          // 0: CSA, 1: HCA
  const int grp = y - slot * APPEND_GROUPS;
  const int arrivals = APPEND_GROUPS * n_layers;     // work-groups that read pos[b]
  const bool own = (c >> 6) == grp;  // channel c is this work-group's (uniform per wave)
  float wcol[DIM];
  if (own) load_wcol(C, layer, c, wcol);  // requested first: it does not depend on the position
  const int64_t p = C.pos[b];
  if (p < 0) {  // inactive sequence (uniform per work-group): decodes nothing, keeps its state
    if (slot == 0 && grp == 0 && c == 0) q_pos[b] = p;
    return;
  }
  // CSA entry ci = (p+1)/4 - 1 completes at p: slots s = 0..7 hold tokens p-7+s
  // (slots with a negative position are left out of the softmax).  The seven
  // earlier slots and the biases are requested before the gate product.
  const bool csa_done = layer == 0 && (p + 1) % 4 == 0 && (p + 1) / 4 - 1 < C.csa_cap;  // uniform
  const int64_t ci = (p + 1) / 4 - 1;
  if (csa_done && grp != 0) {  // CSA work-group 0 takes this step's channels
    __syncthreads();            // every thread of this work-group has read pos[b]
    if (advance && c == 0 && atomicAdd(&arrive[b], 1) == arrivals - 1) {
      arrive[b] = 0;
      C.pos[b] = p + 1;
    }
    return;
  }
  const bool mine = csa_done || own;  // this work-group writes channel c
  if (!own && csa_done) load_wcol(C, layer, c, wcol);
  const float xv = load_x(layer ? x_hca : x_csa, x_dtype, (int64_t)b * DIM + c);
  float gz[8], xz[8], bz[8];
  if (csa_done) {
#pragma unroll
    for (int s = 0; s < 7; ++s) {
      const int64_t j = p - 7 + s;
      gz[s] = xz[s] = 0.0f;
      if (j >= 0) {
        const int64_t r = (int64_t)b * CSA_RING + j % CSA_RING;
        gz[s] = C.csa_logits[r * DIM + c];
        xz[s] = bf16_to_f32(C.csa_raw[r * DIM + c]);
      }
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) bz[s] = C.csa_pos_bias[s * DIM + c];
  }
  const float g = append_channel(C, layer, b, c, p, xv, mine, mine, xs, wcol, [] { __syncthreads(); });

  if (csa_done) {  // uniform
    // the key projection's weights (column c of w_idx) into the registers the
    // gate column held, requested before the pooling (key widths up to 192)
    const int di = C.idx_dim;
    if (di <= DIM && c < di) {
#pragma unroll
      for (int cc = 0; cc < DIM; ++cc) wcol[cc] = C.csa_w_idx[cc * di + c];
    }
    gz[7] = g;
    xz[7] = xs[c];
    float z[8], mx = -INFINITY;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const bool valid = p - 7 + s >= 0;
      z[s] = valid ? gz[s] + bz[s] : -INFINITY;
      mx = fmaxf(mx, z[s]);
    }
    float den = 0.0f, num = 0.0f;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const float pe = z[s] == -INFINITY ? 0.0f : expf(z[s] - mx);
      den += pe;
      num = fmaf(pe, xz[s], num);
    }
    const float v = num / den;
    const int64_t ent = entry_row(csa_entry_pages(C), C.csa_cap, b, ci);  // row of the entry (and of its key)
    store_entry_channel(C.csa_kv + ent * CSA_MIXED_ROW_BYTES, CSA_KV_MIXED, c, v);
    cs[c] = v;
    __syncthreads();
    // key k[t] = sum_c cs[c] * w_idx[c][t], c ascending (one thread per t)
    if (di <= DIM) {
      if (c < di) {
        float k = 0.0f;
#pragma unroll
        for (int cc = 0; cc < DIM; ++cc) k = fmaf(cs[cc], wcol[cc], k);
        kq[c] = k;
      }
    } else {
      for (int t = c; t < di; t += DIM) {
        float k = 0.0f;
#pragma unroll 16
        for (int cc = 0; cc < DIM; ++cc) k = fmaf(cs[cc], C.csa_w_idx[cc * di + t], k);
        kq[t] = k;
      }
    }
    __syncthreads();
    // MXFP4 (the rule of mxfp4_quantize), one value per thread: block maximum,
    // shared exponent, E2M1 code; then 8 codes per 32-bit word
    for (int t = c; t < di; t += DIM) {
      const float* blk = kq + (t & ~(MXB - 1));
      float amax = 0.0f;
#pragma unroll
      for (int u = 0; u < MXB; ++u) amax = fmaxf(amax, fabsf(blk[u]));
      const int ex = mx_scale_exp(amax);
      codes[t] = (uint8_t)e2m1_code(ldexpf(kq[t], -ex));
      if ((t & (MXB - 1)) == 0) C.csa_key_scales[ent * (di / MXB) + t / MXB] = (uint8_t)(ex + 127);
    }
    __syncthreads();
    for (int t = c; t < di / 8; t += DIM) {
      uint32_t word = 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) word |= (uint32_t)codes[8 * t + u] << (4 * u);
      reinterpret_cast<uint32_t*>(C.csa_keys + ent * (di / 2))[t] = word;
    }
  }

  // HCA entry hi = (p+1)/128 - 1 completes at p: slot s = token 128*hi + s = ring row s.
  // Sums in the prefill compressor's order: eight partial sums over the slots
  // t, t+8, .., t+120, then the partials in order t = 0..7.
  const bool hca_done = layer == 1 && (p + 1) % HCA_RING == 0 && (p + 1) / HCA_RING - 1 < C.hca_cap;  // uniform
  const int64_t hi = (p + 1) / HCA_RING - 1;
  if (hca_done && mine) {
    const int64_t r0 = (int64_t)b * HCA_RING;
    float mx = -INFINITY;
#pragma unroll 32
    for (int s = 0; s < HCA_RING; ++s)
      mx = fmaxf(mx, C.hca_logits[(r0 + s) * DIM + c] + C.hca_pos_bias[s * DIM + c]);
    float den = 0.0f, num = 0.0f;
    for (int t = 0; t < 8; ++t) {
      float dt = 0.0f, nt = 0.0f;
#pragma unroll
      for (int r = 0; r < HCA_RING / 8; ++r) {
        const int s = t + 8 * r;
        const float a = C.hca_logits[(r0 + s) * DIM + c] + C.hca_pos_bias[s * DIM + c];
        const float pe = expf(a - mx);
        dt += pe;
        nt = fmaf(pe, bf16_to_f32(C.hca_raw[(r0 + s) * DIM + c]), nt);
      }
      den += dt;
      num += nt;
    }
    store_entry_channel(C.hca_kv + entry_row(hca_entry_pages(C), C.hca_cap, b, hi) * CSA_MIXED_ROW_BYTES,
                        CSA_KV_MIXED, c, num / den);
  }

  __syncthreads();  // every thread of this work-group has read pos[b]
  if (c == 0) {
    if (grp == 0) {
      if (slot == 0) q_pos[b] = p;
      if (layer == 0) {
        if ((p + 1) % 4 == 0) C.csa_entries[b] = (int32_t)(ci + 1 < C.csa_cap ? ci + 1 : C.csa_cap);
      } else if ((p + 1) % HCA_RING == 0) {
        C.hca_entries[b] = (int32_t)(hi + 1 < C.hca_cap ? hi + 1 : C.hca_cap);
      }
    }
    if (advance && atomicAdd(&arrive[b], 1) == arrivals - 1) {  // every layer work-group has read pos[b]
      arrive[b] = 0;
      C.pos[b] = p + 1;
    }
  }
}

// grid (B, n_tok), block 384: token t of sequence b at position pos[b]-n_tok+t
// into both layers' rings (no compression, pos unchanged).  Only the tokens
// that stay in a ring are written to it, so no two work-groups share a row.
__global__ void __launch_bounds__(DEC_THREADS) decode_prime_kernel(csa_decode_cache C, const void* __restrict__ x_csa,
                                                                   const void* __restrict__ x_hca, int x_dtype,
                                                                   int n_tok) {
  __shared__ float xs[2][DIM];
  const int b = blockIdx.x;
  const int t = blockIdx.y;
  const int layer = threadIdx.x >= DIM ? 1 : 0;
  const int c = threadIdx.x - layer * DIM;
  const int64_t end = C.pos[b];
  const int64_t p = end - n_tok + t;
  if (p < 0) return;  // uniform per work-group
  const float xv = load_x(layer ? x_hca : x_csa, x_dtype, ((int64_t)b * n_tok + t) * DIM + c);
  const bool to_ring = p >= end - (layer ? HCA_RING : CSA_RING);
  const bool to_win = p >= end - C.win_rows;
  float wcol[DIM];
  if (to_ring) load_wcol(C, layer, c, wcol);
  append_channel(C, layer, b, c, p, xv, to_ring, to_win, xs[layer], wcol, [] { __syncthreads(); });
}

// Copy n16 16-byte words from src to dst, grid-strided over blockIdx.x.
__device__ __forceinline__ void copy_words(const void* src, void* dst, int64_t n16) {
  const uint4* s = static_cast<const uint4*>(src);
  uint4* d = static_cast<uint4*>(dst);
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (int64_t)gridDim.x * blockDim.x)
    d[i] = s[i];
}
__device__ __forceinline__ void copy_bytes(const uint8_t* src, uint8_t* dst, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

// Sequence dst takes sequence src's state (paged caches).  blockIdx.y picks
// the part: 0..5 the rings, 6 position, counts and the shared page-table
// entries, 7..9 the rows of a partly filled last page (CSA rows, CSA keys and
// scales, HCA rows).  Nothing read here is written here: src's state is only
// read, and the table entries written (dst's pages below the count) are not
// the ones the partial copies read (dst's page at the count).
__global__ void __launch_bounds__(256) decode_fork_kernel(csa_decode_cache C, int src, int dst) {
  const int part = blockIdx.y;
  const int64_t P = C.page_entries;
  const int sh = 31 - __builtin_clz((unsigned)C.page_entries);
  const int64_t nc = C.csa_entries[src], nh = C.hca_entries[src];
  switch (part) {
    case 0: copy_words(C.csa_raw + (int64_t)src * CSA_RING * DIM, C.csa_raw + (int64_t)dst * CSA_RING * DIM,
                       CSA_RING * DIM * 2 / 16); break;
    case 1: copy_words(C.csa_logits + (int64_t)src * CSA_RING * DIM, C.csa_logits + (int64_t)dst * CSA_RING * DIM,
                       CSA_RING * DIM * 4 / 16); break;
    case 2: copy_words(C.hca_raw + (int64_t)src * HCA_RING * DIM, C.hca_raw + (int64_t)dst * HCA_RING * DIM,
                       HCA_RING * DIM * 2 / 16); break;
    case 3: copy_words(C.hca_logits + (int64_t)src * HCA_RING * DIM, C.hca_logits + (int64_t)dst * HCA_RING * DIM,
                       HCA_RING * DIM * 4 / 16); break;
    case 4: copy_words(C.csa_win + src * C.win_rows * ROW_BYTES, C.csa_win + dst * C.win_rows * ROW_BYTES,
                       C.win_rows * ROW_BYTES / 16); break;
    case 5: copy_words(C.hca_win + src * C.win_rows * ROW_BYTES, C.hca_win + dst * C.win_rows * ROW_BYTES,
                       C.win_rows * ROW_BYTES / 16); break;
    case 6: {
      const int64_t tc = C.csa_cap >> sh, th = C.hca_cap >> sh;
      const int64_t fc = nc >> sh, fh = nh >> sh;  // full pages: shared
      for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < fc + fh;
           i += (int64_t)gridDim.x * blockDim.x) {
        if (i < fc) C.csa_pages[dst * tc + i] = C.csa_pages[src * tc + i];
        else C.hca_pages[dst * th + (i - fc)] = C.hca_pages[src * th + (i - fc)];
      }
      if (blockIdx.x == 0 && threadIdx.x == 0) {
        C.pos[dst] = C.pos[src];
        C.csa_entries[dst] = (int32_t)nc;
        C.hca_entries[dst] = (int32_t)nh;
      }
      break;
    }
    default: {  // the partly filled page, if any
      const bool hca = part == 9;
      const int64_t n = hca ? nh : nc;
      const int64_t rows = n & (P - 1);
      if (rows == 0) break;
      const EntryPages m = hca ? hca_entry_pages(C) : csa_entry_pages(C);
      const int64_t cap = hca ? C.hca_cap : C.csa_cap;
      const int64_t first = n - rows;  // entry at the start of the page
      const int64_t rs = entry_row(m, cap, src, first), rd = entry_row(m, cap, dst, first);
      if (part == 8) {
        const int kb = C.idx_dim / 2, sb = C.idx_dim / 32;
        copy_bytes(C.csa_keys + rs * kb, C.csa_keys + rd * kb, rows * kb);
        copy_bytes(C.csa_key_scales + rs * sb, C.csa_key_scales + rd * sb, rows * sb);
      } else {
        uint8_t* kv = hca ? C.hca_kv : C.csa_kv;
        copy_words(kv + rs * ROW_BYTES, kv + rd * ROW_BYTES, rows * ROW_BYTES / 16);
      }
    }
  }
}

hipError_t launch_decode_fork(const csa_decode_cache& c, int src, int dst, hipStream_t s) {
  hipLaunchKernelGGL(decode_fork_kernel, dim3(16, 10), dim3(256), 0, s, c, src, dst);
  return hipGetLastError();
}

hipError_t launch_decode_append(const csa_decode_cache& c, const void* x_csa, const void* x_hca, int x_dtype,
                                int64_t* q_pos, int32_t* arrive, const float* q_idx, uint8_t* q_codes,
                                uint8_t* q_scales, hipStream_t s, int layers, bool advance) {
  const int n_layers = (layers & 1) + (layers >> 1);
  const int groups = APPEND_GROUPS * n_layers + (layers & 1);
  hipLaunchKernelGGL(decode_append_kernel, dim3(c.batch, groups), dim3(DIM), 0, s, c, x_csa, x_hca, x_dtype, q_pos,
                     arrive, q_idx, q_codes, q_scales, layers, advance ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_decode_prime(const csa_decode_cache& c, const void* x_csa, const void* x_hca, int x_dtype,
                               int n_tok, hipStream_t s) {
  hipLaunchKernelGGL(decode_prime_kernel, dim3(c.batch, n_tok), dim3(DEC_THREADS), 0, s, c, x_csa, x_hca, x_dtype,
                     n_tok);
  return hipGetLastError();
}

}  // namespace csa
