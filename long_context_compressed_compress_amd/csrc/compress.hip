// CSA and HCA compressors: softmax-gated pooling of raw token KV into one
// entry per block of tokens.
//   CSA (「论文解读｜DeepSeek-V4：百万 token 上下文的效率革命」, blog.tripbot.top,
//   §3.1 第一步 + Figure 3; gitcode.csdn.net DeepSeek-V4 解读 §1.1 工程细节):
//   m = 4, entry i reads the previous block C^b (tokens 4i-4..4i-1, slots 0..3)
//   and its own block C^a (tokens 4i..4i+3, slots 4..7).
//   HCA (blog.tripbot.top §3.2): m' = 128, entry i reads tokens 128i..128i+127.
// Per channel c: z[s,c] = x_{j(s)} . w_gate[:,c] + bias[s,c]; weights = softmax
// over the existing slots; entry[c] = sum_s weight[s,c] * x_{j(s)}[c].
// All arithmetic in float32; the entry is rounded to its storage format once.
#include "common.h"

namespace csa {

namespace {

__device__ __forceinline__ float load_raw(const uint8_t* row, int x_dtype, int d) {
  if (x_dtype == CSA_F32) return reinterpret_cast<const float*>(row)[d];
  return bf16_to_f32(reinterpret_cast<const uint16_t*>(row)[d]);
}

constexpr int MAX_DIDX = 256;  // largest indexer key width
constexpr int WROWS = 64;      // weight rows staged in LDS per round

// Cooperative copy of rows [r0, r0 + nr) of a row-major float32 matrix with
// `cols` columns (cols % 4 == 0, 16-byte aligned) into LDS, 16 bytes at a time.
__device__ __forceinline__ void stage_rows(const float* __restrict__ w, int cols, int r0, int nr, float* lds,
                                           int tid, int nthr) {
  const int n4 = nr * cols / 4;
  const float4* src = reinterpret_cast<const float4*>(w + (size_t)r0 * cols);
  float4* dst = reinterpret_cast<float4*>(lds);
#pragma unroll 16
  for (int i = tid; i < n4; i += nthr) dst[i] = src[i];
}

// NTOK consecutive raw tokens of one sequence into LDS as float32 rows
// (xs[n][DIM]), from a 16-byte aligned ring: 16-byte pieces (8 BF16 or 4
// float32 values), each thread requesting up to 12 pieces before it stores
// the first, so the loads' latencies overlap instead of adding up.
// row_of(n) is token n's ring row, or -1 for a token that is stored as zeros.
template <int NTHR, int NTOK, bool F32, typename RowOf>
__device__ __forceinline__ void stage_tokens(const uint8_t* __restrict__ ring, RowOf row_of, float* xs, int tid) {
  constexpr int PPR = F32 ? DIM / 4 : DIM / 8;  // pieces per row
  constexpr int TOTAL = NTOK * PPR;
  constexpr int PER = (TOTAL + NTHR - 1) / NTHR;
  constexpr int G = PER < 12 ? PER : 12;
  constexpr int RB = F32 ? DIM * 4 : DIM * 2;
  for (int k0 = 0; k0 < PER; k0 += G) {
    uint4 v[G];
    bool ok[G];
#pragma unroll
    for (int k = 0; k < G; ++k) {
      const int q = tid + NTHR * (k0 + k);
      const int n = q / PPR, part = q - n * PPR;
      const int64_t r = (q < TOTAL && k0 + k < PER) ? row_of(n) : -1;
      // absent tokens read ring row 0 (always present) and are zeroed when stored
      v[k] = *reinterpret_cast<const uint4*>(ring + (r >= 0 ? r : 0) * RB + 16 * part);
      ok[k] = r >= 0;
    }
#pragma unroll
    for (int k = 0; k < G; ++k) {
      const int q = tid + NTHR * (k0 + k);
      if (q >= TOTAL || k0 + k >= PER) continue;
      const int n = q / PPR, part = q - n * PPR;
      const uint32_t keep = ok[k] ? 0xffffffffu : 0u;
      const uint32_t w[4] = {v[k].x & keep, v[k].y & keep, v[k].z & keep, v[k].w & keep};
      if constexpr (F32) {
        *reinterpret_cast<uint4*>(xs + n * DIM + 4 * part) = make_uint4(w[0], w[1], w[2], w[3]);
      } else {
        float4* dst = reinterpret_cast<float4*>(xs + n * DIM + 8 * part);
        dst[0] = make_float4(__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u),
                             __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xffff0000u));
        dst[1] = make_float4(__uint_as_float(w[2] << 16), __uint_as_float(w[2] & 0xffff0000u),
                             __uint_as_float(w[3] << 16), __uint_as_float(w[3] & 0xffff0000u));
      }
    }
  }
}

__device__ __forceinline__ bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

// grid: (ceil(n_new / EPB), batch); block: 192 threads, thread c owns channel c.
// EPB entries per block read 4*EPB + 4 distinct tokens; the gate and key
// weights stream through LDS in rounds of WROWS rows.
template <int EPB>
__global__ void __launch_bounds__(192) csa_compress_kernel(
    const uint8_t* __restrict__ x, int x_dtype, int64_t raw_rows, int64_t raw_base,
    const float* __restrict__ w_gate, const float* __restrict__ pos_bias, int64_t entry_begin, int n_new,
    uint8_t* __restrict__ kv_out, int kv_dtype, int64_t n_cap, const float* __restrict__ w_idx, int d_idx,
    uint8_t* __restrict__ key_out, uint8_t* __restrict__ key_scales, int key_dtype) {
  constexpr int TOK = 4 * EPB + 4;                        // distinct tokens the block's entries read
  constexpr int KQ = (EPB * MAX_DIDX + DIM - 1) / DIM;    // key outputs per thread
  extern __shared__ float smem[];
  float* xs = smem;                    // [TOK][DIM] raw tokens, float32
  float* wsm = xs + TOK * DIM;         // [WROWS][<= MAX_DIDX] weight rows of the current round
  float* cs = wsm + WROWS * MAX_DIDX;  // [EPB][DIM] pooled entries (for the key projection)
  float* ks = cs + EPB * DIM;          // [EPB][MAX_DIDX] projected keys

  const int b = blockIdx.y;
  const int c = threadIdx.x;
  const int64_t i0 = entry_begin + (int64_t)blockIdx.x * EPB;
  const int ne = (int)min<int64_t>(EPB, entry_begin + n_new - i0);
  const int64_t j0 = 4 * (i0 - 1);  // token of slot 0 of the first entry
  const int ntok = 4 * ne + 4;
  const int xb = x_dtype == CSA_F32 ? 4 : 2;

  // Ring row of token j0 + n: one 64-bit remainder per work-group, then the
  // block's consecutive tokens step through the ring (they fit in it, so
  // they wrap at most once); tokens before position 0 or the ring's base
  // read as zero.
  const int64_t rel0 = j0 - raw_base;
  const int64_t m0 = rel0 >= 0 ? rel0 % raw_rows : rel0;
  auto row_of = [&](int n) -> int64_t {
    if (n >= ntok || j0 + n < 0 || rel0 + n < 0) return -1;
    const int64_t r = m0 + n;
    return r >= raw_rows ? r - raw_rows : r;
  };
  const uint8_t* ring = x + (int64_t)b * raw_rows * DIM * xb;
  if (aligned16(x)) {
    if (x_dtype == CSA_F32) stage_tokens<DIM, TOK, true>(ring, row_of, xs, c);
    else stage_tokens<DIM, TOK, false>(ring, row_of, xs, c);
  } else {
    for (int n = 0; n < TOK; ++n) {
      const int64_t r = row_of(n);
      xs[n * DIM + c] = r >= 0 ? load_raw(ring + r * DIM * xb, x_dtype, c) : 0.0f;
    }
  }

  // Gate logits for every token of the block, channel c: g[n] = x_n . w_gate[:, c] (d ascending)
  float g[TOK];
#pragma unroll
  for (int n = 0; n < TOK; ++n) g[n] = 0.0f;
  for (int d0 = 0; d0 < DIM; d0 += WROWS) {
    __syncthreads();  // previous round consumed (and xs complete)
    stage_rows(w_gate, DIM, d0, WROWS, wsm, c, DIM);
    __syncthreads();
    for (int d = 0; d < WROWS; d += 4) {  // four dims per LDS read of a token (same d order per sum)
      const float w0 = wsm[d * DIM + c], w1 = wsm[(d + 1) * DIM + c];
      const float w2 = wsm[(d + 2) * DIM + c], w3 = wsm[(d + 3) * DIM + c];
#pragma unroll
      for (int n = 0; n < TOK; ++n) {
        const float4 xv = *reinterpret_cast<const float4*>(xs + n * DIM + d0 + d);
        g[n] = fmaf(xv.x, w0, g[n]);
        g[n] = fmaf(xv.y, w1, g[n]);
        g[n] = fmaf(xv.z, w2, g[n]);
        g[n] = fmaf(xv.w, w3, g[n]);
      }
    }
  }

  float bias[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) bias[s] = pos_bias[s * DIM + c];

#pragma unroll
  for (int e = 0; e < EPB; ++e) {
    if (e >= ne) break;
    const int64_t i = i0 + e;
    float z[8], mx = -INFINITY;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const bool valid = 4 * (i - 1) + s >= 0;
      z[s] = valid ? g[4 * e + s] + bias[s] : -INFINITY;
      mx = fmaxf(mx, z[s]);
    }
    float den = 0.0f, num = 0.0f;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const float p = z[s] == -INFINITY ? 0.0f : expf(z[s] - mx);
      den += p;
      num = fmaf(p, xs[(4 * e + s) * DIM + c], num);
    }
    const float v = num / den;
    store_entry_channel(kv_out + ((int64_t)b * n_cap + i) * row_bytes(kv_dtype), kv_dtype, c, v);
    cs[e * DIM + c] = v;
  }

  if (w_idx == nullptr) return;
  // Key projection k[e][d] = sum_c cs[e][c] * w_idx[c][d] (c ascending)
  float kacc[KQ];
#pragma unroll
  for (int q = 0; q < KQ; ++q) kacc[q] = 0.0f;
  for (int c0 = 0; c0 < DIM; c0 += WROWS) {
    __syncthreads();
    stage_rows(w_idx, d_idx, c0, WROWS, wsm, c, DIM);
    __syncthreads();
#pragma unroll
    for (int q = 0; q < KQ; ++q) {
      const int p = c + DIM * q;
      if (p < ne * d_idx) {
        const int e = p / d_idx, d = p % d_idx;
        float acc = kacc[q];
        for (int cc = 0; cc < WROWS; ++cc) acc = fmaf(cs[e * DIM + c0 + cc], wsm[cc * d_idx + d], acc);
        kacc[q] = acc;
      }
    }
  }
#pragma unroll
  for (int q = 0; q < KQ; ++q) {
    const int p = c + DIM * q;
    if (p < ne * d_idx) ks[(p / d_idx) * MAX_DIDX + p % d_idx] = kacc[q];
  }
  __syncthreads();
  if (key_dtype == CSA_F32) {
    for (int p = c; p < ne * d_idx; p += DIM) {
      const int e = p / d_idx, d = p % d_idx;
      reinterpret_cast<float*>(key_out)[((int64_t)b * n_cap + i0 + e) * d_idx + d] = ks[e * MAX_DIDX + d];
    }
  } else {  // MXFP4: one thread per 32-element block
    const int nblk = d_idx / MXB;
    for (int p = c; p < ne * nblk; p += DIM) {
      const int e = p / nblk, bk = p % nblk;
      const float* kv = ks + e * MAX_DIDX + bk * MXB;
      float amax = 0.0f;
      for (int t = 0; t < MXB; ++t) amax = fmaxf(amax, fabsf(kv[t]));
      const int ex = mx_scale_exp(amax);
      uint32_t w[4] = {0, 0, 0, 0};
      for (int t = 0; t < MXB; ++t) w[t / 8] |= e2m1_code(ldexpf(kv[t], -ex)) << (4 * (t % 8));
      const int64_t ent = (int64_t)b * n_cap + i0 + e;
      *reinterpret_cast<uint4*>(key_out + ent * (d_idx / 2) + bk * (MXB / 2)) = make_uint4(w[0], w[1], w[2], w[3]);
      key_scales[ent * nblk + bk] = (uint8_t)(ex + 127);
    }
  }
}

// HCA: grid (n_new * 6, batch): each block pools 32 channels of one entry over 128 slots.
// block: 256 threads; LDS holds the 128 raw tokens (float32) and the 32-channel gate slice.
constexpr int HCA_M = 128;
constexpr int HCA_CB = 32;  // channels per block

__global__ void __launch_bounds__(256) hca_compress_kernel(
    const uint8_t* __restrict__ x, int x_dtype, int64_t raw_rows, int64_t raw_base,
    const float* __restrict__ w_gate, const float* __restrict__ pos_bias, int64_t entry_begin,
    uint8_t* __restrict__ kv_out, int kv_dtype, int64_t n_cap) {
  extern __shared__ float smem[];
  float* xs = smem;                          // [128][DIM]
  float* ws = xs + HCA_M * DIM;              // [DIM][HCA_CB]
  float* red = ws + DIM * HCA_CB;            // [8][HCA_CB] partial reductions
  float* zs = red + 8 * HCA_CB;              // [8][HCA_CB] partial reductions

  const int b = blockIdx.y;
  const int64_t i = entry_begin + blockIdx.x / (DIM / HCA_CB);
  const int c0 = (blockIdx.x % (DIM / HCA_CB)) * HCA_CB;
  const int tid = threadIdx.x;
  const int xb = x_dtype == CSA_F32 ? 4 : 2;

  // ring rows of the entry's 128 consecutive tokens: one 64-bit remainder per
  // work-group, then steps through the ring (at most one wrap)
  const int64_t rel0 = HCA_M * i - raw_base;
  const int64_t m0 = rel0 >= 0 ? rel0 % raw_rows : rel0;
  auto row_of = [&](int s) -> int64_t {
    if (rel0 + s < 0) return -1;
    const int64_t r = m0 + s;
    return r >= raw_rows ? r - raw_rows : r;
  };
  const uint8_t* ring = x + (int64_t)b * raw_rows * DIM * xb;
  if (aligned16(x)) {
    if (x_dtype == CSA_F32) stage_tokens<256, HCA_M, true>(ring, row_of, xs, tid);
    else stage_tokens<256, HCA_M, false>(ring, row_of, xs, tid);
  } else {
    for (int p = tid; p < HCA_M * DIM; p += 256) {
      const int s = p / DIM, d = p % DIM;
      const int64_t r = row_of(s);
      xs[p] = r >= 0 ? load_raw(ring + r * DIM * xb, x_dtype, d) : 0.0f;
    }
  }
  // the channel slice of w_gate: row d, columns c0 .. c0+31 (eight 16-byte
  // pieces per row, six per thread, all requested before the first store)
  if (aligned16(w_gate)) {
    constexpr int PW = DIM * HCA_CB / 4 / 256;
    float4 wv[PW];
#pragma unroll
    for (int k = 0; k < PW; ++k) {
      const int q = tid + 256 * k, d = q / (HCA_CB / 4), part = q % (HCA_CB / 4);
      wv[k] = *reinterpret_cast<const float4*>(w_gate + d * DIM + c0 + 4 * part);
    }
#pragma unroll
    for (int k = 0; k < PW; ++k) reinterpret_cast<float4*>(ws)[tid + 256 * k] = wv[k];
  } else {
    for (int p = tid; p < DIM * HCA_CB; p += 256) ws[p] = w_gate[(p / HCA_CB) * DIM + c0 + p % HCA_CB];
  }
  __syncthreads();

  // z[s][c] for 16 slots s = sg + 8r of channel cc
  const int cc = tid % HCA_CB, sg = tid / HCA_CB;
  float acc[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
  for (int d = 0; d < DIM; d += 4) {  // four dims per LDS read of a token (same d order per sum)
    const float w0 = ws[d * HCA_CB + cc], w1 = ws[(d + 1) * HCA_CB + cc];
    const float w2 = ws[(d + 2) * HCA_CB + cc], w3 = ws[(d + 3) * HCA_CB + cc];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float4 xv = *reinterpret_cast<const float4*>(xs + (sg + 8 * r) * DIM + d);
      acc[r] = fmaf(xv.x, w0, acc[r]);
      acc[r] = fmaf(xv.y, w1, acc[r]);
      acc[r] = fmaf(xv.z, w2, acc[r]);
      acc[r] = fmaf(xv.w, w3, acc[r]);
    }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int s = sg + 8 * r;
    acc[r] += pos_bias[s * DIM + c0 + cc];
    mx = fmaxf(mx, acc[r]);
  }
  red[sg * HCA_CB + cc] = mx;
  __syncthreads();
  mx = -INFINITY;
  for (int t = 0; t < 8; ++t) mx = fmaxf(mx, red[t * HCA_CB + cc]);
  float den = 0.0f, num = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int s = sg + 8 * r;
    const float p = expf(acc[r] - mx);
    den += p;
    num = fmaf(p, xs[s * DIM + c0 + cc], num);
  }
  __syncthreads();
  red[sg * HCA_CB + cc] = den;
  zs[sg * HCA_CB + cc] = num;
  __syncthreads();
  if (sg == 0) {
    float D = 0.0f, Nm = 0.0f;
    for (int t = 0; t < 8; ++t) {
      D += red[t * HCA_CB + cc];
      Nm += zs[t * HCA_CB + cc];
    }
    store_entry_channel(kv_out + ((int64_t)b * n_cap + i) * row_bytes(kv_dtype), kv_dtype, c0 + cc, Nm / D);
  }
}

hipError_t launch_csa_compress(const void* x, int x_dtype, int batch, int64_t raw_rows, int64_t raw_base,
                               const float* w_gate, const float* pos_bias, int64_t entry_begin, int n_new,
                               void* kv_out, int kv_dtype, int64_t n_cap, const float* w_idx, int d_idx,
                               void* key_out, uint8_t* key_scales, int key_dtype, hipStream_t s) {
  if (n_new == 0 || batch == 0) return hipSuccess;
  auto go = [&](auto kernel, int epb) -> hipError_t {
    const size_t smem = sizeof(float) * ((size_t)(4 * epb + 4) * DIM + WROWS * MAX_DIDX + epb * DIM + epb * MAX_DIDX);
    hipError_t e = hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    dim3 grid((n_new + epb - 1) / epb, batch);
    hipLaunchKernelGGL(kernel, grid, dim3(DIM), smem, s, (const uint8_t*)x, x_dtype, raw_rows, raw_base, w_gate,
                       pos_bias, entry_begin, n_new, (uint8_t*)kv_out, kv_dtype, n_cap, w_idx, d_idx,
                       (uint8_t*)key_out, key_scales, key_dtype);
    return hipGetLastError();
  };
  // a few entries (decode): one entry per block; many (prefill): two, sharing their
  // tokens.  Measured at 1,024 entries from a BF16 ring: eight entries per block
  // (128 work-groups) 61 us, four 33 us, two 27 us, one 45 us.
  if (n_new <= 16) return go(csa_compress_kernel<1>, 1);
  return go(csa_compress_kernel<2>, 2);
}

hipError_t launch_hca_compress(const void* x, int x_dtype, int batch, int64_t raw_rows, int64_t raw_base,
                               const float* w_gate, const float* pos_bias, int64_t entry_begin, int n_new,
                               void* kv_out, int kv_dtype, int64_t n_cap, hipStream_t s) {
  if (n_new == 0 || batch == 0) return hipSuccess;
  const size_t smem = sizeof(float) * (HCA_M * DIM + DIM * HCA_CB + 2 * 8 * HCA_CB);
  hipError_t e = hipFuncSetAttribute((const void*)hca_compress_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)smem);
  if (e != hipSuccess) return e;
  dim3 grid(n_new * (DIM / HCA_CB), batch);
  hipLaunchKernelGGL(hca_compress_kernel, grid, dim3(256), smem, s, (const uint8_t*)x, x_dtype, raw_rows, raw_base,
                     w_gate, pos_bias, entry_begin, (uint8_t*)kv_out, kv_dtype, n_cap);
  return hipGetLastError();
}

}  // namespace csa
