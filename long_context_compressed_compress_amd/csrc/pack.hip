// Storage-format kernels: KV row packing (RoPE dims BF16, other dims FP8 E4M3 —
// gitcode.csdn.net DeepSeek-V4 解读, 核心创新一 §1.4 存储格式混合) and MXFP4
// block quantisation (austery.github.io DeepSeek-V4 notes, 全栈工程优化).
#include "common.h"

namespace csa {

// 8 consecutive dims d0..d0+7 of a row: load as float, store in a row format.
__device__ __forceinline__ void load_row8(const uint8_t* src, int x_dtype, int d0, float (&v)[8]) {
  if (x_dtype == CSA_F32) {
    const float4 a = *reinterpret_cast<const float4*>(src + 4 * d0);
    const float4 b = *reinterpret_cast<const float4*>(src + 4 * d0 + 16);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    const uint4 a = *reinterpret_cast<const uint4*>(src + 2 * d0);
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_to_f32(w[i] & 0xffffu);
      v[2 * i + 1] = bf16_to_f32(w[i] >> 16);
    }
  }
}

__device__ __forceinline__ void store_row8(const float (&v)[8], int out_dtype, uint8_t* dst, int d0) {
  if (out_dtype == CSA_F32) {
    *reinterpret_cast<float4*>(dst + 4 * d0) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(dst + 4 * d0 + 16) = make_float4(v[4], v[5], v[6], v[7]);
  } else if (out_dtype == CSA_BF16 || d0 >= DIM_NOPE) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = f32_to_bf16_rne(v[2 * i]) | (f32_to_bf16_rne(v[2 * i + 1]) << 16);
    const int off = out_dtype == CSA_BF16 ? 2 * d0 : DIM_NOPE + 2 * (d0 - DIM_NOPE);
    *reinterpret_cast<uint4*>(dst + off) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {  // mixed row, FP8 part
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo |= f32_to_fp8_sat(v[i]) << (8 * i);
      hi |= f32_to_fp8_sat(v[4 + i]) << (8 * i);
    }
    *reinterpret_cast<uint2*>(dst + d0) = make_uint2(lo, hi);
  }
}

// One thread converts 8 consecutive dims of one row (24 threads per row).
__global__ void __launch_bounds__(256) kv_pack_kernel(const uint8_t* __restrict__ x, int x_dtype, int64_t n_rows,
                                                      int64_t x_stride_bytes, uint8_t* __restrict__ out,
                                                      int out_dtype, int64_t out_stride_bytes) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = gid / 24;
  const int grp = (int)(gid % 24);
  if (row >= n_rows) return;
  float v[8];
  load_row8(x + row * x_stride_bytes, x_dtype, grp * 8, v);
  store_row8(v, out_dtype, out + row * out_stride_bytes, grp * 8);
}

// Decode append: thread (b, ring, grp) writes dims 8grp..8grp+7 of sequence b's
// new row into ring `ring` (0 = raw, 1 = window) at row (pos[b] - base) mod rows.
struct RingArgs {
  uint8_t* data;
  int dtype;
  int64_t rows, base;
};
__global__ void __launch_bounds__(256) kv_append_kernel(const uint8_t* __restrict__ x, int x_dtype, int batch,
                                                        const int64_t* __restrict__ pos, RingArgs raw,
                                                        RingArgs win) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int b = (int)(gid / 48);
  const int rem = (int)(gid % 48);
  if (b >= batch) return;
  const RingArgs& r = rem < 24 ? raw : win;
  if (!r.data) return;
  const int64_t rel = pos[b] - r.base;
  if (rel < 0) return;
  const int grp = rem % 24;
  float v[8];
  load_row8(x + (int64_t)b * DIM * (x_dtype == CSA_F32 ? 4 : 2), x_dtype, grp * 8, v);
  const int rb = row_bytes(r.dtype);
  store_row8(v, r.dtype, r.data + ((int64_t)b * r.rows + rel % r.rows) * rb, grp * 8);
}

hipError_t launch_kv_append(const void* x, int x_dtype, int batch, const int64_t* pos, void* raw_ring, int raw_dtype,
                            int64_t raw_rows, int64_t raw_base, void* win_ring, int win_dtype, int64_t win_rows,
                            int64_t win_base, hipStream_t s) {
  if (batch == 0) return hipSuccess;
  const int64_t threads = (int64_t)batch * 48;
  RingArgs raw{(uint8_t*)raw_ring, raw_dtype, raw_rows, raw_base};
  RingArgs win{(uint8_t*)win_ring, win_dtype, win_rows, win_base};
  hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                     (const uint8_t*)x, x_dtype, batch, pos, raw, win);
  return hipGetLastError();
}

hipError_t launch_kv_pack(const void* x, int x_dtype, int64_t n_rows, int64_t x_stride, void* out, int out_dtype,
                          int64_t out_stride, hipStream_t s) {
  if (n_rows == 0) return hipSuccess;
  const int64_t threads = n_rows * 24;
  const int64_t blocks = (threads + 255) / 256;
  const int64_t xsb = x_stride * (x_dtype == CSA_F32 ? 4 : 2);
  hipLaunchKernelGGL(kv_pack_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (const uint8_t*)x, x_dtype, n_rows,
                     xsb, (uint8_t*)out, out_dtype, out_stride);
  return hipGetLastError();
}

// One thread per 32-element block: amax -> shared exponent -> 32 E2M1 codes.
__global__ void __launch_bounds__(256) mxfp4_quantize_kernel(const float* __restrict__ x, int64_t n_blocks,
                                                             uint8_t* __restrict__ codes,
                                                             uint8_t* __restrict__ scales) {
  const int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (blk >= n_blocks) return;
  const float4* src = reinterpret_cast<const float4*>(x + blk * MXB);
  float v[MXB];
#pragma unroll
  for (int i = 0; i < MXB / 4; ++i) {
    const float4 a = src[i];
    v[4 * i] = a.x; v[4 * i + 1] = a.y; v[4 * i + 2] = a.z; v[4 * i + 3] = a.w;
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < MXB; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int e = mx_scale_exp(amax);
  uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < MXB; ++i) w[i / 8] |= e2m1_code(ldexpf(v[i], -e)) << (4 * (i % 8));
  *reinterpret_cast<uint4*>(codes + blk * (MXB / 2)) = make_uint4(w[0], w[1], w[2], w[3]);
  scales[blk] = (uint8_t)(e + 127);
}

hipError_t launch_mxfp4_quantize(const float* x, int64_t n_rows, int d, uint8_t* codes, uint8_t* scales,
                                 hipStream_t s) {
  const int64_t nb = n_rows * (d / MXB);
  if (nb == 0) return hipSuccess;
  hipLaunchKernelGGL(mxfp4_quantize_kernel, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, s, x, nb, codes,
                     scales);
  return hipGetLastError();
}

}  // namespace csa
