// Per-query top-k over index scores (「论文解读｜DeepSeek-V4：百万 token 上下文的效率革命」,
// blog.tripbot.top, §3.1 第二步: keep the k best compressed entries; k = 1024 for
// V4-Pro, 512 for V4-Flash).  Exact and deterministic: scores map to
// order-preserving unsigned keys (BF16 -> 16 bits, FP32 -> 32 bits), an 8-bit
// MSB-first radix select finds the k-th largest key tau and how many tau-ties
// to take, and an index-ordered compaction emits every key > tau plus the
// lowest-index ties, in ascending index order.
#include "common.h"

namespace csa {

namespace {

constexpr uint32_t INVALID = 0xffffffffu;  // marker for -inf (never selected)

template <bool BF16>
__device__ __forceinline__ uint32_t score_key(const void* row, int64_t i) {
  if (BF16) {
    uint32_t u = reinterpret_cast<const uint16_t*>(row)[i];
    if (u == 0xff80u) return INVALID;                 // -inf
    if ((u & 0x7fffu) == 0) u = 0;                     // -0 ties with +0
    return (u & 0x8000u) ? (~u & 0xffffu) : (u | 0x8000u);
  } else {
    uint32_t u = reinterpret_cast<const uint32_t*>(row)[i];
    if (u == 0xff800000u) return INVALID;
    if ((u & 0x7fffffffu) == 0) u = 0;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  }
}
// For 32-bit keys the all-ones pattern is NaN's image; scores are never NaN,
// and 16-bit keys never reach it.

template <int BS>
struct BlockScan {
  static constexpr int NW = BS / 64;
  uint32_t wave_cnt[NW];
};

// Exclusive prefix of a predicate over the block in thread order; returns the
// rank and writes the block total.  Two barriers.
template <int BS>
__device__ __forceinline__ uint32_t block_rank(bool pred, BlockScan<BS>& sc, uint32_t& total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const uint64_t m = __ballot(pred);
  const uint32_t in_wave = __popcll(m & ((1ull << lane) - 1ull));
  if (lane == 0) sc.wave_cnt[wv] = __popcll(m);
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < BlockScan<BS>::NW; ++i) {
    const uint32_t c = sc.wave_cnt[i];
    before += i < wv ? c : 0u;
    tot += c;
  }
  __syncthreads();
  total = tot;
  return before + in_wave;
}

}  // namespace

// grid (n_q, batch), block BS threads: one block selects one query row.
template <bool BF16, int BS>
__global__ void __launch_bounds__(BS) topk_row_kernel(const void* __restrict__ scores, int n_q, int64_t n_cap,
                                                     const int32_t* __restrict__ n_entries,
                                                     const int64_t* __restrict__ q_pos, int ratio, int k,
                                                     int32_t* __restrict__ idx_out) {
  constexpr int KEYBITS = BF16 ? 16 : 32;
  constexpr int NPASS = KEYBITS / 8;
  __shared__ uint32_t hist[256];
  __shared__ uint32_t s_prefix, s_need, s_all;
  __shared__ BlockScan<BS> sc;

  const int b = blockIdx.y;
  const int64_t row = (int64_t)b * n_q + blockIdx.x;
  const int64_t n = visible_entries(n_entries[b], q_pos[row], ratio, n_cap);
  const uint8_t* srow = reinterpret_cast<const uint8_t*>(scores) + row * n_cap * (BF16 ? 2 : 4);
  int32_t* out = idx_out + row * k;
  const int tid = threadIdx.x, lane = tid & 63;

  uint32_t prefix = 0, need = (uint32_t)k;
  bool take_all = false;
  for (int p = 0; p < NPASS; ++p) {
    const int shift = KEYBITS - 8 * (p + 1);
    for (int i = tid; i < 256; i += BS) hist[i] = 0;
    __syncthreads();
    for (int64_t i = tid; i < n; i += BS) {
      const uint32_t key = score_key<BF16>(srow, i);
      if (key == INVALID) continue;
      if (p > 0 && (key >> (shift + 8)) != prefix) continue;
      atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      // lane holds bins 4*lane .. 4*lane+3; suffix sums from the top bin down
      const uint32_t h0 = hist[4 * lane], h1 = hist[4 * lane + 1], h2 = hist[4 * lane + 2], h3 = hist[4 * lane + 3];
      const uint32_t c = h0 + h1 + h2 + h3;
      uint32_t suf = c;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t v = __shfl_down(suf, o, 64);
        if (lane + o < 64) suf += v;
      }
      const uint32_t total = __shfl(suf, 0, 64);
      if (p == 0 && total <= (uint32_t)k) {
        if (lane == 0) s_all = 1u;
      } else {
        const uint64_t ge = __ballot(suf >= need);
        const int L = 63 - __clzll(ge);  // highest lane whose suffix still covers `need`
        if (lane == L) {
          uint32_t above = suf - c;
          const uint32_t hb[4] = {h0, h1, h2, h3};
          int d = 3;
          for (; d > 0; --d) {
            if (above + hb[d] >= need) break;
            above += hb[d];
          }
          s_prefix = (prefix << 8) | (uint32_t)(4 * lane + d);
          s_need = need - above;
          s_all = 0u;
        }
      }
    }
    __syncthreads();
    if (s_all) {
      take_all = true;
      break;
    }
    prefix = s_prefix;
    need = s_need;
    __syncthreads();
  }

  // Index-ordered compaction.
  const uint32_t tau = prefix;
  uint32_t base = 0, ties_seen = 0;
  for (int64_t start = 0; start < n; start += BS) {
    const int64_t i = start + tid;
    const uint32_t key = i < n ? score_key<BF16>(srow, i) : INVALID;
    const bool valid = key != INVALID;
    bool sel;
    if (take_all) {
      sel = valid;
    } else {
      const bool eq = valid && key == tau;
      uint32_t n_eq;
      const uint32_t eq_rank = block_rank<BS>(eq, sc, n_eq);
      sel = (valid && key > tau) || (eq && ties_seen + eq_rank < need);
      ties_seen += n_eq;
    }
    uint32_t n_sel;
    const uint32_t pos = block_rank<BS>(sel, sc, n_sel);
    if (sel) out[base + pos] = (int32_t)i;
    base += n_sel;
    if (base >= (uint32_t)k) break;  // block-uniform
  }
  for (int64_t j = (int64_t)base + tid; j < k; j += BS) out[j] = -1;
  (void)lane;
}

size_t topk_ws_bytes(int batch, int n_q, int64_t n_cap, int k, int score_dtype) {
  (void)batch; (void)n_q; (void)n_cap; (void)k; (void)score_dtype;
  return 0;
}

hipError_t launch_topk(const void* scores, int score_dtype, int batch, int n_q, int64_t n_cap,
                       const int32_t* n_entries, const int64_t* q_pos, int ratio, int k, int32_t* idx_out, void* ws,
                       hipStream_t s) {
  (void)ws;
  if (batch == 0 || n_q == 0) return hipSuccess;
  dim3 grid(n_q, batch);
  if (score_dtype == CSA_BF16)
    hipLaunchKernelGGL((topk_row_kernel<true, 512>), grid, dim3(512), 0, s, scores, n_q, n_cap, n_entries, q_pos,
                       ratio, k, idx_out);
  else
    hipLaunchKernelGGL((topk_row_kernel<false, 512>), grid, dim3(512), 0, s, scores, n_q, n_cap, n_entries, q_pos,
                       ratio, k, idx_out);
  return hipGetLastError();
}

}  // namespace csa
