// Per-query top-k over index scores (「论文解读｜DeepSeek-V4：百万 token 上下文的效率革命」,
// blog.tripbot.top, §3.1 第二步: keep the k best compressed entries; k = 1024 for
// V4-Pro, 512 for V4-Flash).  Exact and deterministic: scores map to
// order-preserving unsigned keys (BF16 -> 16 bits, FP32 -> 32 bits), an 8-bit
// MSB-first radix select finds the k-th largest key tau and how many tau-ties
// to take, and an index-ordered compaction emits every key > tau plus the
// lowest-index ties, in ascending index order.
//
// Two schedules give the same (exact) result:
//   * row path   — one work-group per query row (many rows: prefill);
//   * split path — BF16 scores, few long rows (decode): every row is cut into
//     chunks of 4096 keys, one work-group per (row, chunk), three launches
//     (histogram of the high byte, histogram of the low byte inside the chosen
//     high bin, selection).  Row totals are integer atomics (exact in any
//     order); every work-group derives the digit choices from them itself and
//     the selection launch places each chunk's output from the per-chunk counts
//     of the chunks before it, so no work-group ever waits for another and no
//     device-wide cache fence is needed inside a launch.
#include "common.h"

namespace csa {

namespace {

template <bool BF16>
__device__ __forceinline__ uint32_t score_key(const void* row, int64_t i) {
  if (BF16) return bf16_key(reinterpret_cast<const uint16_t*>(row)[i]);
  uint32_t u = reinterpret_cast<const uint32_t*>(row)[i];
  if (u == 0xff800000u) return INVALID;
  if ((u & 0x7fffffffu) == 0) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
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

// Exclusive prefix sum of a per-thread count over the block (thread order).
template <int BS>
__device__ __forceinline__ uint32_t block_excl_sum(uint32_t v, BlockScan<BS>& sc, uint32_t& total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  uint32_t inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t t = __shfl_up(inc, o, 64);
    if (lane >= o) inc += t;
  }
  if (lane == 63) sc.wave_cnt[wv] = inc;
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
  return before + inc - v;
}

// The same over 64-bit counts (two 32-bit counts packed, one per half).
template <int BS>
struct BlockScan64 {
  static constexpr int NW = BS / 64;
  uint64_t wave_sum[NW];
};

template <int BS>
__device__ __forceinline__ uint64_t block_excl_sum64(uint64_t v, BlockScan64<BS>& sc, uint64_t& total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  uint64_t inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint64_t t = __shfl_up(inc, o, 64);
    if (lane >= o) inc += t;
  }
  if (lane == 63) sc.wave_sum[wv] = inc;
  __syncthreads();
  uint64_t before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < BlockScan64<BS>::NW; ++i) {
    const uint64_t c = sc.wave_sum[i];
    before += i < wv ? c : 0ull;
    tot += c;
  }
  __syncthreads();
  total = tot;
  return before + inc - v;
}

struct DigitChoice {
  uint32_t prefix;  // decided key bits so far
  uint32_t need;    // how many keys still to take among those matching `prefix`
  uint32_t all;     // 1: at most k valid keys exist, take them all
};

// Run by one wave (64 lanes) over a 256-bin histogram of the current digit.
// Picks the digit d* where the count from the top reaches `need`.
__device__ __forceinline__ void choose_digit(const uint32_t* hist, uint32_t prefix, uint32_t need, bool first,
                                             uint32_t k, DigitChoice* out) {
  const int lane = threadIdx.x & 63;
  const uint32_t h0 = hist[4 * lane], h1 = hist[4 * lane + 1], h2 = hist[4 * lane + 2], h3 = hist[4 * lane + 3];
  const uint32_t c = h0 + h1 + h2 + h3;
  uint32_t suf = c;  // keys in bins >= 4*lane
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t v = __shfl_down(suf, o, 64);
    if (lane + o < 64) suf += v;
  }
  const uint32_t total = __shfl(suf, 0, 64);
  if (first && total <= k) {
    if (lane == 0) *out = DigitChoice{0u, 0u, 1u};
    return;
  }
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
    *out = DigitChoice{(prefix << 8) | (uint32_t)(4 * lane + d), need - above, 0u};
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// Row path: grid (n_q, batch), block BS threads: one block selects one query row.
// ---------------------------------------------------------------------------
template <bool BF16, int BS>
__global__ void __launch_bounds__(BS) topk_row_kernel(const void* __restrict__ scores, int n_q, int64_t n_cap,
                                                     const int32_t* __restrict__ n_entries,
                                                     const int64_t* __restrict__ q_pos, int ratio, int k,
                                                     int32_t* __restrict__ idx_out) {
  constexpr int KEYBITS = BF16 ? 16 : 32;
  constexpr int NPASS = KEYBITS / 8;
  __shared__ uint32_t hist[256];
  __shared__ DigitChoice ch;
  __shared__ BlockScan<BS> sc;

  const int b = blockIdx.y;
  const int64_t row = (int64_t)b * n_q + blockIdx.x;
  const int64_t n = visible_entries(n_entries[b], q_pos[row], ratio, n_cap);
  const uint8_t* srow = reinterpret_cast<const uint8_t*>(scores) + row * n_cap * (BF16 ? 2 : 4);
  int32_t* out = idx_out + row * k;
  const int tid = threadIdx.x;

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
    if (tid < 64) choose_digit(hist, prefix, need, p == 0, (uint32_t)k, &ch);
    __syncthreads();
    if (ch.all) {
      take_all = true;
      break;
    }
    prefix = ch.prefix;
    need = ch.need;
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
}

// ---------------------------------------------------------------------------
// Split path (BF16 keys).  No work-group waits for or signals another; each
// launch boundary publishes the previous launch's results.
// Workspace layout (32-bit words):
//   fixed region, SPLIT_MAX_ROWS rows: total0[256] + total1[256] (row totals of
//     the two digit histograms; zero at rest: the caller zero-fills once, the
//     first launch clears total1 for the call, the last launch clears total0)
//   then per row: state (DigitChoice of the high byte), per chunk:
//     suf1[257] (suffix sums of the chunk's low-byte counts in the chosen high
//     bin: suf1[d] = keys with low byte >= d), above0 (keys of the chunk whose
//     high byte is above the chosen bin, or its valid keys when all are taken)
// A work-group owns chunk c = keys [c*CH, (c+1)*CH) of its row, CH = 4096*R;
// each thread holds 16 consecutive keys per round (two 16-byte loads).
// ---------------------------------------------------------------------------
constexpr int SBS = 256;                 // threads per split work-group
constexpr int SKT = 16;                  // keys per thread per round
constexpr int SROUND = SBS * SKT;        // 4096 keys per round
constexpr int SPLIT_MAX_ROWS = 128;
constexpr size_t SPLIT_FIXED_ROW_WORDS = 512;
constexpr size_t SPLIT_FIXED_WORDS = (size_t)SPLIT_MAX_ROWS * SPLIT_FIXED_ROW_WORDS;
constexpr int SUF = 258;                 // words per chunk: suf1[257] + above0

struct SplitPlan {
  int chunks;   // C
  int rounds;   // R: chunk = R * 4096 keys
  size_t row_words;
};

__host__ __device__ inline SplitPlan topk_split_plan(int64_t n_cap) {
  SplitPlan p;
  int64_t rounds = (n_cap + (int64_t)256 * SROUND - 1) / ((int64_t)256 * SROUND);  // at most 256 chunks
  if (rounds < 1) rounds = 1;
  const int64_t chunk = rounds * SROUND;
  p.rounds = (int)rounds;
  p.chunks = (int)((n_cap + chunk - 1) / chunk);
  p.row_words = 4 + (size_t)p.chunks * SUF;
  return p;
}

static bool use_split(int64_t rows, int64_t n_cap, int score_dtype) {
  return score_dtype == CSA_BF16 && rows < SPLIT_MAX_ROWS && n_cap >= 16384;
}

struct SplitView {
  uint32_t* total0;    // [256]
  uint32_t* total1;    // [256]
  DigitChoice* state;  // high-byte choice
  uint32_t* chunk;     // [C][SUF]
};

__device__ __forceinline__ SplitView split_view(void* ws, int64_t row, const SplitPlan& p) {
  uint32_t* w = reinterpret_cast<uint32_t*>(ws);
  SplitView v;
  v.total0 = w + row * SPLIT_FIXED_ROW_WORDS;
  v.total1 = v.total0 + 256;
  uint32_t* base = w + SPLIT_FIXED_WORDS + row * p.row_words;
  v.state = reinterpret_cast<DigitChoice*>(base);
  v.chunk = base + 4;
  return v;
}

// The 16 keys [i, i+16) of a thread (i a multiple of 16); keys at or beyond n are INVALID.
// Keys of 16 consecutive BF16 scores held in two 16-byte pieces.
__device__ __forceinline__ void unpack16(const uint4& a, const uint4& b, uint32_t (&key)[SKT]) {
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    key[2 * j] = bf16_key(w[j] & 0xffffu);
    key[2 * j + 1] = bf16_key(w[j] >> 16);
  }
}

__device__ __forceinline__ void load16(const uint16_t* srow, int64_t i, int64_t n, uint32_t (&key)[SKT]) {
  // vector loads need 16-byte alignment: true for every thread of a row whose start is aligned
  if (i + SKT <= n && (reinterpret_cast<uintptr_t>(srow) & 15u) == 0) {
    unpack16(*reinterpret_cast<const uint4*>(srow + i), *reinterpret_cast<const uint4*>(srow + i + 8), key);
  } else {
#pragma unroll
    for (int j = 0; j < SKT; ++j) key[j] = i + j < n ? bf16_key(srow[i + j]) : INVALID;
  }
}

// Keys i..i+15 of a row as loaded by load16 with bound n, from keys loaded
// earlier with the row's capacity as bound (so the loads could be issued
// before n was known).
__device__ __forceinline__ void mask16(uint32_t (&key)[SKT], int64_t i, int64_t n) {
  const int64_t r = n - i;
  const int rem = r <= 0 ? 0 : (r >= SKT ? SKT : (int)r);
#pragma unroll
  for (int j = 0; j < SKT; ++j) key[j] = j < rem ? key[j] : INVALID;
}

// Work-group barrier for LDS data only: unlike __syncthreads it does not wait
// for the global loads in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// choose_digit for one wave holding the 256-bin histogram in registers (lane l:
// bins 4l .. 4l+3); every lane gets the choice, so no work-group exchange is needed.
__device__ __forceinline__ DigitChoice choose_digit_wave(const uint4 hb, uint32_t prefix, uint32_t need, bool first,
                                                         uint32_t k) {
  const int lane = threadIdx.x & 63;
  const uint32_t c = hb.x + hb.y + hb.z + hb.w;
  uint32_t suf = c;  // keys in bins >= 4*lane
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t v = __shfl_down(suf, o, 64);
    if (lane + o < 64) suf += v;
  }
  const uint32_t total = (uint32_t)__builtin_amdgcn_readfirstlane(__shfl(suf, 0, 64));
  if (first && total <= k) return DigitChoice{0u, 0u, 1u};
  const uint64_t ge = __ballot(suf >= need);
  const int L = 63 - __clzll(ge);  // highest lane whose suffix still covers `need`
  uint32_t above = __shfl(suf - c, L, 64);
  const uint32_t hL[4] = {__shfl(hb.x, L, 64), __shfl(hb.y, L, 64), __shfl(hb.z, L, 64), __shfl(hb.w, L, 64)};
  int d = 3;
  for (; d > 0; --d) {
    if (above + hL[d] >= need) break;
    above += hL[d];
  }
  // the same on every lane: kept in scalar registers so branches on it are uniform
  return DigitChoice{(uint32_t)__builtin_amdgcn_readfirstlane((prefix << 8) | (uint32_t)(4 * L + d)),
                     (uint32_t)__builtin_amdgcn_readfirstlane(need - above), 0u};
}

// launch 1: row totals of the high byte of every valid key; clears total1 for launch 2
__global__ void __launch_bounds__(SBS) topk_split_hist0(const uint16_t* __restrict__ scores, int n_q, int64_t n_cap,
                                                        const int32_t* __restrict__ n_entries,
                                                        const int64_t* __restrict__ q_pos, int ratio,
                                                        void* __restrict__ ws, SplitPlan p) {
  __shared__ uint32_t hist[256 * HREP];
  const int c = blockIdx.x;
  const int64_t row = blockIdx.y;
  const int b = (int)(row / n_q);
  const int tid = threadIdx.x;
  const int64_t n = visible_entries(n_entries[b], q_pos[row], ratio, n_cap);
  const SplitView v = split_view(ws, row, p);
  const uint16_t* srow = scores + row * n_cap;
  if (c == 0) v.total1[tid] = 0u;
  rep_clear(hist, tid);
  __syncthreads();
  for (int r = 0; r < p.rounds; ++r) {
    const int64_t i = ((int64_t)c * p.rounds + r) * SROUND + (int64_t)tid * SKT;
    if (i >= n) break;
    uint32_t key[SKT];
    load16(srow, i, n, key);
#pragma unroll
    for (int j = 0; j < SKT; ++j)
      if (key[j] != INVALID) rep_add(hist, key[j] >> 8, tid);
  }
  __syncthreads();
  const uint32_t t = rep_total(hist, tid);
  if (t) atomicAdd(&v.total0[tid], t);
}

// Launches 2 and 3 run on a 1-D grid that places every chunk of row r on XCD
// r mod 8 (work-groups are dealt to the 8 XCDs round-robin by linear id): the
// per-chunk counts that launch 2 writes and every chunk of launch 3 reads then
// stay in one XCD's L2, and a chunk's keys are read by both launches on the
// same XCD (measured: passes 2-3 17.2 -> 16.7 us at 8 x 262,144).  Returns
// false for the padding work-groups of XCDs with fewer rows.
__device__ __forceinline__ bool split_slot(int rows, int chunks, int& c, int64_t& row) {
  const uint32_t id = blockIdx.x, x = id % 8u, k = id / 8u;
  const uint32_t nr = (uint32_t)rows > x ? ((uint32_t)rows - x + 7u) / 8u : 0u;
  if (k >= nr * (uint32_t)chunks) return false;
  row = x + 8 * (int64_t)(k / (uint32_t)chunks);
  c = (int)(k % (uint32_t)chunks);
  return true;
}

// launch 2: every wave picks the high byte from the row totals; counts of the
// low byte inside that bin (per chunk, as suffix sums, and into the row totals)
// and of the keys above it.
__global__ void __launch_bounds__(SBS) topk_split_hist1(const uint16_t* __restrict__ scores, int n_q, int64_t n_cap,
                                                        const int32_t* __restrict__ n_entries,
                                                        const int64_t* __restrict__ q_pos, int ratio, int k,
                                                        void* __restrict__ ws, SplitPlan p, int rows) {
  __shared__ uint32_t rhist[256 * HREP];
  __shared__ BlockScan64<SBS> sc;
  int c;
  int64_t row;
  if (!split_slot(rows, p.chunks, c, row)) return;
  const int b = (int)(row / n_q);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const SplitView v = split_view(ws, row, p);
  // everything that does not depend on the digit is requested first, so the
  // waits overlap: this row's visibility, the first round's keys, the totals
  const int32_t ne_b = n_entries[b];
  const int64_t qp = q_pos[row];
  const uint16_t* srow = scores + row * n_cap;
  const int64_t i0 = (int64_t)c * p.rounds * SROUND + (int64_t)tid * SKT;
  const uint4 hb = reinterpret_cast<const uint4*>(v.total0)[lane];
  uint32_t key0[SKT];
  load16(srow, i0, n_cap, key0);
  rep_clear(rhist, tid);
  lds_barrier();
  const DigitChoice st = choose_digit_wave(hb, 0u, (uint32_t)k, true, (uint32_t)k);
  if (c == 0 && tid == 0) *v.state = st;
  const int64_t n = visible_entries(ne_b, qp, ratio, n_cap);
  uint32_t above = 0;
  for (int r = 0; r < p.rounds; ++r) {
    const int64_t i = ((int64_t)c * p.rounds + r) * SROUND + (int64_t)tid * SKT;
    if (i >= n) break;
    uint32_t key[SKT];
    if (r == 0) {
#pragma unroll
      for (int j = 0; j < SKT; ++j) key[j] = key0[j];
      mask16(key, i, n);
    } else {
      load16(srow, i, n, key);
    }
    if (st.all) {  // uniform: every valid key is taken
#pragma unroll
      for (int j = 0; j < SKT; ++j) above += key[j] != INVALID ? 1u : 0u;
    } else {
#pragma unroll
      for (int j = 0; j < SKT; ++j) {
        const uint32_t hi = key[j] >> 8;  // INVALID's image is above every bin
        above += (hi > st.prefix && key[j] != INVALID) ? 1u : 0u;
        if (hi == st.prefix) rep_add(rhist, key[j] & 255u, tid);
      }
    }
  }
  lds_barrier();
  // one scan gives both the suffix sums of the chunk's low-byte counts (low
  // half: thread tid takes bin 255-tid) and the chunk's count above the bin
  // (high half)
  const uint32_t h = rep_total(rhist, 255 - tid);
  uint64_t tot;
  const uint64_t before = block_excl_sum64<SBS>(((uint64_t)above << 32) | h, sc, tot);
  uint32_t* cw = v.chunk + (size_t)c * SUF;
  cw[255 - tid] = (uint32_t)before + h;  // suf[d] = keys with low byte >= d
  if (tid == 0) {
    cw[256] = 0u;
    cw[257] = (uint32_t)(tot >> 32);
  }
  if (h) atomicAdd(&v.total1[255 - tid], h);
}

// launch 3: every wave picks tau from the row totals and computes where its
// chunk's selections start from the per-chunk counts of the chunks before it;
// the work-group writes its selected indices (index order) into the output.
__global__ void __launch_bounds__(SBS) topk_split_select(const uint16_t* __restrict__ scores, int n_q, int64_t n_cap,
                                                         const int32_t* __restrict__ n_entries,
                                                         const int64_t* __restrict__ q_pos, int ratio, int k,
                                                         void* __restrict__ ws, SplitPlan p,
                                                         int32_t* __restrict__ idx_out, int rows) {
  __shared__ BlockScan<SBS> sc;
  int c;
  int64_t row;
  if (!split_slot(rows, p.chunks, c, row)) return;
  const int b = (int)(row / n_q);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const SplitView v = split_view(ws, row, p);
  // requested first (none depends on tau): visibility, the first round's keys,
  // the pass-1 state, the low-byte totals and each chunk's count above the bin
  const int32_t ne_b = n_entries[b];
  const int64_t qp = q_pos[row];
  const uint16_t* srow = scores + row * n_cap;
  const int64_t i0 = (int64_t)c * p.rounds * SROUND + (int64_t)tid * SKT;
  const DigitChoice st0 = *v.state;
  const uint4 hb = reinterpret_cast<const uint4*>(v.total1)[lane];
  // lane l holds chunks 4l .. 4l+3 (p.chunks <= 256)
  uint32_t ab[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int cc = 4 * lane + u;
    ab[u] = cc < p.chunks ? v.chunk[(size_t)cc * SUF + 257] : 0u;
  }
  uint32_t key0[SKT];
  load16(srow, i0, n_cap, key0);
  const bool take_all = st0.all != 0u;
  uint32_t tau = 0, need = 0;
  if (!take_all) {
    const DigitChoice ch = choose_digit_wave(hb, st0.prefix, st0.need, false, 0u);
    tau = ch.prefix;
    need = ch.need;
  }
  // per chunk: ties (keys == tau) and keys above tau; exclusive sums over the
  // chunks before this one, within the wave
  const uint32_t lo = tau & 255u;
  uint32_t eq[4], gt[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int cc = 4 * lane + u;
    uint32_t s_lo = 0, s_hi = 0;
    if (!take_all && cc < p.chunks) {
      const uint32_t* cw = v.chunk + (size_t)cc * SUF;
      s_lo = cw[lo];
      s_hi = cw[lo + 1];
    }
    eq[u] = s_lo - s_hi;
    gt[u] = ab[u] + s_hi;
  }
  const int cu = c & 3, cl = c >> 2;
  uint32_t e4 = 0, g4 = 0, e_in = 0, g_in = 0;  // lane sums; sums of the sub-chunks before cu
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    e_in += u < cu ? eq[u] : 0u;
    g_in += u < cu ? gt[u] : 0u;
    e4 += eq[u];
    g4 += gt[u];
  }
  uint32_t ei = e4, gi = g4;  // inclusive scans over lanes
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t te = __shfl_up(ei, o, 64), tg = __shfl_up(gi, o, 64);
    if (lane >= o) {
      ei += te;
      gi += tg;
    }
  }
  const uint32_t ties_before = __shfl(ei - e4 + e_in, cl, 64);
  const uint32_t gt_before = __shfl(gi - g4 + g_in, cl, 64);
  const uint32_t e_tot = __shfl(ei, 63, 64), g_tot = __shfl(gi, 63, 64);
  const uint32_t offset = gt_before + min(ties_before, need);
  const uint32_t sel_tot = g_tot + min(e_tot, need);
  int32_t* out = idx_out + row * k;
  if (c == 0) {
    for (int64_t j = (int64_t)min<uint32_t>(sel_tot, (uint32_t)k) + tid; j < k; j += SBS) out[j] = -1;
    if (tid < 256) v.total0[tid] = 0u;  // launch 1 of the next call starts from zero
  }

  const int64_t n = visible_entries(ne_b, qp, ratio, n_cap);
  uint32_t base = offset, ties_seen = ties_before;
  for (int r = 0; r < p.rounds; ++r) {
    const int64_t r0 = ((int64_t)c * p.rounds + r) * SROUND;
    if (r0 >= n) break;  // block-uniform
    const int64_t i = r0 + (int64_t)tid * SKT;
    uint32_t key[SKT];
    if (r == 0) {
#pragma unroll
      for (int j = 0; j < SKT; ++j) key[j] = key0[j];
      mask16(key, i, n);
    } else {
      load16(srow, i, n, key);
    }
    uint32_t n_eq = 0, n_gt = 0;
#pragma unroll
    for (int j = 0; j < SKT; ++j) {
      n_eq += (!take_all && key[j] == tau) ? 1u : 0u;
      n_gt += (key[j] != INVALID && (take_all || key[j] > tau)) ? 1u : 0u;
    }
    // one scan of both counts (each half's round total is at most 4096); ties
    // are taken greedily in index order, so the ties taken before a thread are
    // min(ties before it, ties still needed)
    uint32_t tot;
    const uint32_t pre = block_excl_sum<SBS>((n_eq << 16) | n_gt, sc, tot);
    const uint32_t e_t = pre >> 16, g_t = pre & 0xffffu;
    const uint32_t rem = need > ties_seen ? need - ties_seen : 0u;
    // ties taken by the threads before this one, then by this one (written so
    // that no subtraction can wrap: a conditional rem - e_t let the optimiser
    // assume e_t <= rem and drop the first minimum)
    const uint32_t tb = min(e_t, rem);
    const uint32_t take_eq = min(n_eq, rem - tb);
    uint32_t pos = base + g_t + tb;
    if (n_gt + take_eq) {
      uint32_t eq_taken = 0;
#pragma unroll
      for (int j = 0; j < SKT; ++j) {
        bool sel = key[j] != INVALID && (take_all || key[j] > tau);
        if (!take_all && key[j] == tau) {
          sel = eq_taken < take_eq;
          eq_taken += 1u;
        }
        if (sel && pos < (uint32_t)k) out[pos] = (int32_t)(i + j);
        pos += sel ? 1u : 0u;
      }
    }
    base += (tot & 0xffffu) + min(tot >> 16, rem);
    ties_seen += tot >> 16;
  }
}

// ---------------------------------------------------------------------------
// Row path for BF16 rows of at most RR_MAX_ROUNDS * 4096 keys (prefill): one
// work-group of SBS threads per row, the row read once into registers (16
// consecutive keys per thread per round, R rounds), both digit histograms
// built from the registers (replicated LDS histograms), and the compaction in
// index order from one packed scan per round.  Same result as topk_row_kernel.
// ---------------------------------------------------------------------------
constexpr int RR_MAX_ROUNDS = 8;

template <int R>
__global__ void __launch_bounds__(SBS) topk_row_regs_kernel(const uint16_t* __restrict__ scores, int n_q,
                                                            int64_t n_cap, const int32_t* __restrict__ n_entries,
                                                            const int64_t* __restrict__ q_pos, int ratio, int k,
                                                            int32_t* __restrict__ idx_out) {
  __shared__ uint32_t hist[256 * HREP];
  __shared__ BlockScan64<SBS> sc;
  const int b = blockIdx.y;
  const int64_t row = (int64_t)b * n_q + blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // the row's keys are requested before its visible count is back (bounded
  // by the capacity, masked below)
  const int32_t ne_b = n_entries[b];
  const int64_t qp = q_pos[row];
  const uint16_t* srow = scores + row * n_cap;
  uint32_t key[R][SKT];
  if ((reinterpret_cast<uintptr_t>(srow) & 15u) == 0 && n_cap >= SKT) {
    // every round's two pieces are requested before any is unpacked (a piece
    // past the row's capacity reads the row's first 16 keys; the one piece
    // that straddles the capacity is read element by element)
    uint4 raw[R][2];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t i = (int64_t)r * SROUND + (int64_t)tid * SKT;
      const uint16_t* src = srow + (i + SKT <= n_cap ? i : 0);
      raw[r][0] = *reinterpret_cast<const uint4*>(src);
      raw[r][1] = *reinterpret_cast<const uint4*>(src + 8);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t i = (int64_t)r * SROUND + (int64_t)tid * SKT;
      if (i + SKT <= n_cap) unpack16(raw[r][0], raw[r][1], key[r]);
      else load16(srow, i, n_cap, key[r]);
    }
  } else {
#pragma unroll
    for (int r = 0; r < R; ++r) load16(srow, (int64_t)r * SROUND + (int64_t)tid * SKT, n_cap, key[r]);
  }
  rep_clear(hist, tid);
  const int64_t n = visible_entries(ne_b, qp, ratio, n_cap);
#pragma unroll
  for (int r = 0; r < R; ++r) mask16(key[r], (int64_t)r * SROUND + (int64_t)tid * SKT, n);
  lds_barrier();

  // high byte: histogram of every valid key; every wave picks the digit.
  // Rounds that start past the visible count hold no valid key and are
  // skipped here and below (a uniform branch: n is the row's).
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if ((int64_t)r * SROUND >= n) break;
#pragma unroll
    for (int j = 0; j < SKT; ++j)
      if (key[r][j] != INVALID) rep_add(hist, key[r][j] >> 8, tid);
  }
  lds_barrier();
  uint4 hb = make_uint4(rep_total(hist, 4 * lane), rep_total(hist, 4 * lane + 1), rep_total(hist, 4 * lane + 2),
                        rep_total(hist, 4 * lane + 3));
  const DigitChoice st = choose_digit_wave(hb, 0u, (uint32_t)k, true, (uint32_t)k);
  uint32_t tau = 0, need = 0;
  if (!st.all) {  // uniform
    // low byte among the keys in the chosen high bin
    lds_barrier();  // every wave has read the first histogram
    rep_clear(hist, tid);
    lds_barrier();
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if ((int64_t)r * SROUND >= n) break;
#pragma unroll
      for (int j = 0; j < SKT; ++j)
        if ((key[r][j] >> 8) == st.prefix) rep_add(hist, key[r][j] & 255u, tid);
    }
    lds_barrier();
    hb = make_uint4(rep_total(hist, 4 * lane), rep_total(hist, 4 * lane + 1), rep_total(hist, 4 * lane + 2),
                    rep_total(hist, 4 * lane + 3));
    const DigitChoice st2 = choose_digit_wave(hb, st.prefix, st.need, false, (uint32_t)k);
    tau = st2.prefix;  // the k-th largest key
    need = st2.need;   // how many keys equal to tau are taken (the lowest-index ones)
  }

  // Compaction in index order: a key's place is the number of selected keys
  // before it, i.e. the keys above tau before it plus min(ties before it,
  // need).  Round r holds keys r*4096 + 16*tid + j, so rounds are in index
  // order and, within a round, threads are.
  int32_t* out = idx_out + row * k;
  uint32_t gt_before = 0, eq_before = 0;  // over the previous rounds
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if ((int64_t)r * SROUND >= n) break;
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int j = 0; j < SKT; ++j) {
      const bool valid = key[r][j] != INVALID;
      gt += (valid && (st.all || key[r][j] > tau)) ? 1u : 0u;
      eq += (valid && !st.all && key[r][j] == tau) ? 1u : 0u;
    }
    uint64_t tot;
    const uint64_t pre = block_excl_sum64<SBS>(((uint64_t)eq << 32) | gt, sc, tot);
    uint32_t g = gt_before + (uint32_t)pre, e = eq_before + (uint32_t)(pre >> 32);
    const int64_t i0 = (int64_t)r * SROUND + (int64_t)tid * SKT;
#pragma unroll
    for (int j = 0; j < SKT; ++j) {
      const bool valid = key[r][j] != INVALID;
      const bool above = valid && (st.all || key[r][j] > tau);
      const bool tie = valid && !st.all && key[r][j] == tau;
      const uint32_t pos = g + min(e, need);
      if (above || (tie && e < need)) out[pos] = (int32_t)(i0 + j);
      g += above ? 1u : 0u;
      e += tie ? 1u : 0u;
    }
    gt_before += (uint32_t)tot;
    eq_before += (uint32_t)(tot >> 32);
  }
  const uint32_t taken = gt_before + min(eq_before, need);
  for (uint32_t j = taken + tid; j < (uint32_t)k; j += SBS) out[j] = -1;
}

size_t topk_ws_bytes(int batch, int n_q, int64_t n_cap, int k, int score_dtype) {
  (void)k;
  const int64_t rows = (int64_t)batch * n_q;
  if (!use_split(rows, n_cap, score_dtype)) return 0;
  return (SPLIT_FIXED_WORDS + topk_split_plan(n_cap).row_words * (size_t)rows) * 4;
}

bool topk_uses_split(int64_t rows, int64_t n_cap, int score_dtype) { return use_split(rows, n_cap, score_dtype); }

uint32_t* topk_split_totals(void* ws, int* row_words) {
  *row_words = (int)SPLIT_FIXED_ROW_WORDS;
  return reinterpret_cast<uint32_t*>(ws);
}

hipError_t launch_topk(const void* scores, int score_dtype, int batch, int n_q, int64_t n_cap,
                       const int32_t* n_entries, const int64_t* q_pos, int ratio, int k, int32_t* idx_out, void* ws,
                       hipStream_t s, bool pass1_done) {
  if (batch == 0 || n_q == 0) return hipSuccess;
  const int64_t rows = (int64_t)batch * n_q;
  if (use_split(rows, n_cap, score_dtype)) {
    const SplitPlan p = topk_split_plan(n_cap);
    const uint16_t* sc = reinterpret_cast<const uint16_t*>(scores);
    dim3 grid(p.chunks, (unsigned)rows);
    if (!pass1_done) {  // else the scores' producer already accumulated total0 and cleared total1
      hipLaunchKernelGGL(topk_split_hist0, grid, dim3(SBS), 0, s, sc, n_q, n_cap, n_entries, q_pos, ratio, ws, p);
      const hipError_t e0 = hipGetLastError();
      if (e0 != hipSuccess) return e0;
    }
    hipError_t e;
    const dim3 xgrid((unsigned)(8 * ((rows + 7) / 8) * p.chunks));
    hipLaunchKernelGGL(topk_split_hist1, xgrid, dim3(SBS), 0, s, sc, n_q, n_cap, n_entries, q_pos, ratio, k, ws, p,
                       (int)rows);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_split_select, xgrid, dim3(SBS), 0, s, sc, n_q, n_cap, n_entries, q_pos, ratio, k, ws, p,
                       idx_out, (int)rows);
    return hipGetLastError();
  }
  dim3 grid(n_q, batch);
  if (score_dtype == CSA_BF16 && n_cap <= (int64_t)RR_MAX_ROUNDS * SROUND) {
    const uint16_t* sc = reinterpret_cast<const uint16_t*>(scores);
    const int64_t rounds = (n_cap + SROUND - 1) / SROUND;
#define CSA_TOPK_RR(R) \
  hipLaunchKernelGGL((topk_row_regs_kernel<R>), grid, dim3(SBS), 0, s, sc, n_q, n_cap, n_entries, q_pos, ratio, k, idx_out)
    if (rounds <= 1) CSA_TOPK_RR(1);
    else if (rounds <= 2) CSA_TOPK_RR(2);
    else if (rounds <= 4) CSA_TOPK_RR(4);
    else CSA_TOPK_RR(8);
#undef CSA_TOPK_RR
  } else if (score_dtype == CSA_BF16)
    hipLaunchKernelGGL((topk_row_kernel<true, 512>), grid, dim3(512), 0, s, scores, n_q, n_cap, n_entries, q_pos,
                       ratio, k, idx_out);
  else
    hipLaunchKernelGGL((topk_row_kernel<false, 512>), grid, dim3(512), 0, s, scores, n_q, n_cap, n_entries, q_pos,
                       ratio, k, idx_out);
  return hipGetLastError();
}

}  // namespace csa
