// Attention over compressed entries plus the sliding window.
//   CSA (「论文解读｜DeepSeek-V4：百万 token 上下文的效率革命」, blog.tripbot.top,
//   §3.1 + §3.3 + Figure 3): keys = the top-k selected entries U the last W raw
//   tokens (t-W+1 .. t); HCA (same page, §3.2): keys = every visible entry U the
//   window.  One joint softmax per (query, head); the value is the stored row
//   itself (MQA: all query heads share the single KV row); an optional
//   learnable sink adds exp(sink_h) to head h's denominator (§3.3).
//
// Two implementations:
//   * attn_valu_kernel — float32 vector path for any dtype (used for float32
//     rows/queries and head counts that are not a multiple of 32).
//   * attn_mfma_kernel / attn_mfma_pair_kernel — matrix-core path (q BF16,
//     rows FP8/BF16 mixed): S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (exact
//     BF16 inputs) and O^T = V^T P^T on v_mfma_f32_32x32x16_f16 (P and V in
//     FP16), fp32 accumulation and an fp32 online softmax.  When there are too
//     few queries to fill the chip, a query's key list is cut into segments
//     run by separate work-groups (the pair kernel, placed per XCD), and their
//     partial (max, sum, O) are merged by attn_merge_pair_kernel.
#include "common.h"

namespace csa {

namespace {

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// Where key number j of a query's list lives: pointer to its stored row, or null.
// Counts and indices are 32-bit (the host bounds a list at 2^31 - 1 keys and a
// ring at 2^30 rows); only the sequence's base pointers are 64-bit.
struct KeyList {
  const uint8_t* kv;     // batch slice of the entry rows (paged: the page pool)
  const uint8_t* win;    // batch slice of the window ring
  const uint8_t* any;    // some readable row (for loads whose result is discarded)
  const int32_t* idx;    // query's selected list (null = dense)
  const int32_t* pages;  // the sequence's page table (null = contiguous entries)
  int k;                 // length of the selected list (dense: n_vis)
  int nv;                // visible entries
  int cap;               // entry capacity of the sequence
  int window;
  int win_rows;
  int w_lo;              // window keys w < w_lo are not stored (position < 0 or below the ring's base)
  int m0;                // ring row of window key 0 (negative when the ring starts after it)
  int rb;                // row bytes
  int pshift;            // log2 of the entries per page
  int pool_pages;
  __device__ __forceinline__ int len() const { return k + window; }
  // Row of entry e (0 <= e < cap) in kv: e itself, or its place in the pool.
  __device__ __forceinline__ int64_t entry_row(int e) const {
    if (!pages) return e;
    int pg = pages[e >> pshift];
    pg = pg < 0 ? 0 : (pg >= pool_pages ? pool_pages - 1 : pg);
    return ((int64_t)pg << pshift) | (e & ((1 << pshift) - 1));
  }
  // Ring row of window key w (0 <= w < window <= win_rows), -1 if not stored.
  __device__ __forceinline__ int win_row(int w) const {
    if (w < w_lo) return -1;
    const int x = m0 + w;  // in [0, 2 win_rows)
    return x >= win_rows ? x - win_rows : x;
  }
  __device__ __forceinline__ const uint8_t* row(int j) const {
    if (j < k) {
      const int e = idx ? idx[j] : j;
      return (e >= 0 && e < nv) ? kv + entry_row(e) * rb : nullptr;
    }
    const int r = win_row(j - k);
    return r < 0 ? nullptr : win + (int64_t)r * rb;
  }
};

// The list in two steps: the parts given by the arguments alone (so that the
// selected indices of a first block can be requested at once), then those that
// need the query's position and the sequence's entry count, which the caller
// requests together (list_position).
__device__ __forceinline__ KeyList list_base(const AttnArgs& a, int b, int64_t row) {
  KeyList L;
  L.rb = row_bytes(a.kv_dtype);
  L.pages = a.pages.pages ? a.pages.pages + (int64_t)b * (a.n_cap >> a.pages.shift) : nullptr;
  L.pshift = a.pages.shift;
  L.pool_pages = a.pages.pool_pages;
  L.cap = (int)a.n_cap;
  L.kv = reinterpret_cast<const uint8_t*>(a.kv) + (L.pages ? 0 : (int64_t)b * a.n_cap * L.rb);
  L.win = reinterpret_cast<const uint8_t*>(a.win) + (int64_t)b * a.win_rows * L.rb;
  L.any = a.n_cap > 0 ? L.kv : L.win;
  L.idx = a.idx ? a.idx + row * a.k : nullptr;
  L.k = a.idx ? a.k : 0;
  L.window = a.window;
  L.win_rows = (int)a.win_rows;
  return L;
}
struct ListPos {
  int64_t t, n_entries;
};
__device__ __forceinline__ ListPos list_position(const AttnArgs& a, int b, int64_t row) {
  ListPos p;
  p.t = a.q_pos[row];
  p.n_entries = a.n_cap > 0 ? a.n_entries[b] : 0;  // no entries: window only
  return p;
}
__device__ __forceinline__ void list_finish(KeyList& L, const AttnArgs& a, ListPos p) {
  L.nv = a.n_cap > 0 ? (int)visible_entries(p.n_entries, p.t, a.ratio, a.n_cap) : 0;
  if (!a.idx) L.k = L.nv;
  const int64_t p0 = p.t - a.window + 1;  // position of window key 0
  const int64_t rel0 = p0 - a.win_base;   // its place relative to the ring's base
  // keys below position 0 or below the base are absent
  int64_t lo = 0;
  if (-p0 > lo) lo = -p0;
  if (-rel0 > lo) lo = -rel0;
  L.w_lo = lo > a.window ? a.window : (int)lo;
  // rel0 mod win_rows; a power-of-two ring (the usual case) takes a mask
  // instead of a 64-bit division.  A ring starting after key 0 maps key w to
  // row rel0 + w directly (rel0 + w < window <= win_rows, no wrap).
  const int64_t wr = a.win_rows;
  L.m0 = (wr <= 0 || rel0 < -(int64_t)a.window) ? 0
         : rel0 < 0                              ? (int)rel0
         : (wr & (wr - 1)) == 0                  ? (int)(rel0 & (wr - 1))
                                                 : (int)(rel0 % wr);
}
__device__ __forceinline__ KeyList make_list(const AttnArgs& a, int b, int64_t row) {
  KeyList L = list_base(a, b, row);
  list_finish(L, a, list_position(a, b, row));
  return L;
}

__device__ __forceinline__ float load_row_elem(const uint8_t* r, int dtype, int d) {
  if (dtype == CSA_F32) return reinterpret_cast<const float*>(r)[d];
  if (dtype == CSA_BF16) return bf16_to_f32(reinterpret_cast<const uint16_t*>(r)[d]);
  return d < DIM_NOPE ? fp8_to_f32(r[d]) : bf16_to_f32(reinterpret_cast<const uint16_t*>(r + DIM_NOPE)[d - DIM_NOPE]);
}

__device__ __forceinline__ void store_out(void* out, int dtype, int64_t off, float v) {
  if (dtype == CSA_F32) reinterpret_cast<float*>(out)[off] = v;
  else reinterpret_cast<uint16_t*>(out)[off] = (uint16_t)f32_to_bf16_rne(v);
}

// Final normalisation with the optional sink: out = o_un * c for every dim of a
// head, o_un the unnormalised output, m the running max (natural-log units), l
// the sum of exp(logit - m).  Without a sink c = 1 / l; with sink logit s,
// c = e^(m-M) / (l e^(m-M) + e^(s-M)), M = max(m, s).  One division per head:
// a division per output element (an IEEE sequence of about ten instructions)
// would cost more than the attention itself on short key lists.
__device__ __forceinline__ float finish_scale(float m, float l, float sink, bool has_sink) {
  if (!has_sink) return l > 0.0f ? 1.0f / l : 0.0f;
  const float ms = fmaxf(m, sink);
  const float f = m == -INFINITY ? 0.0f : expf(m - ms);
  const float den = l * f + expf(sink - ms);
  return f / den;
}

}  // namespace

// ---------------------------------------------------------------------------
// float32 vector path: grid (n_q, batch, ceil(n_heads/16)), block 192 (thread = dim)
// ---------------------------------------------------------------------------
constexpr int VHG = 16;  // heads per block
constexpr int VKC = 32;  // keys per chunk

__global__ void __launch_bounds__(192) attn_valu_kernel(AttnArgs a) {
  __shared__ float qs[VHG][DIM];
  __shared__ float ks[VKC][DIM + 1];
  __shared__ float ls[VHG][VKC];
  __shared__ float m_s[VHG], l_s[VHG], al_s[VHG];
  __shared__ int valid[VKC];
  __shared__ const uint8_t* rows_s[VKC];

  const int b = blockIdx.y;
  const int64_t row = (int64_t)b * a.n_q + blockIdx.x;
  const int h0 = blockIdx.z * VHG;
  const int hg = min(VHG, a.n_heads - h0);
  const int d = threadIdx.x;
  const KeyList L = make_list(a, b, row);

  {  // every head's load in flight before the first store
    uint32_t qv[VHG];
    const int64_t q0 = (row * a.n_heads + h0) * DIM + d;
    if (a.q_dtype == CSA_F32) {
#pragma unroll
      for (int h = 0; h < VHG; ++h) qv[h] = reinterpret_cast<const uint32_t*>(a.q)[q0 + min(h, hg - 1) * DIM];
    } else {
#pragma unroll
      for (int h = 0; h < VHG; ++h)
        qv[h] = (uint32_t)reinterpret_cast<const uint16_t*>(a.q)[q0 + min(h, hg - 1) * DIM] << 16;
    }
#pragma unroll
    for (int h = 0; h < VHG; ++h)
      if (h < hg) qs[h][d] = __uint_as_float(qv[h]);
  }
  if (d < VHG) {
    m_s[d] = -INFINITY;
    l_s[d] = 0.0f;
  }
  float acc[VHG];
#pragma unroll
  for (int h = 0; h < VHG; ++h) acc[h] = 0.0f;
  __syncthreads();

  const int64_t n = L.len();
  for (int64_t c0 = 0; c0 < n; c0 += VKC) {
    const int nk = (int)min<int64_t>(VKC, n - c0);
    // the chunk's rows (one key's selected index and row per thread), then
    // every dim load of the chunk in flight at once (absent keys read some
    // row and store zeros)
    if (d < VKC) {
      const uint8_t* r = d < nk ? L.row(c0 + d) : nullptr;
      rows_s[d] = r;
      valid[d] = r != nullptr;
    }
    __syncthreads();
    {
      float v[VKC];
      auto src = [&](int j) { const uint8_t* r = rows_s[j]; return r ? r : L.any; };
      if (a.kv_dtype == CSA_F32) {
#pragma unroll
        for (int j = 0; j < VKC; ++j) v[j] = reinterpret_cast<const float*>(src(j))[d];
      } else if (a.kv_dtype == CSA_BF16 || d >= DIM_NOPE) {  // BF16 rows, or the BF16 RoPE dims of mixed rows
        const int o = a.kv_dtype == CSA_BF16 ? 2 * d : DIM_NOPE + 2 * (d - DIM_NOPE);
        uint32_t u[VKC];
#pragma unroll
        for (int j = 0; j < VKC; ++j) u[j] = *reinterpret_cast<const uint16_t*>(src(j) + o);
#pragma unroll
        for (int j = 0; j < VKC; ++j) v[j] = bf16_to_f32(u[j]);
      } else {  // FP8 dims of mixed rows
        uint32_t u[VKC];
#pragma unroll
        for (int j = 0; j < VKC; ++j) u[j] = src(j)[d];
#pragma unroll
        for (int j = 0; j < VKC; ++j) v[j] = fp8_to_f32(u[j]);
      }
#pragma unroll
      for (int j = 0; j < VKC; ++j) ks[j][d] = valid[j] ? v[j] : 0.0f;
    }
    __syncthreads();
    for (int p = d; p < hg * nk; p += DIM) {
      const int h = p / nk, j = p % nk;
      float dot = 0.0f;
      for (int e = 0; e < DIM; ++e) dot = fmaf(qs[h][e], ks[j][e], dot);
      ls[h][j] = valid[j] ? dot * a.scale : -INFINITY;
    }
    __syncthreads();
    if (d < hg) {
      float mx = -INFINITY;
      for (int j = 0; j < nk; ++j) mx = fmaxf(mx, ls[d][j]);
      const float m_new = fmaxf(m_s[d], mx);
      const float alpha = m_new == -INFINITY ? 1.0f : expf(m_s[d] - m_new);
      float sum = 0.0f;
      for (int j = 0; j < nk; ++j) {
        const float p = ls[d][j] == -INFINITY ? 0.0f : expf(ls[d][j] - m_new);
        ls[d][j] = p;
        sum += p;
      }
      l_s[d] = l_s[d] * alpha + sum;
      m_s[d] = m_new;
      al_s[d] = alpha;
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < VHG; ++h) {
      if (h < hg) {
        float s = acc[h] * al_s[h];
        for (int j = 0; j < nk; ++j) s = fmaf(ls[h][j], ks[j][d], s);
        acc[h] = s;
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int h = 0; h < VHG; ++h) {
    if (h < hg) {
      const float sink = a.sink ? a.sink[h0 + h] : 0.0f;
      const float o = acc[h] * finish_scale(m_s[h], l_s[h], sink, a.sink != nullptr);
      store_out(a.out, a.out_dtype, (row * a.n_heads + h0 + h) * DIM + d, o);
    }
  }
  if (a.lse && d < hg) a.lse[row * a.n_heads + h0 + d] = l_s[d] > 0.0f ? m_s[d] + logf(l_s[d]) : -INFINITY;
}

// ---------------------------------------------------------------------------
// BF16 matrix-core path
// ---------------------------------------------------------------------------
// Per block of 32 keys, in LDS (double-buffered):
//   Ks [key][dim] BF16  — A operand of S^T = K Q^T (FP8 dims widened exactly,
//                         RoPE dims copied), read with 16-byte loads;
//   Vs [key][dim] FP16  — V for O^T = V^T P^T (FP8 dims exact in FP16, RoPE
//                         dims clamped to +-65504, below 2^-14 rounded toward
//                         zero), read transposed with ds_read_b64_tr_b16.
// Later blocks' rows are loaded into registers while the current block is
// computed; one barrier per block.
constexpr int KB = 32;         // keys per block (one 32x32 MFMA tile)
constexpr int KSTR = DIM + 8;  // K tile row stride (bf16 elements): 400 B rows
// V tile row stride (fp16 elements).  A transposed read takes, per 16-lane
// group, 8 bytes at rows kbase..kbase+3 and byte offsets 0, 8, 16, 24 within a
// 32-byte column slice, and the next 16 lanes the next slice; LDS serves 32
// lanes of 8 bytes over its 64 four-byte banks at once.  Rows of 448 B (a
// stride of 112 banks, == 48 mod 64) put the four rows 16 banks apart, so the
// 32 lanes cover the 64 banks once (416-byte rows leave 2-way conflicts:
// bank-conflict cycles 759K -> 304K per decode launch).  They are used with
// four head waves (128 heads), where registers hold a CU to two work-groups
// anyway; with fewer waves rows stay 416 B, so that three work-groups' tiles
// fit a CU's 160 KB of LDS (448-byte rows allow two: the 64-head chunked
// prefill ran 265 -> 350 us).
template <int NW>
constexpr int vstr() { return NW == 4 ? DIM + 32 : DIM + 16; }
constexpr float RESCALE_SLACK = 8.0f;  // log2 units

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

struct MfmaSplit {
  int splits;
  int keys_per_split;
};

// How a query's key list is cut into independently processed segments.  The
// plan depends only on per-sequence quantities (queries per sequence, longest
// list), never on the batch size, so a sequence gets bitwise the same result
// alone or inside any batch.  Many queries per sequence (prefill): one
// segment.  Few (decode): segments of at least SPLIT_MIN_BLOCKS key blocks and
// at most SPLIT_MAX segments per query.  A decode row's segments are placed on
// one XCD (32 CUs), so SPLIT_MAX is that XCD's CU count.  SPLIT_MIN_BLOCKS
// bounds how short a segment gets: each carries a fixed cost (key list and
// query loads, the FP16 partial store, its share of the merge).  At 1M context
// a decode CSA list (1,152 keys, 36 blocks of KB) gets 18 segments of 2 blocks,
// a top-512 one (640 keys) 10 of 2, and an HCA list (8,320 keys, 260 blocks)
// 29 of 9 blocks.  At most 32 was the fastest of the limits measured on the
// batch-8 decode layers (27, 32, 48, 64); at least 2 blocks instead of 4 left
// the top-1,024 step unchanged and made the top-512 one 1.8 % faster.
constexpr int SPLIT_MAX = 32;
constexpr int SPLIT_MIN_BLOCKS = 2;

__host__ __device__ inline MfmaSplit plan_split(int n_q, int n_heads, int64_t max_keys) {
  (void)n_heads;
  MfmaSplit p;
  const int64_t blocks = (max_keys + KB - 1) / KB;
  if (n_q >= 64 || blocks <= SPLIT_MIN_BLOCKS) {
    p.splits = 1;
    p.keys_per_split = (int)((blocks > 0 ? blocks : 1) * KB);
    return p;
  }
  int64_t bps = (blocks + SPLIT_MAX - 1) / SPLIT_MAX;
  if (bps < SPLIT_MIN_BLOCKS) bps = SPLIT_MIN_BLOCKS;
  p.keys_per_split = (int)(bps * KB);
  p.splits = (int)((blocks + bps - 1) / bps);
  return p;
}

// Staging of one block.  In round u a thread takes row r = i/8 and p = i%8 of
// the block, i = tid + u*NT: the FP8 piece p (bytes 16p.. of the stored row,
// dims 16p..16p+15) and the BF16 piece p (bytes 128+16p.., dims 128+8p..+7), so
// every thread runs both conversions and the wave never diverges.  Rows that do
// not exist are read from a readable dummy row and zeroed.
template <int NT>
struct Stage {
  static constexpr int ROUNDS = (KB * 8 + NT - 1) / NT;
  uint4 f8[ROUNDS], b16[ROUNDS];
  bool ok[ROUNDS];
};

// Selected entry indices of a thread's staged rows, loaded one block ahead of
// their use so that waiting for them never drains the row loads in flight.
// With paged entries the look-ahead holds the entries (-1 outside the
// capacity) and their pool pages as read from the page table (pools hold
// fewer than 2^31 rows).  Paged lists come from the decode step, whose
// selections hold visible entries only, so the row alone decides.
template <int NT>
struct IdxAhead {
  int32_t e[Stage<NT>::ROUNDS];
  int32_t pg[Stage<NT>::ROUNDS];  // paged lists: the entry's pool page, as read from the table
};

template <int NT>
__device__ __forceinline__ void idx_load(const KeyList& L, int jb, int tid, IdxAhead<NT>& ia) {
  // No branch around the load: a dense list reads some readable word instead
  // (the value is not used).  A load under a branch ends in a copy at the
  // join, which makes the compiler wait for it at once.
  const bool sel = L.idx && L.k > 0;
#pragma unroll
  for (int u = 0; u < Stage<NT>::ROUNDS; ++u) {
    int j = jb + ((tid + u * NT) >> 3);
    j = j < L.k ? j : L.k - 1;  // in bounds; positions past the selection are window keys
    const int32_t* ip = sel ? L.idx + j : reinterpret_cast<const int32_t*>(L.any);
    ia.e[u] = *ip;
  }
}

// Paged lists: a block's rows in two steps, so that the deep loop never waits
// for a read it has just issued.  idx_ids reads the block's entries (selected
// indices; a dense list reads a word it ignores), idx_rows, an iteration
// later, turns them into entries and reads their pages, and stage_load,
// another iteration later, forms the pool rows.  Values are used only after
// the iteration that read them: the compiler waits for a load when its value
// is first used, and reads under a branch or followed at once by arithmetic
// would be waited for at the read.
template <int NT>
__device__ __forceinline__ void idx_ids(const KeyList& L, int jb, int tid, IdxAhead<NT>& ia) {
  const bool sel = L.idx && L.k > 0;
#pragma unroll
  for (int u = 0; u < Stage<NT>::ROUNDS; ++u) {
    const int j = jb + ((tid + u * NT) >> 3);
    const int jc = j < L.k ? j : L.k - 1;
    const int32_t* ip = sel ? L.idx + jc : reinterpret_cast<const int32_t*>(L.any);
    ia.e[u] = *ip;
  }
}
template <int NT>
__device__ __forceinline__ void idx_rows(const KeyList& L, int jb, int tid, IdxAhead<NT>& ia) {
#pragma unroll
  for (int u = 0; u < Stage<NT>::ROUNDS; ++u) {
    const int j = jb + ((tid + u * NT) >> 3);
    const int e = L.idx ? (L.k > 0 ? ia.e[u] : -1) : j;
    const bool in = e >= 0 && e < L.cap;  // the table is read inside its bounds only
    ia.e[u] = in ? e : -1;
    const int32_t* pp = L.cap > 0 ? L.pages + ((in ? e : 0) >> L.pshift) : reinterpret_cast<const int32_t*>(L.any);
    ia.pg[u] = *pp;
  }
}
// A block's look-ahead in one go (prologue, short-stage loop).
template <int NT, bool PAGED>
__device__ __forceinline__ void idx_full(const KeyList& L, int jb, int tid, IdxAhead<NT>& ia) {
  if constexpr (PAGED) {
    idx_ids<NT>(L, jb, tid, ia);
    idx_rows<NT>(L, jb, tid, ia);
  } else {
    idx_load<NT>(L, jb, tid, ia);
  }
}

template <int NT, bool PAGED>
__device__ __forceinline__ void stage_load(const KeyList& L, int jb, int j_end, int tid, const IdxAhead<NT>& ia,
                                           Stage<NT>& st) {
#pragma unroll
  for (int u = 0; u < Stage<NT>::ROUNDS; ++u) {
    const int i = tid + u * NT;
    const int p = i & 7;
    const int j = jb + (i >> 3);
    const uint8_t* src = nullptr;
    if (i < KB * 8 && j < j_end) {
      if (j < L.k) {
        if constexpr (PAGED) {
          const int e = ia.e[u];
          if (e >= 0) {
            int pg = ia.pg[u];
            pg = pg < 0 ? 0 : (pg >= L.pool_pages ? L.pool_pages - 1 : pg);
            src = L.kv + (((int64_t)pg << L.pshift) | (e & ((1 << L.pshift) - 1))) * L.rb;
          }
        } else {
          const int e = L.idx ? ia.e[u] : j;
          if (e >= 0 && e < L.nv) src = L.kv + (int64_t)e * L.rb;
        }
      } else {
        const int wr = L.win_row(j - L.k);
        if (wr >= 0) src = L.win + (int64_t)wr * L.rb;
      }
    }
    st.ok[u] = src != nullptr;
    const uint8_t* rd = src ? src : L.any;
    st.f8[u] = *reinterpret_cast<const uint4*>(rd + 16 * p);
    st.b16[u] = *reinterpret_cast<const uint4*>(rd + DIM_NOPE + 16 * p);
  }
}

template <int NT, int VSTR>
__device__ __forceinline__ void stage_store(const Stage<NT>& st, int tid, uint16_t* Ks, uint16_t* Vs, int* valid) {
#pragma unroll
  for (int u = 0; u < Stage<NT>::ROUNDS; ++u) {
    const int i = tid + u * NT;
    if (i >= KB * 8) break;  // wave-uniform
    const int r = i >> 3, p = i & 7;
    if (p == 0) valid[r] = st.ok[u];
    // A row that does not exist was read from some real row; it is masked out
    // of the softmax, and its value is zeroed so that a non-finite value
    // stored there cannot reach the output (0 * inf).  Integer masks, not a
    // conditional copy of the vectors (which the compiler turns into a
    // memory temporary).
    const uint32_t keep = st.ok[u] ? 0xffffffffu : 0u;
    const uint4 f8 = make_uint4(st.f8[u].x & keep, st.f8[u].y & keep, st.f8[u].z & keep, st.f8[u].w & keep);
    const uint4 bf = make_uint4(st.b16[u].x & keep, st.b16[u].y & keep, st.b16[u].z & keep, st.b16[u].w & keep);
    {  // 16 FP8 values, dims 16p .. 16p+15: K as BF16, V as FP16 (both exact)
      const uint32_t w[4] = {f8.x, f8.y, f8.z, f8.w};
      uint32_t kb[8], vh[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        auto b0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[q], 1.0f, false);
        auto b1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[q], 1.0f, true);
        auto h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[q], 1.0f, false);
        auto h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[q], 1.0f, true);
        __builtin_memcpy(&kb[2 * q], &b0, 4);
        __builtin_memcpy(&kb[2 * q + 1], &b1, 4);
        __builtin_memcpy(&vh[2 * q], &h0, 4);
        __builtin_memcpy(&vh[2 * q + 1], &h1, 4);
      }
      const int d0 = 16 * p;
      uint4* kd = reinterpret_cast<uint4*>(Ks + r * KSTR + d0);
      kd[0] = make_uint4(kb[0], kb[1], kb[2], kb[3]);
      kd[1] = make_uint4(kb[4], kb[5], kb[6], kb[7]);
      uint2* vd = reinterpret_cast<uint2*>(Vs + r * VSTR + d0);
      vd[0] = make_uint2(vh[0], vh[1]);
      vd[1] = make_uint2(vh[2], vh[3]);
      vd[2] = make_uint2(vh[4], vh[5]);
      vd[3] = make_uint2(vh[6], vh[7]);
    }
    {  // 8 BF16 values, dims 128 + 8p .. +7: K copied, V to FP16 (clamped to +-65504)
      const int d0 = DIM_NOPE + 8 * p;
      *reinterpret_cast<uint4*>(Ks + r * KSTR + d0) = bf;
      const uint32_t w[4] = {bf.x, bf.y, bf.z, bf.w};
      uint32_t vh[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float lo = __builtin_amdgcn_fmed3f(__uint_as_float(w[q] << 16), -65504.0f, 65504.0f);
        const float hi = __builtin_amdgcn_fmed3f(__uint_as_float(w[q] & 0xffff0000u), -65504.0f, 65504.0f);
        auto h = __builtin_amdgcn_cvt_pkrtz(lo, hi);
        __builtin_memcpy(&vh[q], &h, 4);
      }
      uint2* vd = reinterpret_cast<uint2*>(Vs + r * VSTR + d0);
      vd[0] = make_uint2(vh[0], vh[1]);
      vd[1] = make_uint2(vh[2], vh[3]);
    }
  }
}

// Work-group barrier for LDS data only: unlike __syncthreads it does not wait
// for the global loads in flight (the next blocks' rows).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Swap-add across the two 32-lane halves of a wave: every lane gets
// x[l % 32] + x[l % 32 + 32] (v_permlane32_swap, no LDS round trip).
__device__ __forceinline__ float half_sum(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}
__device__ __forceinline__ float half_max(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}

// Two floats as FP16 (round to nearest even), packed low / high.
__device__ __forceinline__ uint32_t half2_bits(float lo, float hi) {
  const _Float16 a = (_Float16)lo, b = (_Float16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}
__device__ __forceinline__ float half_lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu)); }
__device__ __forceinline__ float half_hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }
// Bytes of the FP16 O / l partials of a split launch (the (m, l) pairs follow).
__host__ __device__ inline int64_t partial_o_bytes(int64_t rows, int splits, int n_heads) {
  return rows * splits * (int64_t)n_heads * DIM * 2;
}

// LDS of one work-group: two K tiles and two V tiles (double buffering) and
// the row-validity flags.
constexpr int LDS_K = KB * KSTR * 2;  // bytes of one K tile
template <int NW>
constexpr int lds_v() { return KB * vstr<NW>() * 2; }  // bytes of one V tile
template <int NW>
constexpr int lds_bytes() { return 2 * LDS_K + 2 * lds_v<NW>() + 2 * KB * 4; }
// Output staging of a wave's 32 heads x 192 dims (unsplit lists, BF16 output):
// row strides padded by 16 bytes, one area per wave in the tiles' space.
constexpr int OUT_ROW_BF16 = DIM * 2 + 16;
constexpr int OUT_AREA_BF16 = 32 * OUT_ROW_BF16;
static_assert(4 * OUT_AREA_BF16 <= lds_bytes<4>() && 3 * OUT_AREA_BF16 <= lds_bytes<3>(), "output staging fits");

// Work-group of NW waves; wave w owns heads 32w .. 32w+31 and every wave
// takes every key block of the segment (the K and V tiles are shared through
// LDS).  Work-group (sp, qy, b) of one attention problem: split sp of query qy
// of sequence b; rows = batch * n_q.  The kernels below map block indices onto
// it.  (Two key groups per work-group, taking alternate blocks and combining
// their states at the end, were measured: at batch 8 within 2 % either way,
// at batch 32 22 % slower: one work-group per CU, and the groups meet at
// every barrier.)
template <int NW, bool PAGED>
__device__ __forceinline__ void attn_mfma_body(const AttnArgs& a, int splits, int keys_per_split, int sp, int qy,
                                               int b, int64_t rows, uint8_t* lds) {
  constexpr int NT = 64 * NW;  // threads of the work-group
  const int64_t row = (int64_t)b * a.n_q + qy;
  const int lane = threadIdx.x & 63;
  const int tid = threadIdx.x;
  const int wv = tid >> 6;
  const int g = lane >> 5, col = lane & 31;
  const int head = 32 * wv + col;
  constexpr int VSTR = vstr<NW>();
  constexpr int LDS_V = lds_v<NW>();
  uint8_t* my = lds;
  auto Kt = [&](int buf) { return reinterpret_cast<uint16_t*>(my + buf * LDS_K); };
  auto Vt = [&](int buf) { return reinterpret_cast<uint16_t*>(my + 2 * LDS_K + buf * LDS_V); };
  auto valid = [&](int buf) { return reinterpret_cast<int*>(my + 2 * LDS_K + 2 * LDS_V + buf * KB * 4); };

  // Requests that need only the arguments go out first: the query's position
  // and entry count, its Q rows, and the selected indices of this group's first
  // block (their positions in the list do not depend on the query position).
  KeyList L = list_base(a, b, row);
  const ListPos lp = list_position(a, b, row);
  // Q^T fragments: B operand, lane holds head `col` and dims 16*ks + 8*g .. +7
  v8bf qf[12];
  {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + (row * a.n_heads + head) * DIM;
#pragma unroll
    for (int ks = 0; ks < 12; ++ks) qf[ks] = *reinterpret_cast<const v8bf*>(qp + 16 * ks + 8 * g);
  }
  IdxAhead<NT> ia;
  idx_full<NT, PAGED>(L, sp * keys_per_split, tid, ia);
  list_finish(L, a, lp);
  const int n = L.len();
  const int j_begin = sp * keys_per_split;
  const int j_end = min(n, j_begin + keys_per_split);
  const int nblk = j_end > j_begin ? (j_end - j_begin + KB - 1) / KB : 0;
  // transposed-read addressing of the V tile (see the lane mapping of ds_read_b64_tr_b16:
  // within each 16-lane group, lane s supplies the 4 values at row kbase + s/4, dims
  // dbase + 4*(s%4) .. +3; lane d receives dim dbase + d of rows kbase .. kbase+3)
  const int l16 = lane >> 4, s16 = lane & 15;
  const int v_off = (4 * g + (s16 >> 2)) * VSTR + 16 * (l16 & 1) + 4 * (s16 & 3);

  const float sl2 = a.scale * LOG2E;
  float m = -INFINITY, l = 0.0f;  // m in log2 units
  v16f o[6];
#pragma unroll
  for (int nt = 0; nt < 6; ++nt) o[nt] = v16f{};

  // Rows are staged two blocks ahead of their use through a ring of two
  // register stages: while block i is computed, block i+1 (requested an
  // iteration earlier) is converted into the other LDS tile at the end of the
  // iteration and block i+2 is requested.  The requests are unconditional
  // (blocks past the segment read a real row and are marked absent), so the
  // compiler's waits count exactly the loads still needed; barriers wait for
  // LDS only, keeping the next block's rows in flight.
  // The selected indices of a block are requested one iteration before its
  // rows (two index registers take turns), after that iteration's row
  // requests: a wait the compiler places at the head of an iteration (it
  // reuses registers of the rows in flight) then covers the previous
  // iteration's requests only, never an index just requested (measured: the
  // 4,096-query CSA prefill chunk 608 -> 565 us).
  // With fewer threads (fewer than 128 heads) each thread stages two pieces
  // per block and a second stage does not fit the register budget: rows are
  // then staged one block ahead.
  constexpr bool DEEP = Stage<NT>::ROUNDS == 1;
  Stage<NT> sa, sb;
  IdxAhead<NT> ia1;
  {
    const int jb0 = j_begin;  // the first block (its indices requested above)
    stage_load<NT, PAGED>(L, jb0, j_end, tid, ia, sa);
    if constexpr (DEEP) {
      idx_full<NT, PAGED>(L, jb0 + KB, tid, ia1);
      stage_load<NT, PAGED>(L, jb0 + KB, j_end, tid, ia1, sb);
      idx_full<NT, PAGED>(L, jb0 + 2 * KB, tid, ia);
      if constexpr (PAGED) idx_ids<NT>(L, jb0 + 3 * KB, tid, ia1);
    } else {
      idx_full<NT, PAGED>(L, jb0 + KB, tid, ia);
    }
    if (nblk > 0) stage_store<NT, VSTR>(sa, tid, Kt(0), Vt(0), valid(0));
  }
  lds_barrier();

  auto compute = [&](int buf) {
    const uint16_t* K = Kt(buf);
    const uint16_t* V = Vt(buf);
    const int* vld = valid(buf);

    // ---- S^T[key][head] = K Q^T  (A = K rows, B = Q^T), one accumulation chain.
    // The key's validity flag is read first, and the K fragments three ahead
    // of their products: left to itself the scheduler reads each fragment into
    // the same four registers right before its product and waits for it there,
    // so every read's latency adds up along the chain (measured: 3 % on the
    // decode attention, batch 8 and 32).
    const int vcol = vld[col];
    v16f s = v16f{};
    {
      constexpr int KPRE = 3;
      v8bf kf[12];
#pragma unroll
      for (int ks = 0; ks < 12; ++ks) kf[ks] = *reinterpret_cast<const v8bf*>(K + col * KSTR + 16 * ks + 8 * g);
#pragma unroll
      for (int ks = 0; ks < 12; ++ks) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[ks], s, 0, 0, 0);
      // LDS reads (mask 0x100) and products (0x008) in the order: the flag and
      // KPRE fragments, then product / read pairs, then the last products
      __builtin_amdgcn_sched_group_barrier(0x100, KPRE + 1, 0);
#pragma unroll
      for (int i = 0; i < 12 - KPRE; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
#pragma unroll
      for (int i = 0; i < KPRE; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    // The V^T fragments of the first k-step are requested now, so that their
    // latency overlaps the products and the softmax; the second k-step's come
    // with the first k-step's products (both at once do not fit the
    // two-waves-per-SIMD register budget next to the staged rows).
    // k-step ks2 pairs A's k index 8g+i with key 16*ks2 + 4g + (i%4) + 8*(i/4),
    // which is exactly what P register 8*ks2+i of this lane holds.
    v8h vf[2][6];
    auto v_read = [&](int ks2) {
#pragma unroll
      for (int nt = 0; nt < 6; ++nt) {
        const uint16_t* vb = V + 16 * ks2 * VSTR + 32 * nt + v_off;
        const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(vb));
        const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(vb + 8 * VSTR));
        const v8s vv = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        __builtin_memcpy(&vf[ks2][nt], &vv, 16);
      }
    };
    v_read(0);
    // lane holds head `col`, keys 8*(r/4) + 4*g + r%4.  s stays unscaled; the
    // scale (> 0, so it commutes with max) is applied inside the exponent.
    if (!__all(vcol)) {  // wave-uniform: some key of the block does not exist
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 8 * (r >> 2) + 4 * g + (r & 3);
        s[r] = vld[key] ? s[r] : -INFINITY;
      }
    }
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = half_max(mx) * sl2;  // block max in log2 units
    // Lazy rescaling: the reference max m of a head moves only when a block's
    // max exceeds it by more than RESCALE_SLACK, so probabilities stay <= 2^8
    // (exact enough in FP16, far from its range limit) and the accumulators are
    // rescaled only on those rare blocks (wave-uniform branch).
    const bool grow = mx > m + RESCALE_SLACK;
    if (__any(grow)) {
      const float m_new = grow ? mx : m;
      const float alpha = grow ? __builtin_amdgcn_exp2f(m - m_new) : 1.0f;  // m = -inf -> 0
      l *= alpha;
#pragma unroll
      for (int nt = 0; nt < 6; ++nt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[nt][r] *= alpha;
      m = m_new;
    }
    const float mref = m == -INFINITY ? 0.0f : m;  // no finite logit yet: every p is 0
    float psum = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = __builtin_amdgcn_exp2f(fmaf(s[r], sl2, -mref));  // exp2(-inf) = 0
      s[r] = p;
      psum += p;
    }
    l += half_sum(psum);

    // ---- O^T[dim][head] += V^T[dim][key] P^T[key][head]
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
      if (ks2 == 1) v_read(1);
      v8h pf;  // P in FP16 (p in [0, 2^8]: 11 significant bits)
#pragma unroll
      for (int i = 0; i < 8; ++i) pf[i] = (_Float16)s[8 * ks2 + i];
#pragma unroll
      for (int nt = 0; nt < 6; ++nt) o[nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf[ks2][nt], pf, o[nt], 0, 0, 0);
    }
  };

  // One iteration: `next` holds block bi+1 (in flight), `free_` receives
  // block bi+2, whose indices are in `ia_use`; `ia_load` receives those of
  // block bi+3.
  auto iteration = [&](int bi, Stage<NT>& next, Stage<NT>& free_, IdxAhead<NT>& ia_use, IdxAhead<NT>& ia_load) {
    const int buf = bi & 1;
    const int jb = j_begin + bi * KB;
    stage_load<NT, PAGED>(L, jb + 2 * KB, j_end, tid, ia_use, free_);
    if constexpr (PAGED) {
      idx_rows<NT>(L, jb + 3 * KB, tid, ia_load);  // block bi+3: its entries (read an iteration ago), their pages
      idx_ids<NT>(L, jb + 4 * KB, tid, ia_use);    // block bi+4: its entries
    } else {
      idx_load<NT>(L, jb + 3 * KB, tid, ia_load);
    }
    compute(buf);
    if (bi + 1 < nblk) stage_store<NT, VSTR>(next, tid, Kt(buf ^ 1), Vt(buf ^ 1), valid(buf ^ 1));
    lds_barrier();
  };
  const int iters = nblk;
  if constexpr (DEEP) {
    for (int it = 0; it < iters; it += 2) {  // unrolled by two: the stages swap roles
      iteration(it, sb, sa, ia, ia1);
      if (it + 1 < iters) iteration(it + 1, sa, sb, ia1, ia);
    }
  } else {
    for (int bi = 0; bi < iters; ++bi) {  // one block ahead, one stage
      const int buf = bi & 1;
      const int jb = j_begin + bi * KB;
      const bool more = bi + 1 < nblk;
      if (more) {
        stage_load<NT, PAGED>(L, jb + KB, j_end, tid, ia, sa);
        idx_full<NT, PAGED>(L, jb + 2 * KB, tid, ia);
      }
      compute(buf);
      if (more) stage_store<NT, VSTR>(sa, tid, Kt(buf ^ 1), Vt(buf ^ 1), valid(buf ^ 1));
      lds_barrier();
    }
  }

  // lane holds head `col`, dims 32*nt + 8*(r/4) + 4*g + r%4
  if (splits == 1) {
    const float sink = a.sink ? a.sink[head] : 0.0f;
    const float c = finish_scale(m * LN2, l, sink, a.sink != nullptr);  // m in natural-log units
    const bool f32 = a.out_dtype == CSA_F32;
    if (!f32) {
      // The wave's 32 heads are one contiguous run of the output row
      // ([head][dim]).  The values pass through LDS (the wave's own area in
      // the tiles' space, free after the loop's last barrier), so that each
      // store instruction writes 64 consecutive 16-byte pieces rather than 64
      // pieces of 8 bytes one head row (384 B) apart.
      uint8_t* ob = lds + wv * OUT_AREA_BF16;
#pragma unroll
      for (int nt = 0; nt < 6; ++nt) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int d0 = 32 * nt + 8 * q4 + 4 * g;
          float v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = o[nt][4 * q4 + i] * c;
          *reinterpret_cast<uint2*>(ob + col * OUT_ROW_BF16 + 2 * d0) =
              make_uint2(f32x2_to_bf16x2_rne(v[0], v[1]), f32x2_to_bf16x2_rne(v[2], v[3]));
        }
      }
      // lanes read what other lanes of the same wave wrote (a wave's LDS
      // operations complete in issue order; the fences order them for the compiler)
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      constexpr int run = DIM * 2;  // bytes of one head's output
      uint4* dst = reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(a.out) +
                                            (row * a.n_heads + 32 * wv) * (int64_t)run);
#pragma unroll
      for (int s = 0; s < 12; ++s) {
        const int piece = lane + 64 * s;
        const int h = piece * 16 / run, w = piece * 16 - h * run;
        dst[piece] = *reinterpret_cast<const uint4*>(ob + h * OUT_ROW_BF16 + w);
      }
    } else {
#pragma unroll
      for (int nt = 0; nt < 6; ++nt) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int d0 = 32 * nt + 8 * q4 + 4 * g;
          float v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = o[nt][4 * q4 + i] * c;
          const int64_t off = (row * a.n_heads + head) * DIM + d0;
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + off) = make_float4(v[0], v[1], v[2], v[3]);
        }
      }
    }
    if (a.lse && g == 0) a.lse[row * a.n_heads + head] = l > 0.0f ? (m + log2f(l)) * LN2 : -INFINITY;
  } else {
    // partials: the split's own output O / l (|O / l| <= max |v| <= 65504, the V
    // tile's range) as FP16, [rows][splits][n_heads/32][24][64] x 4 halves in lane
    // order (each store instruction writes 512 B contiguous), then (m, l)
    // [rows][splits][n_heads] float2
    const int nw = a.n_heads / 32;
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;  // a split without keys stores 0
    uint2* po = reinterpret_cast<uint2*>(a.ws) + (((row * splits + sp) * nw + wv) * 24) * 64 + lane;
#pragma unroll
    for (int nt = 0; nt < 6; ++nt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        po[(nt * 4 + q4) * 64] = make_uint2(half2_bits(o[nt][4 * q4] * inv, o[nt][4 * q4 + 1] * inv),
                                            half2_bits(o[nt][4 * q4 + 2] * inv, o[nt][4 * q4 + 3] * inv));
    if (g == 0) {
      float2* pml = reinterpret_cast<float2*>(reinterpret_cast<uint8_t*>(a.ws) + partial_o_bytes(rows, splits, a.n_heads));
      pml[(row * splits + sp) * a.n_heads + head] = make_float2(m, l);
    }
  }
}

// grid (1, n_q, batch): one segment per row (rows with split lists go through
// the pair kernel); block NW waves.
template <int NW>
__global__ void __launch_bounds__(64 * NW, 2) attn_mfma_kernel(AttnArgs a, int splits, int keys_per_split) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[lds_bytes<NW>()];
  const int64_t rows = (int64_t)a.batch * a.n_q;
  if (a.pages.pages) attn_mfma_body<NW, true>(a, splits, keys_per_split, blockIdx.x, blockIdx.y, blockIdx.z, rows, lds);
  else attn_mfma_body<NW, false>(a, splits, keys_per_split, blockIdx.x, blockIdx.y, blockIdx.z, rows, lds);
}

// Work-groups are dealt to the chip's XCDs round-robin by linear id (id mod 8),
// each XCD with its own L2.  The paired kernels place every work-group of a
// query row on XCD (row mod 8): the row's split partials, written by the
// attention kernel, are then read back by the merge from the same L2.
constexpr int N_XCD = 8;
struct XcdSlot {
  int problem;  // 0 or 1, -1 = no work
  int64_t row;
  int item;  // split (attention) or head block (merge)
};
// Slot k of XCD x when XCD x takes, in order, per0 items of each problem-0 row
// r = x, x+8, .. < rows0, then per1 items of each problem-1 row likewise.
// All quantities fit in 32 bits (the launch has fewer than 2^31 work-groups and
// rows * items bounds it), so the divisions are 32-bit ones: a 64-bit division
// is a long instruction sequence at the head of every work-group.
__device__ __forceinline__ XcdSlot xcd_slot(int64_t id64, int64_t rows0_64, int per0, int64_t rows1_64, int per1) {
  XcdSlot w;
  const uint32_t id = (uint32_t)id64, rows0 = (uint32_t)rows0_64, rows1 = (uint32_t)rows1_64;
  const uint32_t x = id % N_XCD;
  const uint32_t k = id / N_XCD;
  const uint32_t n0 = rows0 > x ? (rows0 - x + N_XCD - 1) / N_XCD : 0;  // problem-0 rows on this XCD
  const uint32_t n1 = rows1 > x ? (rows1 - x + N_XCD - 1) / N_XCD : 0;
  w.problem = -1;
  w.row = 0;
  w.item = 0;
  if (k < n0 * (uint32_t)per0) {
    w.problem = 0;
    w.row = x + N_XCD * (k / (uint32_t)per0);
    w.item = (int)(k % (uint32_t)per0);
  } else if (k - n0 * (uint32_t)per0 < n1 * (uint32_t)per1) {
    const uint32_t k1 = k - n0 * (uint32_t)per0;
    w.problem = 1;
    w.row = x + N_XCD * (k1 / (uint32_t)per1);
    w.item = (int)(k1 % (uint32_t)per1);
  }
  return w;
}
inline int64_t xcd_grid(int64_t rows0, int per0, int64_t rows1, int per1) {
  int64_t most = 0;
  for (int x = 0; x < N_XCD; ++x) {
    const int64_t n0 = rows0 > x ? (rows0 - x + N_XCD - 1) / N_XCD : 0;
    const int64_t n1 = rows1 > x ? (rows1 - x + N_XCD - 1) / N_XCD : 0;
    const int64_t v = n0 * per0 + n1 * per1;
    most = v > most ? v : most;
  }
  return most * N_XCD;
}

// Two independent problems with the same head count in one launch (a decode
// step's CSA and HCA attention), work-groups placed by xcd_slot.
template <int NW>
__global__ void __launch_bounds__(64 * NW, 2) attn_mfma_pair_kernel(AttnArgs a0, int s0, int k0, AttnArgs a1,
                                                                         int s1, int k1) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[lds_bytes<NW>()];
  const int64_t rows0 = (int64_t)a0.batch * a0.n_q, rows1 = (int64_t)a1.batch * a1.n_q;
  const XcdSlot w = xcd_slot(blockIdx.x, rows0, s0, rows1, s1);  // uniform per work-group
  // (a problem's paging is uniform over the launch)
  if (w.problem == 0) {
    const int qy = (int)(w.row % a0.n_q), b = (int)(w.row / a0.n_q);
    if (a0.pages.pages) attn_mfma_body<NW, true>(a0, s0, k0, w.item, qy, b, rows0, lds);
    else attn_mfma_body<NW, false>(a0, s0, k0, w.item, qy, b, rows0, lds);
  } else if (w.problem == 1) {
    const int qy = (int)(w.row % a1.n_q), b = (int)(w.row / a1.n_q);
    if (a1.pages.pages) attn_mfma_body<NW, true>(a1, s1, k1, w.item, qy, b, rows1, lds);
    else attn_mfma_body<NW, false>(a1, s1, k1, w.item, qy, b, rows1, lds);
  }
}

// Merge of one row's split partials, four FP16 values of the partial record per
// thread: a work-group takes MERGE_CHUNK consecutive entries of the record
// ([n_heads/32][24][64] in the attention kernel's lane order), so each split's
// read is one contiguous run.  Entry f holds head 32*(f/1536) + (f%64)%32,
// dims 32*nt + 8*q4 + 4*g .. +3 with (nt, q4) = ((f/64)%24) / 4, % 4 and
// g = (f%64)/32.  Splits are combined in split order (deterministic); every
// split's record is requested before any is used.
constexpr int MERGE_CHUNK = 256;
__device__ __forceinline__ void attn_merge_body(const AttnArgs& a, int splits, int64_t rows, int64_t row,
                                                int chunk) {
  const int f = chunk * MERGE_CHUNK + threadIdx.x;
  const int rec = a.n_heads * (DIM / 4);  // 4-value entries per (row, split) record
  if (f >= rec) return;
  const int lane = f & 63, jj = f >> 6;
  const int wv = jj / 24, r24 = jj - wv * 24;
  const int head = 32 * wv + (lane & 31);
  const int d0 = 32 * (r24 >> 2) + 8 * (r24 & 3) + 4 * (lane >> 5);
  const uint2* po = reinterpret_cast<const uint2*>(a.ws) + row * splits * rec + f;
  const float2* pml = reinterpret_cast<const float2*>(reinterpret_cast<const uint8_t*>(a.ws) +
                                                      partial_o_bytes(rows, splits, a.n_heads)) +
                      row * splits * a.n_heads + head;
  float2 ml[SPLIT_MAX];
  uint2 v[SPLIT_MAX];
#pragma unroll
  for (int sp = 0; sp < SPLIT_MAX; ++sp) {
    if (sp < splits) {
      ml[sp] = pml[(int64_t)sp * a.n_heads];
      v[sp] = po[(int64_t)sp * rec];
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int sp = 0; sp < SPLIT_MAX; ++sp)
    if (sp < splits) M = fmaxf(M, ml[sp].x);
  float Lsum = 0.0f;
  float4 O = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
  for (int sp = 0; sp < SPLIT_MAX; ++sp) {
    if (sp < splits) {
      const float fct = ml[sp].x == -INFINITY ? 0.0f : exp2f(ml[sp].x - M);
      const float wl = ml[sp].y * fct;  // the split's weight: its sum of exp, rescaled
      Lsum += wl;
      O.x += half_lo(v[sp].x) * wl;
      O.y += half_hi(v[sp].x) * wl;
      O.z += half_lo(v[sp].y) * wl;
      O.w += half_hi(v[sp].y) * wl;
    }
  }
  const float sink = a.sink ? a.sink[head] : 0.0f;
  const float c = finish_scale(M * LN2, Lsum, sink, a.sink != nullptr);
  const int64_t off = (row * a.n_heads + head) * DIM + d0;
  const float r0 = O.x * c, r1 = O.y * c, r2 = O.z * c, r3 = O.w * c;
  if (a.out_dtype == CSA_F32) {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + off) = make_float4(r0, r1, r2, r3);
  } else {
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.out) + off) =
        make_uint2(f32x2_to_bf16x2_rne(r0, r1), f32x2_to_bf16x2_rne(r2, r3));
  }
  if (a.lse && d0 == 0) a.lse[row * a.n_heads + head] = Lsum > 0.0f ? (M + log2f(Lsum)) * LN2 : -INFINITY;
}

// Merge of one or two problems' split rows: 1-D grid placed by xcd_slot (items
// = record chunks), so a row is merged on the XCD that computed it.  A problem
// without splits has r = 0 rows to merge.
__global__ void __launch_bounds__(MERGE_CHUNK) attn_merge_pair_kernel(AttnArgs a0, int s0, int64_t r0, AttnArgs a1,
                                                                      int s1, int64_t r1, int chunks) {
  const XcdSlot w = xcd_slot(blockIdx.x, r0, chunks, r1, chunks);
  if (w.problem == 0) attn_merge_body(a0, s0, r0, w.row, w.item);
  else if (w.problem == 1) attn_merge_body(a1, s1, r1, w.row, w.item);
}

static bool use_mfma(int q_dtype, int kv_dtype, int n_heads) {
  return q_dtype == CSA_BF16 && kv_dtype == CSA_KV_MIXED && n_heads % 32 == 0 && n_heads <= 128 && n_heads > 0;
}

size_t attn_ws_bytes(int batch, int n_q, int n_heads, int64_t max_keys, int q_dtype, int kv_dtype) {
  if (!use_mfma(q_dtype, kv_dtype, n_heads)) return 0;
  const int64_t rows = (int64_t)batch * n_q;
  const MfmaSplit p = plan_split(n_q, n_heads, max_keys);
  if (p.splits == 1) return 0;
  return (size_t)partial_o_bytes(rows, p.splits, n_heads) + (size_t)rows * p.splits * n_heads * 2 * sizeof(float);
}

hipError_t launch_attention_xcd(const AttnArgs& a0, int64_t max_keys0, const AttnArgs& a1, int64_t max_keys1,
                                hipStream_t s);

hipError_t launch_attention(const AttnArgs& a, int64_t max_keys, hipStream_t s) {
  const int64_t rows = (int64_t)a.batch * a.n_q;
  if (rows == 0 || a.n_heads == 0) return hipSuccess;
  if (!use_mfma(a.q_dtype, a.kv_dtype, a.n_heads)) {
    dim3 grid(a.n_q, a.batch, (a.n_heads + VHG - 1) / VHG);
    hipLaunchKernelGGL(attn_valu_kernel, grid, dim3(DIM), 0, s, a);
    return hipGetLastError();
  }
  const MfmaSplit p = plan_split(a.n_q, a.n_heads, max_keys);
  if (p.splits > 1) {  // split rows: every work-group of a row, and its merge, on the row's XCD
    AttnArgs none = a;
    none.batch = 0;
    return launch_attention_xcd(a, max_keys, none, 0, s);
  }
  dim3 grid(1, a.n_q, a.batch);
  const int nw = a.n_heads / 32;
#define CSA_ATTN_LAUNCH(NW) \
  hipLaunchKernelGGL((attn_mfma_kernel<NW>), grid, dim3(64 * NW), 0, s, a, p.splits, p.keys_per_split)
  switch (nw) {
    case 1: CSA_ATTN_LAUNCH(1); break;
    case 2: CSA_ATTN_LAUNCH(2); break;
    case 3: CSA_ATTN_LAUNCH(3); break;
    default: CSA_ATTN_LAUNCH(4); break;
  }
#undef CSA_ATTN_LAUNCH
  return hipGetLastError();
}

hipError_t launch_attention_pair(const AttnArgs& a0, int64_t max_keys0, const AttnArgs& a1, int64_t max_keys1,
                                 hipStream_t s) {
  const int64_t rows0 = (int64_t)a0.batch * a0.n_q, rows1 = (int64_t)a1.batch * a1.n_q;
  const bool pair = rows0 > 0 && rows1 > 0 && a0.n_heads == a1.n_heads &&
                    use_mfma(a0.q_dtype, a0.kv_dtype, a0.n_heads) && use_mfma(a1.q_dtype, a1.kv_dtype, a1.n_heads);
  if (!pair) {
    hipError_t e = launch_attention(a0, max_keys0, s);
    return e != hipSuccess ? e : launch_attention(a1, max_keys1, s);
  }
  return launch_attention_xcd(a0, max_keys0, a1, max_keys1, s);
}

// One or two matrix-core problems (a1 may have no rows) with the XCD-aware
// placement of xcd_slot, then one merge of the split rows, placed alike.
hipError_t launch_attention_xcd(const AttnArgs& a0, int64_t max_keys0, const AttnArgs& a1, int64_t max_keys1,
                                hipStream_t s) {
  const int64_t rows0 = (int64_t)a0.batch * a0.n_q, rows1 = (int64_t)a1.batch * a1.n_q;
  const MfmaSplit p0 = plan_split(a0.n_q, a0.n_heads, max_keys0);
  const MfmaSplit p1 = plan_split(a1.n_q, a1.n_heads, max_keys1);
  const int64_t n = xcd_grid(rows0, p0.splits, rows1, p1.splits);
  if (n > 0x7fffffff) return hipErrorInvalidConfiguration;
  const int nw = a0.n_heads / 32;
  dim3 grid((unsigned)n);
#define CSA_ATTN_PAIR(NW)                                                                                          \
  hipLaunchKernelGGL((attn_mfma_pair_kernel<NW>), grid, dim3(64 * NW), 0, s, a0, p0.splits, p0.keys_per_split, a1, \
                     p1.splits, p1.keys_per_split)
  switch (nw) {
    case 1: CSA_ATTN_PAIR(1); break;
    case 2: CSA_ATTN_PAIR(2); break;
    case 3: CSA_ATTN_PAIR(3); break;
    default: CSA_ATTN_PAIR(4); break;
  }
#undef CSA_ATTN_PAIR
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t m0 = p0.splits > 1 ? rows0 : 0, m1 = p1.splits > 1 ? rows1 : 0;
  if (m0 + m1 == 0) return hipSuccess;
  const int ch = (a0.n_heads * (DIM / 4) + MERGE_CHUNK - 1) / MERGE_CHUNK;
  const int64_t nm = xcd_grid(m0, ch, m1, ch);
  if (nm > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(attn_merge_pair_kernel, dim3((unsigned)nm), dim3(MERGE_CHUNK), 0, s, a0, p0.splits, m0, a1,
                     p1.splits, m1, ch);
  return hipGetLastError();
}

}  // namespace csa
