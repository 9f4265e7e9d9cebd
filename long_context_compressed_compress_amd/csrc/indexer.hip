// Lightning Indexer: I[t,s] = sum_h w[t,h] * max(0, q[t,h,:] . k[s,:]) over the
// visible compressed entries (「论文解读｜DeepSeek-V4：百万 token 上下文的效率革命」,
// blog.tripbot.top, §3.1 第二步).  The MXFP4 path runs QK on the gfx950 scaled
// FP4 matrix cores and rounds the float32 score to BF16 (gitcode.csdn.net
// DeepSeek-V4 解读, 核心创新一 §1.4; austery.github.io notes, 全栈工程优化).
#include <hip/hip_ext.h>

#include "common.h"

namespace csa {

// ---------------------------------------------------------------------------
// FP32 path (vector ALU).  grid (ceil(n_cap/256), n_q, batch); one thread per entry.
// Summation order: d ascending inside a head, heads ascending.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) indexer_f32_kernel(const float* __restrict__ q, const float* __restrict__ w,
                                                          const float* __restrict__ k, int n_q, int n_heads, int d_idx,
                                                          int64_t n_cap, const int32_t* __restrict__ n_entries,
                                                          const int64_t* __restrict__ q_pos, int ratio,
                                                          float* __restrict__ scores) {
  extern __shared__ float sm[];
  float* qs = sm;                       // [n_heads][d_idx]
  float* ws = sm + n_heads * d_idx;     // [n_heads]
  const int b = blockIdx.z, t = blockIdx.y;
  const int64_t row = (int64_t)b * n_q + t;
  for (int p = threadIdx.x; p < n_heads * d_idx; p += 256) qs[p] = q[row * n_heads * d_idx + p];
  for (int p = threadIdx.x; p < n_heads; p += 256) ws[p] = w[row * n_heads + p];
  __syncthreads();
  const int64_t s = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (s >= n_cap) return;
  const int64_t nv = visible_entries(n_entries[b], q_pos[row], ratio, n_cap);
  float acc = -INFINITY;
  if (s < nv) {
    const float* kr = k + ((int64_t)b * n_cap + s) * d_idx;
    acc = 0.0f;
    for (int h = 0; h < n_heads; ++h) {
      float dot = 0.0f;
      for (int d = 0; d < d_idx; ++d) dot = fmaf(qs[h * d_idx + d], kr[d], dot);
      acc = fmaf(ws[h], fmaxf(dot, 0.0f), acc);
    }
  }
  scores[row * n_cap + s] = acc;
}

hipError_t launch_indexer_f32(const float* q, const float* w, const float* k, int batch, int n_q, int n_heads,
                              int d_idx, int64_t n_cap, const int32_t* n_entries, const int64_t* q_pos, int ratio,
                              float* scores, hipStream_t s) {
  if (batch == 0 || n_q == 0 || n_cap == 0) return hipSuccess;
  dim3 grid((unsigned)((n_cap + 255) / 256), n_q, batch);
  const size_t smem = sizeof(float) * ((size_t)n_heads * d_idx + n_heads);
  hipLaunchKernelGGL(indexer_f32_kernel, grid, dim3(256), smem, s, q, w, k, n_q, n_heads, d_idx, n_cap, n_entries,
                     q_pos, ratio, scores);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// MXFP4 path on v_mfma_scale_f32_32x32x64_f8f6f4 (both operands E2M1, one E8M0
// scale per lane and 32-element K block).
//   A = q rows (32 heads of one query) x K = 64 index dims
//   B = K x 32 entries                       -> C[head][entry], 16 heads per lane
// A lane holds row (lane % 32) and the 32-element block (lane / 32) of a 64-wide
// K step: bytes [16*(lane/32), +16) of the packed row, and that block's scale.
// Output lane layout (32x32 tiles): column = lane % 32, rows
// 8*(r/4) + 4*(lane/32) + r%4 for r = 0..15.
// Epilogue per lane: sum over its 16 heads of w_h * ReLU(c), then the partner
// lane (lane ^ 32) holding the other heads of the same entry is added.
//
// grid (n_chunks, n_q * batch); block 256 = 4 waves.  Wave wv of a block takes
// the wv-th contiguous quarter of the chunk's 32-entry blocks.  Each wave runs a
// software pipeline P blocks deep: the key rows of block j+P are requested right
// after block j's products are issued, so HBM latency hides behind the
// ReLU/weight epilogue.  Blocks past the last visible entry are not read; their
// scores are written as -inf.
// ---------------------------------------------------------------------------
// max(x, 0) as one integer max on the bit pattern: non-negative floats order
// like their bits as signed integers and every negative float (and -0) is a
// negative integer.  fmaxf costs a second instruction to quiet signalling NaNs.
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// VGPRs per lane besides the pipeline (an estimate calibrated on the compiled
// kernels): query fragments, two result tiles, weight reads and addressing.
// Each pipeline stage adds 5 VGPRs per 64-wide K step.
constexpr int idx_fixed_vgprs(int nt, int ks) { return 4 * nt * ks + 16 * nt + 64; }
// 4 waves per SIMD (128 VGPRs) when a two-block pipeline fits, else 2.
constexpr int idx_waves_per_simd(int nt, int ks) { return idx_fixed_vgprs(nt, ks) + 20 * ks <= 128 ? 4 : 2; }
// Work-groups per launch when rows allow: 4 per CU, all of equal work, so that
// no CU carries a fifth of the chip's load more than another.
constexpr int IDX_WG_TARGET = 1024;
// Pipeline depth in 32-entry blocks (even: scores are stored two blocks at a
// time).  Two: the other waves of the SIMD hide the key rows' latency, and a
// deeper ring pushed the 64-head kernel against its 128-register budget
// (measured: depth 4 with the top-k histogram staging spilled and ran slower).
constexpr int IDX_DEPTH = 2;

// Fused top-k, first pass: every stored visible score's order-preserving key
// is binned by its high byte as it is stored (one LDS add per distinct value
// across the wave: decode scores of 64 entries take one to three values), and
// at the end the work-group adds its bins to the row totals tot[0..255];
// work-group 0 of the row clears the second pass's totals tot[256..511].

template <int NT, int KS, bool QF>  // NT = n_heads / 32, KS = d_idx / 64
__global__ void __launch_bounds__(256, idx_waves_per_simd(NT, KS)) indexer_mx_kernel(const void* __restrict__ qv, const uint8_t* __restrict__ qs,
                                                            const float* __restrict__ w, const uint8_t* __restrict__ k,
                                                            const uint8_t* __restrict__ ks, int n_q, int64_t n_cap,
                                                            const int32_t* __restrict__ n_entries,
                                                            const int64_t* __restrict__ q_pos, int ratio,
                                                            uint16_t* __restrict__ scores, int chunk_blocks,
                                                            uint32_t* __restrict__ hist, int hist_row_words,
                                                            EntryPages pg) {
  constexpr int H = 32 * NT;
  constexpr int D = 64 * KS;
  constexpr int RB = D / 2;    // packed bytes per row
  constexpr int SB = D / 32;   // scale bytes per row
  constexpr int P = IDX_DEPTH;  // pipeline depth in 32-entry blocks
  const int row = blockIdx.y;  // b * n_q + t
  const int b = row / n_q;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5, col = lane & 31;
  // The query's position and entry count are requested first and used only
  // after the key rows and query fragments have been requested (below).
  const int64_t t_pos = q_pos[row];
  const int32_t n_ent = n_entries[b];

  // Wave wv takes the contiguous quarter [wb0, wb1) of the chunk (chunk_blocks
  // is a multiple of 8, so every quarter starts on an even block).
  const int64_t n_blk = (n_cap + 31) / 32;
  const int64_t b0 = (int64_t)blockIdx.x * chunk_blocks;
  // The row's last chunk also takes the blocks past the last whole chunk (its
  // last wave does them).
  const int64_t b1 = blockIdx.x == gridDim.x - 1 ? n_blk : min(b0 + chunk_blocks, n_blk);
  const int64_t wb0 = b0 + (int64_t)wv * (chunk_blocks / 4);
  const int64_t wb1 = wv == 3 ? b1 : min(wb0 + chunk_blocks / 4, b1);
  // Set once the position is back (after the prologue): visible entries, the
  // wave's visible blocks, and its first n_full blocks, whose 32 entries are
  // all visible (so below n_cap too): their loads and stores need no bounds.
  int64_t nv = 0, bvis = 0;
  int nj = 0, n_full = 0;
  const uint8_t* kb = k + (int64_t)b * n_cap * RB;
  const uint8_t* ksb = ks + (int64_t)b * n_cap * SB;
  uint16_t* out = scores + (int64_t)row * n_cap;
  // Codes and scales of the 32-entry block starting at entry e0 (a multiple of
  // 32).  Paged keys: a page holds a power of two >= 32 entries, so the block
  // is 32 consecutive rows of one page.
  auto block_rows = [&](int64_t e0, const uint8_t*& kp, const uint8_t*& sp) {
    if (pg.pages) {
      const int64_t r = entry_row(pg, n_cap, b, e0);
      kp = k + r * RB;
      sp = ks + r * SB;
    } else {
      kp = kb + e0 * RB;
      sp = ksb + e0 * SB;
    }
  };

  v8i A[NT][KS];
  int As[NT][KS];
  __shared__ __attribute__((aligned(16))) float wl[H];
  __shared__ uint32_t hl[256];          // top-k first-pass bins (with `hist`)
  if (hist) hl[threadIdx.x] = 0u;       // published by the barrier before the scoring loop
  // Prefetches past the wave's last visible block re-read that block (a cache
  // hit), so every stage issues its loads unconditionally and the ring of key
  // registers needs no loop-carried copies.
  v4i Bv[P][KS];
  int Bs[P][KS];
  auto load = [&](v4i (&bv)[KS], int (&bs)[KS], int j) {
    j = min(j, nj - 1);
    const int64_t e0 = nj > 0 ? (wb0 + j) * 32 : 0;  // first entry of the block (wave-uniform)
    const uint8_t *kp, *sp;
    block_rows(e0, kp, sp);
    unsigned e = (unsigned)col;
    if (j >= n_full) {  // wave-uniform: a block that may reach past n_cap
      const int64_t left = n_cap - 1 - e0;
      const int lim = left < 31 ? (int)left : 31;
      e = (unsigned)(col < lim ? col : lim);  // rows past n_cap re-read the last row
    }
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      bv[kk] = *reinterpret_cast<const v4i*>(kp + (e * RB + 32 * kk + 16 * g));
      bs[kk] = sp[e * SB + 2 * kk + g];
    }
  };
  // Products of one head tile, then the ReLU/weight epilogue of the previous
  // tile while the next tile's products run (two result tiles live at a time).
  auto mma = [&](const v4i (&bv)[KS], const int (&bs)[KS], int th) {
    v16f c = {};
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const v8i b8 = v8i{bv[kk].x, bv[kk].y, bv[kk].z, bv[kk].w, 0, 0, 0, 0};
      c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A[th][kk], b8, c, 4, 4, 0, As[th][kk], 0, bs[kk]);
    }
    return c;
  };
  // Score of entry col of the block in every lane (lanes l and l^32 agree).
  auto block = [&](v4i (&bv)[KS], int (&bs)[KS], bool refill, int j_next) {
    float acc = 0.0f;
    v16f c = mma(bv, bs, 0);
#pragma unroll
    for (int th = 0; th < NT; ++th) {
      v16f cn;
      if (th + 1 < NT) cn = mma(bv, bs, th + 1);
      if (th + 1 == NT && refill) load(bv, bs, j_next);
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 wq = *reinterpret_cast<const float4*>(&wl[32 * th + 8 * q4 + 4 * g]);
        acc = fmaf(wq.x, relu(c[4 * q4]), acc);
        acc = fmaf(wq.y, relu(c[4 * q4 + 1]), acc);
        acc = fmaf(wq.z, relu(c[4 * q4 + 2]), acc);
        acc = fmaf(wq.w, relu(c[4 * q4 + 3]), acc);
      }
      if (th + 1 < NT) c = cn;
    }
    // lanes l and l^32 hold the two halves of the heads of entry l%32
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc), __float_as_uint(acc), false, false);
    return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  };
  // Scores are written two blocks at a time, 64 entries = one 128-byte line:
  // lane l writes entry e0 + l (block j0 in lanes 0..31, block j0+1 in 32..63).
  auto bin_scores = [&](uint32_t bits, bool stored) {  // top-k's first pass (see above)
    const uint32_t key = bf16_key(bits);
    const uint32_t bin = key >> 8;
    uint64_t rem = __ballot(stored && key != INVALID);
    while (rem) {  // wave-uniform
      const int leader = __builtin_ctzll(rem);
      const uint32_t lb = (uint32_t)__builtin_amdgcn_readlane((int)bin, leader);
      const uint64_t m = __ballot(bin == lb) & rem;
      if (lane == leader) atomicAdd(&hl[lb], (uint32_t)__builtin_popcountll(m));
      rem &= ~m;
    }
  };
  auto store = [&](int j0, float s_lo, float s_hi, bool pair) {
    const int64_t e0 = (wb0 + j0) * 32;  // wave-uniform, as are the two bounds below
    const float v = g == 0 ? s_lo : s_hi;
    if (pair && j0 + 1 < n_full) {  // wave-uniform: 64 visible entries
      const uint32_t bits = f32_to_bf16_rne(v);  // hardware RNE; scores are never NaN
      out[e0 + lane] = (uint16_t)bits;
      if (hist) bin_scores(bits, true);
      return;
    }
    const int64_t dv = nv - e0, dc = n_cap - e0;
    const int n_vis64 = dv < 0 ? 0 : (dv > 64 ? 64 : (int)dv);
    const int n_cap64 = dc < 0 ? 0 : (dc > 64 ? 64 : (int)dc);
    const uint32_t bits = f32_to_bf16_rne(lane < n_vis64 ? v : -INFINITY);
    if ((pair || g == 0) && lane < n_cap64) out[e0 + lane] = (uint16_t)bits;
    if (hist) bin_scores(bits, (pair || g == 0) && lane < n_vis64);
  };
  // Float32 query: each thread's first block is requested before the key rows
  // (vector-memory waits count in issue order, so waiting for the query then
  // leaves the key rows in flight).
  constexpr int NB = H * SB;  // MXFP4 blocks of the query row
  float qv0[MXB];
  const float wt = threadIdx.x < H ? w[(int64_t)row * H + threadIdx.x] : 0.0f;
  if constexpr (QF) {
    if (threadIdx.x < NB) {
      const float4* src = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(qv) +
                                                          ((int64_t)row * H * D + (int64_t)threadIdx.x * MXB));
#pragma unroll
      for (int i = 0; i < MXB / 4; ++i) {
        const float4 t = src[i];
        qv0[4 * i] = t.x; qv0[4 * i + 1] = t.y; qv0[4 * i + 2] = t.z; qv0[4 * i + 3] = t.w;
      }
    }
  }
  // The first P blocks of the wave's range are requested before the query
  // fragments are built and before the query's position is back (their
  // addresses do not depend on it; blocks that turn out invisible are simply
  // not used), so their latency overlaps the query's loads (and quantization).
  // Unconditional: a branch here would make every later wait assume nothing
  // is in flight.
  {
    const int nb = wb1 > wb0 ? (int)(wb1 - wb0) : 0;
#pragma unroll
    for (int u = 0; u < P; ++u) {
      const int j = min(u, nb - 1);
      const int64_t e0 = nb > 0 ? (wb0 + j) * 32 : 0;
      const int64_t left = n_cap - 1 - e0;
      const int lim = left < 31 ? (int)left : 31;
      const unsigned e = (unsigned)(col < lim ? col : lim);
      const uint8_t *kp, *sp;
      block_rows(e0, kp, sp);
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        Bv[u][kk] = *reinterpret_cast<const v4i*>(kp + (e * RB + 32 * kk + 16 * g));
        Bs[u][kk] = sp[e * SB + 2 * kk + g];
      }
      __builtin_amdgcn_sched_barrier(0);  // keep the stages' loads in order
    }
  }
  if constexpr (QF) {
    // The work-group quantizes the query row once: thread t encodes blocks
    // t, t+256, ... (block b = 32 values of head b / SB) into LDS.
    __shared__ v4i qcodes[NB];
    __shared__ int qscale[NB];
    for (int bk = threadIdx.x; bk < NB; bk += 256) {
      float v[MXB];
      if (bk == (int)threadIdx.x) {
#pragma unroll
        for (int i = 0; i < MXB; ++i) v[i] = qv0[i];
      } else {
        const float4* src = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(qv) +
                                                            ((int64_t)row * H * D + (int64_t)bk * MXB));
#pragma unroll
        for (int i = 0; i < MXB / 4; ++i) {
          const float4 t = src[i];
          v[4 * i] = t.x; v[4 * i + 1] = t.y; v[4 * i + 2] = t.z; v[4 * i + 3] = t.w;
        }
      }
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < MXB; ++i) amax = fmaxf(amax, fabsf(v[i]));
      const int e = mx_scale_exp(amax);
      uint32_t c[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < MXB; ++i) c[i / 8] |= e2m1_code(ldexpf(v[i], -e)) << (4 * (i % 8));
      qcodes[bk] = v4i{(int)c[0], (int)c[1], (int)c[2], (int)c[3]};
      qscale[bk] = e + 127;
    }
    if (threadIdx.x < H) wl[threadIdx.x] = wt;
    // LDS-only barrier: the key rows already requested stay in flight
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
#pragma unroll
    for (int th = 0; th < NT; ++th)
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const int bk = (32 * th + col) * SB + 2 * kk + g;  // block 2kk+g of head 32th+col
        const v4i a = qcodes[bk];
        A[th][kk] = v8i{a.x, a.y, a.z, a.w, 0, 0, 0, 0};
        As[th][kk] = qscale[bk];
      }
  } else {
    const uint8_t* q = reinterpret_cast<const uint8_t*>(qv);
#pragma unroll
    for (int th = 0; th < NT; ++th) {
      const int64_t qrow = (int64_t)row * H + 32 * th + col;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const v4i a = *reinterpret_cast<const v4i*>(q + qrow * RB + 32 * kk + 16 * g);
        A[th][kk] = v8i{a.x, a.y, a.z, a.w, 0, 0, 0, 0};
        As[th][kk] = qs[qrow * SB + 2 * kk + g];
      }
    }
  }
  if constexpr (!QF) {
    if (threadIdx.x < H) wl[threadIdx.x] = wt;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  }

  __builtin_amdgcn_sched_barrier(0);  // the requests above go out before the position is needed
  nv = visible_entries(n_ent, t_pos, ratio, n_cap);
  bvis = min(b1, (nv + 31) / 32);  // blocks below bvis hold a visible entry
  nj = wb0 < bvis ? (int)(min(wb1, bvis) - wb0) : 0;
  {
    const int64_t fv = nv / 32 - wb0;
    n_full = fv <= 0 ? 0 : (fv >= nj ? nj : (int)fv);
  }

  if (nj > 0) {
    float pend = 0.0f;  // score of the even block awaiting its odd partner
    int j0 = 0;
    for (; j0 + P <= nj; j0 += P) {
#pragma unroll
      for (int u = 0; u < P; ++u) {  // P is even: j0 + u has the parity of u
        const float sc = block(Bv[u], Bs[u], true, j0 + u + P);
        if (u & 1) store(j0 + u - 1, pend, sc, true);
        else pend = sc;
      }
    }
#pragma unroll
    for (int u = 0; u < P - 1; ++u) {
      if (j0 + u < nj) {  // wave-uniform
        // reloaded rather than taken from the loop's prefetch ring, so no key
        // register has to live across the loop (the tail is at most P-1 blocks)
        v4i tb[KS];
        int ts[KS];
        load(tb, ts, j0 + u);
        const float sc = block(tb, ts, false, 0);
        if (u & 1) store(j0 + u - 1, pend, sc, true);
        else pend = sc;
      }
    }
    if (nj & 1) store(nj - 1, pend, pend, false);  // the last block has no partner
  }
  // Blocks with no visible entry.
  const uint16_t ninf = (uint16_t)f32_to_bf16_rne(-INFINITY);
  for (int64_t bi = max(wb0, bvis); bi < wb1; ++bi) {
    const int64_t n = bi * 32 + col;
    if (g == 0 && n < n_cap) out[n] = ninf;
  }
  if (hist) {  // the work-group's bins into the row totals; work-group 0 clears the second pass's
    const int tid = wv * 64 + lane;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();  // LDS only: the score stores stay in flight
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    uint32_t* tot = hist + (int64_t)row * hist_row_words;
    const uint32_t t = hl[tid];
    if (t) atomicAdd(&tot[tid], t);
    if (blockIdx.x == 0) tot[256 + tid] = 0u;
  }
}

hipError_t launch_indexer_mxfp4(const void* q, bool q_f32, const uint8_t* q_scales, const float* w, const uint8_t* k,
                                const uint8_t* k_scales, int batch, int n_q, int n_heads, int d_idx, int64_t n_cap,
                                const int32_t* n_entries, const int64_t* q_pos, int ratio, uint16_t* scores,
                                hipStream_t s, uint32_t* hist, int hist_row_words, hipEvent_t ev_start,
                                hipEvent_t ev_stop, EntryPages pg) {
  if (batch == 0 || n_q == 0 || n_cap == 0) return hipSuccess;
  const int64_t rows = (int64_t)batch * n_q;
  const int64_t n_blk = (n_cap + 31) / 32;
  // Equal work-groups, IDX_WG_TARGET of them over the chip when rows allow:
  // chunk = the row's blocks over its share of work-groups, a multiple of 8
  // (four even quarters) and at least 16 blocks (so each wave's pipeline runs
  // a few stages); the last chunk of a row also takes the blocks past the last
  // whole chunk (fewer than a chunk more).
  const int64_t per_row = rows >= IDX_WG_TARGET ? 1 : IDX_WG_TARGET / rows;
  int64_t chunk = n_blk / per_row / 8 * 8;
  if (chunk < 16) chunk = 16;
  if (chunk > n_blk) chunk = n_blk;
  const int64_t n_chunks = n_blk / chunk;
  if (n_chunks > 0x7fffffff || rows > 65535) return hipErrorInvalidConfiguration;
  dim3 grid((unsigned)n_chunks, (unsigned)rows);
  // with events, the dispatch itself records them at the kernel's start and end
#define CSA_IDX_LAUNCH(NT, KS)                                                                                     \
  if (q_f32)                                                                                                         \
    hipExtLaunchKernelGGL((indexer_mx_kernel<NT, KS, true>), grid, dim3(256), 0, s, ev_start, ev_stop, 0, q,         \
                          q_scales, w, k, k_scales, n_q, n_cap, n_entries, q_pos, ratio, scores, (int)chunk, hist,  \
                          hist_row_words, pg);                                                                       \
  else                                                                                                               \
    hipExtLaunchKernelGGL((indexer_mx_kernel<NT, KS, false>), grid, dim3(256), 0, s, ev_start, ev_stop, 0, q,        \
                          q_scales, w, k, k_scales, n_q, n_cap, n_entries, q_pos, ratio, scores, (int)chunk, hist,  \
                          hist_row_words, pg)
  const int nt = n_heads / 32, kss = d_idx / 64;
  switch (nt * 8 + kss) {
    case 8 + 1: CSA_IDX_LAUNCH(1, 1); break;
    case 8 + 2: CSA_IDX_LAUNCH(1, 2); break;
    case 8 + 4: CSA_IDX_LAUNCH(1, 4); break;
    case 16 + 1: CSA_IDX_LAUNCH(2, 1); break;
    case 16 + 2: CSA_IDX_LAUNCH(2, 2); break;
    case 16 + 4: CSA_IDX_LAUNCH(2, 4); break;
    case 24 + 1: CSA_IDX_LAUNCH(3, 1); break;
    case 24 + 2: CSA_IDX_LAUNCH(3, 2); break;
    case 24 + 4: CSA_IDX_LAUNCH(3, 4); break;
    case 32 + 1: CSA_IDX_LAUNCH(4, 1); break;
    case 32 + 2: CSA_IDX_LAUNCH(4, 2); break;
    case 32 + 4: CSA_IDX_LAUNCH(4, 4); break;
    default: return hipErrorInvalidValue;
  }
#undef CSA_IDX_LAUNCH
  return hipGetLastError();
}

}  // namespace csa
