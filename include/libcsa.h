/*
 * libcsa — CSA + HCA compressed attention (the DeepSeek-V4 hybrid long-context
 * attention) for AMD MI355X (gfx950 / CDNA4).
 *
 * The method (as the web pages summarising the DeepSeek-V4 report describe it;
 * the bracketed tags are how the comments below cite them):
 *   [TRIPBOT] 「论文解读｜DeepSeek-V4：百万 token 上下文的效率革命」(blog.tripbot.top):
 *       §3.1 + Figure 3  CSA: compress every m=4 tokens, Lightning Indexer, top-k
 *       §3.2             HCA: compress every m'=128 tokens, dense attention
 *       §3.3             128-token sliding-window branch, learnable attention sink
 *   [CSDN] gitcode.csdn.net DeepSeek-V4 解读, 核心创新一:
 *       §1.1 工程细节     overlapped compression (C^a current block + C^b previous block)
 *       §1.4              KV storage: RoPE dims BF16, other dims FP8; indexer QK in
 *                         FP4, index scores FP32 -> BF16
 *   [AUSTERY] austery.github.io DeepSeek-V4 notes, 全栈工程优化: the indexer QK path
 *       is MXFP4; the inference framework keeps a heterogeneous KV cache for the
 *       hybrid attention
 *   [YANBAOKE] 研报客「DeepSeek-V4 详细总结」(pc.yanbaoke.cn), §5 训练与推理优化:
 *       heterogeneous KV cache structure
 *
 * Conventions for every call
 * --------------------------
 *  - Every tensor pointer is a DEVICE pointer; small per-sequence arrays
 *    (n_entries, q_pos) are device arrays too.  The caller allocates and owns
 *    all memory, including workspaces sized by the *_workspace_size calls.
 *    The library allocates no device memory and keeps no state between calls
 *    apart from an immutable per-device property cache and the fixed-size
 *    device array that topk_select_noalloc uses as its workspace.
 *  - Calls are asynchronous, ordered on `stream` (a hipStream_t; NULL = the
 *    default stream).  Buffers must stay alive until the stream reaches the call.
 *  - Arguments are validated on the host before anything is enqueued.  A call
 *    that returns a status other than CSA_OK or CSA_ERR_HIP has enqueued
 *    nothing and written nothing; after CSA_ERR_HIP, kernels launched before
 *    the failing one may have run.
 *    No exception crosses this boundary; there are no device-side asserts.
 *  - Data-dependent conditions are defined, not errors: a selected index that
 *    is < 0 or not visible is skipped (so -1 padding is legal); a query with no
 *    visible entry still attends to its window.
 *  - Results are deterministic and independent of batch composition: the same
 *    inputs give the same bits, run alone or inside a larger batch.
 *  - Threads: every call may be made concurrently from several host threads.
 *  - Tensors are plain pointers with explicit sizes (batch, rows, capacities)
 *    and a dtype code where a call accepts more than one element type; every
 *    tensor is dense and row-major in the shape its call lists (no strides).
 *  - A top-k selection is a set: its indices come in ascending index order
 *    (not score order), padded with -1 when fewer than k entries are visible.
 *
 * Fixed geometry
 * --------------
 *  A KV row (raw token or compressed entry) has CSA_DIM = 192 values: dims
 *  [0,128) carry no position, dims [128,192) are the RoPE dims.  Row formats:
 *    CSA_F32       192 x float32                       (768 bytes)
 *    CSA_BF16      192 x bfloat16                      (384 bytes)
 *    CSA_KV_MIXED  bytes [0,128): dims 0..127 as FP8 E4M3 (OCP e4m3fn: bias 7,
 *                  max 448, no inf; round to nearest even, saturating);
 *                  bytes [128,256): dims 128..191 as BF16 (RNE), little-endian
 *                                                      (256 bytes)
 *  MXFP4 tensors come as two arrays: E2M1 codes packed two per byte (the even
 *  element in the low nibble, sign in bit 3 of each nibble), and one E8M0
 *  scale byte (2^(byte-127)) per 32 consecutive elements along the last axis.
 *  Scale rule (OCP MX v1.0): e = floor(log2(max|v|)) - 2 clamped to
 *  [-127,127], all-zero block -> e = -127; codes = E2M1 RNE of v / 2^e,
 *  saturating at +-6.
 *
 * Positions and ring buffers
 * --------------------------
 *  Raw-token buffers (compressor input, sliding window) are rings: token at
 *  absolute position p lives in row (p - base) mod rows of its sequence's
 *  slice; positions below `base` are absent.  A plain contiguous buffer of
 *  positions [base, base+rows) is the special case with no wrap-around.
 *  A compressed entry i of ratio m is visible to a query at position t iff its
 *  last token m*i+m-1 <= t and i < n_entries[b]:
 *      n_vis(b,t) = min(n_entries[b], (t+1)/m).
 *  The sliding window of a query at t is tokens max(0,t-W+1) .. t inclusive.
 */
#ifndef LIBCSA_H
#define LIBCSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum csa_status {
  CSA_OK = 0,
  CSA_ERR_NULL = 1,        /* a required pointer is NULL                                */
  CSA_ERR_SHAPE = 2,       /* a size is out of range or inconsistent                    */
  CSA_ERR_DTYPE = 3,       /* unsupported dtype or dtype combination                    */
  CSA_ERR_ALIGN = 4,       /* pointer or stride not 16-byte aligned                     */
  CSA_ERR_RANGE = 5,       /* requested tokens/entries lie outside the supplied buffers */
  CSA_ERR_WORKSPACE = 6,   /* workspace missing or smaller than *_workspace_size        */
  CSA_ERR_UNSUPPORTED = 7, /* valid request this library does not implement             */
  CSA_ERR_HIP = 8,         /* the HIP runtime reported an error (see csa_last_hip_error) */
  CSA_ERR_IO = 9,          /* a snapshot file could not be opened, read or written      */
  CSA_ERR_FORMAT = 10      /* a snapshot file is not one, is truncated or damaged, or
                              does not fit the cache it is loaded into                  */
};

enum csa_dtype { CSA_F32 = 0, CSA_BF16 = 1, CSA_KV_MIXED = 2, CSA_MXFP4 = 3 };

#define CSA_DIM 192
#define CSA_DIM_NOPE 128
#define CSA_DIM_ROPE 64
#define CSA_MIXED_ROW_BYTES 256
#define CSA_MX_BLOCK 32

/* Human-readable name of a status code (static string, never NULL). */
const char* csa_status_string(int status);

/* hipError_t of the last CSA_ERR_HIP returned on the calling thread (0 if none). */
int csa_last_hip_error(void);

/*
 * kv_pack — convert KV rows between storage formats ([CSDN] 核心创新一 §1.4:
 * RoPE dims BF16, other dims FP8).
 *   x        [n_rows] rows of 192 values, dtype x_dtype (CSA_F32 | CSA_BF16);
 *            row r starts at element r * x_row_stride.
 *   out      [n_rows] rows in out_dtype (CSA_F32 | CSA_BF16 | CSA_KV_MIXED);
 *            row r starts at byte r * out_row_stride.
 *   Strides and both base pointers must be 16-byte aligned.  Used for the
 *   window append at decode (out_row_stride = ring_rows * row bytes) and to
 *   store raw tokens.  Rounding: RNE; FP8 saturates at +-448.
 */
int kv_pack(const void* x, int32_t x_dtype, int64_t n_rows, int64_t x_row_stride,
            void* out, int32_t out_dtype, int64_t out_row_stride, void* stream);

/*
 * kv_append — decode-time append of every sequence's newest token to its rings,
 * in one launch ([TRIPBOT] §3.3: the sliding window of the last raw tokens;
 * [CSDN] 核心创新一 §1.4: stored rows FP8 + BF16).  For b < batch, with
 * p = pos[b]:
 *   raw_ring[b, (p - raw_base) mod raw_rows] = x[b] in raw_dtype
 *       (CSA_F32 | CSA_BF16: the raw tokens the compressors read),
 *   win_ring[b, (p - win_base) mod win_rows] = x[b] in win_dtype
 *       (CSA_F32 | CSA_BF16 | CSA_KV_MIXED: the stored window row),
 * both rounded exactly as kv_pack does.  A sequence with p < base skips that
 * ring.  Either ring may be NULL (not written).
 *   x   [batch, 192] contiguous rows, x_dtype CSA_F32 | CSA_BF16
 *   pos [batch] int64, device memory (read by the kernel, so the call can be
 *       replayed unchanged from step to step)
 *   rings [batch, rows] rows of their row bytes; base pointers 16-byte aligned.
 * Errors: CSA_ERR_DTYPE, CSA_ERR_SHAPE (batch < 0, rows < 1 for a given ring),
 * CSA_ERR_NULL (x or pos NULL), CSA_ERR_ALIGN.
 */
int kv_append(const void* x, int32_t x_dtype, int32_t batch, const int64_t* pos, void* raw_ring,
              int32_t raw_dtype, int64_t raw_rows, int64_t raw_base, void* win_ring, int32_t win_dtype,
              int64_t win_rows, int64_t win_base, void* stream);

/*
 * mxfp4_quantize — MXFP4 block quantisation of float32 rows ([AUSTERY]
 * 全栈工程优化: indexer QK path in MXFP4; [CSDN] §1.4).
 *   x [n_rows, d] float32 contiguous, d a multiple of 32;
 *   codes [n_rows, d/2] bytes; scales [n_rows, d/32] bytes.
 */
int mxfp4_quantize(const float* x, int64_t n_rows, int32_t d, uint8_t* codes, uint8_t* scales,
                   void* stream);

/*
 * csa_compress — CSA compressor ([TRIPBOT] §3.1 第一步 + Figure 3; [CSDN] §1.1 工程细节).
 * Entry i pools the 8 raw tokens 4(i-1) .. 4i+3: slots 0..3 are the previous
 * block C^b, slots 4..7 the entry's own block C^a.  Per channel c:
 *     z[s,c] = sum_d x_{j(s)}[d] * w_gate[d,c] + pos_bias[s,c]
 *     C_i[c] = sum_s softmax_s(z[.,c])[s] * x_{j(s)}[c]
 * over the slots whose token exists (j >= 0: entry 0 pools its own block only).
 *   x_raw      [batch, raw_rows, 192] raw token ring (CSA_F32 | CSA_BF16), base raw_base
 *   w_gate     [192, 192] float32 row-major (d, c);  pos_bias [8, 192] float32
 *   entries entry_begin .. entry_begin+n_new-1 are written to
 *   kv_out     [batch, n_cap] rows of kv_dtype (CSA_F32 | CSA_BF16 | CSA_KV_MIXED)
 *   Optional indexer key (all three NULL/0 to skip): k_i = C_i @ w_idx with
 *   w_idx [192, d_idx] float32, written to key_out [batch, n_cap, d_idx] as
 *   key_dtype CSA_F32, or CSA_MXFP4 (key_out = codes [batch, n_cap, d_idx/2],
 *   key_scales = [batch, n_cap, d_idx/32]).
 *   Pooling and the key projection run in float32; the entry is rounded to
 *   kv_dtype once at the end.
 *   CSA_ERR_RANGE if a needed token precedes raw_base or the needed tokens do
 *   not fit in raw_rows, or entry_begin + n_new > n_cap.
 */
int csa_compress(const void* x_raw, int32_t x_dtype, int32_t batch, int64_t raw_rows,
                 int64_t raw_base, const float* w_gate, const float* pos_bias,
                 int64_t entry_begin, int32_t n_new, void* kv_out, int32_t kv_dtype,
                 int64_t n_cap, const float* w_idx, int32_t d_idx, void* key_out,
                 uint8_t* key_scales, int32_t key_dtype, void* stream);

/*
 * hca_compress — HCA compressor ([TRIPBOT] §3.2; [CSDN] 核心创新一 §1.2).
 * Entry i pools tokens 128i .. 128i+127 (no overlap) with the same
 * softmax-gated rule; pos_bias is [128, 192].  Other arguments as csa_compress.
 */
int hca_compress(const void* x_raw, int32_t x_dtype, int32_t batch, int64_t raw_rows,
                 int64_t raw_base, const float* w_gate, const float* pos_bias,
                 int64_t entry_begin, int32_t n_new, void* kv_out, int32_t kv_dtype,
                 int64_t n_cap, void* stream);

/*
 * indexer_score — Lightning Indexer ([TRIPBOT] §3.1 第二步; [CSDN] §1.4).
 *   I[b,t,s] = sum_h w[b,t,h] * max(0, q[b,t,h,:] . k[b,s,:])   for s < n_vis(b,t)
 *   I[b,t,s] = -inf                                             for n_vis <= s < n_cap
 * One key per entry, shared by all heads.
 *   FP32 path : q_dtype = k_dtype = CSA_F32, score_dtype = CSA_F32.
 *               q [batch, n_q, n_heads, d_idx], k [batch, n_cap, d_idx] float32;
 *               q_scales, k_scales NULL.  Accumulation in float32.
 *   MXFP4 path: q_dtype = k_dtype = CSA_MXFP4, score_dtype = CSA_BF16.
 *               q codes [batch, n_q, n_heads, d_idx/2] + scales [.., d_idx/32];
 *               k codes [batch, n_cap, d_idx/2] + scales [batch, n_cap, d_idx/32];
 *               products exact, sums in float32 (matrix cores), then RNE to BF16.
 *               Needs n_heads % 32 == 0 (<= 128) and d_idx % 64 == 0 (<= 256).
 *               q_dtype = CSA_F32 with k_dtype = CSA_MXFP4: q float32
 *               [batch, n_q, n_heads, d_idx] (16-byte aligned) is quantized to
 *               MXFP4 inside the call exactly as mxfp4_quantize would (q_scales
 *               NULL), then scored as above.
 *   w [batch, n_q, n_heads] float32 (any sign); n_entries [batch] int32;
 *   q_pos [batch, n_q] int64; ratio = m of the compressor (4 for CSA).
 *   scores [batch, n_q, n_cap] of score_dtype.
 */
int indexer_score(const void* q, const uint8_t* q_scales, int32_t q_dtype, const float* w,
                  const void* k, const uint8_t* k_scales, int32_t k_dtype, int32_t batch,
                  int32_t n_q, int32_t n_heads, int32_t d_idx, int64_t n_cap,
                  const int32_t* n_entries, const int64_t* q_pos, int32_t ratio, void* scores,
                  int32_t score_dtype, void* stream);

/*
 * topk_select — per-query top-k ([TRIPBOT] §3.1 第二步: k = 1024 for V4-Pro,
 * 512 for V4-Flash).  Among the visible entries s < n_vis(b,t) whose score is
 * not -inf, keep the k with the largest score, ties going to the lower index.
 * idx_out [batch, n_q, k] int32 receives the chosen indices in ascending index
 * order, followed by -1 when fewer than k qualify.  Scores (score_dtype
 * CSA_BF16 or CSA_F32, never NaN) are compared exactly as numbers, so -0 and
 * +0 tie.
 * Workspace: at least topk_workspace_size(...) bytes, 16-byte aligned, and
 * zero-filled before its first use; every call that returns CSA_OK leaves the
 * part that must start at zero (per-row histogram totals) at zero again, so
 * one zeroing at allocation suffices, also when the workspace is reused for
 * other shapes.  Calls sharing a workspace must not overlap.
 * Few long BF16 rows (decode) are split over several work-groups per row;
 * the result is exact either way.
 */
size_t topk_workspace_size(int32_t batch, int32_t n_q, int64_t n_cap, int32_t k,
                           int32_t score_dtype);
int topk_select(const void* scores, int32_t score_dtype, int32_t batch, int32_t n_q,
                int64_t n_cap, const int32_t* n_entries, const int64_t* q_pos, int32_t ratio,
                int32_t k, int32_t* idx_out, void* workspace, size_t ws_bytes, void* stream);

/*
 * topk_select_noalloc — topk_select with no workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid the allocator).  The workspace is a
 * fixed array of CSA_TOPK_NOALLOC_MAX_BYTES in device memory that the library
 * owns: each GPU the library runs on holds its own copy until the process
 * ends.  Arguments, results and errors are those of topk_select; a shape
 * whose topk_workspace_size exceeds the array returns CSA_ERR_WORKSPACE
 * (nothing enqueued; use topk_select with a workspace).  The first call on a
 * device enqueues a clear of the array on `stream` (a fill kernel).  Every
 * call on a GPU shares that GPU's array: calls that overlap on one GPU (other
 * streams, other host threads) race and must be serialized by the caller.
 * The call allocates nothing.  Eight rows of 262144 BF16 scores (decode at
 * 1M context) need about 0.8 MiB of the array.
 */
#define CSA_TOPK_NOALLOC_MAX_BYTES (4u << 20)
int topk_select_noalloc(const void* scores, int32_t score_dtype, int32_t batch, int32_t n_q,
                        int64_t n_cap, const int32_t* n_entries, const int64_t* q_pos,
                        int32_t ratio, int32_t k, int32_t* idx_out, void* stream);

/*
 * indexer_topk — indexer_score followed by topk_select on its scores, in one
 * call ([TRIPBOT] §3.1 第二步: score every visible entry, keep the top k).
 * Arguments are those of the two calls (score_dtype and scores as for
 * indexer_score, topk = k and the workspace as for topk_select); the results
 * are identical to the two calls made in sequence: scores is written and
 * idx_out receives the selection.  On the MXFP4 path with few long rows
 * (decode) the indexer also builds top-k's first histogram pass, so one launch
 * fewer runs.  The workspace contract of topk_select applies.
 * stage_events: NULL, or two hipEvent_t (owned by the caller, created with
 * timing) that the scoring kernel's dispatch records at its start and its end,
 * for callers that time the scoring stage on its own; both must be non-NULL
 * (else CSA_ERR_NULL).
 */
int indexer_topk(const void* q, const uint8_t* q_scales, int32_t q_dtype, const float* w,
                 const void* k, const uint8_t* k_scales, int32_t k_dtype, int32_t batch,
                 int32_t n_q, int32_t n_heads, int32_t d_idx, int64_t n_cap,
                 const int32_t* n_entries, const int64_t* q_pos, int32_t ratio, void* scores,
                 int32_t score_dtype, int32_t topk, int32_t* idx_out, void* workspace,
                 size_t ws_bytes, void* const* stage_events, void* stream);

/*
 * sparse_window_attn — CSA attention ([TRIPBOT] §3.1 + §3.3 + Figure 3).
 * For each query (b,t) and head h: one joint softmax over the key set
 *     { entry rows idx[b,t,j] : 0 <= idx < n_vis(b,t) }  U  { window rows t-W+1..t }
 * logits scale * q.kappa, value = the same stored row (all 192 dims, MQA: every
 * query head shares the one KV row).  With sink != NULL, exp(sink[h]) is added
 * to head h's denominator (the learnable attention sink of [TRIPBOT] §3.3).
 *   q    [batch, n_q, n_heads, 192] (q_dtype CSA_F32 | CSA_BF16)
 *   kv   [batch, n_cap] entry rows (kv_dtype CSA_F32 | CSA_KV_MIXED)
 *   idx  [batch, n_q, k] int32;  n_entries [batch]; ratio (4)
 *   win  [batch, win_rows] raw-token ring in kv_dtype, base win_base
 *   q_pos [batch, n_q] int64; window = W (>= 0)
 *   scale: logit scale, finite and > 0 (CSA_ERR_RANGE otherwise; 1/sqrt(192)
 *   in the method)
 *   out  [batch, n_q, n_heads, 192] (out_dtype CSA_F32 | CSA_BF16)
 *   lse_out [batch, n_q, n_heads] float32 = log sum exp of the logits (keys
 *   only, no sink), or NULL.
 *   Matrix-core path: q_dtype CSA_BF16, kv_dtype CSA_KV_MIXED, n_heads % 32 == 0
 *   (<= 128); otherwise a float32 vector path (n_heads <= 16 per block of heads).
 *   Value range on the matrix-core path: the logits use the stored row
 *   exactly, but the row enters P.V as FP16, so a BF16 (RoPE-dim) value
 *   beyond +-65504 acts as +-65504 in the output sum, and one below 2^-14 in
 *   magnitude keeps FP16's subnormal precision (rounded toward zero); the
 *   FP8 dims are exact.  N(0,1)-scaled KV is far inside this range; callers
 *   whose rows may exceed it use the float32 path.  The same holds for
 *   hca_dense_attn, swa_attn and decode_step.
 *   Workspace: attn_workspace_size(batch, n_q, n_heads, k + window, q_dtype, kv_dtype).
 */
size_t attn_workspace_size(int32_t batch, int32_t n_q, int32_t n_heads, int64_t max_keys,
                           int32_t q_dtype, int32_t kv_dtype);
int sparse_window_attn(const void* q, int32_t q_dtype, int32_t batch, int32_t n_q,
                       int32_t n_heads, const void* kv, int32_t kv_dtype, int64_t n_cap,
                       const int32_t* n_entries, int32_t ratio, const int32_t* idx, int32_t k,
                       const void* win, int64_t win_rows, int64_t win_base,
                       const int64_t* q_pos, int32_t window, float scale, const float* sink,
                       void* out, int32_t out_dtype, float* lse_out, void* workspace,
                       size_t ws_bytes, void* stream);

/*
 * hca_dense_attn — HCA attention ([TRIPBOT] §3.2 + §3.3): as sparse_window_attn
 * with the key set = every visible entry { 0 .. n_vis(b,t)-1 } U window.
 * Workspace: attn_workspace_size(batch, n_q, n_heads, n_cap + window, q_dtype, kv_dtype).
 */
int hca_dense_attn(const void* q, int32_t q_dtype, int32_t batch, int32_t n_q, int32_t n_heads,
                   const void* kv, int32_t kv_dtype, int64_t n_cap, const int32_t* n_entries,
                   int32_t ratio, const void* win, int64_t win_rows, int64_t win_base,
                   const int64_t* q_pos, int32_t window, float scale, const float* sink,
                   void* out, int32_t out_dtype, float* lse_out, void* workspace,
                   size_t ws_bytes, void* stream);

/*
 * swa_attn — attention over the sliding window alone, the pure-SWA layers
 * ([TRIPBOT] §3.3 window of 128 raw tokens; the V4-Flash layer schedule of
 * §3 puts such layers first): for each query (b,t) and head h one softmax over
 * the window rows t-W+1..t (those stored, positions >= 0), value = the row.
 * Arguments as for hca_dense_attn without entries; window >= 1 (else
 * CSA_ERR_SHAPE).  A window of at most 288 keys needs no workspace (NULL, 0);
 * longer windows: attn_workspace_size(batch, n_q, n_heads, window, q_dtype,
 * win_dtype).
 */
int swa_attn(const void* q, int32_t q_dtype, int32_t batch, int32_t n_q, int32_t n_heads,
             const void* win, int32_t win_dtype, int64_t win_rows, int64_t win_base,
             const int64_t* q_pos, int32_t window, float scale, const float* sink, void* out,
             int32_t out_dtype, float* lse_out, void* workspace, size_t ws_bytes, void* stream);

/*
 * Decode over a device-resident cache ([AUSTERY] 全栈工程优化 and [YANBAOKE] §5:
 * the hybrid attention keeps a heterogeneous KV cache; the pages give no
 * layout, so this one is a reading).  One CSA layer and one HCA layer per
 * cache, every sequence of the batch at its own position.  Per sequence b the
 * cache holds
 *   - pos[b]: the position the next decode step appends and decodes;
 *   - the compressor state of each layer: the raw KV of the last m tokens
 *     (CSA m = 8 rows: two overlapped blocks; HCA m = 128) as BF16 and their
 *     gate logits x.W_gate as float32, ring row = position mod m;
 *   - the sliding-window rows of each layer (CSA_KV_MIXED), ring row =
 *     position mod win_rows;
 *   - the compressed entries of each layer (CSA_KV_MIXED) with their counts,
 *     and the CSA entries' MXFP4 indexer keys.
 * Every array is a device array the caller allocates (sizes below) and owns;
 * the library only reads and writes them.  Positions, counts and the
 * compress-on-boundary decisions live on the device, so a step enqueues the
 * same launches whatever the positions are.
 *
 * Paged entries (optional).  With page_entries = P > 0 the compressed entries
 * of both layers live in pools of fixed-size pages of P entries, addressed
 * through per-sequence page tables ([YANBAOKE] §5 and [AUSTERY] 全栈工程优化
 * name a paged, heterogeneous KV cache; its layout is this library's):
 *   csa_kv [csa_pool_pages, P, 256], csa_keys [csa_pool_pages, P, idx_dim/2],
 *   csa_key_scales [csa_pool_pages, P, idx_dim/32] (a CSA page holds its
 *   entries' rows and MXFP4 keys), hca_kv [hca_pool_pages, P, 256];
 *   csa_pages [B, csa_cap/P], hca_pages [B, hca_cap/P]: entry e of sequence b
 *   is row e mod P of physical page csa_pages[b][e / P] (hca likewise).
 * P is a power of two >= 32 dividing csa_cap and hca_cap.  Page ids are read
 * on the device and clamped to [0, pool_pages): a bad table gives wrong rows,
 * never an access outside the pools.  Every call gives bit for bit the results
 * of the contiguous layout holding the same entries.  Sequences may share
 * physical pages (decode_fork): a step writes only the page holding a
 * sequence's next entry (logical page count / P), so pages below it can be
 * shared read-only; a page that a step writes must belong to one sequence.
 * With page_entries = 0 the page fields are ignored and every entry array is
 * contiguous per sequence as listed below.
 */
typedef struct {
  int32_t batch;         /* B, 1 .. 65535                                        */
  int32_t n_heads;       /* query heads of both layers (MQA: one KV row per entry) */
  int32_t idx_heads;     /* indexer heads, a multiple of 32, <= 128               */
  int32_t idx_dim;       /* indexer key width: 64, 128 or 256                     */
  int32_t topk;          /* CSA entries kept per query, >= 1                      */
  int32_t window;        /* sliding window W, 0 .. win_rows                       */
  int64_t win_rows;      /* rows of each window ring, >= 1                        */
  int64_t csa_cap;       /* CSA entries a sequence can hold, >= 1                 */
  int64_t hca_cap;       /* HCA entries a sequence can hold, >= 1                 */
  float scale;           /* softmax logit scale (> 0, finite)                     */
  /* weights, float32 row-major */
  const float* csa_w_gate;    /* [192, 192]                                       */
  const float* csa_pos_bias;  /* [8, 192]                                         */
  const float* csa_w_idx;     /* [192, idx_dim]  indexer key projection           */
  const float* hca_w_gate;    /* [192, 192]                                       */
  const float* hca_pos_bias;  /* [128, 192]                                       */
  const float* csa_sink;      /* [n_heads] attention sink, or NULL                */
  const float* hca_sink;      /* [n_heads] or NULL                                */
  /* per-sequence state */
  int64_t* pos;               /* [B]                                              */
  int32_t* csa_entries;       /* [B] entries stored                               */
  int32_t* hca_entries;       /* [B]                                              */
  /* compressor rings */
  uint16_t* csa_raw;          /* [B, 8, 192]    BF16                              */
  float* csa_logits;          /* [B, 8, 192]                                      */
  uint16_t* hca_raw;          /* [B, 128, 192]  BF16                              */
  float* hca_logits;          /* [B, 128, 192]                                    */
  /* sliding-window rings, 16-byte aligned */
  uint8_t* csa_win;           /* [B, win_rows, 256]                               */
  uint8_t* hca_win;           /* [B, win_rows, 256]                               */
  /* compressed entries, 16-byte aligned */
  uint8_t* csa_kv;            /* [B, csa_cap, 256]                                */
  uint8_t* csa_keys;          /* [B, csa_cap, idx_dim/2]  MXFP4 codes             */
  uint8_t* csa_key_scales;    /* [B, csa_cap, idx_dim/32] E8M0                    */
  uint8_t* hca_kv;            /* [B, hca_cap, 256]                                */
  /* paged entries (page_entries = 0: contiguous, the fields below unused)     */
  int32_t page_entries;       /* P: a power of two >= 32 dividing both caps, or 0 */
  int32_t csa_pool_pages;     /* pages in the CSA pools, >= 1 when paged          */
  int32_t hca_pool_pages;     /* pages in the HCA pool, >= 1 when paged           */
  int32_t* csa_pages;         /* [B, csa_cap / P] physical page ids               */
  int32_t* hca_pages;         /* [B, hca_cap / P]                                 */
} csa_decode_cache;

/*
 * decode_fork — sequence dst takes sequence src's state at src's position p,
 * sharing src's full entry pages (paged caches only: [CSDN] 共享前缀场景的推理
 * 复用 reuses a shared prefix's compressed entries instead of recomputing
 * them).  Enqueued on `stream`, no host synchronisation:
 *   - pos[dst] = pos[src], the entry counts, both layers' compressor rings
 *     and window rings are copied;
 *   - for each layer, dst's page-table entries of the logical pages wholly
 *     below the entry count (count / P of them) are set to src's, so those
 *     physical pages are then shared (the pages dst's table named there are
 *     no longer referenced by dst: the caller may reuse them);
 *   - the rows of a partly filled last page (count mod P of them) are copied
 *     from src's page into the page dst's table already names for it, which
 *     must be dst's own (a page later steps of dst write).
 * Later steps of src and dst then run independently and give the results an
 * unshared copy would give, bit for bit.  src == dst is a no-op.  Errors:
 * CSA_ERR_NULL, CSA_ERR_SHAPE (src or dst out of range), CSA_ERR_UNSUPPORTED
 * (page_entries = 0), CSA_ERR_HIP.
 */
int decode_fork(const csa_decode_cache* cache, int32_t src, int32_t dst, void* stream);

/*
 * decode_prime — write the last n_tok tokens before pos[b] into the rings of
 * every sequence b: positions pos[b]-n_tok .. pos[b]-1 (those >= 0), raw KV
 * x_csa / x_hca [B, n_tok, 192] (x_dtype CSA_F32 | CSA_BF16).  Raw rings get
 * the BF16 value, logit rings its gate logits, window rings its stored row.
 * Nothing is compressed and pos is not changed: the entries of the prefix
 * come from csa_compress / hca_compress.  1 <= n_tok <= 65535.
 */
int decode_prime(const csa_decode_cache* cache, const void* x_csa, const void* x_hca,
                 int32_t x_dtype, int32_t n_tok, void* stream);

/*
 * decode_step — one decode token for every sequence b, at position p = pos[b]:
 *   1. append ([TRIPBOT] §3.3 window; [CSDN] 核心创新一 §1.4 storage): the
 *      token's raw KV x_csa[b] / x_hca[b] goes to each layer's raw, logit and
 *      window rings;
 *   2. compress on a boundary ([TRIPBOT] §3.1 第一步, §3.2): when p+1 is a
 *      multiple of 4, CSA entry (p+1)/4-1 is pooled from tokens p-7..p with its
 *      MXFP4 key; when p+1 is a multiple of 128, HCA entry (p+1)/128-1 from
 *      tokens p-127..p; the counts follow (an entry at or past the capacity is
 *      not stored and its count stays at the capacity);
 *   3. index and select ([TRIPBOT] §3.1 第二步): scores of the float32
 *      indexer query q_idx [B, idx_heads, idx_dim] with head weights
 *      w [B, idx_heads] over the visible CSA entries, top `topk`;
 *   4. attend ([TRIPBOT] §3.1, §3.2, §3.3): CSA layer over the selected
 *      entries + window with q_csa, HCA layer over every visible entry +
 *      window with q_hca ([B, n_heads, 192], q_dtype CSA_F32 | CSA_BF16),
 *      into out_csa / out_hca ([B, n_heads, 192], out_dtype CSA_F32 | CSA_BF16);
 *   5. pos[b] = p + 1.
 * A sequence whose pos[b] is negative is inactive: nothing is appended or
 * compressed, pos[b] stays, and its outputs are zero (it has no key).
 * The results equal those of kv_append, csa_compress (with its key),
 * hca_compress, indexer_topk, sparse_window_attn and hca_dense_attn called in
 * that order on the same state, bit for bit.
 * Workspace: decode_workspace_size(cache, q_dtype) bytes, 256-byte aligned
 * and zero-filled before its first use; it holds the step's scores,
 * selection and partial results and stays valid for the next step (the part
 * that must start at zero — per-sequence arrival counters and top-k totals,
 * at fixed offsets in the first 512 KiB — is left at zero, so one zeroing
 * suffices, also when the workspace later serves a cache of another shape).
 * Steps sharing a cache or a workspace must not overlap.
 * stage_events: as for indexer_topk (bracket the scoring kernel), or NULL.
 */
size_t decode_workspace_size(const csa_decode_cache* cache, int32_t q_dtype);
int decode_step(const csa_decode_cache* cache, const void* x_csa, const void* x_hca,
                int32_t x_dtype, const float* q_idx, const float* w, const void* q_csa,
                const void* q_hca, int32_t q_dtype, void* out_csa, void* out_hca,
                int32_t out_dtype, void* workspace, size_t ws_bytes,
                void* const* stage_events, void* stream);

/*
 * decode_csa_layer, decode_hca_layer — the same token split by layer, for a
 * model that runs its layers one after the other (the HCA layer's raw KV and
 * query come from the CSA layer's output, so its work cannot start before the
 * CSA layer's attention has finished).  For each token call decode_csa_layer,
 * then decode_hca_layer, with the same cache and workspace:
 *   decode_csa_layer: steps 1-4 of decode_step for the CSA layer at p = pos[b]
 *     (append, compress a CSA entry with its key on a boundary, index, select,
 *     attend into out_csa); pos is not changed;
 *   decode_hca_layer: steps 1, 2 and 4 for the HCA layer at p = pos[b], then
 *     pos[b] = p + 1 (step 5).
 * Arguments as for decode_step (the workspace is decode_workspace_size's).
 * The pair of calls gives decode_step's results bit for bit.
 */
int decode_csa_layer(const csa_decode_cache* cache, const void* x_csa, int32_t x_dtype,
                     const float* q_idx, const float* w, const void* q_csa, int32_t q_dtype,
                     void* out_csa, int32_t out_dtype, void* workspace, size_t ws_bytes,
                     void* const* stage_events, void* stream);
int decode_hca_layer(const csa_decode_cache* cache, const void* x_hca, int32_t x_dtype,
                     const void* q_hca, int32_t q_dtype, void* out_hca, int32_t out_dtype,
                     void* workspace, size_t ws_bytes, void* stream);

/*
 * Prefix reuse ([CSDN] 共享前缀场景的推理复用: a shared prefix's compressed
 * entries are kept on disk and reused instead of prefilling it again; for the
 * uncompressed sliding-window KV the pages list full caching, periodic
 * checkpointing and no caching at all).
 *
 * prefix_save writes sequence `seq` of the cache, at its current position p,
 * to the file `path` (created or replaced): `parts` is a mask of
 *   CSA_PREFIX_ENTRIES  the compressed entries of both layers with the CSA
 *                       MXFP4 keys (everything tokens 0 .. p-1 were compressed
 *                       into: the counts stored in the cache);
 *   CSA_PREFIX_RINGS    the uncompressed state: both layers' window rings and
 *                       compressor rings (raw BF16 KV and gate logits).
 * Full caching saves both; a periodic checkpoint is a snapshot with rings taken
 * every so many tokens; with no SWA caching only entries are saved.
 *
 * prefix_load restores such a file into sequence `seq` of a cache for a prefix
 * of `prefix_len` tokens (-1: the file's own p), and sets pos[seq] to it:
 *   ENTRIES: the entries of the prefix, i.e. the first min(count, prefix_len/4)
 *            CSA and min(count, prefix_len/128) HCA entries of the file
 *            (prefix_len <= p; a longer saved prefix serves a shorter one);
 *   RINGS:   the file's rings, which describe positions below p, so p <=
 *            prefix_len is required.
 * *prime_from (may be NULL) receives the first position whose raw KV the
 * caller must still write with decode_prime on this sequence alone (positions
 * *prime_from .. prefix_len-1; none when it equals prefix_len): the rings hold
 * the last max(128, win_rows) positions, so without RINGS that is
 * max(0, prefix_len - max(128, win_rows)), and with RINGS from a snapshot at
 * p it is max(p, prefix_len - max(128, win_rows)).  Entries past the prefix
 * and rings not loaded are left as they were (they are rewritten before use).
 * The file must match the cache's idx_dim (and, for RINGS, win_rows), and the
 * restored counts must fit the cache's capacities.  With paged entries the
 * rows go to (and are saved from) the pages the sequence's tables name; a
 * page id there outside its pool is refused with CSA_ERR_RANGE before
 * anything is written (loading into pages that other sequences share changes
 * their entries too).
 *
 * Both calls synchronise `stream` and copy through host memory (host I/O
 * around the path, not a kernel).  Format (version 2): a 144-byte header
 * (magic "CSAPFX01", version, parts, p, counts, sizes, a 64-bit checksum per
 * section, and last a 64-bit checksum of the header's own 136 bytes), then
 * the sections in the order above, each the sequence's rows as stored in the
 * cache; no other bytes.  Errors: CSA_ERR_NULL, CSA_ERR_SHAPE (seq out of range, parts empty or
 * unknown), CSA_ERR_IO, CSA_ERR_FORMAT (bad magic, version, sizes or
 * either checksum, parts missing from the file), CSA_ERR_RANGE (prefix_len outside
 * what the file can serve, counts over the capacities), CSA_ERR_HIP.  Every
 * check of the file is made before the cache is written.
 */
#define CSA_PREFIX_ENTRIES 1
#define CSA_PREFIX_RINGS 2
int prefix_save(const csa_decode_cache* cache, int32_t seq, const char* path, int32_t parts, void* stream);
int prefix_load(const csa_decode_cache* cache, int32_t seq, const char* path, int32_t parts,
                int64_t prefix_len, int64_t* prime_from, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBCSA_H */
