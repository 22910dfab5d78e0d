/*
 * bsx.h: C ABI of libbsx, block-sparse draft-query cross-attention on MI355X (gfx950).
 *
 * What is computed.  "Split-KV: Efficient Context Parallelism for Training
 * Diffusion Drafters" (Abstract): a diffusion drafter's training builds compact
 * draft queries by anchor sampling and cross-attends a much longer context under
 * a block-sparse mask; the context-parallel scheme keeps key/value shards local,
 * moves only query-sized tensors, is exact, and balances context KV chunks over
 * ranks by realized attention cost with longest-processing-time-first (LPT)
 * planning.  Attention itself is softmax(Q K^T / sqrt(d)) V ("Flash-dLLM:
 * IO-Aware KV Caching and Parallel Decoding for Diffusion LLMs", section
 * "Method 1: I/O-Aware Fused KV-Cache Kernel").  This library is one GPU's share
 * of that scheme: every draft query against the local KV chunks.
 *
 * Notation and the mask.
 *   n_blocks anchors, each owning a block of B = block_size draft queries:
 *   query q belongs to block b = q / B, N_q = n_blocks * B.
 *   Query head h reads KV head g = h / (H_q / H_kv) (contiguous GQA groups).
 *   Every query of block b sees
 *     - the context keys at packed positions [ctx_begin[b], anchor[b]): its own
 *       sample's keys before its anchor (ctx_begin[b] = start of that sample, 0
 *       for one sample), and
 *     - bidirectionally, the B keys of its own draft block, given separately as
 *       k_self/v_self rows b*B .. b*B+B-1.
 *
 * Layouts (row-major, contiguous, 16-byte aligned):
 *   q, d_o          [N_q][H_q][d]        dtype of the shape (f32 or bf16)
 *   k, v            [n_local][H_kv][d]   the local chunks back to back, in chunk index order
 *   k_self, v_self  [N_q][H_kv][d]
 *   o_part          [n_out][N_q][H_q][d] f32,  lse_part [n_out][N_q][H_q] f32
 *   merged o        [rows][d] f32 or bf16, merged lse [rows] f32  (rows = N_q * H_q)
 *   anchor, ctx_begin  [n_blocks] int64 (device)
 * LSE values are natural logarithms.  A partial is normalized within its own key set:
 * O_T = sum_{k in T} exp(s_k - LSE_T) v_k.
 *
 * Memory and ownership.  "device" pointers are caller-owned GPU memory; "host"
 * pointers are caller-owned CPU memory read during the call only.  The library
 * allocates nothing and keeps no state between calls.  Calls that take a
 * workspace need at least the bytes the matching *_workspace query returns, on
 * the device, 256-byte aligned; a workspace must not be shared by calls in flight
 * at the same time.  Device work is enqueued on `stream` (a hipStream_t; NULL is
 * the default stream) and is asynchronous; host buffers may be reused as soon as
 * the call returns.
 *
 * Errors.  Every call checks its arguments first and returns a bsx_status; on
 * any error nothing is launched and bsx_last_error() (per thread) describes it.
 * A failed launch returns BSX_E_DEVICE.  No C++ exception crosses this ABI.
 */
#ifndef BSX_H_
#define BSX_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BSX_ABI_VERSION 2

typedef enum {
  BSX_OK = 0,
  BSX_E_INVALID = 1,      /* an argument is null, negative, out of range or inconsistent */
  BSX_E_UNSUPPORTED = 2,  /* valid, but not implemented (head_dim, dtype) */
  BSX_E_WORKSPACE = 3,    /* workspace smaller than the *_workspace query */
  BSX_E_DEVICE = 4        /* the HIP runtime reported an error at launch */
} bsx_status;

typedef enum { BSX_F32 = 0, BSX_BF16 = 1 } bsx_dtype;

/* Problem shape shared by the attention calls. */
typedef struct {
  int32_t n_blocks;    /* anchors (query blocks), >= 0 */
  int32_t block_size;  /* B, draft queries per block, 1 .. 256 */
  int32_t n_q_heads;   /* H_q, a multiple of n_kv_heads */
  int32_t n_kv_heads;  /* H_kv >= 1 */
  int32_t head_dim;    /* d; 128 is implemented */
  int32_t dtype;       /* bsx_dtype of q, k, v, k_self, v_self, d_o */
  int64_t ctx_len;     /* S: packed context length; positions are [0, S) */
  float scale;         /* softmax scale; <= 0 selects 1/sqrt(head_dim) */
} bsx_shape;

/* KV chunking (host arrays).  Chunk i covers packed positions
 * [start[i], start[i] + len[i]) and sits in the local K/V buffer right after
 * chunks 0 .. i-1, so n_local = sum(len) (below 2^32; larger local buffers return
 * BSX_E_UNSUPPORTED).  Each chunk feeds output slot slot[i]
 * (NULL: slot i, which needs n_slots == n_chunks).  Split-KV page, Abstract:
 * key/value chunks stay where they are and are balanced over ranks; a slot is one
 * chunk (per-chunk partials), one LPT bin (virtual rank), or a rank's whole share. */
typedef struct {
  int32_t n_chunks;       /* >= 0 */
  int32_t n_slots;        /* >= 1 when n_chunks > 0 */
  const int64_t* start;   /* host [n_chunks], 0 <= start, start + len <= S */
  const int64_t* len;     /* host [n_chunks], len >= 0 */
  const int32_t* slot;    /* host [n_chunks] in [0, n_slots), or NULL */
} bsx_chunks;

int bsx_abi_version(void);
/* Text of the last error on this thread ("" when none). */
const char* bsx_last_error(void);
const char* bsx_status_string(int status);

/* ---------------------------------------------------------------------------
 * Host: the block-sparse mask of anchor-sampled draft blocks.  Split-KV page,
 * Abstract: anchor sampling builds compact draft queries, one draft block per
 * anchor, which cross-attend the context under a block-sparse mask.  Block b sees
 * the context positions of its own sample before its anchor:
 *   ctx_begin[b] = sample_start[b]  (0 when sample_start is NULL: one sample)
 *   anchor[b]    = anchor_global[b] (packed position of the anchor)
 * i.e. the interval [ctx_begin[b], anchor[b]) the other calls take, plus (not
 * stored) the block's own B draft keys.
 *   anchor_global, sample_start: host [shape->n_blocks]; sample_start may be NULL
 *   ctx_begin, anchor: host [shape->n_blocks] out, written only on success
 * Returns BSX_E_INVALID, writing nothing, when some block has
 * sample_start < 0, sample_start > anchor_global or anchor_global > S.
 */
bsx_status bsx_mask_from_anchors(const bsx_shape* shape, const int64_t* anchor_global,
                                 const int64_t* sample_start, int64_t* ctx_begin,
                                 int64_t* anchor);

/* ---------------------------------------------------------------------------
 * Host: check a block-sparse mask.  Split-KV page, Abstract (anchor sampling
 * and the block-sparse mask).  Returns BSX_OK when every block satisfies
 * 0 <= ctx_begin[b] <= anchor[b] <= S, BSX_E_INVALID naming the first block
 * that does not.  anchor, ctx_begin: host [shape->n_blocks].
 */
bsx_status bsx_validate_mask(const bsx_shape* shape, const int64_t* anchor,
                             const int64_t* ctx_begin);

/* ---------------------------------------------------------------------------
 * Device: realized cost per (query block, KV chunk).  Split-KV page, Abstract:
 * chunks are balanced by their realized attention cost.  Unit: visible
 * (query, context key) pairs of one head,
 *   counts[b][c]  = B * |[start_c, start_c + len_c) ∩ [ctx_begin_b, anchor_b)|
 *   chunk_cost[c] = sum_b counts[b][c]
 * exact in int64.  The draft block's own keys carry no chunk cost.
 *   anchor, ctx_begin: device [n_blocks]
 *   chunks: host; slot and n_slots are ignored
 *   counts: device [n_blocks][n_chunks] int64, or NULL to skip it
 *   chunk_cost: device [n_chunks] int64
 *   mask_err: device int32, set to 1 if some block's range is not a valid
 *             interval of [0, S] (counts then use the range clamped to it), else 0
 *   ws: device, bsx_cost_workspace(chunks->n_chunks) bytes
 */
size_t bsx_cost_workspace(int32_t n_chunks);
bsx_status bsx_cost(const bsx_shape* shape, const int64_t* anchor, const int64_t* ctx_begin,
                    const bsx_chunks* chunks, int64_t* counts, int64_t* chunk_cost,
                    int32_t* mask_err, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Host: LPT planning.  Split-KV page, Abstract (cost-aware longest-processing-
 * time-first balancing of KV chunks).  Items in order of (cost descending, index
 * ascending) each go to the bin of (load ascending, index ascending).
 *   cost: host [n_items] (>= 0); bin_of: host [n_items] out; bin_load: host [n_bins] out
 *   makespan: max load; imbalance: makespan / (sum / n_bins) - 1, 0 if the sum is 0.
 * Any of bin_load, makespan, imbalance may be NULL.
 */
bsx_status bsx_lpt(int32_t n_items, const int64_t* cost, int32_t n_bins, int32_t* bin_of,
                   int64_t* bin_load, int64_t* makespan, double* imbalance);

/* ---------------------------------------------------------------------------
 * Host: chunk placement by a named rule, for comparing balancing strategies.
 * Split-KV page, Figures & tables (CP comparison table, load-balancing column):
 * Split-KV balances chunks by cost-aware LPT, Ring Attention by zigzag, RingX not
 * at all.  Items are chunks in context order, i = 0 .. n_items - 1, P = n_bins:
 *   BSX_PLACE_LPT          as bsx_lpt
 *   BSX_PLACE_CONTIGUOUS   bin = floor(i * P / n_items): P runs of consecutive chunks
 *   BSX_PLACE_ZIGZAG       s = floor(i * 2P / n_items) (2P runs); bin = s if s < P,
 *                          else 2P - 1 - s: bin r holds runs r and 2P - 1 - r
 *   BSX_PLACE_ROUND_ROBIN  bin = i mod P
 * Only LPT reads the costs to place; every rule reports loads, makespan and
 * imbalance the same way as bsx_lpt.  Arguments as bsx_lpt.
 */
typedef enum {
  BSX_PLACE_LPT = 0,
  BSX_PLACE_CONTIGUOUS = 1,
  BSX_PLACE_ZIGZAG = 2,
  BSX_PLACE_ROUND_ROBIN = 3
} bsx_placement;

bsx_status bsx_place(int32_t mode, int32_t n_items, const int64_t* cost, int32_t n_bins,
                     int32_t* bin_of, int64_t* bin_load, int64_t* makespan, double* imbalance);

/* ---------------------------------------------------------------------------
 * Device: forward partials.  Attention is softmax(Q K^T / sqrt(d)) V (Flash-dLLM
 * page, "Method 1: I/O-Aware Fused KV-Cache Kernel", the attention formula), taken
 * under the block-sparse draft-query mask over a rank's local KV chunks, each
 * chunk group giving a partial that the exact merge combines (Split-KV page,
 * Abstract: exact context parallelism with local key/value shards and a global
 * query view).  For every query row (q, h) and output slot s:
 * the partial (O, LSE) over the visible keys of the chunks mapped to s; with
 * k_self/v_self given, one more slot (index n_slots, last) over the block's own
 * keys.  n_out = n_slots + (k_self ? 1 : 0).  Rows that see no key of a slot get
 * LSE = -inf; their O is unspecified and must be given weight 0 (bsx_lse_merge
 * does so without reading it).
 *   q: device [N_q][H_q][d]; k, v: device [n_local][H_kv][d]
 *   k_self, v_self: device [N_q][H_kv][d], both NULL for no self slot
 *   anchor, ctx_begin: device [n_blocks]; a range outside [0, S] is clamped to it
 *   o_part: device [n_out][N_q][H_q][d] f32; lse_part: device [n_out][N_q][H_q] f32
 *   ws: device, bsx_fwd_workspace(shape, chunks) bytes
 * bf16 inputs use bf16 matrix cores with f32 accumulation and an f32 softmax;
 * f32 inputs use f32 arithmetic throughout.
 */
size_t bsx_fwd_workspace(const bsx_shape* shape, const bsx_chunks* chunks);
bsx_status bsx_attn_fwd(const bsx_shape* shape, const void* q, const void* k, const void* v,
                        const void* k_self, const void* v_self, const int64_t* anchor,
                        const int64_t* ctx_begin, const bsx_chunks* chunks, float* o_part,
                        float* lse_part, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Device: bsx_attn_fwd without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, results and errors as bsx_attn_fwd, minus ws/ws_bytes:
 * its scratch (the uploaded chunk table and the launch order) lives in a file-scope
 * device array of BSX_NOALLOC_SCRATCH_BYTES that each GPU holds from the library's
 * load until the process ends.  The call allocates nothing: no hipMalloc/hipFree and
 * no host heap.  Limits (BSX_E_UNSUPPORTED beyond them, nothing launched): at most
 * BSX_NOALLOC_MAX_CHUNKS chunks and slots, and a launch whose table and launch order
 * fit the scratch.  Launches with few (KV head, slot) pairs run without the split of
 * long items that bsx_attn_fwd may use (same results within rounding).  Every call
 * on a GPU shares that GPU's scratch, which keeps the last call's contents: calls
 * that overlap on one GPU (on different streams or threads) race and must be
 * serialized by the caller.
 */
#define BSX_NOALLOC_MAX_CHUNKS 1024
#define BSX_NOALLOC_SCRATCH_BYTES (1 << 20)
bsx_status bsx_attn_fwd_noalloc(const bsx_shape* shape, const void* q, const void* k,
                                const void* v, const void* k_self, const void* v_self,
                                const int64_t* anchor, const int64_t* ctx_begin,
                                const bsx_chunks* chunks, float* o_part, float* lse_part,
                                void* stream);

/* ---------------------------------------------------------------------------
 * Device: exact LSE merge of partials.  Split-KV page, Abstract (exact method,
 * query-sized exchange).  Per row, over the partials p in ascending order:
 *   M = max_p LSE_p, LSE = M + log sum_p exp(LSE_p - M), O = sum_p exp(LSE_p - LSE) O_p,
 * where partials with LSE_p = -inf are skipped and their O_p is not read; a row
 * whose partials are all -inf merges to (O = 0, LSE = -inf).
 *   o_parts: device [n_parts][n_rows][head_dim] f32; lse_parts: device [n_parts][n_rows] f32
 *   out_dtype: BSX_F32 or BSX_BF16, the element type of o_out
 *   o_out: device [n_rows][head_dim] of out_dtype (BSX_BF16: the f32 result rounded to
 *          nearest, ties to even); lse_out: device [n_rows] f32
 * head_dim: a multiple of 4, at most 512.  n_parts: 1 .. 4096 (BSX_F32), 1 .. 128
 * (BSX_BF16; more returns BSX_E_UNSUPPORTED).
 */
bsx_status bsx_lse_merge(int32_t n_parts, int64_t n_rows, int32_t head_dim,
                         const float* o_parts, const float* lse_parts, int32_t out_dtype,
                         void* o_out, float* lse_out, void* stream);

/* ---------------------------------------------------------------------------
 * Device: backward of the attention.  Split-KV page, Abstract: the method trains
 * diffusion drafters, so the attention (Flash-dLLM page, "Method 1", the
 * attention formula) needs its gradients; the pages print none, and this is the
 * analytic gradient of the unchunked masked softmax attention with respect to
 * q, k, v, k_self, v_self, using the merged forward results: P = exp(s - LSE), D = rowsum(dO * O), dS = P (dO.v - D),
 * dQ = scale dS K, dK = scale dS^T Q (summed over the query heads of a KV head),
 * dV = P^T dO.  Over a chunk subset (one rank's local keys) dK/dV are exact for
 * the local keys and dQ is this share's contribution (shares sum to the full dQ).
 *   o, lse: device merged forward outputs, [N_q][H_q][d] and [N_q][H_q] f32
 *   d_o: device [N_q][H_q][d], dtype of the shape
 *   dq: device [N_q][H_q][d] f32; dk, dv: device [n_local][H_kv][d] f32
 *   dk_self, dv_self: device [N_q][H_kv][d] f32 (required iff k_self is given)
 *   All gradient outputs are overwritten.
 *   ws: device, bsx_bwd_workspace(shape, chunks) bytes.  bf16 inputs only.
 */
size_t bsx_bwd_workspace(const bsx_shape* shape, const bsx_chunks* chunks);
bsx_status bsx_attn_bwd(const bsx_shape* shape, const void* q, const void* k, const void* v,
                        const void* k_self, const void* v_self, const float* o,
                        const float* lse, const void* d_o, const int64_t* anchor,
                        const int64_t* ctx_begin, const bsx_chunks* chunks, float* dq,
                        float* dk, float* dv, float* dk_self, float* dv_self, void* ws,
                        size_t ws_bytes, void* stream);

#ifdef __cplusplus
}  /* extern "C" */
#endif

#endif  /* BSX_H_ */
