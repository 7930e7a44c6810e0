/*
 * sa.h -- C ABI of the MI355X (gfx950) sparse-attention library (libsa.so).
 *
 * Training-free block/stripe-sparse attention for long-context prefill, and top-K
 * block-sparse decode.  The operations follow the review pages:
 *
 *  - AnchorAttention: Difference-Aware Sparse Attention with Stripe Granularity
 *    (arXiv 2505.23520): Eq. (1) anchor = max score over the initial and local key regions;
 *    Eq. (2) mask = I(avgpool(x_a) - avgpool(Q) K^T / sqrt(d) <= theta); Eq. (3) the index
 *    set I per query block; "Core claim": stripe granularity and discrete K/V loading.
 *  - SALE: Low-bit Estimation for Efficient Sparse Attention in Long-context LLM Prefilling
 *    (arXiv 2505.24179): low-precision Q.K^T estimate, sink (32 tokens) and local (256
 *    tokens) areas, block skipping, log-domain compare; drop-in replacement of the
 *    attention module (inputs Q, K, V; output O).
 *  - SpotAttention: Plug-In Block-Sparse Routing for Pretrained Long-Context Transformers
 *    (arXiv 2606.22874), Figure 2: decode attends to a sink prefix, a recency window and the
 *    top-scoring blocks, gathered from the cache.
 *  - KVpop (arXiv 2607.05061), referee minor comment 4: query heads sharing a KV head are
 *    aggregated with max.
 *
 * Conventions shared by every entry point
 *  - Memory: every tensor pointer is DEVICE memory owned by the caller (the library never
 *    allocates or frees on these paths and keeps no mutable global state; calls on
 *    different streams are independent).  `sa_shape`, `sa_sparse_params`,
 *    `sa_decode_params` and `sa_lists` themselves are HOST structs read during the call.
 *  - Layout: Q, K, V, O are bf16 with head_dim contiguous; the (batch, token, head)
 *    strides are given in ELEMENTS and must be multiples of 8 (16-byte rows); base
 *    pointers must be 16-byte aligned.  Query head h uses KV head kv_head_of_q[h] (sa_shape),
 *    by default h / (Hq / Hkv).
 *  - Execution: asynchronous on `stream`.  All validation happens on the host before any
 *    launch; on an error nothing is launched and no output is touched.
 *  - Errors: returned as `sa_status`; no exception or abort crosses the ABI.  A HIP launch
 *    failure is reported as SA_ERR_DEVICE.
 *  - Supported (v1): head_dim in {64, 128}; block_q in {64, 128}; block_k in {32, 64} for
 *    block lists (SALE's configuration is block_q 64, block_k 32) and 64 for stripes and the
 *    anchor-state pair; n_q_heads <= 128 and n_q_heads / n_kv_heads in {1, 2, 4, 8}; the token
 *    strides of K and V (k_stride[1], v_stride[1]) below 2^24 elements.
 *  - Sizes: batch, head counts, seq_q and seq_k are at least 1; an empty problem is
 *    SA_ERR_SHAPE (there is nothing to launch: callers skip the call).  seq_q < 2^30; at most
 *    8192 key blocks for decode.
 */
#ifndef SA_H_
#define SA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SA_OK = 0,
  SA_ERR_NULL = 1,         /* a required pointer is NULL                                   */
  SA_ERR_SHAPE = 2,        /* inconsistent sizes, strides or alignment                     */
  SA_ERR_PARAM = 3,        /* bad parameter value (theta NaN, negative sink, ...)          */
  SA_ERR_UNSUPPORTED = 4,  /* valid but not implemented (head_dim, block sizes, group size)*/
  SA_ERR_CAPACITY = 5,     /* list stride too small for a block list                       */
  SA_ERR_WORKSPACE = 6,    /* workspace NULL or smaller than sa_workspace_size()           */
  SA_ERR_DEVICE = 7,       /* a HIP call or kernel launch failed                           */
  SA_ERR_CHECK = 8         /* debug build only: a kernel found invalid caller data         */
} sa_status;

enum { SA_BLOCK = 0, SA_STRIPE = 1 };
enum { SA_OP_ESTIMATE = 0, SA_OP_PREFILL = 1, SA_OP_DECODE = 2, SA_OP_CALIBRATE = 3,
       SA_OP_ESTIMATE_STATE = 4 };

#define SA_MAX_Q_HEADS 128

/* Problem statement: batch, heads, head_dim, query/key lengths, the GQA head map and
 * element strides of the (batch, token, head) dimensions of each tensor.  For decode, seq_q is
 * 1 and seq_k is the cache capacity (tokens per sequence in the cache buffers); q/o strides
 * use the token stride slot unused.
 *
 * kv_head_of_q (HOST int32 [n_q_heads], nullable; read during the call): the KV head each
 * query head attends with (grouped-query attention; KVpop, referee minor comment 4: the query
 * heads sharing a KV head are aggregated with max, so a list row is per KV head).  NULL means
 * h / (n_q_heads / n_kv_heads).  Every value must lie in [0, n_kv_heads) (else SA_ERR_PARAM)
 * and every KV head must have exactly n_q_heads / n_kv_heads query heads (the kernels pack a
 * group's heads onto one K/V tile; otherwise SA_ERR_UNSUPPORTED).  The heads of a group may sit
 * anywhere in the head dimension of Q and O; per-query-head inputs and outputs (theta, O, LSE,
 * the anchor state, calibration results) stay indexed by the query head itself. */
typedef struct {
  int32_t batch, n_q_heads, n_kv_heads, head_dim, seq_q, seq_k;
  const int32_t* kv_head_of_q;
  int64_t q_stride[3], k_stride[3], v_stride[3], o_stride[3];
} sa_shape;

/* Sparse prefill parameters.  `theta` (HOST array [n_q_heads], logit units) is the Eq. (2)
 * threshold per query head: +inf keeps every causal block (dense causal attention), -inf
 * keeps only the forced sink and local blocks; NaN is rejected.  softmax_scale <= 0 means
 * 1/sqrt(head_dim) (rounded once to fp32).  sink_tokens >= 0 and local_tokens >= 1. */
typedef struct {
  int32_t block_q, block_k, sink_tokens, local_tokens;
  int32_t granularity;            /* SA_BLOCK or SA_STRIPE */
  const float* theta;             /* host [n_q_heads] */
  float softmax_scale;
  int32_t estimator;              /* SA_EST_POOLED (0) or SA_EST_RELATIVE (1) */
  int32_t step;                   /* query-block group size of the identification, 0 or 1: none */
} sa_sparse_params;

/* step (AnchorAttention, "Assumptions & free parameters": query blocks are identified in
 * groups of `step`, 16 in its experiments, and a key selected by any block of a group is
 * active for every block of it): with step > 1 the list of query block i holds its forced
 * entries and every causal candidate of i that passes the threshold for some block of i's
 * group {floor(i / step) * step, ...}.  Margins, when requested, stay per block.
 * step < 0: SA_ERR_PARAM. */

/* Estimators of sa_estimate_mask.
 * SA_EST_POOLED (AnchorAttention Eq. 1-2): per query block, the anchor (row max over each
 *   row's sink and local keys, averaged over the block) against int8 scores of the pooled
 *   query: margin = score - (anchor - theta).  Block and stripe granularity.
 * SA_EST_RELATIVE (SALE, "What carries the argument" and referee major comment 1): every
 *   (row, key) pair of the block is estimated from int8 Q (one scale per row) and int8 K
 *   tiles; a key block is kept when, for some row r and causal key j in it,
 *   S~[r, j] - LSE_r >= -theta, with LSE_r the log-sum-exp of S~ over row r's sink and local
 *   keys (theta = -ln tau of SALE's relative score).  Block granularity only
 *   (SA_ERR_UNSUPPORTED for stripes); its workspace also holds the int8 queries
 *   (B * seq * n_q_heads * (head_dim + 4) bytes). */
enum { SA_EST_POOLED = 0, SA_EST_RELATIVE = 1, SA_EST_RELATIVE_MXFP4 = 2 };
/* SA_EST_RELATIVE_MXFP4: the relative-score estimate with 4-bit operands (the pages' estimate
 *   is 4-bit): Q and K rows quantised to MXFP4 as the OCP Microscaling (MX) v1.0
 *   specification defines it (per 32 head dims a shared scale 2^e, e = floor(log2 max|x|) - 2,
 *   elements E2M1 round-to-nearest-even, saturating at 6), dot products on the block-scaled
 *   fp4 MFMA, S~ = fp32(dot) * c.  Block granularity only; the workspace holds the 4-bit rows
 *   (B * seq * (n_q_heads + n_kv_heads) * (head_dim / 2 + head_dim / 32) bytes and more). */

/* Per-row kept lists (the index set I of Eq. (3)), one row per (batch, KV head, query
 * block), rows ordered (b, g, i).  Row r holds counts[r] ascending key-block ids (block
 * granularity, blocks of block_k keys) or key-column ids (stripe granularity) in
 * idx[r*stride ...].  Lists given to sa_sparse_prefill may come from the caller: entries must
 * be ascending and lie in [0, ceil(seq_k / block_k)) (columns: [0, seq_k)); entries outside
 * that range are clamped into it on the device (memory stays in bounds; the result for such a
 * list is unspecified).  Forced sink and
 * local entries are included.  counts always receives the true count; entries past
 * `stride` are dropped (stripe lists only -- block lists require stride >= ceil(seq_k /
 * block_k)), so a caller detects stripe overflow as counts[r] > stride after the call.
 * margins (nullable, DEVICE float [rows * n_cand], n_cand = ceil(seq_k/block_k) for blocks or
 * seq_k for stripes) receives, for each causal candidate, max over the group's heads of
 * (score - (anchor - theta)); entries of non-candidates are left untouched. */
typedef struct {
  int32_t* counts;                /* device [B * Hkv * nQB]           */
  int32_t* idx;                   /* device [B * Hkv * nQB * stride]  */
  int32_t stride;
  float* margins;                 /* device, nullable                 */
} sa_lists;

/* Decode parameters: key-block size of the summaries and of the selection, number of
 * selected blocks K (forced blocks count toward K), sink and local (recency) sizes in
 * tokens, number of split-K partitions (0 = library choice), softmax scale as above.
 * top_p (SpotAttention abstract and Figure 2: a top-p rule reads each query's budget from the
 * selector's distribution over blocks): 0 selects exactly min(K, blocks) blocks; in (0, 1]
 * the forced blocks plus the fewest others, in (score desc, block asc) order, whose share of
 * pi_J = softmax over the cache's blocks of score_J brings the cumulative share to at least
 * top_p -- at most K blocks in all.  Other values: SA_ERR_PARAM.
 * K (top_k_blocks) must hold the whole forced set at every cache length, i.e. be at least
 * ceil(sink / block_k) + floor((local - 1) / block_k) + 2 (the sink blocks plus the most blocks
 * a window of `local` tokens can overlap), unless it covers every block of seq_k; a smaller K
 * is SA_ERR_PARAM (6 for block_k 64, sink 32, local 256; 10 for block_k 32). */
typedef struct {
  int32_t block_k, top_k_blocks, sink_tokens, local_tokens, n_splits;
  float softmax_scale;
  float top_p;
} sa_decode_params;

/* Workspace bytes an operation needs (op = SA_OP_ESTIMATE, SA_OP_ESTIMATE_STATE or
 * SA_OP_CALIBRATE with sa_sparse_params, or SA_OP_DECODE with sa_decode_params;
 * SA_OP_PREFILL needs none).
 * Returns 0 for an invalid request. */
size_t sa_workspace_size(int op, const sa_shape* shape, const void* params);

/* Estimation pass (AnchorAttention Eq. (1)-(3); SALE low-precision estimate):
 *  1. anchor x_a[r] = max over keys j <= r with j < sink or j > r - local of
 *     c * q_r . k_j (bf16 MFMA, fp32 accumulate), averaged over the query block;
 *  2. pooled query avgpool(Q) (fp64 sum, one rounding to fp32, fp32 divide), quantised to
 *     int8 with one symmetric scale per vector; keys quantised per block_k-key tile;
 *  3. exact int32 score D = qbar_q . k_q; s = fp32(D) * fp32(fp32(s_q * s_k) * c);
 *     block granularity takes the max over the block's causal columns;
 *  4. keep when max over the group's heads of s - (anchor - theta_h) >= 0 (ties keep), or
 *     when the block/column is forced (overlaps [0, sink) or the query block's local
 *     windows); compact into ascending lists.
 * q: device bf16 [B, seq, Hq, d]; k: device bf16 [B, seq, Hkv, d]; seq_q == seq_k.
 * ws: device scratch of at least sa_workspace_size(SA_OP_ESTIMATE, ...) bytes, 256-byte
 * aligned, owned by the caller, may be reused after the stream passes this call. */
sa_status sa_estimate_mask(const sa_shape* shape, const sa_sparse_params* params,
                           const void* q, const void* k, const sa_lists* out,
                           void* ws, size_t ws_bytes, hipStream_t stream);

/* Computation pass (SALE "Computation-Pass"; AnchorAttention discrete K/V loading): for
 * every query row r of head h in query block i, attention over the tokens named by the
 * list of (b, h / (Hq/Hkv), i) with j <= r, online softmax on bf16 MFMA.  Block lists name
 * key blocks; stripe lists name key columns (gathered row by row).  o: device bf16
 * [B, seq, Hq, d] (o_stride); lse: nullable device fp32 [B, Hq, seq], natural log.  A row
 * with no visible key gets O = 0 and LSE = -inf.  Only the first min(counts, stride)
 * entries of a row are read. */
sa_status sa_sparse_prefill(const sa_shape* shape, const sa_sparse_params* params /* theta unused, may be NULL */,
                            const void* q, const void* k, const void* v,
                            const sa_lists* lists, void* o, float* lse, hipStream_t stream);

/* Anchor-state reuse (AnchorAttention, "What carries the argument": the anchor kernel's
 * intermediates are kept for the sparse kernel; referee major comment 1: per query row the
 * anchor kernel holds the running max M and the p.V accumulator Acc; referee minor comment 2:
 * the sparse loop starts past the initial block, which the anchor covers).  The state of row r
 * of query head h is the softmax attention over its anchor region
 * A(r) = {j <= r : j < sink or j >= r - local + 1} (the token set of Eq. (1)'s max), kept as
 *   o   device bf16 [B, seq, Hq, d], contiguous: the normalised output over A(r), i.e. Acc / l;
 *   lse device fp32 [B, Hq, seq]: its log-sum-exp, natural log (M + ln l).
 * Both buffers are owned by the caller (B * seq * Hq * (2 d + 4) bytes). */
typedef struct {
  void* o;
  float* lse;
} sa_anchor_state;

/* sa_estimate_mask (pooled estimator, block_k 64, block or column lists; SA_ERR_UNSUPPORTED
 * otherwise) preceded by the anchor-state pass: one bf16 MFMA online softmax over each row's anchor
 * region writes `state` and hands the per-row anchors x_a (the same MFMA sequence, so the
 * same values and the same lists as sa_estimate_mask) to the estimate.  v: device bf16
 * [B, seq, Hkv, d] (v_stride).  ws: at least sa_workspace_size(SA_OP_ESTIMATE_STATE, ...)
 * bytes (the estimate's workspace plus B * seq * Hq * 4 bytes of anchors). */
sa_status sa_estimate_mask_anchor_state(const sa_shape* shape, const sa_sparse_params* params,
                                        const void* q, const void* k, const void* v,
                                        const sa_lists* out, const sa_anchor_state* state,
                                        void* ws, size_t ws_bytes, hipStream_t stream);

/* sa_sparse_prefill resuming from an anchor state (block_k 64; block or column lists): row r
 * starts from state (o, lse) and adds the listed tokens j <= r outside A(r) (sink_tokens and
 * local_tokens of params define A(r); they and softmax_scale must be the ones the state was
 * made with); block tiles that lie wholly inside every row's anchor region, and listed
 * columns inside it, are skipped.  The result is the attention over A(r) and the listed
 * causal tokens, which for lists of the estimate (they hold the forced blocks or columns, a
 * superset of A(r)) is sa_sparse_prefill's result.  o, lse as in sa_sparse_prefill; the
 * state is read only. */
sa_status sa_sparse_prefill_resume(const sa_shape* shape, const sa_sparse_params* params,
                                   const void* q, const void* k, const void* v,
                                   const sa_lists* lists, const sa_anchor_state* state, void* o,
                                   float* lse, hipStream_t stream);

/* Block summaries for decode (SALE "The reading": one representative per key block):
 * kbar[b, J, g, :] = mean of the cached keys of block J (fp64 sum and divide, rounded to
 * fp32 then to bf16); blocks at or past cache_len[b] are written as zeros.
 * k_cache: device bf16 [B, seq_k, Hkv, d] (k_stride); cache_len: device int32 [B] with
 * cache_len[b] in [0, seq_k] (values outside are clamped on the device to that range); k_summary:
 * device bf16 [B, ceil(seq_k/block_k), Hkv, d],
 * contiguous. */
sa_status sa_build_block_summary(const sa_shape* shape, int32_t block_k,
                                 const void* k_cache, const int32_t* cache_len,
                                 void* k_summary, hipStream_t stream);

/* Sparse decode (SpotAttention Figure 2 with a training-free block score): per (b, g)
 * score every block J < ceil(cache_len[b]/block_k) by max over the group's heads of
 * c * q_h . kbar_J; select the forced blocks (overlapping [0, sink) or
 * [cache_len-local, cache_len-1]) plus the highest-scoring others (ties to the lower
 * block) up to top_k_blocks; then split-K attention of the single query (position
 * cache_len-1, seeing every cached token) over the selected blocks and an LSE merge.
 * q: device bf16 [B, Hq, d] (q_stride[0] = batch stride, q_stride[2] = head stride);
 * o: device bf16 [B, Hq, d] likewise (o_stride); lse: nullable device fp32 [B, Hq];
 * selected: nullable device int32 [B, Hkv, top_k_blocks], ascending, padded with -1 (with
 * top_p the number of entries before the padding is each (b, g)'s budget).  An empty cache
 * (cache_len[b] = 0 after clamping) selects nothing and gives o = 0 and lse = -inf.
 * ws: at least sa_workspace_size(SA_OP_DECODE, ...) bytes. */
sa_status sa_sparse_decode(const sa_shape* shape, const sa_decode_params* params,
                           const void* q, const void* k_cache, const void* v_cache,
                           const void* k_summary, const int32_t* cache_len,
                           void* o, float* lse, int32_t* selected,
                           void* ws, size_t ws_bytes, hipStream_t stream);

/* sa_sparse_decode without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  The call's scratch (block scores, the selection, per-split partial outputs)
 * lives in a static device array of SA_NOALLOC_SCRATCH_BYTES that the library holds on each GPU
 * it runs on until the process ends; its address is looked up once per device, on the first
 * call with that device current, and no call allocates or frees memory.  Every call on a GPU
 * uses that GPU's one array and may leave data in it: calls that overlap on one GPU (other
 * streams, other host threads) race, so the caller serialises them.  Arguments, results and
 * errors as sa_sparse_decode, plus SA_ERR_WORKSPACE when the call needs more scratch than
 * SA_NOALLOC_SCRATCH_BYTES (sa_workspace_size(SA_OP_DECODE, ...) gives the need: about 1.6 MB
 * at batch 16, 32/8 heads, a 128K-token cache, K = 64) and SA_ERR_DEVICE when the array's
 * device address cannot be obtained. */
#define SA_NOALLOC_SCRATCH_BYTES (16u << 20)
sa_status sa_sparse_decode_noalloc(const sa_shape* shape, const sa_decode_params* params,
                                   const void* q, const void* k_cache, const void* v_cache,
                                   const void* k_summary, const int32_t* cache_len,
                                   void* o, float* lse, int32_t* selected, hipStream_t stream);

/* 4-bit block summaries (SpotAttention, "Key findings": quantising the selector's key cache
 * to INT4 / FP4 shrinks it 3.5x at no accuracy cost).  From bf16 summaries (as written by
 * sa_build_block_summary, contiguous [B, ceil(seq_k/block_k), Hkv, d]) each row is cut into
 * groups of 32 dims; a group with a = max |x| gets scale = fp32(a / 7) rounded to bf16 and
 * codes clamp(rint_even(fp32(x * fp32(7 / a))), -7, 7) (zeros and scale 0 when a = 0).
 * codes: device uint8 [B, nKB, Hkv, d/2] holding offset-binary nibbles u = code + 8 (1..15):
 * each little-endian 32-bit word covers 8 consecutive dims, dim 2j in nibble j and dim 2j+1
 * in nibble j+4 (j = 0..3); scales: device bf16 [B, nKB, Hkv, d/32].  4.5 bits per dim.
 * Errors: the shape checks common to every entry point, SA_ERR_NULL for a null pointer,
 * SA_ERR_PARAM for block_k < 1, SA_ERR_SHAPE for a pointer not 16-byte aligned.
 * Asynchronous on the stream. */
sa_status sa_quantize_block_summary(const sa_shape* shape, int32_t block_k, const void* k_summary,
                                    void* codes, void* scales, hipStream_t stream);

/* sa_sparse_decode scoring the blocks from 4-bit summaries (scale * code per dim) instead
 * of bf16 ones; everything else as sa_sparse_decode, with the same workspace size. */
sa_status sa_sparse_decode_q4(const sa_shape* shape, const sa_decode_params* params,
                              const void* q, const void* k_cache, const void* v_cache,
                              const void* summary_codes, const void* summary_scales,
                              const int32_t* cache_len, void* o, float* lse, int32_t* selected,
                              void* ws, size_t ws_bytes, hipStream_t stream);

/* FP4 block summaries (SpotAttention, "Key findings": the selector's key cache quantised to
 * INT4 or FP4 microscale is 3.5x smaller at no accuracy cost), in the OCP Microscaling v1.0
 * MXFP4 format.  From bf16 summaries (contiguous [B, ceil(seq_k/block_k), Hkv, d], as
 * written by sa_build_block_summary) each row is cut into groups of 32 dims; a group with
 * a = max |x| gets the shared exponent e = floor(log2 a) - 2 clamped to [-127, 127] (-127
 * when a = 0 or a is subnormal) and each x the E2M1 code of |x| * 2^-e (grid 0, 0.5, 1, 1.5,
 * 2, 3, 4, 6 as codes 0..7, nearest with ties to the even code, saturating at 6) with the
 * sign bit of x in bit 3, so the summary is read as code value * 2^e.
 * codes: device uint8 [B, nKB, Hkv, d/2], dim 2k in the low and dim 2k+1 in the high nibble
 * of byte k of its row; exps: device uint8 [B, nKB, Hkv, d/32], the E8M0 byte e + 127.
 * 4.25 bits per dim.  Errors as sa_quantize_block_summary.  Asynchronous on the stream. */
sa_status sa_quantize_block_summary_fp4(const sa_shape* shape, int32_t block_k,
                                        const void* k_summary, void* codes, void* exps,
                                        hipStream_t stream);

/* sa_sparse_decode scoring the blocks from FP4 summaries (E2M1 value * 2^e per dim, from
 * sa_quantize_block_summary_fp4) instead of bf16 ones; everything else as sa_sparse_decode,
 * with the same workspace size.  SA_ERR_NULL for a null codes or exps pointer. */
sa_status sa_sparse_decode_fp4(const sa_shape* shape, const sa_decode_params* params,
                               const void* q, const void* k_cache, const void* v_cache,
                               const void* summary_codes, const void* summary_exps,
                               const int32_t* cache_len, void* o, float* lse, int32_t* selected,
                               void* ws, size_t ws_bytes, hipStream_t stream);

/* Per-head threshold calibration (SALE, "Assumptions & free parameters": the per-head
 * threshold tau starts at 0.008 and is halved until the L1 output error
 * Err(tau) = ||O - O~||_1 / N meets a user-chosen bound; the relative-score test keeps a
 * block when its score is at least tau times the anchor's, i.e. theta = -ln tau in the
 * logit units of Eq. (2)).  With this library's own passes: O is the attention with every
 * causal block kept (theta = +inf), O~ the estimate + sparse prefill with the current
 * thetas; Err_h = sum over batch, rows and head dims of |O - O~| for query head h, divided
 * by batch * seq (the rows).  Starting from theta_h = -ln(tau0), every head whose Err_h is
 * not below err_bound gets theta_h = -ln(tau0) + k_h ln 2 with k_h one larger, and the loop
 * repeats, at most max_halvings times; all heads are evaluated together each round (the
 * lists are unions over a KV head's query heads, so raising one head's theta can lower its
 * group mates' errors).  Block granularity only (SA_ERR_UNSUPPORTED for stripes).
 * params->theta is ignored.  theta_out: HOST float [n_q_heads], the calibrated thetas;
 * err_out: nullable HOST float [n_q_heads], each head's Err at its final theta;
 * halvings_out: nullable HOST int32 [n_q_heads], the k_h.  q, k, v as for
 * sa_sparse_prefill; ws: at least sa_workspace_size(SA_OP_CALIBRATE, ...) bytes (it holds
 * both outputs and the lists).  Unlike the other entry points this call is synchronous: it
 * reads the errors back every round and returns after the last one. */
sa_status sa_calibrate_theta(const sa_shape* shape, const sa_sparse_params* params,
                             const void* q, const void* k, const void* v,
                             float tau0, float err_bound, int32_t max_halvings,
                             float* theta_out, float* err_out, int32_t* halvings_out,
                             void* ws, size_t ws_bytes, hipStream_t stream);

/* Static description of a status code. */
const char* sa_status_string(sa_status status);

/* Debug build (libsa_debug.so, the same sources compiled with -DSA_DEBUG), for callers that
 * build their own lists or cache lengths.  The kernels then check the data that the release
 * kernels clamp -- each list's count in [0, stride], its entries inside the sequence's key
 * blocks (columns for stripe lists) and strictly ascending, each cache length in [0, seq_k] --
 * and sa_sparse_prefill(_resume), sa_sparse_decode(_q4, _fp4, _noalloc) and
 * sa_build_block_summary wait for their stream after the launches and return SA_ERR_CHECK when
 * a check failed (results are then those of the clamped data).  Bits of the last such call:
 * 1 a count outside [0, stride], 2 an entry out of range, 4 entries not strictly ascending,
 * 8 a cache length outside [0, seq_k].  The debug build allocates one 4-byte word per device on
 * its first checked call; the release build checks nothing, never waits and returns 0 here. */
uint32_t sa_debug_flags(void);

#ifdef __cplusplus
}
#endif
#endif /* SA_H_ */
