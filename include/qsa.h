/*
 * qsa.h -- C ABI of libqsa.so, the MI355X (gfx950) decode path of QSA
 * (Qwen Sparse Attention).
 *
 * Sources (web pages) cited below:
 *   [QSA-DCP]  "Qwen 4 QSA 迎来解码上下文并行：深入解读 vLLM 针对 Qwen3.8-Flash-Next 的
 *              草稿 PR" (orcarouter.ai blog), section "拉取请求实际改变了什么" (what the
 *              pull request actually changes): a lightweight indexer compresses keys
 *              into micro-blocks at ratio 4, scores them, keeps the best 512 blocks
 *              (about 2,048 tokens) and runs the final softmax and value aggregation
 *              over the uncompressed K/V at those positions; with decode context
 *              parallelism each rank reads its own slice of the main KV cache and
 *              the partial attention results are merged at the end; the selector
 *              and the main KV cache live in one cache group so they cannot drift;
 *              synthetic (dummy) batches must not write the indexer's side cache.
 *   [PR53896]  "PR #53896 完整报告" (prhub.com.cn report on vLLM PR #53896), section
 *              "实现拆解" (implementation breakdown): startup check that the compress
 *              ratio divides the KV block size; the indexer writes token keys into a
 *              raw-key ring and pools them by the compress ratio into a compressed
 *              key cache, then does a weight-free top-k on the compressed keys.
 *              Section "关键源码片段" (key source snippets), QSAIndexer: fixed-width
 *              int32 output padded with -1; a paged KV cache is required; a later
 *              MTP step may reuse the first step's selection.
 *
 * Conventions for every entry point
 *   - All array arguments are DEVICE pointers to caller-owned memory.  The
 *     library never allocates, frees or synchronises; every call only enqueues
 *     kernels on `stream` (0 = the null stream) and returns.
 *   - Arguments are validated on the host before anything is enqueued.  A
 *     failed check returns a status and enqueues nothing.  QSA_ERR_HIP means a
 *     launch failed (hipGetLastError after the launch); later kernels of the
 *     same call are then not enqueued.  qsa_last_error() describes the last
 *     failure on the calling thread.  No C++ exception crosses this ABI.
 *   - Data-dependent contracts (page ids inside the pool, seq_len within the
 *     block-table capacity, the bounds stated per call) are not checked on the
 *     device; violating them is undefined behaviour.
 *   - Calls that share a workspace, ring or output buffer must be ordered
 *     (same stream, or synchronised); overlapping calls on them race.
 *
 * Layouts (all row-major, innermost last)
 *   block_table  int32 [num_reqs, max_pages_per_req]: logical page -> physical page.
 *                One table serves both the K/V cache and the compressed-key cache
 *                ([QSA-DCP]: selector and main KV in one cache group).
 *   K/V cache    [num_pages, H_kv, page_size, head_dim]; bf16, or fp8 E4M3 (OCP)
 *                bytes with k_scale / v_scale fp32 [num_pages, page_size] (one
 *                scale per token per tensor).  Token t of request b is at page
 *                block_table[b][t / page_size], slot t % page_size.
 *   ckey cache   int8 [num_pages, page_size/4 * (D + D/4)]: micro-block j of a request
 *                lives in page block_table[b][4j / page_size], slot j % (page_size/4).
 *                Its exact integer key C (sum of 4 int8 keys, |C| <= 512) is stored
 *                losslessly in 10 bits per dimension: with v = C + 512,
 *                s = (v mod 256) - 128 (int8) and b0, b1 = bits 8 and 9 of v,
 *                C = 256*(2*b1 + b0) + s - 384.  Page layout: first the s plane as
 *                D/16 runs of [page_size/4 slots][16 bytes] (run r holds dims
 *                [16r, 16r+16) of every slot), then per slot D/4 mask bytes (b0 of
 *                dims 0..D-1, then b1; dim i is bit i%8 of byte i/8).
 *                Size: qsa_ckey_cache_bytes().
 *   ring         int8 [num_reqs, 8, D]: the raw keys of each request's last 8
 *                tokens (slot t % 8).  Only the open block's tokens are ever read.
 */
#ifndef QSA_H_
#define QSA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QSA_OK = 0,
  QSA_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, ratio != 4, ...     */
  QSA_ERR_UNSUPPORTED = 2,      /* valid but not built: head_dim, index_dim, ... */
  QSA_ERR_WORKSPACE = 3,        /* workspace missing or too small               */
  QSA_ERR_HIP = 4               /* a HIP launch failed                          */
} qsa_status;

typedef enum { QSA_KV_BF16 = 0, QSA_KV_FP8_E4M3 = 1 } qsa_kv_dtype;

/* Static shape of one QSA layer. */
typedef struct {
  int32_t num_q_heads;       /* H_q; a multiple of num_kv_heads                    */
  int32_t num_kv_heads;      /* H_kv; query head h reads KV head h / (H_q/H_kv)    */
  int32_t head_dim;          /* d: 64 or 128                                       */
  int32_t index_dim;         /* D: 32, 64 or 128                                   */
  int32_t compress_ratio;    /* tokens per micro-block; must be 4 ([QSA-DCP])      */
  int32_t topk_blocks;       /* k: 1..2048 (512 in [QSA-DCP])                      */
  int32_t page_size;         /* tokens per page: power of two, >= 16 ([PR53896]:
                                the ratio must divide the block size)             */
  int32_t max_pages_per_req; /* row stride of block_table                         */
  int32_t ring_size;         /* slots of the raw-key ring per request: must be 8
                                (QSA_RING_SIZE; [PR53896]: the indexer keeps the
                                latest token keys in a ring before pooling)       */
  int32_t kv_dtype;          /* qsa_kv_dtype                                       */
  float softmax_scale;       /* logits are scale * q.k (1/sqrt(d) usually)         */
} qsa_config;

/* Raw-key ring slots per request (qsa_config.ring_size): the last 8 tokens. */
#define QSA_RING_SIZE 8

/* Largest context one row may have: 2^21 micro-blocks (8,388,608 tokens). */
#define QSA_MAX_SEQ_LEN (4 * (1 << 21))

/* Bytes of the compressed-key cache for `num_pages` pages; 0 on a bad config. */
size_t qsa_ckey_cache_bytes(const qsa_config* cfg, int64_t num_pages);

/*
 * qsa_compress -- append new tokens' indexer keys; close micro-blocks.
 *   [QSA-DCP] keys are compressed into micro-blocks of 4 tokens; [PR53896] the
 *   raw keys go through a ring and are pooled into the compressed key cache.
 *
 * Request b (0 <= b < num_reqs) appends rows [new_cu[b], new_cu[b+1]) of
 * new_keys (int8 [T_new, D]) as tokens seq_len_before[b], seq_len_before[b]+1, ...
 * Every micro-block j whose last token 4j+3 is among them gets
 * C_j = k_{4j} + k_{4j+1} + k_{4j+2} + k_{4j+3} written to ckey_cache; keys of
 * tokens before seq_len_before[b] that C_j needs come from ring[b]; the last
 * (up to 8) new tokens are written to ring[b].  Any number of new tokens and
 * any seq_len_before are handled (bulk prefill and decode alike).
 * Rollback ([PR53896]: MTP draft steps keep updating the side cache, and
 * rejected draft tokens must not stay in it): a call may restart from an
 * earlier length L (seq_len_before[b] = L after the caller drops rejected
 * tokens) if the last call that wrote request b ended at most
 * 4*floor(L/4) + 8 tokens in, i.e. up to 8 - L%4 (>= 5) tokens are dropped.
 * Blocks that the dropped tokens closed are rewritten when they close again;
 * scans never read them before (they lie past floor(L/4)).
 * Requests with seq_len_before[b] < 0 or no new tokens write nothing
 * ([QSA-DCP]: dummy batches must not write the side cache).
 *   max_new_tokens: host-side upper bound of new_cu[b+1]-new_cu[b] (sizes the grid;
 *                   a larger count is still handled correctly, just slower).
 * Errors: INVALID_ARGUMENT (null pointer, num_reqs < 0, bad config),
 *         UNSUPPORTED (index_dim), HIP.
 */
qsa_status qsa_compress(const qsa_config* cfg, int32_t num_reqs, int32_t max_new_tokens,
                        const int8_t* new_keys, const int32_t* new_cu,
                        const int32_t* seq_len_before, const int32_t* block_table,
                        int8_t* ring, int8_t* ckey_cache, hipStream_t stream);

/*
 * Workspace of qsa_index_topk for num_sel_rows rows of context <= max_seq_len.
 * Returns 0 on a bad argument.  Before its FIRST use a workspace must be
 * cleared with qsa_index_topk_workspace_init(), and again before it serves
 * calls with another num_sel_rows or max_seq_len (its layout follows them).
 * Every call that selects (an index call with topk != NULL, or
 * qsa_select_sparse_decode after a scoring call) leaves it ready for the next
 * call, so later calls need no clearing.
 */
size_t qsa_index_topk_workspace_size(const qsa_config* cfg, int32_t num_sel_rows,
                                     int32_t max_seq_len);
qsa_status qsa_index_topk_workspace_init(void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * qsa_index_topk -- score every closed micro-block against the indexer query
 * and keep the best k.  [QSA-DCP]: keep the best 512 blocks; [PR53896]:
 * weight-free top-k over the compressed keys, fixed-width int32 output padded
 * with -1.
 *
 * Selecting row s (0 <= s < num_sel_rows) belongs to request sel_req[s] and has
 * context L = sel_seq_len[s] (all cached tokens, its own included).  Blocks
 * j < floor(L/4) are scored exactly: score_j = sum_i q_index[s][i] * C_j[i]
 * (int32, no overflow for D <= 128).  The best min(k, floor(L/4)) blocks by
 * (score descending, block index ascending) are written to topk[s] (int32 [S, k])
 * in ascending block order, followed by -1.  Rows with L < 4 get all -1.
 * Ties are broken towards the lower block index, so the result is unique.
 * sel_req[s] must be a row of block_table even for a row with nothing to
 * select (a dummy row is sel_seq_len[s] = 0 with any valid request id): the
 * calls read that row's page-table entries.
 *   max_seq_len: host-side bound of sel_seq_len (<= QSA_MAX_SEQ_LEN); it sizes
 *                the grid and the workspace.  Rows longer than it are treated
 *                as max_seq_len long.
 *   topk == NULL: score only.  The exact int32 scores are left in the first
 *                num_sel_rows * nb_stride * 4 bytes of the workspace
 *                (row s, block j at int32 index s * nb_stride + j, nb_stride =
 *                max_seq_len/4 rounded up to a multiple of 1024).  Nothing is
 *                selected, and the histogram counters stay set: the workspace
 *                is then ready for qsa_select_sparse_decode only; any other
 *                call on it needs qsa_index_topk_workspace_init() first.
 * Errors: INVALID_ARGUMENT, UNSUPPORTED (index_dim), WORKSPACE, HIP.
 */
qsa_status qsa_index_topk(const qsa_config* cfg, int32_t num_sel_rows, int32_t max_seq_len,
                          const int8_t* q_index, const int32_t* sel_req,
                          const int32_t* sel_seq_len, const int32_t* block_table,
                          const int8_t* ckey_cache, int32_t* topk,
                          void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * qsa_index_topk_noalloc -- qsa_index_topk without a caller workspace, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  The work space is
 * the library's own device array of QSA_NOALLOC_SCRATCH_BYTES (16 MiB), one per
 * GPU, held until the process ends; the call allocates and frees nothing.
 *   Arguments and results as qsa_index_topk, except that topk is required.
 *   The scratch is shared by every call on a GPU and keeps the last call's
 *   contents (each call first zeroes the part it reads before writing, with a
 *   fill kernel): calls that overlap on one GPU race, so order them (one
 *   stream, or synchronised).  Sizes: qsa_index_topk_workspace_size(cfg,
 *   num_sel_rows, max_seq_len) must not exceed the scratch (for example 12
 *   selecting rows of 262,144 tokens fit).
 * Errors: INVALID_ARGUMENT, UNSUPPORTED (index_dim), WORKSPACE (too large for
 *         the scratch), HIP.
 */
#define QSA_NOALLOC_SCRATCH_BYTES (16u << 20)

qsa_status qsa_index_topk_noalloc(const qsa_config* cfg, int32_t num_sel_rows, int32_t max_seq_len,
                                  const int8_t* q_index, const int32_t* sel_req, const int32_t* sel_seq_len,
                                  const int32_t* block_table, const int8_t* ckey_cache, int32_t* topk,
                                  hipStream_t stream);

/*
 * qsa_compress_index_topk -- qsa_compress followed by qsa_index_topk, in one
 * scan launch (plus the selection), for decode-sized appends.  [QSA-DCP]: each
 * decode step appends the new tokens' keys to the compressed side cache and
 * the indexer then keeps the best 512 blocks; [PR53896]: ring, pooling into
 * the compressed cache, weight-free top-k with -1 padding.
 *
 * The arguments are those of the two calls (cfg and block_table are shared):
 * request b < num_reqs appends rows [new_cu[b], new_cu[b+1]) of new_keys after
 * seq_len_before[b] tokens, and selecting row s < num_sel_rows (request
 * sel_req[s], context sel_seq_len[s]) is scored over the cache as it stands
 * after the append.  ring, ckey_cache, topk and the workspace end exactly as
 * after qsa_compress(...) then qsa_index_topk(...) on the same stream, bit for
 * bit; the rollback rule of qsa_compress holds unchanged.
 *   max_new_tokens: 0..5, a bound on every request's new token count (that
 *                   many tokens never overwrite the ring slots that the scan
 *                   reads for the block straddling seq_len_before[b]).  A
 *                   request with more new tokens than that is undefined.
 *   sel_req[s] outside [0, num_reqs) reads the cache as it stands (no tokens
 *                   of this call).
 *   new_keys, ring: 4-byte aligned; topk == NULL scores only, as in
 *                   qsa_index_topk.  num_sel_rows = 0 only appends (as
 *                   qsa_compress), num_reqs = 0 only selects.
 * Errors: INVALID_ARGUMENT (as either call, or max_new_tokens > 5),
 *         UNSUPPORTED (index_dim), WORKSPACE, HIP.
 */
qsa_status qsa_compress_index_topk(const qsa_config* cfg, int32_t num_reqs, int32_t max_new_tokens,
                                   const int8_t* new_keys, const int32_t* new_cu,
                                   const int32_t* seq_len_before, int8_t* ring,
                                   int32_t num_sel_rows, int32_t max_seq_len,
                                   const int8_t* q_index, const int32_t* sel_req,
                                   const int32_t* sel_seq_len, const int32_t* block_table,
                                   int8_t* ckey_cache, int32_t* topk,
                                   void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * qsa_prefill_index_topk -- qsa_index_topk for a chunk of prefill query rows:
 * many rows per request, each with its own causal length (sparse / chunked
 * prefill; [QSA-DCP], section on why the pull request matters, names a native
 * sparse-prefill kernel for the QSA path as companion work).  [QSA-DCP]: the
 * indexer keeps the best 512 compressed blocks per query; [PR53896]:
 * weight-free top-k, fixed-width int32 output padded with -1.
 *
 * Rows r in [row_cu[b], row_cu[b+1]) belong to request b (row_cu int32 [B+1],
 * row_cu[0] = 0, row_cu[B] = num_rows, at most max_rows_per_req rows per
 * request); row r has context L = row_seq_len[r].  topk[r] is exactly what
 * qsa_index_topk gives for a selecting row with sel_req = b and sel_seq_len =
 * row_seq_len[r].  The scan is a GEMM (int8 MFMA, 16 rows x 16 blocks per
 * instruction): each compressed block is read once per 16 rows instead of once
 * per row.
 *   q_index int8 [num_rows, D] (16-byte aligned); workspace: from
 *   qsa_index_topk_workspace_size(cfg, num_rows, max_seq_len), initialised
 *   once; topk == NULL leaves the scores (layout as for qsa_index_topk) and
 *   histogram counters set.
 * Errors: INVALID_ARGUMENT, UNSUPPORTED (index_dim), WORKSPACE, HIP.
 */
qsa_status qsa_prefill_index_topk(const qsa_config* cfg, int32_t num_reqs, int32_t num_rows,
                                  int32_t max_rows_per_req, int32_t max_seq_len,
                                  const int8_t* q_index, const int32_t* row_cu,
                                  const int32_t* row_seq_len, const int32_t* block_table,
                                  const int8_t* ckey_cache, int32_t* topk,
                                  void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * qsa_sparse_decode -- attention of the query rows over the selected tokens,
 * as num_splits partial results.  [QSA-DCP]: softmax and value aggregation over
 * the uncompressed K/V at the kept positions; with decode context parallelism
 * each rank reads its own slice of the main KV cache and yields a partial
 * result, merged at the end (qsa_merge_partials).
 *
 * Query row r (0 <= r < num_rows) uses selecting row s = row_sel[r]: request
 * sel_req[s], selection topk[s] ([PR53896]: a later MTP step reuses the first
 * step's selection; any number of draft rows per request, in any order).  It
 * attends tokens {4j..4j+3 : j in topk[s], j >= 0} plus its own tail
 * [4*floor(sel_seq_len[s]/4), row_seq_len[r]) (the open block the selecting
 * row could not score); row_seq_len[r] >= sel_seq_len[s] is required.
 *   row_sel  int32 [num_rows], or NULL: row r is selecting row r (then
 *            num_rows == num_sel_rows and max_rows_per_sel == 1).  Rows with
 *            row_sel[r] outside [0, num_sel_rows), and rows past the first
 *            max_rows_per_sel (in index order) of one selecting row, are not
 *            attended: their o_part / lse_part entries are not written.
 * Split p of P owns a contiguous stretch of the selecting row's context: the
 * run of entries [floor(p*n/P), floor((p+1)*n/P)) of its n = min(k, nb)
 * ascending selected blocks (nb = floor(sel_seq_len/4)), so every split takes
 * a near-equal share of the selection; split P-1 also owns the tail.  For
 * query head h (KV head h / (H_q/H_kv)):
 *   z_t = softmax_scale * q[r][h] . K_t   (fp8: times k_scale of token t)
 *   lse_part[p][r][h] = log sum_t exp(z_t)                 (natural log)
 *   o_part[p][r][h][:] = sum_t exp(z_t - lse) V_t          (fp8: V_t * v_scale_t)
 * A split without tokens gives o_part = 0, lse_part = -inf.
 *   q        bf16 [num_rows, H_q, d]
 *   topk     int32 [num_sel_rows, k]: ascending block ids, then -1 (as qsa_index_topk writes)
 *   o_part   fp32 [P, num_rows, H_q, d];  lse_part fp32 [P, num_rows, H_q]
 *   num_splits in [1, 64]; max_rows_per_sel * (H_q/H_kv) <= 64.
 *   k_scale / v_scale are required for fp8 and ignored for bf16.
 * Errors: INVALID_ARGUMENT, UNSUPPORTED (head_dim, group size), HIP.
 */
qsa_status qsa_sparse_decode(const qsa_config* cfg, int32_t num_rows, int32_t num_sel_rows,
                             int32_t max_rows_per_sel, int32_t num_splits, const void* q,
                             const int32_t* row_sel, const int32_t* row_seq_len,
                             const int32_t* sel_req, const int32_t* sel_seq_len,
                             const int32_t* topk, const int32_t* block_table,
                             const void* k_cache, const void* v_cache,
                             const float* k_scale, const float* v_scale,
                             float* o_part, float* lse_part, hipStream_t stream);

/*
 * qsa_select_sparse_decode -- the selection step of qsa_index_topk and
 * qsa_sparse_decode on its result, in one call ([QSA-DCP]: keep the best 512
 * blocks, then softmax and value aggregation over the kept positions, as
 * context-parallel partials).  Its outputs are exactly those of
 *   qsa_index_topk(..., topk, workspace, ...)   (the selection half), then
 *   qsa_sparse_decode(cfg, num_rows, num_sel_rows, max_rows_per_sel, num_splits, ...)
 * on a workspace left by a scoring call with topk == NULL (qsa_index_topk,
 * qsa_compress_index_topk or qsa_prefill_index_topk) for the same
 * num_sel_rows, max_seq_len and sel_seq_len; topk (int32 [S, k]) is written as
 * that selection would write it, and the partials are the same, bit for bit.
 * The workspace is left clean (as after a selecting call).  One kernel does
 * both (qsa_select_sparse_decode_launches returns 1) when the grid of
 * P x H_kv x row groups x S workgroups has fewer than 512 (row groups: the
 * fewest groups of query rows whose heads fit one workgroup, 8 heads at
 * head_dim 128 and 16 at 64) and a row's selection bitmap fits the LDS
 * (max_seq_len up to about 1,048,576 tokens): each workgroup finds its row's
 * selection itself and lists only its own run, so the attention starts
 * without a launch boundary.  Otherwise the two kernels run one after the
 * other.
 *   Arguments as in the two calls: workspace from
 *   qsa_index_topk_workspace_size(cfg, num_sel_rows, max_seq_len); topk is
 *   required; num_rows = 0 only selects.
 * Errors: INVALID_ARGUMENT, UNSUPPORTED (index_dim, head_dim, group size),
 *         WORKSPACE, HIP.
 */
qsa_status qsa_select_sparse_decode(const qsa_config* cfg, int32_t num_rows, int32_t num_sel_rows,
                                    int32_t max_rows_per_sel, int32_t num_splits, int32_t max_seq_len,
                                    const void* q, const int32_t* row_sel, const int32_t* row_seq_len,
                                    const int32_t* sel_req, const int32_t* sel_seq_len,
                                    const int32_t* block_table, const void* k_cache, const void* v_cache,
                                    const float* k_scale, const float* v_scale, int32_t* topk,
                                    float* o_part, float* lse_part,
                                    void* workspace, size_t ws_bytes, hipStream_t stream);

/* Kernel launches qsa_select_sparse_decode makes for this shape: 1 (selection
 * and attention in one kernel) or 2 (finalize, then attention); 0 on a bad
 * argument.  Enqueues nothing. */
int32_t qsa_select_sparse_decode_launches(const qsa_config* cfg, int32_t num_sel_rows, int32_t max_rows_per_sel,
                                          int32_t num_splits, int32_t max_seq_len);

/*
 * qsa_merge_partials -- log-sum-exp merge of the split partials ([QSA-DCP]:
 * partial attention results of the context partitions are merged at the end).
 *   lse[r][h] = M + log sum_p exp(lse_part[p][r][h] - M),  M = max_p lse_part
 *   out[r][h] = sum_p exp(lse_part[p][r][h] - lse[r][h]) * o_part[p][r][h]
 * If every split is empty (all -inf): out = 0, lse = -inf.
 *   o_part fp32 [P, R, H, d], lse_part fp32 [P, R, H], lse fp32 [R, H];
 *   out [R, H, d] is fp32 (out_dtype QSA_OUT_F32) or bf16 rounded to nearest
 *   even from the same fp32 value (QSA_OUT_BF16).
 *   num_splits in [1, 64]; head_dim 64 or 128.
 * Errors: INVALID_ARGUMENT, UNSUPPORTED (head_dim), HIP.
 */
typedef enum { QSA_OUT_F32 = 0, QSA_OUT_BF16 = 1 } qsa_out_dtype;

qsa_status qsa_merge_partials(int32_t num_splits, int32_t num_rows, int32_t num_heads,
                              int32_t head_dim, const float* o_part, const float* lse_part,
                              void* out, int32_t out_dtype, float* lse, hipStream_t stream);

/*
 * qsa_indexer_project -- the indexer front end: hidden states to the int8
 * indexer query and keys that qsa_index_topk / qsa_compress take.
 * [PR53896] (key source snippets, QSAIndexer): Q and K are projected from the
 * hidden states, normalised with a Gemma-style RMSNorm and rotated by a 1-D
 * rotary embedding before K enters the raw-key ring and Q selects.  For token
 * t at position positions[t]:
 *   [q | k] = hidden[t] . w_qk^T     (w_qk bf16 [2D, H]: rows 0..D-1 give q, D..2D-1 give k)
 *   x = x / sqrt(mean(x^2) + 1e-6) * (1 + g)            (g_q fp32 [D] for q, g_k for k)
 *   (x_i, x_{i+D/2}) rotated by positions[t] * rope_base^(-2i/D), i < D/2
 *   out = clamp(round-half-even(x * scale), -127, 127)  (q_scale, k_scale)
 *   hidden bf16 [T, H] (H a multiple of 32), 16-byte aligned like w_qk;
 *   q_index, keys int8 [T, D]; index_dim D in {32, 64, 128}.
 * Sums are fp32 over bf16 products (slices of H summed in a fixed order, so
 * results are deterministic): a value within ~1e-4 of a rounding boundary may
 * round either way.
 *   workspace: device scratch of at least
 *   qsa_indexer_project_workspace_size(num_tokens, hidden_dim, index_dim) bytes,
 *   16-byte aligned, no initialisation; calls sharing it must be ordered.
 * Errors: INVALID_ARGUMENT, UNSUPPORTED (index_dim), WORKSPACE, HIP.
 */
size_t qsa_indexer_project_workspace_size(int32_t num_tokens, int32_t hidden_dim, int32_t index_dim);
qsa_status qsa_indexer_project(int32_t num_tokens, int32_t hidden_dim, int32_t index_dim, const void* hidden,
                               const int32_t* positions, const void* w_qk, const float* g_q, const float* g_k,
                               float rope_base, float q_scale, float k_scale, int8_t* q_index, int8_t* keys,
                               void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * qsa_indexer_project_mrope -- qsa_indexer_project with the multimodal rotary
 * embedding.  [PR53896] (key source snippets, QSAIndexer): the AMD indexer
 * combines the Gemma RMSNorm with a 1-D or an MRoPE rotation, and its forward
 * takes positions with a leading component axis (positions[..., :num_tokens]).
 * Here positions is int32 [3, T]: the temporal, height and width components of
 * every token (row c, column t).  The D/2 rotation frequencies are split into
 * three contiguous sections of section_t, section_h and section_w frequencies;
 * pair (x_i, x_{i+D/2}) turns by p_c[t] * rope_base^(-2i/D) with c the section
 * of i (0 for i < section_t, 1 for i < section_t + section_h, else 2).  A
 * token whose three components are equal (text) gets exactly what
 * qsa_indexer_project gives at that position.  Everything else, the
 * workspace included, as qsa_indexer_project.
 *   section_t, section_h, section_w >= 0 with sum index_dim / 2.
 * Errors: INVALID_ARGUMENT (also for the sections), UNSUPPORTED, WORKSPACE, HIP.
 */
qsa_status qsa_indexer_project_mrope(int32_t num_tokens, int32_t hidden_dim, int32_t index_dim, const void* hidden,
                                     const int32_t* positions, int32_t section_t, int32_t section_h,
                                     int32_t section_w, const void* w_qk, const float* g_q, const float* g_k,
                                     float rope_base, float q_scale, float k_scale, int8_t* q_index, int8_t* keys,
                                     void* workspace, size_t ws_bytes, hipStream_t stream);

/* Human-readable name of a status. */
const char* qsa_status_string(qsa_status status);

/* Description of the last failed call on this thread ("" if none). */
const char* qsa_last_error(void);

/* Library version, e.g. "qsa-mi355x 0.1.0". */
const char* qsa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QSA_H_ */
