// Host entry points of libqsa.so: argument validation, then kernel launches.
// Every check runs before anything is enqueued; see include/qsa.h for the
// contract of each call.
#include <cmath>
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "qsa.h"
#include "qsa_internal.h"

namespace qsa {

static thread_local char g_err[512];

qsa_status fail(qsa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

qsa_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(QSA_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return QSA_OK;
}

static bool is_pow2(int32_t x) { return x > 0 && (x & (x - 1)) == 0; }
static bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Shape checks common to the calls that take a qsa_config.
static qsa_status check_config(const qsa_config* c, bool need_index, bool need_attn) {
  if (!c) return fail(QSA_ERR_INVALID_ARGUMENT, "cfg is NULL");
  if (c->compress_ratio != 4)
    return fail(QSA_ERR_INVALID_ARGUMENT, "compress_ratio must be 4 (got %d)", c->compress_ratio);
  if (c->ring_size != QSA_RING_SIZE)
    return fail(QSA_ERR_INVALID_ARGUMENT, "ring_size must be %d (got %d)", QSA_RING_SIZE, c->ring_size);
  if (c->page_size < 16 || !is_pow2(c->page_size) || c->page_size % c->compress_ratio)
    return fail(QSA_ERR_INVALID_ARGUMENT,
                "page_size must be a power of two >= 16 divisible by the compress ratio (got %d)",
                c->page_size);
  if (c->max_pages_per_req < 1)
    return fail(QSA_ERR_INVALID_ARGUMENT, "max_pages_per_req must be >= 1 (got %d)", c->max_pages_per_req);
  if (c->topk_blocks < 1 || c->topk_blocks > 2048)
    return fail(QSA_ERR_INVALID_ARGUMENT, "topk_blocks must be in [1, 2048] (got %d)", c->topk_blocks);
  if (need_index) {
    if (c->index_dim < 1)
      return fail(QSA_ERR_INVALID_ARGUMENT, "index_dim must be positive (got %d)", c->index_dim);
    if (c->index_dim != 32 && c->index_dim != 64 && c->index_dim != 128)
      return fail(QSA_ERR_UNSUPPORTED, "index_dim %d not built (32, 64, 128)", c->index_dim);
  }
  if (need_attn) {
    if (c->num_kv_heads < 1 || c->num_q_heads < 1 || c->num_q_heads % c->num_kv_heads)
      return fail(QSA_ERR_INVALID_ARGUMENT, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                  c->num_q_heads, c->num_kv_heads);
    if (c->num_kv_heads > 65535) return fail(QSA_ERR_INVALID_ARGUMENT, "num_kv_heads too large");
    if (c->head_dim < 1) return fail(QSA_ERR_INVALID_ARGUMENT, "head_dim must be positive (got %d)", c->head_dim);
    if (c->head_dim != 64 && c->head_dim != 128)
      return fail(QSA_ERR_UNSUPPORTED, "head_dim %d not built (64, 128)", c->head_dim);
    if (c->kv_dtype != QSA_KV_BF16 && c->kv_dtype != QSA_KV_FP8_E4M3)
      return fail(QSA_ERR_UNSUPPORTED, "kv_dtype %d not supported", c->kv_dtype);
    if (!(c->softmax_scale > 0.f) || c->softmax_scale > 1e30f)
      return fail(QSA_ERR_INVALID_ARGUMENT, "softmax_scale must be positive and finite");
  }
  return QSA_OK;
}

}  // namespace qsa

using namespace qsa;

extern "C" {

size_t qsa_ckey_cache_bytes(const qsa_config* cfg, int64_t num_pages) {
  if (check_config(cfg, true, false) != QSA_OK || num_pages < 0) return 0;
  // per micro-block: D bytes of the s plane + D/4 bytes of the two bit-masks
  return (size_t)num_pages * (size_t)cfg->page_size / 4 * ((size_t)cfg->index_dim + (size_t)cfg->index_dim / 4);
}

qsa_status qsa_compress(const qsa_config* cfg, int32_t num_reqs, int32_t max_new_tokens,
                        const int8_t* new_keys, const int32_t* new_cu,
                        const int32_t* seq_len_before, const int32_t* block_table,
                        int8_t* ring, int8_t* ckey_cache, hipStream_t stream) {
  qsa_status st = check_config(cfg, true, false);
  if (st != QSA_OK) return st;
  if (num_reqs < 0 || num_reqs > 65535)
    return fail(QSA_ERR_INVALID_ARGUMENT, "num_reqs must be in [0, 65535] (got %d)", num_reqs);
  if (max_new_tokens < 0)
    return fail(QSA_ERR_INVALID_ARGUMENT, "max_new_tokens must be >= 0 (got %d)", max_new_tokens);
  if (num_reqs == 0) return QSA_OK;
  if (!new_cu || !seq_len_before || !block_table || !ring || !ckey_cache)
    return fail(QSA_ERR_INVALID_ARGUMENT, "qsa_compress: NULL array argument");
  if (!new_keys && max_new_tokens > 0)
    return fail(QSA_ERR_INVALID_ARGUMENT, "qsa_compress: new_keys is NULL");
  if (!aligned(ckey_cache, 16) || !aligned(ring, 4) || (new_keys && !aligned(new_keys, 4)))
    return fail(QSA_ERR_INVALID_ARGUMENT, "qsa_compress: ckey_cache needs 16-byte, ring/new_keys 4-byte alignment");
  return launch_compress(*cfg, num_reqs, max_new_tokens, new_keys, new_cu, seq_len_before,
                         block_table, ring, ckey_cache, stream);
}

size_t qsa_index_topk_workspace_size(const qsa_config* cfg, int32_t num_sel_rows, int32_t max_seq_len) {
  if (check_config(cfg, true, false) != QSA_OK) return 0;
  if (num_sel_rows < 0 || num_sel_rows > 65535 || max_seq_len < 0 || max_seq_len > QSA_MAX_SEQ_LEN) return 0;
  return topk_workspace_layout(num_sel_rows, max_seq_len).total;
}

qsa_status qsa_index_topk_workspace_init(void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (!workspace) return fail(QSA_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned(workspace, 256)) return fail(QSA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  return launch_ws_clear(workspace, ws_bytes, stream);
}

qsa_status qsa_index_topk(const qsa_config* cfg, int32_t num_sel_rows, int32_t max_seq_len,
                          const int8_t* q_index, const int32_t* sel_req,
                          const int32_t* sel_seq_len, const int32_t* block_table,
                          const int8_t* ckey_cache, int32_t* topk,
                          void* workspace, size_t ws_bytes, hipStream_t stream) {
  qsa_status st = check_config(cfg, true, false);
  if (st != QSA_OK) return st;
  if (num_sel_rows < 0 || num_sel_rows > 65535)
    return fail(QSA_ERR_INVALID_ARGUMENT, "num_sel_rows must be in [0, 65535] (got %d)", num_sel_rows);
  if (max_seq_len < 0 || max_seq_len > QSA_MAX_SEQ_LEN)
    return fail(QSA_ERR_INVALID_ARGUMENT, "max_seq_len must be in [0, %d] (got %d)", QSA_MAX_SEQ_LEN, max_seq_len);
  if (num_sel_rows == 0) return QSA_OK;
  if (!q_index || !sel_req || !sel_seq_len || !block_table || !ckey_cache)
    return fail(QSA_ERR_INVALID_ARGUMENT, "qsa_index_topk: NULL array argument");
  if (!aligned(ckey_cache, 16) || !aligned(q_index, 4))
    return fail(QSA_ERR_INVALID_ARGUMENT, "qsa_index_topk: ckey_cache needs 16-byte, q_index 4-byte alignment");
  TopkWorkspace lay = topk_workspace_layout(num_sel_rows, max_seq_len);
  if (!workspace) return fail(QSA_ERR_WORKSPACE, "qsa_index_topk: workspace is NULL");
  if (!aligned(workspace, 256)) return fail(QSA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < lay.total)
    return fail(QSA_ERR_WORKSPACE, "qsa_index_topk: workspace has %zu bytes, needs %zu", ws_bytes, lay.total);
  return launch_index_topk(*cfg, num_sel_rows, max_seq_len, q_index, sel_req, sel_seq_len,
                           block_table, ckey_cache, topk, lay, workspace, stream);
}

qsa_status qsa_index_topk_noalloc(const qsa_config* cfg, int32_t num_sel_rows, int32_t max_seq_len,
                                  const int8_t* q_index, const int32_t* sel_req, const int32_t* sel_seq_len,
                                  const int32_t* block_table, const int8_t* ckey_cache, int32_t* topk,
                                  hipStream_t stream) {
  qsa_status st = check_config(cfg, true, false);
  if (st != QSA_OK) return st;
  if (num_sel_rows < 0 || num_sel_rows > 65535)
    return fail(QSA_ERR_INVALID_ARGUMENT, "num_sel_rows must be in [0, 65535] (got %d)", num_sel_rows);
  if (max_seq_len < 0 || max_seq_len > QSA_MAX_SEQ_LEN)
    return fail(QSA_ERR_INVALID_ARGUMENT, "max_seq_len must be in [0, %d] (got %d)", QSA_MAX_SEQ_LEN, max_seq_len);
  if (num_sel_rows == 0) return QSA_OK;
  if (!q_index || !sel_req || !sel_seq_len || !block_table || !ckey_cache || !topk)
    return fail(QSA_ERR_INVALID_ARGUMENT, "qsa_index_topk_noalloc: NULL array argument");
  if (!aligned(ckey_cache, 16) || !aligned(q_index, 4))
    return fail(QSA_ERR_INVALID_ARGUMENT,
                "qsa_index_topk_noalloc: ckey_cache needs 16-byte, q_index 4-byte alignment");
  const size_t need = topk_workspace_layout(num_sel_rows, max_seq_len).total;
  if (need > (size_t)QSA_NOALLOC_SCRATCH_BYTES)
    return fail(QSA_ERR_WORKSPACE,
                "qsa_index_topk_noalloc: %d rows of up to %d tokens need %zu bytes of scratch, more than the "
                "library's %zu; use qsa_index_topk with a workspace of qsa_index_topk_workspace_size bytes",
                num_sel_rows, max_seq_len, need, (size_t)QSA_NOALLOC_SCRATCH_BYTES);
  return launch_index_topk_noalloc(*cfg, num_sel_rows, max_seq_len, q_index, sel_req, sel_seq_len, block_table,
                                   ckey_cache, topk, stream);
}

qsa_status qsa_compress_index_topk(const qsa_config* cfg, int32_t num_reqs, int32_t max_new_tokens,
                                   const int8_t* new_keys, const int32_t* new_cu,
                                   const int32_t* seq_len_before, int8_t* ring,
                                   int32_t num_sel_rows, int32_t max_seq_len,
                                   const int8_t* q_index, const int32_t* sel_req,
                                   const int32_t* sel_seq_len, const int32_t* block_table,
                                   int8_t* ckey_cache, int32_t* topk,
                                   void* workspace, size_t ws_bytes, hipStream_t stream) {
  qsa_status st = check_config(cfg, true, false);
  if (st != QSA_OK) return st;
  if (num_reqs < 0 || num_reqs > 65535)
    return fail(QSA_ERR_INVALID_ARGUMENT, "num_reqs must be in [0, 65535] (got %d)", num_reqs);
  if (max_new_tokens < 0 || max_new_tokens > 5)
    return fail(QSA_ERR_INVALID_ARGUMENT,
                "qsa_compress_index_topk: max_new_tokens must be in [0, 5] (got %d); use qsa_compress and "
                "qsa_index_topk for longer appends", max_new_tokens);
  if (num_sel_rows < 0 || num_sel_rows > 65535)
    return fail(QSA_ERR_INVALID_ARGUMENT, "num_sel_rows must be in [0, 65535] (got %d)", num_sel_rows);
  if (max_seq_len < 0 || max_seq_len > QSA_MAX_SEQ_LEN)
    return fail(QSA_ERR_INVALID_ARGUMENT, "max_seq_len must be in [0, %d] (got %d)", QSA_MAX_SEQ_LEN, max_seq_len);
  if (num_reqs == 0 && num_sel_rows == 0) return QSA_OK;
  if (!block_table || !ckey_cache)
    return fail(QSA_ERR_INVALID_ARGUMENT, "qsa_compress_index_topk: NULL array argument");
  if (num_reqs > 0) {
    if (!new_cu || !seq_len_before || !ring)
      return fail(QSA_ERR_INVALID_ARGUMENT, "qsa_compress_index_topk: NULL append argument");
    if (!new_keys && max_new_tokens > 0)
      return fail(QSA_ERR_INVALID_ARGUMENT, "qsa_compress_index_topk: new_keys is NULL");
    if (!aligned(ring, 4) || (new_keys && !aligned(new_keys, 4)))
      return fail(QSA_ERR_INVALID_ARGUMENT, "qsa_compress_index_topk: ring and new_keys need 4-byte alignment");
  }
  if (!aligned(ckey_cache, 16))
    return fail(QSA_ERR_INVALID_ARGUMENT, "qsa_compress_index_topk: ckey_cache needs 16-byte alignment");
  if (num_sel_rows > 0) {
    if (!q_index || !sel_req || !sel_seq_len)
      return fail(QSA_ERR_INVALID_ARGUMENT, "qsa_compress_index_topk: NULL selection argument");
    if (!aligned(q_index, 4))
      return fail(QSA_ERR_INVALID_ARGUMENT, "qsa_compress_index_topk: q_index needs 4-byte alignment");
  }
  TopkWorkspace lay = topk_workspace_layout(num_sel_rows, max_seq_len);
  if (num_sel_rows > 0) {
    if (!workspace) return fail(QSA_ERR_WORKSPACE, "qsa_compress_index_topk: workspace is NULL");
    if (!aligned(workspace, 256)) return fail(QSA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (ws_bytes < lay.total)
      return fail(QSA_ERR_WORKSPACE, "qsa_compress_index_topk: workspace has %zu bytes, needs %zu", ws_bytes,
                  lay.total);
  }
  return launch_compress_index_topk(*cfg, num_reqs, new_keys, new_cu, seq_len_before, ring, ckey_cache,
                                    num_sel_rows, max_seq_len, q_index, sel_req, sel_seq_len, block_table, topk,
                                    lay, workspace, stream);
}

qsa_status qsa_prefill_index_topk(const qsa_config* cfg, int32_t num_reqs, int32_t num_rows,
                                  int32_t max_rows_per_req, int32_t max_seq_len,
                                  const int8_t* q_index, const int32_t* row_cu,
                                  const int32_t* row_seq_len, const int32_t* block_table,
                                  const int8_t* ckey_cache, int32_t* topk,
                                  void* workspace, size_t ws_bytes, hipStream_t stream) {
  qsa_status st = check_config(cfg, true, false);
  if (st != QSA_OK) return st;
  if (num_reqs < 0 || num_reqs > 65535)
    return fail(QSA_ERR_INVALID_ARGUMENT, "num_reqs must be in [0, 65535] (got %d)", num_reqs);
  if (num_rows < 0 || num_rows > 65535)
    return fail(QSA_ERR_INVALID_ARGUMENT, "num_rows must be in [0, 65535] (got %d)", num_rows);
  if (max_rows_per_req < 0 || max_rows_per_req > num_rows)
    return fail(QSA_ERR_INVALID_ARGUMENT, "max_rows_per_req must be in [0, num_rows] (got %d)", max_rows_per_req);
  if (max_seq_len < 0 || max_seq_len > QSA_MAX_SEQ_LEN)
    return fail(QSA_ERR_INVALID_ARGUMENT, "max_seq_len must be in [0, %d] (got %d)", QSA_MAX_SEQ_LEN, max_seq_len);
  if (num_rows == 0 || num_reqs == 0) return QSA_OK;
  if (!q_index || !row_cu || !row_seq_len || !block_table || !ckey_cache)
    return fail(QSA_ERR_INVALID_ARGUMENT, "qsa_prefill_index_topk: NULL array argument");
  if (!aligned(ckey_cache, 16) || !aligned(q_index, 16))
    return fail(QSA_ERR_INVALID_ARGUMENT, "qsa_prefill_index_topk: ckey_cache and q_index need 16-byte alignment");
  TopkWorkspace lay = topk_workspace_layout(num_rows, max_seq_len);
  if (!workspace) return fail(QSA_ERR_WORKSPACE, "qsa_prefill_index_topk: workspace is NULL");
  if (!aligned(workspace, 256)) return fail(QSA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < lay.total)
    return fail(QSA_ERR_WORKSPACE, "qsa_prefill_index_topk: workspace has %zu bytes, needs %zu", ws_bytes, lay.total);
  return launch_prefill_index_topk(*cfg, num_reqs, num_rows, max_rows_per_req, max_seq_len, q_index, row_cu,
                                   row_seq_len, block_table, ckey_cache, topk, lay, workspace, stream);
}

}  // extern "C"

// Argument checks of the attention half (qsa_sparse_decode and the fused call);
// `what` names the call in the messages.
static qsa_status check_decode(const qsa_config* cfg, int32_t num_rows, int32_t num_sel_rows,
                               int32_t max_rows_per_sel, int32_t num_splits, const void* q, const int32_t* row_sel,
                               const int32_t* row_seq_len, const int32_t* sel_req, const int32_t* sel_seq_len,
                               const int32_t* topk, const int32_t* block_table, const void* k_cache,
                               const void* v_cache, const float* k_scale, const float* v_scale,
                               const float* o_part, const float* lse_part, const char* what) {
  if (num_sel_rows < 0 || num_sel_rows > 65535)
    return fail(QSA_ERR_INVALID_ARGUMENT, "num_sel_rows must be in [0, 65535] (got %d)", num_sel_rows);
  if (num_rows < 0 || num_rows > (1 << 24))
    return fail(QSA_ERR_INVALID_ARGUMENT, "num_rows must be in [0, 2^24] (got %d)", num_rows);
  if (num_splits < 1 || num_splits > 64)
    return fail(QSA_ERR_INVALID_ARGUMENT, "num_splits must be in [1, 64] (got %d)", num_splits);
  if (max_rows_per_sel < 1)
    return fail(QSA_ERR_INVALID_ARGUMENT, "max_rows_per_sel must be >= 1 (got %d)", max_rows_per_sel);
  const int G = cfg->num_q_heads / cfg->num_kv_heads;
  if ((int64_t)G * max_rows_per_sel > 64)
    return fail(QSA_ERR_UNSUPPORTED, "max_rows_per_sel * (num_q_heads/num_kv_heads) = %lld exceeds 64",
                (long long)G * max_rows_per_sel);
  if (!row_sel && (num_rows != num_sel_rows || max_rows_per_sel != 1))
    return fail(QSA_ERR_INVALID_ARGUMENT,
                "%s: without row_sel every row is its own selecting row (num_rows == num_sel_rows, "
                "max_rows_per_sel == 1)", what);
  if (num_sel_rows == 0 || num_rows == 0) return QSA_OK;
  if (!q || !row_seq_len || !sel_req || !sel_seq_len || !topk || !block_table || !k_cache || !v_cache ||
      !o_part || !lse_part)
    return fail(QSA_ERR_INVALID_ARGUMENT, "%s: NULL array argument", what);
  if (cfg->kv_dtype == QSA_KV_FP8_E4M3 && (!k_scale || !v_scale))
    return fail(QSA_ERR_INVALID_ARGUMENT, "%s: fp8 K/V need k_scale and v_scale", what);
  if (cfg->kv_dtype == QSA_KV_FP8_E4M3 && (!aligned(k_scale, 16) || !aligned(v_scale, 16)))
    return fail(QSA_ERR_INVALID_ARGUMENT, "%s: k_scale and v_scale need 16-byte alignment", what);
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16))
    return fail(QSA_ERR_INVALID_ARGUMENT, "%s: q, k_cache, v_cache need 16-byte alignment", what);
  return QSA_OK;
}

extern "C" {

qsa_status qsa_sparse_decode(const qsa_config* cfg, int32_t num_rows, int32_t num_sel_rows,
                             int32_t max_rows_per_sel, int32_t num_splits, const void* q,
                             const int32_t* row_sel, const int32_t* row_seq_len,
                             const int32_t* sel_req, const int32_t* sel_seq_len,
                             const int32_t* topk, const int32_t* block_table,
                             const void* k_cache, const void* v_cache,
                             const float* k_scale, const float* v_scale,
                             float* o_part, float* lse_part, hipStream_t stream) {
  qsa_status st = check_config(cfg, false, true);
  if (st != QSA_OK) return st;
  st = check_decode(cfg, num_rows, num_sel_rows, max_rows_per_sel, num_splits, q, row_sel, row_seq_len, sel_req,
                    sel_seq_len, topk, block_table, k_cache, v_cache, k_scale, v_scale, o_part, lse_part,
                    "qsa_sparse_decode");
  if (st != QSA_OK || num_sel_rows == 0 || num_rows == 0) return st;
  return launch_sparse_decode(*cfg, num_rows, num_sel_rows, max_rows_per_sel, num_splits, q, row_sel, row_seq_len,
                              sel_req, sel_seq_len, topk, block_table, k_cache, v_cache, k_scale, v_scale,
                              o_part, lse_part, stream);
}

qsa_status qsa_select_sparse_decode(const qsa_config* cfg, int32_t num_rows, int32_t num_sel_rows,
                                    int32_t max_rows_per_sel, int32_t num_splits, int32_t max_seq_len,
                                    const void* q, const int32_t* row_sel, const int32_t* row_seq_len,
                                    const int32_t* sel_req, const int32_t* sel_seq_len,
                                    const int32_t* block_table, const void* k_cache, const void* v_cache,
                                    const float* k_scale, const float* v_scale, int32_t* topk,
                                    float* o_part, float* lse_part,
                                    void* workspace, size_t ws_bytes, hipStream_t stream) {
  qsa_status st = check_config(cfg, true, true);
  if (st != QSA_OK) return st;
  if (max_seq_len < 0 || max_seq_len > QSA_MAX_SEQ_LEN)
    return fail(QSA_ERR_INVALID_ARGUMENT, "max_seq_len must be in [0, %d] (got %d)", QSA_MAX_SEQ_LEN, max_seq_len);
  st = check_decode(cfg, num_rows, num_sel_rows, max_rows_per_sel, num_splits, q, row_sel, row_seq_len, sel_req,
                    sel_seq_len, topk, block_table, k_cache, v_cache, k_scale, v_scale, o_part, lse_part,
                    "qsa_select_sparse_decode");
  if (st != QSA_OK || num_sel_rows == 0) return st;
  if (num_rows == 0 && !topk) return fail(QSA_ERR_INVALID_ARGUMENT, "qsa_select_sparse_decode: topk is NULL");
  TopkWorkspace lay = topk_workspace_layout(num_sel_rows, max_seq_len);
  if (!workspace) return fail(QSA_ERR_WORKSPACE, "qsa_select_sparse_decode: workspace is NULL");
  if (!aligned(workspace, 256)) return fail(QSA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < lay.total)
    return fail(QSA_ERR_WORKSPACE, "qsa_select_sparse_decode: workspace has %zu bytes, needs %zu", ws_bytes,
                lay.total);
  return launch_select_decode(*cfg, num_rows, num_sel_rows, max_rows_per_sel, num_splits, max_seq_len, q, row_sel,
                              row_seq_len, sel_req, sel_seq_len, block_table, k_cache, v_cache, k_scale, v_scale,
                              topk, o_part, lse_part, lay, workspace, stream);
}

int32_t qsa_select_sparse_decode_launches(const qsa_config* cfg, int32_t num_sel_rows, int32_t max_rows_per_sel,
                                          int32_t num_splits, int32_t max_seq_len) {
  if (check_config(cfg, true, true) != QSA_OK) return 0;
  if (num_sel_rows < 1 || num_sel_rows > 65535 || max_rows_per_sel < 1 || num_splits < 1 || num_splits > 64 ||
      max_seq_len < 0 || max_seq_len > QSA_MAX_SEQ_LEN)
    return 0;
  const int G = cfg->num_q_heads / cfg->num_kv_heads;
  if ((int64_t)G * max_rows_per_sel > 64) return 0;
  return select_decode_launches(*cfg, num_sel_rows, max_rows_per_sel, num_splits, max_seq_len);
}

qsa_status qsa_merge_partials(int32_t num_splits, int32_t num_rows, int32_t num_heads,
                              int32_t head_dim, const float* o_part, const float* lse_part,
                              void* out, int32_t out_dtype, float* lse, hipStream_t stream) {
  if (num_splits < 1 || num_splits > 64)
    return fail(QSA_ERR_INVALID_ARGUMENT, "num_splits must be in [1, 64] (got %d)", num_splits);
  if (num_rows < 0 || num_heads < 1)
    return fail(QSA_ERR_INVALID_ARGUMENT, "num_rows must be >= 0 and num_heads >= 1");
  if ((int64_t)num_rows * num_heads > (int64_t)1 << 30)
    return fail(QSA_ERR_INVALID_ARGUMENT, "num_rows * num_heads too large");
  if (head_dim < 1) return fail(QSA_ERR_INVALID_ARGUMENT, "head_dim must be positive (got %d)", head_dim);
  if (head_dim != 64 && head_dim != 128)
    return fail(QSA_ERR_UNSUPPORTED, "head_dim %d not built (64, 128)", head_dim);
  if (out_dtype != QSA_OUT_F32 && out_dtype != QSA_OUT_BF16)
    return fail(QSA_ERR_INVALID_ARGUMENT, "out_dtype must be QSA_OUT_F32 or QSA_OUT_BF16 (got %d)", out_dtype);
  if (num_rows == 0) return QSA_OK;
  if (!o_part || !lse_part || !out || !lse)
    return fail(QSA_ERR_INVALID_ARGUMENT, "qsa_merge_partials: NULL array argument");
  return launch_merge(num_splits, num_rows, num_heads, head_dim, o_part, lse_part, out,
                      out_dtype == QSA_OUT_BF16, lse, stream);
}

size_t qsa_indexer_project_workspace_size(int32_t num_tokens, int32_t hidden_dim, int32_t index_dim) {
  if (num_tokens < 0 || num_tokens > (1 << 24) || hidden_dim < 32 || hidden_dim % 32 != 0 || hidden_dim > 65536 ||
      (index_dim != 32 && index_dim != 64 && index_dim != 128))
    return 0;
  return qsa::indexer_project_workspace_bytes(num_tokens, hidden_dim, index_dim);
}

namespace {

// Shared by the 1-D and MRoPE front-end calls; name is the caller's, for messages.
qsa_status indexer_project_common(const char* name, int32_t num_tokens, int32_t hidden_dim, int32_t index_dim,
                                  const void* hidden, const int32_t* positions, int32_t pos_stride, int32_t sec1,
                                  int32_t sec2, const void* w_qk, const float* g_q, const float* g_k,
                                  float rope_base, float q_scale, float k_scale, int8_t* q_index, int8_t* keys,
                                  void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (num_tokens < 0 || num_tokens > (1 << 24))
    return fail(QSA_ERR_INVALID_ARGUMENT, "%s: num_tokens must be in [0, 2^24] (got %d)", name, num_tokens);
  if (hidden_dim < 32 || hidden_dim % 32 != 0 || hidden_dim > 65536)
    return fail(QSA_ERR_INVALID_ARGUMENT, "%s: hidden_dim must be a multiple of 32 in [32, 65536] (got %d)", name,
                hidden_dim);
  if (index_dim != 32 && index_dim != 64 && index_dim != 128)
    return fail(QSA_ERR_UNSUPPORTED, "%s: index_dim %d not built (32, 64, 128)", name, index_dim);
  if (!(rope_base > 1.0f) || !(q_scale > 0.0f) || !(k_scale > 0.0f) || !std::isfinite(rope_base) ||
      !std::isfinite(q_scale) || !std::isfinite(k_scale))
    return fail(QSA_ERR_INVALID_ARGUMENT, "%s: rope_base must be > 1 and the scales > 0, all finite", name);
  if (num_tokens == 0) return QSA_OK;
  if (!hidden || !positions || !w_qk || !g_q || !g_k || !q_index || !keys)
    return fail(QSA_ERR_INVALID_ARGUMENT, "%s: NULL array argument", name);
  if (!aligned(hidden, 16) || !aligned(w_qk, 16) || !aligned(q_index, 4) || !aligned(keys, 4))
    return fail(QSA_ERR_INVALID_ARGUMENT, "%s: hidden and w_qk need 16-byte, q_index and keys 4-byte alignment",
                name);
  if (!workspace || !aligned(workspace, 16))
    return fail(QSA_ERR_WORKSPACE, "%s: workspace is NULL or not 16-byte aligned", name);
  const size_t need = indexer_project_workspace_bytes(num_tokens, hidden_dim, index_dim);
  if (ws_bytes < need) return fail(QSA_ERR_WORKSPACE, "%s: workspace has %zu bytes, needs %zu", name, ws_bytes, need);
  return launch_indexer_project(num_tokens, hidden_dim, index_dim, hidden, positions, pos_stride, sec1, sec2, w_qk,
                                g_q, g_k, rope_base, q_scale, k_scale, q_index, keys,
                                reinterpret_cast<float*>(workspace), stream);
}

}  // namespace

qsa_status qsa_indexer_project(int32_t num_tokens, int32_t hidden_dim, int32_t index_dim, const void* hidden,
                               const int32_t* positions, const void* w_qk, const float* g_q, const float* g_k,
                               float rope_base, float q_scale, float k_scale, int8_t* q_index, int8_t* keys,
                               void* workspace, size_t ws_bytes, hipStream_t stream) {
  return indexer_project_common("qsa_indexer_project", num_tokens, hidden_dim, index_dim, hidden, positions, 0,
                                index_dim / 2, index_dim / 2, w_qk, g_q, g_k, rope_base, q_scale, k_scale, q_index,
                                keys, workspace, ws_bytes, stream);
}

qsa_status qsa_indexer_project_mrope(int32_t num_tokens, int32_t hidden_dim, int32_t index_dim, const void* hidden,
                                     const int32_t* positions, int32_t section_t, int32_t section_h,
                                     int32_t section_w, const void* w_qk, const float* g_q, const float* g_k,
                                     float rope_base, float q_scale, float k_scale, int8_t* q_index, int8_t* keys,
                                     void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (section_t < 0 || section_h < 0 || section_w < 0 ||
      (int64_t)section_t + section_h + section_w != index_dim / 2)
    return fail(QSA_ERR_INVALID_ARGUMENT,
                "qsa_indexer_project_mrope: sections (%d, %d, %d) must be >= 0 and sum to index_dim / 2 = %d",
                section_t, section_h, section_w, index_dim / 2);
  return indexer_project_common("qsa_indexer_project_mrope", num_tokens, hidden_dim, index_dim, hidden, positions,
                                num_tokens, section_t, section_t + section_h, w_qk, g_q, g_k, rope_base, q_scale,
                                k_scale, q_index, keys, workspace, ws_bytes, stream);
}

const char* qsa_status_string(qsa_status s) {
  switch (s) {
    case QSA_OK: return "QSA_OK";
    case QSA_ERR_INVALID_ARGUMENT: return "QSA_ERR_INVALID_ARGUMENT";
    case QSA_ERR_UNSUPPORTED: return "QSA_ERR_UNSUPPORTED";
    case QSA_ERR_WORKSPACE: return "QSA_ERR_WORKSPACE";
    case QSA_ERR_HIP: return "QSA_ERR_HIP";
  }
  return "QSA_ERR_UNKNOWN";
}

const char* qsa_last_error(void) { return g_err; }

const char* qsa_version(void) { return "qsa-mi355x 0.1.0"; }

}  // extern "C"
