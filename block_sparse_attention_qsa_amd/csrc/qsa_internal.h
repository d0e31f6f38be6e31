// Host-side internals shared by the QSA translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "qsa.h"

namespace qsa {

// Records a message for qsa_last_error() and returns `st`.
qsa_status fail(qsa_status st, const char* fmt, ...);

// Checks hipGetLastError() after a launch.
qsa_status check_launch(const char* what);

// Workspace layout of qsa_index_topk (offsets in bytes from the base).
struct TopkWorkspace {
  int32_t rows;        // selecting rows it is sized for
  int32_t nb_stride;   // micro-block capacity per row (multiple of the chunk)
  size_t off_scores;   // int32  [rows][nb_stride]
  size_t off_keys;     // uint64 [rows][nb_stride]  each chunk's candidate list, in the chunk's region
  size_t off_bitmap;   // uint64 [rows][nb_stride/64]  (rows too long for the finalize's LDS)
  size_t off_keys2;    // uint64 [rows][nb_stride]  threshold candidates beyond the finalize's LDS
  size_t off_hist;     // uint32 [2][rows][kBins]  two histograms: a call scores into one while the
                       // other is clear (see off_gen)
  size_t off_cinfo;    // uint32 [rows][nb_stride/1024]  per chunk: candidate count << 16 | local bin
  size_t off_gen;      // uint32 [2]  calls scored / calls selected: a scan uses histogram
                       // (selected + 1) & 1 and publishes that count as scored; the selection
                       // reads it, clears the other histogram and publishes it as selected
  size_t total;
};

constexpr int kScoreChunk = 1024;  // micro-blocks per scoring workgroup
constexpr int kMaxChunksPerRow = (QSA_MAX_SEQ_LEN / 4 + kScoreChunk - 1) / kScoreChunk;
constexpr int kBins = 2048;        // histogram bins of the score's top bits
constexpr int kBinShift = 14;      // bin = (score + 2^24) >> 14

TopkWorkspace topk_workspace_layout(int32_t rows, int32_t max_seq_len);

qsa_status launch_compress(const qsa_config& c, int32_t num_reqs, int32_t max_new_tokens,
                           const int8_t* new_keys, const int32_t* new_cu,
                           const int32_t* seq_len_before, const int32_t* block_table,
                           int8_t* ring, int8_t* ckey, hipStream_t stream);

qsa_status launch_index_topk(const qsa_config& c, int32_t S, int32_t max_seq_len,
                             const int8_t* q_index, const int32_t* sel_req,
                             const int32_t* sel_seq_len, const int32_t* block_table,
                             const int8_t* ckey, int32_t* topk, const TopkWorkspace& ws,
                             void* ws_base, hipStream_t stream);

qsa_status launch_compress_index_topk(const qsa_config& c, int32_t num_reqs, const int8_t* new_keys,
                                      const int32_t* new_cu, const int32_t* seq_len_before, int8_t* ring,
                                      int8_t* ckey, int32_t S, int32_t max_seq_len, const int8_t* q_index,
                                      const int32_t* sel_req, const int32_t* sel_seq_len,
                                      const int32_t* block_table, int32_t* topk, const TopkWorkspace& lay,
                                      void* ws_base, hipStream_t stream);
qsa_status launch_prefill_index_topk(const qsa_config& c, int32_t B, int32_t R, int32_t max_rows,
                                     int32_t max_seq_len, const int8_t* q_index, const int32_t* row_cu,
                                     const int32_t* row_seq_len, const int32_t* block_table,
                                     const int8_t* ckey, int32_t* topk, const TopkWorkspace& ws,
                                     void* ws_base, hipStream_t stream);

qsa_status launch_ws_clear(void* ws, size_t bytes, hipStream_t stream);

// qsa_index_topk over the library's own scratch (a file-scope device array).
qsa_status launch_index_topk_noalloc(const qsa_config& c, int32_t S, int32_t max_seq_len, const int8_t* q_index,
                                     const int32_t* sel_req, const int32_t* sel_seq_len, const int32_t* block_table,
                                     const int8_t* ckey, int32_t* topk, hipStream_t stream);

size_t indexer_project_workspace_bytes(int32_t T, int32_t H, int32_t D);

// positions: [T] (pos_stride 0, sec1 = sec2 = D/2) or MRoPE [3, T] (pos_stride T,
// frequency sections [0, sec1), [sec1, sec2), [sec2, D/2))
qsa_status launch_indexer_project(int32_t T, int32_t H, int32_t D, const void* hidden, const int32_t* positions,
                                  int32_t pos_stride, int32_t sec1, int32_t sec2, const void* w_qk, const float* g_q, const float* g_k, float base, float q_scale,
                                  float k_scale, int8_t* q_index, int8_t* keys, float* ws, hipStream_t stream);

qsa_status launch_sparse_decode(const qsa_config& c, int32_t R, int32_t S, int32_t qps, int32_t P,
                                const void* q, const int32_t* row_sel, const int32_t* row_seq_len,
                                const int32_t* sel_req, const int32_t* sel_seq_len, const int32_t* topk,
                                const int32_t* block_table, const void* k_cache,
                                const void* v_cache, const float* k_scale, const float* v_scale,
                                float* o_part, float* lse_part, hipStream_t stream);

// Selection (finalize of a scored workspace) fused with qsa_sparse_decode.
qsa_status launch_select_decode(const qsa_config& c, int32_t R, int32_t S, int32_t qps, int32_t P,
                                int32_t max_seq_len, const void* q, const int32_t* row_sel,
                                const int32_t* row_seq_len, const int32_t* sel_req, const int32_t* sel_seq_len,
                                const int32_t* block_table, const void* k_cache, const void* v_cache,
                                const float* k_scale, const float* v_scale, int32_t* topk, float* o_part,
                                float* lse_part, const TopkWorkspace& lay, void* ws_base, hipStream_t stream);

// Kernel launches qsa_select_sparse_decode makes for this shape: 1 (fused) or 2.
int select_decode_launches(const qsa_config& c, int32_t S, int32_t qps, int32_t P, int32_t max_seq_len);

// The finalize kernel alone (qsa_index_topk's selection step).
qsa_status launch_finalize_ws(const qsa_config& c, int32_t rows, const int32_t* seq_len, int32_t max_seq_len,
                              int32_t* topk, const TopkWorkspace& lay, void* ws_base, hipStream_t stream);

qsa_status launch_merge(int32_t P, int32_t R, int32_t H, int32_t d, const float* o_part,
                        const float* lse_part, void* out, bool out_bf16, float* lse, hipStream_t stream);

}  // namespace qsa
