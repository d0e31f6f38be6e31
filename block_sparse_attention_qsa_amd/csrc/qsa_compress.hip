// qsa_compress: append indexer keys, close 4-token micro-blocks into the paged
// compressed-key cache.
//
// Method ("Qwen 4 QSA 迎来解码上下文并行" blog, section on what the pull request
// changes; "PR #53896 完整报告", implementation breakdown): token keys enter a
// raw-key ring and are pooled by the compress ratio (4) into the compressed key
// cache.  Pooling here is the exact integer sum of the 4 int8 keys,
// C in [-512, 508], stored losslessly in 10 bits per dimension:
//   v = C + 512 in [0, 1023];  s = (v mod 256) - 128 (an int8 plane);
//   b0, b1 = bits 8 and 9 of v (two bit-masks over the dimensions),
// so C = 256*(2*b1 + b0) + s - 384.  The scoring kernel keeps int8 dot
// products for the s plane and adds masked sums of the query for the masks.
//
// Work split: one grid row (blockIdx.y) per request, workgroups stride over the
// micro-blocks that close in this call.  Only the block that straddles the
// previous call (first block, when seq_len_before % 4 != 0) reads the ring;
// the last (up to 8) new tokens are written to it, closed or not, so that a
// caller can roll rejected draft tokens back (the pages' MTP flow: later draft
// steps keep updating the side cache).  Reads and writes happen in workgroup
// 0, reads first, so any number of new tokens is race-free.
#include "qsa_append.h"
#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {

namespace {

constexpr int kThreads = 256;

template <int D>
__global__ __launch_bounds__(kThreads) void compress_kernel(
    const int8_t* __restrict__ new_keys, const int32_t* __restrict__ new_cu,
    const int32_t* __restrict__ seq_len_before, const int32_t* __restrict__ block_table,
    int32_t max_pages, int32_t page_log2, int8_t* __restrict__ ring, int8_t* __restrict__ ckey) {
  append_request<D, kThreads>(blockIdx.y, blockIdx.x, gridDim.x, new_keys, new_cu, seq_len_before, block_table,
                              max_pages, page_log2, ring, ckey);
}

}  // namespace

qsa_status launch_compress(const qsa_config& c, int32_t num_reqs, int32_t max_new_tokens,
                           const int8_t* new_keys, const int32_t* new_cu,
                           const int32_t* seq_len_before, const int32_t* block_table,
                           int8_t* ring, int8_t* ckey, hipStream_t stream) {
  if (num_reqs == 0) return QSA_OK;
  const int page_log2 = __builtin_ctz((unsigned)c.page_size);
  const int groups = c.index_dim / 4;
  const int per_iter = kThreads / groups;
  // closing blocks per request <= max_new_tokens/4 + 1
  int64_t blocks = (int64_t)max_new_tokens / 4 + 1;
  int64_t gx = (blocks + per_iter - 1) / per_iter;
  if (gx < 1) gx = 1;
  if (gx > 4096) gx = 4096;
  dim3 grid((unsigned)gx, (unsigned)num_reqs);
  switch (c.index_dim) {
    case 32:
      hipLaunchKernelGGL(compress_kernel<32>, grid, dim3(kThreads), 0, stream, new_keys, new_cu,
                         seq_len_before, block_table, c.max_pages_per_req, page_log2, ring, ckey);
      break;
    case 64:
      hipLaunchKernelGGL(compress_kernel<64>, grid, dim3(kThreads), 0, stream, new_keys, new_cu,
                         seq_len_before, block_table, c.max_pages_per_req, page_log2, ring, ckey);
      break;
    case 128:
      hipLaunchKernelGGL(compress_kernel<128>, grid, dim3(kThreads), 0, stream, new_keys, new_cu,
                         seq_len_before, block_table, c.max_pages_per_req, page_log2, ring, ckey);
      break;
    default:
      return fail(QSA_ERR_UNSUPPORTED, "index_dim %d not built", c.index_dim);
  }
  return check_launch("qsa_compress");
}

}  // namespace qsa
