// qsa_compress: append indexer keys, close 4-token micro-blocks into the paged
// compressed-key cache.
//
// Method ("Qwen 4 QSA 迎来解码上下文并行" blog, section on what the pull request
// changes; "PR #53896 完整报告", implementation breakdown): token keys enter a
// raw-key ring and are pooled by the compress ratio (4) into the compressed key
// cache.  Pooling here is the exact integer sum of the 4 int8 keys; it is stored
// losslessly as two int8 planes (C = 256*hi + lo), so the scoring kernel keeps
// using int8 dot products and stays bit-exact.
//
// Work split: one grid row (blockIdx.y) per request, workgroups stride over the
// micro-blocks that close in this call.  Only the block that straddles the
// previous call (first block, when seq_len_before % 4 != 0) reads the ring, and
// only the new tokens of the block left open write it; both happen in
// workgroup 0, reads before writes, so any number of new tokens is race-free.
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
  constexpr int kGroups = D / 4;                 // 4-dim groups per block
  constexpr int kBlocksPerIter = kThreads / kGroups;
  const int b = blockIdx.y;
  const int L0 = seq_len_before[b];
  const int base_row = new_cu[b];
  const int n = new_cu[b + 1] - base_row;
  if (L0 < 0 || n <= 0) return;                  // dummy request: writes nothing
  const int jA = L0 >> 2;                        // first block touched
  const int jE = (L0 + n) >> 2;                  // closing blocks are [jA, jE)
  const int bpp_log2 = page_log2 - 2;            // micro-blocks per page (log2)
  const int bpp = 1 << bpp_log2;
  const size_t page_bytes = (size_t)bpp * 2 * D; // 16 B chunks x (2D/16) x bpp
  const int grp = threadIdx.x % kGroups;
  const int sub = threadIdx.x / kGroups;
  const int8_t* ring_b = ring + (size_t)b * kRing * D;

  for (int j = jA + blockIdx.x * kBlocksPerIter + sub; j < jE; j += gridDim.x * kBlocksPerIter) {
    int s[4] = {0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < kRatio; ++e) {
      const int t = 4 * j + e;
      const int8_t* src = (t >= L0) ? new_keys + (size_t)(base_row + (t - L0)) * D
                                    : ring_b + (size_t)(t & (kRing - 1)) * D;
      const uint32_t w = *reinterpret_cast<const uint32_t*>(src + 4 * grp);
#pragma unroll
      for (int i = 0; i < 4; ++i) s[i] += (int32_t)(int8_t)(w >> (8 * i));
    }
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int32_t l = (int32_t)(int8_t)(s[i] & 0xff);  // low byte, signed
      const int32_t h = (s[i] - l) >> 8;                 // exact: s - l is a multiple of 256
      lo |= (uint32_t)(l & 0xff) << (8 * i);
      hi |= (uint32_t)(h & 0xff) << (8 * i);
    }
    const int page = block_table[(size_t)b * max_pages + (j >> bpp_log2)];
    const int slot = j & (bpp - 1);
    int8_t* dst = ckey + (size_t)page * page_bytes + (size_t)slot * 16;
    const int byte = 4 * grp;                     // dims [4grp, 4grp+4)
    const int chunk = byte >> 4;
    *reinterpret_cast<uint32_t*>(dst + (size_t)chunk * bpp * 16 + (byte & 15)) = lo;
    *reinterpret_cast<uint32_t*>(dst + (size_t)(chunk + D / 16) * bpp * 16 + (byte & 15)) = hi;
  }

  if (blockIdx.x != 0) return;
  // New tokens of the block left open go to the ring, after every ring read above.
  __syncthreads();
  const int t0 = max(L0, 4 * jE);
  for (int i = threadIdx.x; i < (L0 + n - t0) * kGroups; i += kThreads) {
    const int t = t0 + i / kGroups;
    const int g = i % kGroups;
    const uint32_t w = *reinterpret_cast<const uint32_t*>(new_keys + (size_t)(base_row + (t - L0)) * D + 4 * g);
    *reinterpret_cast<uint32_t*>(ring + (size_t)b * kRing * D + (size_t)(t & (kRing - 1)) * D + 4 * g) = w;
  }
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
