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
  const size_t page_bytes = (size_t)bpp * (D + D / 4);  // s plane + two bit-masks per block
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
    uint32_t splane = 0, m0 = 0, m1 = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t v = (uint32_t)(s[i] + 512);  // 10 bits
      splane |= ((v & 0xffu) ^ 0x80u) << (8 * i);  // (v mod 256) - 128 as int8
      m0 |= ((v >> 8) & 1u) << i;
      m1 |= ((v >> 9) & 1u) << i;
    }
    // dims 8k..8k+3 (even group) and 8k+4..8k+7 (odd group) form mask byte k
    const uint32_t m0p = __shfl_xor(m0, 1, 64), m1p = __shfl_xor(m1, 1, 64);
    const int page = block_table[(size_t)b * max_pages + (j >> bpp_log2)];
    const int slot = j & (bpp - 1);
    int8_t* pg = ckey + (size_t)page * page_bytes;
    const int byte = 4 * grp;                     // dims [4grp, 4grp+4)
    *reinterpret_cast<uint32_t*>(pg + (size_t)(byte >> 4) * bpp * 16 + (size_t)slot * 16 + (byte & 15)) = splane;
    if ((grp & 1) == 0) {
      uint8_t* mk = reinterpret_cast<uint8_t*>(pg + (size_t)(D / 16) * bpp * 16 + (size_t)slot * (D / 4));
      mk[grp >> 1] = (uint8_t)(m0 | (m0p << 4));
      mk[D / 8 + (grp >> 1)] = (uint8_t)(m1 | (m1p << 4));
    }
  }

  if (blockIdx.x != 0) return;
  // The last kRing new tokens go to the ring, after every ring read above.
  __syncthreads();
  const int t0 = max(L0, L0 + n - kRing);
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
