// Appending tokens to a request's indexer side cache (device side), shared by
// the compress kernel and the scan that does the compression in the same
// launch.  See qsa_compress.hip for the method and the 10-bit block layout.
#pragma once

#include "qsa_device.h"

namespace qsa {

// Close the micro-blocks [jA, jE) that request b's new tokens complete and put
// its last kRing new tokens into the ring.  Called by whole workgroups of NT
// threads: workgroup wg of nwg strides over the blocks; workgroup 0 also writes
// the ring, after every ring read of its own (the only ring reads are of the
// first block, which workgroup 0 handles).
template <int D, int NT>
__device__ __forceinline__ void append_request(int b, int wg, int nwg, const int8_t* __restrict__ new_keys,
                                               const int32_t* __restrict__ new_cu,
                                               const int32_t* __restrict__ seq_len_before,
                                               const int32_t* __restrict__ block_table, int32_t max_pages,
                                               int32_t page_log2, int8_t* __restrict__ ring,
                                               int8_t* __restrict__ ckey) {
  constexpr int kGroups = D / 4;                 // 4-dim groups per block
  constexpr int kBlocksPerIter = NT / kGroups;
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

  for (int j = jA + wg * kBlocksPerIter + sub; j < jE; j += nwg * kBlocksPerIter) {
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
    // dims 8k..8k+3 (even group) and 8k+4..8k+7 (odd group) form mask byte k;
    // partners share `sub`, hence the same trip count of this loop
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

  if (wg != 0) return;
  // The last kRing new tokens go to the ring, after every ring read above.
  __syncthreads();
  const int t0 = max(L0, L0 + n - kRing);
  for (int i = threadIdx.x; i < (L0 + n - t0) * kGroups; i += NT) {
    const int t = t0 + i / kGroups;
    const int g = i % kGroups;
    const uint32_t w = *reinterpret_cast<const uint32_t*>(new_keys + (size_t)(base_row + (t - L0)) * D + 4 * g);
    *reinterpret_cast<uint32_t*>(ring + (size_t)b * kRing * D + (size_t)(t & (kRing - 1)) * D + 4 * g) = w;
  }
}

}  // namespace qsa
