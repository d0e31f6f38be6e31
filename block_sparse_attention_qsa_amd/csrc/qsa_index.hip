// qsa_index_topk: exact block scores and top-k selection.
//
// Method ("Qwen 4 QSA 迎来解码上下文并行" blog, section on what the pull request
// changes): the indexer scores the compressed micro-blocks and keeps the best 512;
// ("PR #53896 完整报告", implementation breakdown / key source snippets) the
// selection is weight-free, on the compressed keys, returned as a fixed-width
// int32 buffer padded with -1.  Ties go to the lower block index, so the
// result is unique and can be compared bit for bit.
//
// Two kernels, both gridded (chunk of 1024 micro-blocks, selecting row):
//   score:  streams the 2-byte compressed keys (the HBM-bound scan), computes
//           score = q.lo + 256 q.hi with v_dot4_i32_i8, stores the int32 score,
//           and adds an LDS histogram of the score's top 11 bits to a per-row
//           global histogram.  The last workgroup of a row finds the threshold
//           bin T: fewer than k scores lie in bins above T, at least k in bins
//           >= T.
//   select: re-reads the scores (L2 / MALL resident), writes a bitmap of the
//           blocks strictly above T and appends 64-bit keys (score, ~index) of
//           the blocks inside T to a candidate list.  The last workgroup of a
//           row radix-selects the missing blocks among the candidates (usually
//           a few hundred), sets their bits, and emits the bitmap in ascending
//           order with a popcount prefix sum, padding with -1.
// Counters and the histogram are cleared by the workgroup that consumed them,
// so the workspace stays clean between calls.
#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kIters = kScoreChunk / kThreads;

struct WsPtrs {
  int32_t* scores;
  uint64_t* keys;
  uint64_t* bitmap;
  uint32_t* hist;
  uint32_t* ctr;
  int32_t* meta;
  int32_t nb_stride;
};

__device__ __forceinline__ int score_bin(int32_t s) {
  return (int)(((uint32_t)(s + (1 << 24))) >> kBinShift);
}

__device__ __forceinline__ uint64_t cand_key(int32_t score, uint32_t j) {
  return ((uint64_t)((uint32_t)score ^ 0x80000000u) << 32) | (uint64_t)(0xffffffffu - j);
}

// Block-wide exclusive prefix sum of one value per thread (256 threads).
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* sh /*[kWaves+1]*/,
                                                    uint32_t* total) {
  const int l = lane_id(), w = threadIdx.x / 64;
  uint32_t inc = wave_incl_scan(v);
  if (l == 63) sh[w] = inc;
  __syncthreads();
  uint32_t off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    const uint32_t x = sh[i];
    off += (i < w) ? x : 0u;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return off + inc - v;
}

template <int D>
__global__ __launch_bounds__(kThreads) void score_kernel(
    const int8_t* __restrict__ q_index, const int32_t* __restrict__ sel_req,
    const int32_t* __restrict__ sel_seq_len, const int32_t* __restrict__ block_table,
    int32_t max_pages, int32_t page_log2, const int8_t* __restrict__ ckey, int32_t k,
    int32_t max_seq_len, WsPtrs ws) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t sh[kWaves + 1];
  __shared__ int is_last;
  const int s = blockIdx.y;
  const int c = blockIdx.x;
  const int L = min(sel_seq_len[s], max_seq_len);
  const int nb = max(L, 0) >> 2;
  const int nchunks = (nb + kScoreChunk - 1) / kScoreChunk;
  if (c >= nchunks) return;
  const int b = sel_req[s];
  const int bpp_log2 = page_log2 - 2;
  const int bpp = 1 << bpp_log2;
  const size_t page_bytes = (size_t)bpp * 2 * D;

  // indexer query: D int8 = D/4 packed dwords, uniform across the workgroup
  int32_t qw[D / 4];
  const int32_t* q32 = reinterpret_cast<const int32_t*>(q_index + (size_t)s * D);
#pragma unroll
  for (int i = 0; i < D / 4; ++i) qw[i] = q32[i];

  for (int i = threadIdx.x; i < kBins; i += kThreads) hist[i] = 0;
  __syncthreads();

  const int32_t* bt = block_table + (size_t)b * max_pages;
  int32_t* srow = ws.scores + (size_t)s * ws.nb_stride;
#pragma unroll 2
  for (int it = 0; it < kIters; ++it) {
    const int j = c * kScoreChunk + it * kThreads + threadIdx.x;
    if (j < nb) {
      const int page = bt[j >> bpp_log2];
      const int8_t* base = ckey + (size_t)page * page_bytes + (size_t)(j & (bpp - 1)) * 16;
      i32x4 v[D / 8];
#pragma unroll
      for (int ch = 0; ch < D / 8; ++ch) v[ch] = ld16(base + (size_t)ch * bpp * 16);
      int32_t lo = 0, hi = 0;
#pragma unroll
      for (int ch = 0; ch < D / 16; ++ch) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          lo = __builtin_amdgcn_sdot4(v[ch][e], qw[4 * ch + e], lo, false);
          hi = __builtin_amdgcn_sdot4(v[ch + D / 16][e], qw[4 * ch + e], hi, false);
        }
      }
      const int32_t score = lo + hi * 256;
      srow[j] = score;
      atomicAdd(&hist[score_bin(score)], 1u);
    }
  }
  __syncthreads();
  uint32_t* ghist = ws.hist + (size_t)s * kBins;
  for (int i = threadIdx.x; i < kBins; i += kThreads) {
    const uint32_t h = hist[i];
    if (h) atomicAdd(&ghist[i], h);
  }
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) is_last = (atomicAdd(&ws.ctr[4 * s + 0], 1u) == (uint32_t)(nchunks - 1));
  __syncthreads();
  if (!is_last) return;
  __threadfence();

  // Last workgroup of the row: threshold bin from the top.
  const uint32_t ks = (uint32_t)min(k, nb);
  constexpr int kPer = kBins / kThreads;  // 8 bins per thread, thread t owns the
  // bins [kBins-1-kPer*t-(kPer-1), kBins-1-kPer*t] (descending from the top)
  uint32_t cnt[kPer];
  uint32_t mine = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int bin = kBins - 1 - (kPer * threadIdx.x + i);
    cnt[i] = ld_acq_u32(&ghist[bin]);
    mine += cnt[i];
  }
  uint32_t total;
  uint32_t above = block_excl_scan(mine, sh, &total);  // count in higher bins
  // The thread whose bins contain the k-th largest records the threshold.
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int bin = kBins - 1 - (kPer * threadIdx.x + i);
    if (above < ks && above + cnt[i] >= ks) {
      ws.meta[2 * s + 0] = bin;
      ws.meta[2 * s + 1] = (int32_t)above;
    }
    above += cnt[i];
  }
  // clear for the next call
  for (int i = threadIdx.x; i < kBins; i += kThreads) ghist[i] = 0;
  if (threadIdx.x == 0) ws.ctr[4 * s + 0] = 0;
}

__global__ __launch_bounds__(kThreads) void select_kernel(
    const int32_t* __restrict__ sel_seq_len, int32_t k, int32_t max_seq_len,
    int32_t* __restrict__ topk, WsPtrs ws) {
  __shared__ uint32_t sh[kWaves + 1];
  __shared__ uint32_t rhist[256];
  __shared__ int is_last;
  __shared__ uint32_t s_info[4];
  const int s = blockIdx.y;
  const int c = blockIdx.x;
  const int L = min(sel_seq_len[s], max_seq_len);
  const int nb = max(L, 0) >> 2;
  int32_t* out = topk + (size_t)s * k;
  if (nb == 0) {
    if (c == 0)
      for (int i = threadIdx.x; i < k; i += kThreads) out[i] = -1;
    return;
  }
  const int nchunks = (nb + kScoreChunk - 1) / kScoreChunk;
  if (c >= nchunks) return;
  const int T = ws.meta[2 * s + 0];
  const int l = lane_id(), w = threadIdx.x / 64;
  const int32_t* srow = ws.scores + (size_t)s * ws.nb_stride;
  uint64_t* bm = ws.bitmap + (size_t)s * (ws.nb_stride / 64);
  uint64_t* keys = ws.keys + (size_t)s * ws.nb_stride;
  uint32_t* ncand = &ws.ctr[4 * s + 2];

  for (int it = 0; it < kIters; ++it) {
    const int j0 = c * kScoreChunk + it * kThreads + w * 64;  // 64-aligned
    const int j = j0 + l;
    const bool valid = j < nb;
    const int32_t score = valid ? srow[j] : 0;
    const int bin = score_bin(score);
    const bool sure = valid && bin > T;
    const bool maybe = valid && bin == T;
    const uint64_t sure_mask = __ballot(sure);
    const uint64_t maybe_mask = __ballot(maybe);
    if (l == 0) bm[j0 >> 6] = sure_mask;
    if (maybe_mask) {
      uint32_t basepos = 0;
      if (l == 0) basepos = atomicAdd(ncand, (uint32_t)__popcll(maybe_mask));
      basepos = __shfl(basepos, 0, 64);
      if (maybe) {
        const uint32_t pos = basepos + (uint32_t)__popcll(maybe_mask & ((1ull << l) - 1ull));
        keys[pos] = cand_key(score, (uint32_t)j);
      }
    }
  }
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) is_last = (atomicAdd(&ws.ctr[4 * s + 1], 1u) == (uint32_t)(nchunks - 1));
  __syncthreads();
  if (!is_last) return;
  __threadfence();

  // ---- last workgroup of the row: resolve the threshold bin, then emit ----
  const uint32_t ks = (uint32_t)min(k, nb);
  const uint32_t n = ld_acq_u32(ncand);
  const uint32_t need = ks - (uint32_t)ws.meta[2 * s + 1];  // 1 <= need <= n
  uint64_t prefix = 0, mask = 0;
  if (need < n) {
    // MSB-first radix select over the 64-bit candidate keys: find the need-th
    // largest key; all candidates share the bits of bin T, so most of the
    // upper digits resolve in one step each.
    uint32_t rem = need;
    for (int shift = 56; shift >= 0; shift -= 8) {
      rhist[threadIdx.x] = 0;
      __syncthreads();
      for (uint32_t i = threadIdx.x; i < n; i += kThreads) {
        const uint64_t key = ld_acq_u64(&keys[i]);
        if ((key & mask) == prefix) atomicAdd(&rhist[(key >> shift) & 0xff], 1u);
      }
      __syncthreads();
      // thread t owns digit 255-t; exclusive scan gives the count of larger digits
      const uint32_t cntd = rhist[255 - threadIdx.x];
      uint32_t tot;
      const uint32_t larger = block_excl_scan(cntd, sh, &tot);
      if (larger < rem && larger + cntd >= rem) {
        s_info[0] = 255 - threadIdx.x;
        s_info[1] = larger;
        s_info[2] = cntd;
      }
      __syncthreads();
      const uint64_t dsel = s_info[0];
      rem -= s_info[1];
      prefix |= dsel << shift;
      mask |= 0xffull << shift;
      const uint32_t eq = s_info[2];
      __syncthreads();
      if (eq == rem) break;  // every remaining candidate with this prefix is kept
    }
  }
  // Mark the kept candidates: masked key > prefix, or == prefix (all of them,
  // by construction of the early exit / exhaustion of the digits).
  for (uint32_t i = threadIdx.x; i < n; i += kThreads) {
    const uint64_t key = ld_acq_u64(&keys[i]);
    if ((key & mask) >= prefix) {
      const uint32_t j = 0xffffffffu - (uint32_t)(key & 0xffffffffull);
      atomicOr(reinterpret_cast<unsigned long long*>(&bm[j >> 6]), 1ull << (j & 63));
    }
  }
  __threadfence();
  __syncthreads();

  // Emit ascending block ids: each thread owns a contiguous run of bitmap words.
  const int nwords = (nb + 63) >> 6;
  const int per = (nwords + kThreads - 1) / kThreads;
  const int w0 = min(nwords, threadIdx.x * per), w1 = min(nwords, w0 + per);
  uint32_t cntw = 0;
  for (int i = w0; i < w1; ++i) cntw += (uint32_t)__popcll(ld_acq_u64(&bm[i]));
  uint32_t tot;
  uint32_t pos = block_excl_scan(cntw, sh, &tot);
  for (int i = w0; i < w1; ++i) {
    uint64_t m = ld_acq_u64(&bm[i]);
    while (m) {
      const int bit = __ffsll((long long)m) - 1;
      m &= m - 1;
      if (pos < (uint32_t)k) out[pos] = i * 64 + bit;
      ++pos;
    }
  }
  for (int i = (int)ks + threadIdx.x; i < k; i += kThreads) out[i] = -1;
  if (threadIdx.x == 0) {
    ws.ctr[4 * s + 1] = 0;
    ws.ctr[4 * s + 2] = 0;
  }
}

__global__ void clear_kernel(uint32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

}  // namespace

TopkWorkspace topk_workspace_layout(int32_t rows, int32_t max_seq_len) {
  TopkWorkspace w{};
  w.rows = rows;
  const int64_t nb = (int64_t)max_seq_len / 4;
  const int64_t chunks = (nb + kScoreChunk - 1) / kScoreChunk;
  w.nb_stride = (int32_t)(chunks < 1 ? kScoreChunk : chunks * kScoreChunk);
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  size_t off = 0;
  w.off_scores = off; off = al(off + (size_t)rows * w.nb_stride * 4);
  w.off_keys = off;   off = al(off + (size_t)rows * w.nb_stride * 8);
  w.off_bitmap = off; off = al(off + (size_t)rows * (w.nb_stride / 64) * 8);
  w.off_hist = off;   off = al(off + (size_t)rows * kBins * 4);
  w.off_ctr = off;    off = al(off + (size_t)rows * 4 * 4);
  w.off_meta = off;   off = al(off + (size_t)rows * 2 * 4);
  w.total = off;
  return w;
}

qsa_status launch_ws_clear(void* ws, size_t bytes, hipStream_t stream) {
  const size_t n = bytes / 4;
  if (n == 0) return QSA_OK;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(clear_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     reinterpret_cast<uint32_t*>(ws), n);
  return check_launch("qsa_index_topk_workspace_init");
}

qsa_status launch_index_topk(const qsa_config& c, int32_t S, int32_t max_seq_len,
                             const int8_t* q_index, const int32_t* sel_req,
                             const int32_t* sel_seq_len, const int32_t* block_table,
                             const int8_t* ckey, int32_t* topk, const TopkWorkspace& lay,
                             void* ws_base, hipStream_t stream) {
  if (S == 0) return QSA_OK;
  char* base = reinterpret_cast<char*>(ws_base);
  WsPtrs ws;
  ws.scores = reinterpret_cast<int32_t*>(base + lay.off_scores);
  ws.keys = reinterpret_cast<uint64_t*>(base + lay.off_keys);
  ws.bitmap = reinterpret_cast<uint64_t*>(base + lay.off_bitmap);
  ws.hist = reinterpret_cast<uint32_t*>(base + lay.off_hist);
  ws.ctr = reinterpret_cast<uint32_t*>(base + lay.off_ctr);
  ws.meta = reinterpret_cast<int32_t*>(base + lay.off_meta);
  ws.nb_stride = lay.nb_stride;
  const int page_log2 = __builtin_ctz((unsigned)c.page_size);
  const int chunks = lay.nb_stride / kScoreChunk;
  dim3 grid(chunks, S);
  switch (c.index_dim) {
    case 32:
      hipLaunchKernelGGL(score_kernel<32>, grid, dim3(kThreads), 0, stream, q_index, sel_req,
                         sel_seq_len, block_table, c.max_pages_per_req, page_log2, ckey,
                         c.topk_blocks, max_seq_len, ws);
      break;
    case 64:
      hipLaunchKernelGGL(score_kernel<64>, grid, dim3(kThreads), 0, stream, q_index, sel_req,
                         sel_seq_len, block_table, c.max_pages_per_req, page_log2, ckey,
                         c.topk_blocks, max_seq_len, ws);
      break;
    case 128:
      hipLaunchKernelGGL(score_kernel<128>, grid, dim3(kThreads), 0, stream, q_index, sel_req,
                         sel_seq_len, block_table, c.max_pages_per_req, page_log2, ckey,
                         c.topk_blocks, max_seq_len, ws);
      break;
    default:
      return fail(QSA_ERR_UNSUPPORTED, "index_dim %d not built", c.index_dim);
  }
  qsa_status st = check_launch("qsa_index_topk(score)");
  if (st != QSA_OK || topk == nullptr) return st;
  hipLaunchKernelGGL(select_kernel, grid, dim3(kThreads), 0, stream, sel_seq_len, c.topk_blocks,
                     max_seq_len, topk, ws);
  return check_launch("qsa_index_topk(select)");
}

}  // namespace qsa
