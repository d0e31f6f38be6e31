// qsa_index_topk: exact block scores and top-k selection.
//
// Method ("Qwen 4 QSA 迎来解码上下文并行" blog, section on what the pull request
// changes): the indexer scores the compressed micro-blocks and keeps the best 512;
// ("PR #53896 完整报告", implementation breakdown / key source snippets) the
// selection is weight-free, on the compressed keys, returned as a fixed-width
// int32 buffer padded with -1.  Ties go to the lower block index, so the
// result is unique and can be compared bit for bit.
//
// Two kernels, no fences and no inter-workgroup waits (the kernel boundary
// publishes the scan's results):
//   score    (grid: chunk of 1024 micro-blocks x selecting row): streams the
//            10-bit compressed keys (the HBM-bound scan: an int8 plane s and two
//            bit-masks b0, b1 per block), computes
//            score = q.s (v_dot4_i32_i8) + 256 (2 q.b1 + q.b0) - 384 sum(q),
//            the masked sums as popcounts of the masks against the query's
//            bit-planes (built per wave with ballots), stores the int32 score,
//            adds an LDS histogram of the score's top 11 bits into the row's
//            histogram with device-scope atomics, and from that LDS histogram
//            writes the chunk's candidate list (every block at or above the
//            bin of its m-th best block; see chunk_candidates).
//   finalize (select_row in qsa_select.h: one workgroup per selecting row
//            here; qsa_select_sparse_decode runs the same steps inside its
//            attention kernel instead): the row's threshold bin T
//            (fewer than k scores above T, at least k at or above it) from the
//            row histogram; the chunks' lists, loaded in one round, are
//            classified against T (a chunk whose list may be short is re-read
//            from its scores); the missing blocks among the bin-T candidates
//            (usually a few hundred) are picked by a radix select; the bitmap
//            is emitted in ascending order with a popcount prefix sum and
//            padded with -1.  The workspace holds two histograms: a scan adds
//            into the one its call count picks, and the selection clears the
//            other, so the workspace stays clean between calls.
#include <mutex>

#include "qsa_append.h"
#include "qsa_device.h"
#include "qsa_internal.h"
#include "qsa_select.h"

namespace qsa {

namespace {

constexpr int kScoreThreads = 512;                     // score kernel
constexpr int kScoreIters = kScoreChunk / kScoreThreads;

// The append half of qsa_compress_index_topk (unused by the plain scan).
struct AppendArgs {
  const int8_t* new_keys;
  const int32_t* new_cu;
  const int32_t* seq_len_before;
  int8_t* ring;
  int8_t* ckey;        // the cache the scan reads, written here
  int32_t num_reqs;
  int32_t num_rows;    // selecting rows: grid rows below it score
  int32_t chunks;      // grid columns; grid rows from num_rows on append, one request per workgroup
};

// Chunk candidates.  Every chunk of 1,024 blocks keeps, as 64-bit keys
// (score, ~index) in its own region of the row's list, all its valid blocks
// whose bin is at or above its local bin: the bin of its m-th best valid block
// (all of them if it has fewer).  cinfo = count << 16 | local bin.  The
// finalize takes the row's threshold bin T from the row histogram: a chunk
// whose local bin is at most T has listed every block of bin >= T; one whose
// local bin is above T is read again from its scores.  m is sized so that the
// list usually fits the finalize's first round of loads (local_m).  The local
// bin is found by one wave walking down from the chunk's highest bin.
template <int NT, int IT>
__device__ __forceinline__ void chunk_candidates(const uint32_t* hist, int maxbin, const int32_t (&sc)[IT], int c,
                                                 int nb, int list_m, uint64_t* keys, uint32_t* cinfo,
                                                 int32_t* s_lb, uint32_t* s_cnt) {
  const int tid = threadIdx.x, l = lane_id();
  const int valid_total = min(kScoreChunk, nb - c * kScoreChunk);
  const uint32_t m = (uint32_t)min(list_m, valid_total);
  // The local bin, by wave 0 alone: 64 bins at a time downward from the
  // chunk's highest occupied bin (one step, as a rule); the count of all bins
  // is valid_total >= m, so the walk ends before bin 0.
  if (tid < 64) {
    int top = maxbin, lb = 0;
    uint32_t acc = 0;
    bool found = false;
    while (!found && top >= 0) {
      const int bin = top - l;
      const uint32_t cnt = bin >= 0 ? hist[bin] : 0u;
      const uint32_t inc = wave_incl_scan(cnt) + acc;
      const uint64_t hit = __ballot(inc >= m);
      if (hit) {
        found = true;
        lb = top - (__ffsll((long long)hit) - 1);
      } else {
        acc = (uint32_t)__builtin_amdgcn_readlane((int)inc, 63);
        top -= 64;
      }
    }
    if (l == 0) { *s_lb = lb; *s_cnt = 0; }
  }
  __syncthreads();
  const int lb = *s_lb;
  // one slot reservation per wave for all its iterations
  bool take[IT];
  uint64_t mask[IT];
  uint32_t total = 0;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int j = c * kScoreChunk + it * NT + tid;
    take[it] = j < nb && score_bin(sc[it]) >= lb;
    mask[it] = __ballot(take[it]);
    total += (uint32_t)__popcll(mask[it]);
  }
  if (total) {
    uint32_t base = 0;
    if (l == 0) base = atomicAdd(s_cnt, total);
    base = __builtin_amdgcn_readfirstlane(base);
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int j = c * kScoreChunk + it * NT + tid;
      if (take[it]) keys[base + lanes_below(mask[it])] = cand_key(sc[it], (uint32_t)j);
      base += (uint32_t)__popcll(mask[it]);
    }
  }
  __syncthreads();
  if (tid == 0) *cinfo = (*s_cnt << 16) | (uint32_t)lb;
}

// Highest bin of this thread's valid scores, merged into s_maxbin (one LDS
// atomic per wave).
template <int IT>
__device__ __forceinline__ void note_max_bin(const int32_t (&sc)[IT], int c, int nt, int nb, int* s_maxbin) {
  int mb = -1;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int j = c * kScoreChunk + it * nt + (int)threadIdx.x;
    mb = max(mb, j < nb ? score_bin(sc[it]) : -1);
  }
  mb = wave_max_i32(mb);
  if (lane_id() == 0) atomicMax(s_maxbin, mb);
}

// With kAppend (qsa_compress_index_topk) the grid has extra rows after the
// selecting rows: each of their workgroups appends one request's new tokens
// (closes its blocks into the cache and writes its ring, as qsa_compress
// does), while the workgroups above score.  A block closed in this call is scored from its raw keys
// (the sum over its 4 tokens of q . k is the same integer as q . C), so the
// scan never depends on the concurrent cache writes: its loads of those blocks
// are dropped.  The raw keys are the new tokens and, for the block straddling
// the previous call, ring slots of tokens before seq_len_before; the append
// writes only the slots of the new tokens, which differ from those while a
// request gets at most 8 - seq_len_before % 4 tokens (at most 5 always fits,
// and closes at most 2 blocks).  The raw loads go out with the cache loads, so
// the closing blocks add no round trip to the workgroups that hold them.
template <int D, bool kAppend>
__global__ __launch_bounds__(kScoreThreads) void score_kernel(
    const int8_t* __restrict__ q_index, const int32_t* __restrict__ sel_req,
    const int32_t* __restrict__ sel_seq_len, const int32_t* __restrict__ block_table,
    int32_t max_pages, int32_t page_log2, const int8_t* ckey,
    int32_t max_seq_len, WsPtrs ws, AppendArgs ap) {
  constexpr int kSChunks = D / 16;       // 16-byte chunks of the s plane
  constexpr int kMaskWords = D / 32;     // dwords per D-bit mask
  constexpr int kMaskLoads = (2 * kMaskWords + 3) / 4;
  __shared__ uint32_t hist[kBins];
  const int s = blockIdx.y;
  const int c = blockIdx.x;
  // (append variant: grid rows past the selecting rows read the last row's
  // entries, unused; num_rows >= 1 whenever it runs)
  const int sr = kAppend ? min(s, ap.num_rows - 1) : s;
  const int Lr = sel_seq_len[sr];
  const int b = sel_req[sr];
  const uint32_t tgen = ws.gen[1] + 1u;  // this call's count; its histogram is tgen & 1
  // Both row loads and the argument pointers in flight together: the compiler
  // would otherwise fetch each only after the exit tests below, one wait each.
  asm volatile("" ::"s"(Lr), "s"(b), "s"(tgen), "s"(block_table), "s"(q_index), "s"(ckey), "s"(max_pages),
               "s"(page_log2), "s"(ws.scores), "s"(ws.hist), "s"(ws.nb_stride));
  if (kAppend) {
    asm volatile("" ::"s"(ap.seq_len_before), "s"(ap.new_cu), "s"(ap.new_keys), "s"(ap.ring), "s"(ap.num_reqs),
                 "s"(ap.chunks), "s"(max_seq_len));
    if (s >= ap.num_rows) {
      const int r = (s - ap.num_rows) * ap.chunks + c;
      if (r < ap.num_reqs)
        append_request<D, kScoreThreads>(r, 0, 1, ap.new_keys, ap.new_cu, ap.seq_len_before, block_table,
                                         max_pages, page_log2, ap.ring, ap.ckey);
      return;
    }
  }
  const int L = min(Lr, max_seq_len);
  const int nb = max(L, 0) >> 2;
  const int nchunks = (nb + kScoreChunk - 1) / kScoreChunk;
  if (c >= nchunks) return;
  const int bpp_log2 = page_log2 - 2;
  const int bpp = 1 << bpp_log2;
  const size_t page_bytes = (size_t)bpp * (D + D / 4);

  // Loads are unconditional (past the row's end they re-read its last block and
  // the result is dropped): a guarded load becomes a branch, and the compiler
  // then drains all outstanding loads at every branch.
  const int32_t* bt = block_table + (size_t)b * max_pages;
  int page[kScoreIters];
#pragma unroll
  for (int it = 0; it < kScoreIters; ++it) {
    const int j = min(c * kScoreChunk + it * kScoreThreads + (int)threadIdx.x, nb - 1);
    page[it] = bt[j >> bpp_log2];
  }
  // This row's request appends after L0 tokens; blocks [jA, jA + nclose) close
  // in this call (nclose <= 2 for appends of at most 5 tokens).  The loads are
  // unconditional (num_reqs >= 1 whenever the append variant runs) and issued
  // after the page-table loads: the exit test above waits for every scalar load
  // in flight.
  int L0 = 0, row0 = 0, jA = 0, nclose = 0;
  if (kAppend) {
    const int bb = min(max(b, 0), ap.num_reqs - 1);
    L0 = ap.seq_len_before[bb];
    row0 = ap.new_cu[bb];
    const int n = ap.new_cu[bb + 1] - row0;
    jA = L0 >> 2;
    nclose = (b == bb && L0 >= 0 && n > 0) ? min(((L0 + n) >> 2) - jA, 2) : 0;
  }

  // All key loads at once (non-temporal: streamed once); each block is scored
  // as soon as its loads have arrived, while the later ones are still in flight.
  i32x4 v[kScoreIters][kSChunks];
  i32x4 mk[kScoreIters][kMaskLoads];
#pragma unroll
  for (int it = 0; it < kScoreIters; ++it) {
    const int j = min(c * kScoreChunk + it * kScoreThreads + (int)threadIdx.x, nb - 1);
    const int slot = j & (bpp - 1);
    const int8_t* pg = ckey + (size_t)page[it] * page_bytes;
#pragma unroll
    for (int ch = 0; ch < kSChunks; ++ch)
      v[it][ch] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(pg + (size_t)ch * bpp * 16 + (size_t)slot * 16));
    const int8_t* mp = pg + (size_t)kSChunks * bpp * 16 + (size_t)slot * (D / 4);
    if (D >= 64) {
#pragma unroll
      for (int m = 0; m < kMaskLoads; ++m)
        mk[it][m] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(mp + 16 * m));
    } else {  // D = 32: 8 mask bytes
      const i32x2 m2 = __builtin_nontemporal_load(reinterpret_cast<const i32x2*>(mp));
      mk[it][0] = i32x4{m2[0], m2[1], 0, 0};
    }
  }
  // Append variant: the raw-key scores of the (up to) two closing blocks, from
  // dword loads issued beside the cache loads.  Dword w = lane + 64 i of the
  // pair is block w / D, token (w % D) / (D/4), dims 4 (w % (D/4)) .. +3; every
  // wave computes both sums itself.  Dwords of blocks that do not close read
  // the query instead (valid memory; their sum is not used).
  constexpr int kRawPerLane = D / 32;     // 2 blocks x D dwords / 64 lanes
  int32_t raw[kRawPerLane], qd[kRawPerLane];
  if (kAppend) {
    const int lane = threadIdx.x & 63;
    const int8_t* qrow = q_index + (size_t)s * D;
#pragma unroll
    for (int i = 0; i < kRawPerLane; ++i) {
      const int w = lane + 64 * i;
      const int blk = w / D, e = (w % D) / (D / 4), g = w % (D / 4);
      const int t = kRatio * (jA + blk) + e;
      const int8_t* src = blk >= nclose ? qrow
                          : (t >= L0 ? ap.new_keys + (size_t)(row0 + (t - L0)) * D
                                     : ap.ring + ((size_t)b * kRing + (t & (kRing - 1))) * D);
      raw[i] = *reinterpret_cast<const int32_t*>(src + 4 * g);
      qd[i] = *reinterpret_cast<const int32_t*>(qrow + 4 * g);
    }
  }
  // Indexer query: D int8 as D/4 packed dwords (uniform across the workgroup),
  // and its bit-planes qp[t][w]: bit k of dword w is bit t of q[32w + k]
  // (two's complement, so plane 7 weighs -128).  Every wave builds them with
  // ballots, lane l holding q[l] (and q[64 + l] when D = 128).
  int32_t qw[D / 4];
  const int32_t* q32 = reinterpret_cast<const int32_t*>(q_index + (size_t)s * D);
#pragma unroll
  for (int i = 0; i < D / 4; ++i) qw[i] = q32[i];
  int32_t qsum = 0;
#pragma unroll
  for (int i = 0; i < D / 4; ++i) qsum = __builtin_amdgcn_sdot4(qw[i], 0x01010101, qsum, false);
  const int lane = threadIdx.x & 63;
  uint32_t qp[8][kMaskWords];
#pragma unroll
  for (int h = 0; h < (D + 63) / 64; ++h) {
    const int dim = 64 * h + lane;
    const int qv = (int)q_index[(size_t)s * D + min(dim, D - 1)];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const uint64_t m = __builtin_amdgcn_ballot_w64(dim < D && ((qv >> t) & 1));
      qp[t][2 * h] = (uint32_t)m;
      if (2 * h + 1 < kMaskWords) qp[t][2 * h + 1] = (uint32_t)(m >> 32);
    }
  }
  // The histogram is cleared while the keys stream in (a barrier does not wait
  // for outstanding loads), so the arithmetic below is followed by no barrier
  // before the histogram updates.
  __shared__ int s_maxbin;
  for (int i = threadIdx.x; i < kBins; i += kScoreThreads) hist[i] = 0;
  if (threadIdx.x == 0) s_maxbin = -1;
  __syncthreads();
  int32_t sc[kScoreIters];
#pragma unroll
  for (int it = 0; it < kScoreIters; ++it) {
    int32_t sd = 0;
#pragma unroll
    for (int ch = 0; ch < kSChunks; ++ch)
#pragma unroll
      for (int e = 0; e < 4; ++e) sd = __builtin_amdgcn_sdot4(v[it][ch][e], qw[4 * ch + e], sd, false);
    // hq = sum_i q[i] (2 b1[i] + b0[i]) = sum_t w_t (2 |Q_t & B1| + |Q_t & B0|)
    int32_t hq = 0;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      uint32_t p0 = 0, p1 = 0;
#pragma unroll
      for (int w = 0; w < kMaskWords; ++w) {
        const int x0 = w, x1 = kMaskWords + w;   // mask dword index of b0, b1
        p0 = __builtin_popcount(qp[t][w] & (uint32_t)mk[it][x0 >> 2][x0 & 3]) + p0;
        p1 = __builtin_popcount(qp[t][w] & (uint32_t)mk[it][x1 >> 2][x1 & 3]) + p1;
      }
      const int32_t xt = (int32_t)(2 * p1 + p0);
      hq += (t == 7) ? -(xt << 7) : (xt << t);
    }
    sc[it] = 256 * hq + sd - 384 * qsum;
  }
  if (kAppend) {
    int32_t p0 = 0, p1 = 0;
#pragma unroll
    for (int i = 0; i < kRawPerLane; ++i) {
      const int32_t p = __builtin_amdgcn_sdot4(raw[i], qd[i], 0, false);
      const bool first = (lane + 64 * i) < D;
      p0 += first ? p : 0;
      p1 += first ? 0 : p;
    }
    p0 = (int32_t)__builtin_amdgcn_readlane((int)wave_incl_scan((uint32_t)p0), 63);
    p1 = (int32_t)__builtin_amdgcn_readlane((int)wave_incl_scan((uint32_t)p1), 63);
#pragma unroll
    for (int it = 0; it < kScoreIters; ++it) {
      const int rel = c * kScoreChunk + it * kScoreThreads + (int)threadIdx.x - jA;
      sc[it] = (rel >= 0 && rel < nclose) ? (rel == 0 ? p0 : p1) : sc[it];
    }
  }
#pragma unroll
  for (int it = 0; it < kScoreIters; ++it) {
    const int j = c * kScoreChunk + it * kScoreThreads + threadIdx.x;
    atomicAdd(&hist[score_bin(sc[it])], j < nb ? 1u : 0u);
  }
  note_max_bin<kScoreIters>(sc, c, kScoreThreads, nb, &s_maxbin);
  __syncthreads();
  // No branches here either: the workspace has score slots up to the chunk's
  // end (slots past the row's end are never read).  The per-row histogram is
  // merged with device-scope atomics, read by the next kernel after this one
  // has finished (no fence needed here).
  int32_t* srow = ws.scores + (size_t)s * ws.nb_stride;
#pragma unroll
  for (int it = 0; it < kScoreIters; ++it) srow[c * kScoreChunk + it * kScoreThreads + threadIdx.x] = sc[it];
  uint32_t* ghist = ws.hist + (size_t)(tgen & 1u) * ws.hist_stride + (size_t)s * kBins;
  if (threadIdx.x == 0) ws.gen[0] = tgen;  // (every scoring workgroup writes the same count)
  for (int i = threadIdx.x; i < kBins; i += kScoreThreads) {
    const uint32_t h = hist[i];
    if (h) atomicAdd(&ghist[i], h);
  }
  // this chunk's candidates for the finalize (no separate filter pass)
  __shared__ int32_t s_lb;
  __shared__ uint32_t s_cnt;
  chunk_candidates<kScoreThreads, kScoreIters>(hist, s_maxbin, sc, c, nb, ws.list_m,
                                               ws.keys + (size_t)s * ws.nb_stride + (size_t)c * kScoreChunk,
                                               ws.cinfo + (size_t)s * (ws.nb_stride / kScoreChunk) + c,
                                               &s_lb, &s_cnt);
}

// Finalize: one workgroup per selecting row (select_row); then the row of the
// next call's histogram is cleared and the count published.
template <bool kBmLds>
__global__ __launch_bounds__(kFinThreads) void finalize_kernel(
    const int32_t* __restrict__ sel_seq_len, int32_t k, int32_t max_seq_len,
    int32_t* __restrict__ topk, WsPtrs ws) {
  const int s = blockIdx.x;
  const uint32_t t = select_row<kBmLds>(s, sel_seq_len, k, max_seq_len, topk + (size_t)s * k, ws);
  // Last, so that no store is outstanding while the phases above wait for
  // their loads (the wait counter covers stores too).
  clear_next_hist(ws, s, t);
  if (s == 0 && threadIdx.x == 0) ws.gen[1] = t;
}

// ---------------------------------------------------------------------------
// Prefill scoring (many query rows per request, each with its own causal
// length): the scan becomes an int8 GEMM, rows x blocks.  A workgroup takes 16
// rows of one request (the MFMA M dimension) and a chunk of 1,024 blocks; each
// of its 4 waves takes 16 tiles of 16 blocks.  Per tile,
//   v_mfma_i32_16x16x64_i8(q, s)  and  v_mfma_i32_16x16x64_i8(q, h),
// h = 2 b1 + b0 expanded from the bit-masks to bytes, give
// score = q.s + 256 q.h - 384 sum(q) exactly in int32.  The B operand of lane l
// is the 16-byte s-plane chunk l/16 of block l%16: a plain 16-byte load from
// the page, no LDS.  Per-row histograms (16-bit counts, two per LDS word) are
// merged into the rows' histograms as in the decode scan, and from them each
// row's candidate list for the chunk is written from the scores still in
// registers (the scores are stored too, for rows whose list may be short);
// the finalize then selects exactly as for qsa_index_topk.
constexpr int kPfThreads = 256;
constexpr int kPfRows = 16;
constexpr int kPfTiles = kScoreChunk / (kPfThreads / 64) / 16;  // block tiles per wave

__device__ __forceinline__ uint32_t spread_nibble(uint32_t n) {  // bit e of n -> byte e (0/1)
  return (n * 0x00204081u) & 0x01010101u;
}

__device__ __forceinline__ int32_t sum_lane_groups(int32_t v) {  // sum over lanes l, l^16, l^32, l^48
  auto a = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
  v = (int32_t)(a[0] + a[1]);
  auto b = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
  return (int32_t)(b[0] + b[1]);
}

template <int D>
__global__ __launch_bounds__(kPfThreads) void prefill_score_kernel(
    const int8_t* __restrict__ q_index, const int32_t* __restrict__ row_cu,
    const int32_t* __restrict__ row_seq_len, const int32_t* __restrict__ block_table,
    int32_t max_pages, int32_t page_log2, const int8_t* ckey, int32_t max_seq_len, WsPtrs ws) {
  constexpr int KS = (D + 63) / 64;  // MFMA k-steps of 64 dims (D = 32: the upper half is zero)
  constexpr int kSChunks = D / 16;
  __shared__ uint32_t hist[kPfRows * kBins / 2];
  const int c = blockIdx.x, tile = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, col = lane & 15;
  const int r_end = row_cu[b + 1];
  const int r0 = row_cu[b] + tile * kPfRows;
  const uint32_t tgen = ws.gen[1] + 1u;  // this call's count; its histogram is tgen & 1
  if (r0 >= r_end) return;
  // Lane col holds row r0+col: its length (0 past the request's rows).
  const int rc = min(r0 + col, r_end - 1);
  const int lr = (r0 + col < r_end) ? min(row_seq_len[rc], max_seq_len) : 0;
  const int nbc = max(lr, 0) >> 2;
  int nbmax = nbc;
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) nbmax = max(nbmax, __shfl_xor(nbmax, o, 64));
  if (c * kScoreChunk >= nbmax) return;  // uniform: every row of the tile ends before this chunk
  const int bpp_log2 = page_log2 - 2;
  const int bpp = 1 << bpp_log2;
  const size_t page_bytes = (size_t)bpp * (D + D / 4);
  const int32_t* bt = block_table + (size_t)b * max_pages;

  // A operand: row r0+col, dims 64 ks + 16 g .. +15 (zero past the request's rows or past D).
  i32x4 qa[KS];
  int32_t qpart = 0;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int dim = 64 * ks + 16 * g;
    const i32x4 v = *reinterpret_cast<const i32x4*>(q_index + (size_t)rc * D + min(dim, D - 16));
    const bool live = (r0 + col < r_end) && dim < D;
    qa[ks] = live ? v : i32x4{0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < 4; ++e) qpart = __builtin_amdgcn_sdot4(qa[ks][e], 0x01010101, qpart, false);
  }
  const int32_t qsum_col = sum_lane_groups(qpart);  // sum(q) of row r0+col
  int32_t qsum_m[4], nb_m[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {  // C rows 4g+i of this lane
    qsum_m[i] = __shfl(qsum_col, 4 * g + i, 64);
    nb_m[i] = __shfl(nbc, 4 * g + i, 64);
  }

  // Page ids of the wave's tiles, then all key loads (blocks clamped to the
  // tile's longest row: they exist in the cache).
  const int jw = c * kScoreChunk + w * (kPfTiles * 16);
  int pg[kPfTiles];
#pragma unroll
  for (int t = 0; t < kPfTiles; ++t) {
    const int jc = min(jw + 16 * t + col, nbmax - 1);
    pg[t] = bt[jc >> bpp_log2];
  }
  i32x4 bs[kPfTiles][KS];
  uint32_t m0[kPfTiles][KS], m1[kPfTiles][KS];
#pragma unroll
  for (int t = 0; t < kPfTiles; ++t) {
    const int jc = min(jw + 16 * t + col, nbmax - 1);
    const int slot = jc & (bpp - 1);
    const int8_t* page = ckey + (size_t)pg[t] * page_bytes;
    const uint8_t* mp = reinterpret_cast<const uint8_t*>(page + (size_t)kSChunks * bpp * 16 + (size_t)slot * (D / 4));
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int ch = min(4 * ks + g, kSChunks - 1);
      bs[t][ks] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(page + (size_t)ch * bpp * 16 + (size_t)slot * 16));
      m0[t][ks] = *reinterpret_cast<const uint16_t*>(mp + 2 * ch);
      m1[t][ks] = *reinterpret_cast<const uint16_t*>(mp + D / 8 + 2 * ch);
    }
  }
  __shared__ int s_pmax[kPfRows];       // per row: highest bin of its valid scores in this chunk
  __shared__ int s_plb[kPfRows];        // per row: local bin of its candidate list
  __shared__ uint32_t s_pcnt[kPfRows];  // per row: list length
  for (int i = threadIdx.x; i < kPfRows * kBins / 2; i += kPfThreads) hist[i] = 0;
  if (threadIdx.x < kPfRows) { s_pmax[threadIdx.x] = -1; s_pcnt[threadIdx.x] = 0; }
  __syncthreads();

  int32_t scv[kPfTiles][4];  // the scores stay here for the candidate lists
  int mb[4] = {-1, -1, -1, -1};
#pragma unroll
  for (int t = 0; t < kPfTiles; ++t) {
    i32x4 cs = {0, 0, 0, 0}, chh = {0, 0, 0, 0};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bool live = 64 * ks + 16 * g < D;
      i32x4 bh;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        bh[e] = (int32_t)(spread_nibble((m0[t][ks] >> (4 * e)) & 15u) + 2u * spread_nibble((m1[t][ks] >> (4 * e)) & 15u));
      const i32x4 bsv = live ? bs[t][ks] : i32x4{0, 0, 0, 0};
      bh = live ? bh : i32x4{0, 0, 0, 0};
      cs = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[ks], bsv, cs, 0, 0, 0);
      chh = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[ks], bh, chh, 0, 0, 0);
    }
    const int j = jw + 16 * t + col;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * g + i;
      const int r = r0 + m;
      const int32_t sc = cs[i] + 256 * chh[i] - 384 * qsum_m[i];
      const bool valid = j < nb_m[i];  // rows past the request's end have nb 0
      const int bin = score_bin(sc);
      atomicAdd(&hist[(m * kBins + bin) >> 1], valid ? ((bin & 1) ? 0x10000u : 1u) : 0u);
      mb[i] = max(mb[i], valid ? bin : -1);
      scv[t][i] = sc;
      if (r < r_end) ws.scores[(size_t)r * ws.nb_stride + j] = sc;
    }
  }
  // highest bin per row: the 16 lanes of a lane group (one DPP row) share its rows
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int v = mb[i];
    v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x111, 0xf, 0xf, false));  // row_shr:1
    v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x112, 0xf, 0xf, false));  // row_shr:2
    v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x114, 0xf, 0xf, false));  // row_shr:4
    v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x118, 0xf, 0xf, false));  // row_shr:8
    if (col == 15) atomicMax(&s_pmax[4 * g + i], v);
  }
  __syncthreads();
  if (threadIdx.x == 0) ws.gen[0] = tgen;  // (every scoring workgroup writes the same count)
  for (int i = threadIdx.x; i < kPfRows * kBins / 2; i += kPfThreads) {
    const uint32_t h = hist[i];
    const int m = (2 * i) / kBins, bin = (2 * i) % kBins;
    if (h && r0 + m < r_end) {
      uint32_t* gh = ws.hist + (size_t)(tgen & 1u) * ws.hist_stride + (size_t)(r0 + m) * kBins + bin;
      if (h & 0xffffu) atomicAdd(gh, h & 0xffffu);
      if (h >> 16) atomicAdd(gh + 1, h >> 16);
    }
  }
  // Each row's candidate list for this chunk, as the decode scan writes it
  // (chunk_candidates): the local bin of its m-th best valid block, found by
  // wave w for rows w, w + 4, w + 8, w + 12 walking down from the row's
  // highest bin; then every valid block at or above it.
  const int lm = ws.list_m;
  for (int m = w; m < kPfRows; m += kPfThreads / 64) {
    const int nbr = __shfl(nbc, m, 64);  // lane m holds row r0 + m's length
    const int valid_total = min(kScoreChunk, nbr - c * kScoreChunk);
    if (valid_total <= 0) continue;       // uniform: the row ends before this chunk
    const uint32_t mm = (uint32_t)min(lm, valid_total);
    int top = s_pmax[m], lb = 0;
    uint32_t acc = 0;
    bool found = false;
    while (!found && top >= 0) {
      const int bin = top - lane;
      const uint32_t cnt = bin >= 0 ? (hist[(m * kBins + bin) >> 1] >> (16 * (bin & 1))) & 0xffffu : 0u;
      const uint32_t inc = wave_incl_scan(cnt) + acc;
      const uint64_t hit = __ballot(inc >= mm);
      if (hit) {
        found = true;
        lb = top - (__ffsll((long long)hit) - 1);
      } else {
        acc = (uint32_t)__builtin_amdgcn_readlane((int)inc, 63);
        top -= 64;
      }
    }
    if (lane == 0) s_plb[m] = lb;
  }
  __syncthreads();
  {
    const int nch = ws.nb_stride / kScoreChunk;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * g + i;
      if (r0 + m >= r_end) continue;
      const int lb = s_plb[m];  // set for every row that reaches this chunk
      uint64_t* keys = ws.keys + (size_t)(r0 + m) * ws.nb_stride + (size_t)c * kScoreChunk;
#pragma unroll
      for (int t = 0; t < kPfTiles; ++t) {
        const int j = jw + 16 * t + col;
        if (j < nb_m[i] && score_bin(scv[t][i]) >= lb) keys[atomicAdd(&s_pcnt[m], 1u)] = cand_key(scv[t][i], (uint32_t)j);
      }
    }
    __syncthreads();
    if (threadIdx.x < kPfRows) {
      const int m = threadIdx.x;
      const int nbr = nbc;  // lane m of wave 0 holds row r0 + m's length
      if (r0 + m < r_end && nbr > c * kScoreChunk)
        ws.cinfo[(size_t)(r0 + m) * nch + c] = (s_pcnt[m] << 16) | (uint32_t)s_plb[m];
    }
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
  w.off_keys2 = off;  off = al(off + (size_t)rows * w.nb_stride * 8);
  w.off_hist = off;   off = al(off + 2 * (size_t)rows * kBins * 4);
  w.off_cinfo = off;  off = al(off + (size_t)rows * (w.nb_stride / kScoreChunk) * 4);
  w.off_gen = off;    off = al(off + 2 * 4);
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

namespace {

template <bool kAppend>
qsa_status launch_scan(const qsa_config& c, dim3 grid, const int8_t* q_index, const int32_t* sel_req,
                       const int32_t* sel_seq_len, const int32_t* block_table, const int8_t* ckey,
                       int32_t max_seq_len, const WsPtrs& ws, const AppendArgs& ap, hipStream_t stream) {
  const int page_log2 = __builtin_ctz((unsigned)c.page_size);
  switch (c.index_dim) {
    case 32:
      hipLaunchKernelGGL((score_kernel<32, kAppend>), grid, dim3(kScoreThreads), 0, stream, q_index, sel_req,
                         sel_seq_len, block_table, c.max_pages_per_req, page_log2, ckey, max_seq_len, ws, ap);
      break;
    case 64:
      hipLaunchKernelGGL((score_kernel<64, kAppend>), grid, dim3(kScoreThreads), 0, stream, q_index, sel_req,
                         sel_seq_len, block_table, c.max_pages_per_req, page_log2, ckey, max_seq_len, ws, ap);
      break;
    case 128:
      hipLaunchKernelGGL((score_kernel<128, kAppend>), grid, dim3(kScoreThreads), 0, stream, q_index, sel_req,
                         sel_seq_len, block_table, c.max_pages_per_req, page_log2, ckey, max_seq_len, ws, ap);
      break;
    default:
      return fail(QSA_ERR_UNSUPPORTED, "index_dim %d not built", c.index_dim);
  }
  return QSA_OK;
}

qsa_status launch_finalize(int32_t rows, const int32_t* seq_len, int32_t k, int32_t max_seq_len, int32_t* topk,
                           const WsPtrs& ws, hipStream_t stream, const char* what) {
  if (ws.nb_stride / 64 <= kWordsLds)
    hipLaunchKernelGGL(finalize_kernel<true>, dim3(rows), dim3(kFinThreads), 0, stream, seq_len, k, max_seq_len,
                       topk, ws);
  else
    hipLaunchKernelGGL(finalize_kernel<false>, dim3(rows), dim3(kFinThreads), 0, stream, seq_len, k, max_seq_len,
                       topk, ws);
  return check_launch(what);
}

}  // namespace

qsa_status launch_finalize_ws(const qsa_config& c, int32_t rows, const int32_t* seq_len, int32_t max_seq_len,
                              int32_t* topk, const TopkWorkspace& lay, void* ws_base, hipStream_t stream) {
  if (rows == 0) return QSA_OK;
  return launch_finalize(rows, seq_len, c.topk_blocks, max_seq_len, topk, ws_ptrs(lay, ws_base), stream,
                         "qsa_select_sparse_decode(finalize)");
}

qsa_status launch_index_topk(const qsa_config& c, int32_t S, int32_t max_seq_len,
                             const int8_t* q_index, const int32_t* sel_req,
                             const int32_t* sel_seq_len, const int32_t* block_table,
                             const int8_t* ckey, int32_t* topk, const TopkWorkspace& lay,
                             void* ws_base, hipStream_t stream) {
  if (S == 0) return QSA_OK;
  const WsPtrs ws = ws_ptrs(lay, ws_base);
  const AppendArgs none{};
  qsa_status st = launch_scan<false>(c, dim3(lay.nb_stride / kScoreChunk, S), q_index, sel_req, sel_seq_len,
                                     block_table, ckey, max_seq_len, ws, none, stream);
  if (st != QSA_OK) return st;
  st = check_launch("qsa_index_topk(score)");
  if (st != QSA_OK || topk == nullptr) return st;
  return launch_finalize(S, sel_seq_len, c.topk_blocks, max_seq_len, topk, ws, stream, "qsa_index_topk(finalize)");
}

qsa_status launch_compress_index_topk(const qsa_config& c, int32_t num_reqs, const int8_t* new_keys,
                                      const int32_t* new_cu, const int32_t* seq_len_before, int8_t* ring,
                                      int8_t* ckey, int32_t S, int32_t max_seq_len, const int8_t* q_index,
                                      const int32_t* sel_req, const int32_t* sel_seq_len,
                                      const int32_t* block_table, int32_t* topk, const TopkWorkspace& lay,
                                      void* ws_base, hipStream_t stream) {
  if (S == 0 && num_reqs == 0) return QSA_OK;
  // nothing to select, or nothing to append: the plain calls
  if (S == 0) return launch_compress(c, num_reqs, 5, new_keys, new_cu, seq_len_before, block_table, ring, ckey, stream);
  if (num_reqs == 0)
    return launch_index_topk(c, S, max_seq_len, q_index, sel_req, sel_seq_len, block_table, ckey, topk, lay,
                             ws_base, stream);
  const WsPtrs ws = ws_ptrs(lay, ws_base);
  const int chunks = lay.nb_stride / kScoreChunk;
  const AppendArgs ap{new_keys, new_cu, seq_len_before, ring, ckey, num_reqs, S, chunks};
  // the append workgroups come after all scoring ones, so that they do not
  // change how the scoring workgroups spread over the compute units
  const int rows = S + (num_reqs + chunks - 1) / chunks;
  if (rows > 65535) {  // beyond the grid's row limit: the two calls, one after the other
    qsa_status st = launch_compress(c, num_reqs, 5, new_keys, new_cu, seq_len_before, block_table, ring, ckey,
                                    stream);
    if (st != QSA_OK) return st;
    return launch_index_topk(c, S, max_seq_len, q_index, sel_req, sel_seq_len, block_table, ckey, topk, lay,
                             ws_base, stream);
  }
  qsa_status st = launch_scan<true>(c, dim3(chunks, rows), q_index, sel_req, sel_seq_len,
                                    block_table, ckey, max_seq_len, ws, ap, stream);
  if (st != QSA_OK) return st;
  st = check_launch("qsa_compress_index_topk(append+score)");
  if (st != QSA_OK || topk == nullptr) return st;
  return launch_finalize(S, sel_seq_len, c.topk_blocks, max_seq_len, topk, ws, stream,
                         "qsa_compress_index_topk(finalize)");
}

// ---- the library's own scratch (qsa_index_topk_noalloc) ----
// A file-scope device array: every GPU the library runs on holds its own copy
// until the process ends.  Host code never passes its name to a kernel (on the
// host it is only a stand-in); the device address comes from
// hipGetSymbolAddress, once per device, with that device current.
namespace {
static __device__ __align__(256) uint8_t scratch[QSA_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

qsa_status noalloc_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(QSA_ERR_HIP, "qsa_index_topk_noalloc: hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(QSA_ERR_UNSUPPORTED, "qsa_index_topk_noalloc: device %d beyond the %d the library tracks", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return fail(QSA_ERR_HIP, "qsa_index_topk_noalloc: hipGetSymbolAddress of the scratch failed: %s",
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return QSA_OK;
}

qsa_status launch_index_topk_noalloc(const qsa_config& c, int32_t S, int32_t max_seq_len, const int8_t* q_index,
                                     const int32_t* sel_req, const int32_t* sel_seq_len, const int32_t* block_table,
                                     const int8_t* ckey, int32_t* topk, hipStream_t stream) {
  if (S == 0) return QSA_OK;
  const TopkWorkspace lay = topk_workspace_layout(S, max_seq_len);
  void* ws = nullptr;
  qsa_status st = noalloc_scratch(&ws);
  if (st != QSA_OK) return st;
  // The scratch keeps the last call's contents, whose layout may differ: the
  // histograms and the call counters (everything the scan reads before it
  // writes) are zeroed first, by a fill kernel.
  st = launch_ws_clear(reinterpret_cast<char*>(ws) + lay.off_hist, lay.off_cinfo - lay.off_hist, stream);
  if (st != QSA_OK) return st;
  st = launch_ws_clear(reinterpret_cast<char*>(ws) + lay.off_gen, lay.total - lay.off_gen, stream);
  if (st != QSA_OK) return st;
  return launch_index_topk(c, S, max_seq_len, q_index, sel_req, sel_seq_len, block_table, ckey, topk, lay, ws,
                           stream);
}

qsa_status launch_prefill_index_topk(const qsa_config& c, int32_t B, int32_t R, int32_t max_rows,
                                     int32_t max_seq_len, const int8_t* q_index, const int32_t* row_cu,
                                     const int32_t* row_seq_len, const int32_t* block_table,
                                     const int8_t* ckey, int32_t* topk, const TopkWorkspace& lay,
                                     void* ws_base, hipStream_t stream) {
  if (R == 0 || B == 0) return QSA_OK;
  const WsPtrs ws = ws_ptrs(lay, ws_base);
  const int page_log2 = __builtin_ctz((unsigned)c.page_size);
  const int chunks = lay.nb_stride / kScoreChunk;
  dim3 grid(chunks, (max_rows + kPfRows - 1) / kPfRows, B);
  switch (c.index_dim) {
    case 32:
      hipLaunchKernelGGL(prefill_score_kernel<32>, grid, dim3(kPfThreads), 0, stream, q_index, row_cu,
                         row_seq_len, block_table, c.max_pages_per_req, page_log2, ckey, max_seq_len, ws);
      break;
    case 64:
      hipLaunchKernelGGL(prefill_score_kernel<64>, grid, dim3(kPfThreads), 0, stream, q_index, row_cu,
                         row_seq_len, block_table, c.max_pages_per_req, page_log2, ckey, max_seq_len, ws);
      break;
    case 128:
      hipLaunchKernelGGL(prefill_score_kernel<128>, grid, dim3(kPfThreads), 0, stream, q_index, row_cu,
                         row_seq_len, block_table, c.max_pages_per_req, page_log2, ckey, max_seq_len, ws);
      break;
    default:
      return fail(QSA_ERR_UNSUPPORTED, "index_dim %d not built", c.index_dim);
  }
  qsa_status st = check_launch("qsa_prefill_index_topk(score)");
  if (st != QSA_OK || topk == nullptr) return st;
  return launch_finalize(R, row_seq_len, c.topk_blocks, max_seq_len, topk, ws, stream,
                         "qsa_prefill_index_topk(finalize)");
}

}  // namespace qsa
