// Row selection from a scored workspace: the finalize step of qsa_index_topk.
//
// Method ("Qwen 4 QSA 迎来解码上下文并行" blog, section on what the pull request
// changes): keep the best 512 micro-blocks of a row; ("PR #53896 完整报告",
// implementation breakdown / key source snippets) weight-free top-k over the
// compressed keys, fixed-width int32 output padded with -1.  Ties go to the
// lower block index.
//
// The scan kernels (qsa_index.hip) leave per row: the exact int32 scores, a
// histogram of the scores' top bits and, per chunk of 1,024 blocks, a candidate
// list.  select_row turns that into the row's ascending top-k in the
// finalize kernel (one workgroup per row); RowSelector below runs the same
// steps at the head of the fused selection + attention kernel (qsa_decode.hip),
// where every workgroup of a row computes the selection into its LDS and
// lists only its own split's run.
#pragma once

#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {

namespace {

constexpr int kFinKeys = 8;  // candidate keys per finalize thread and round

// Finalize threads per chunk in a round: as many as share the 512 threads with
// every chunk of the widest row (one round of loads covers rows of up to 512
// chunks), at most kScoreChunk / kFinKeys (a round never reads past a chunk's
// list region).
__host__ __device__ __forceinline__ int chunk_threads(int nb_stride) {
  const int nch = nb_stride / kScoreChunk;
  int t = 1;
  while (t * 2 * nch <= 512 && t * 2 * kFinKeys <= kScoreChunk) t *= 2;
  return t;
}
// Keys per thread in the fused kernel's first round: 4 where a chunk has at
// least 16 threads (rows of up to 32 chunks, 131,072 tokens), 6 at 8 threads
// (up to 64 chunks, 262,144 tokens), else kFinKeys.
__host__ __device__ __forceinline__ int fused_keys(int nb_stride) {
  const int t = chunk_threads(nb_stride);
  return t >= 16 ? 4 : (t == 8 ? 6 : kFinKeys);
}
// Each chunk lists at least local_m candidates (with the ties of its last
// bin): half as many as the first round's keys per thread, times the threads
// per chunk (tpc).  A top-512 takes about tpc blocks from a row's average
// chunk, so the lists hold 2, 3 or 4 times that (4, 6 or 8 keys), and with the
// ties of their last bin they still fit the round: the count's spread is small
// against 2 x its mean at 16 or more threads per chunk; at 8 (rows of 262,144
// tokens) a 2 x list sends chunks to the score fallback, and a 3 x list with
// its ties needs up to 6 keys per thread (it overflows 4 in about a third of
// the chunks).
__host__ __device__ __forceinline__ int local_m(int nb_stride) {
  const int t = chunk_threads(nb_stride);
  return t * (fused_keys(nb_stride) / 2);
}

struct WsPtrs {
  int32_t* scores;
  uint64_t* keys;
  uint64_t* bitmap;
  uint64_t* keys2;
  uint32_t* hist;       // two histograms of rows x kBins, hist_stride apart
  uint32_t* cinfo;
  uint32_t* gen;        // [0]: calls scored, [1]: calls selected (see TopkWorkspace)
  size_t hist_stride;
  int32_t nb_stride;
  int32_t list_m;       // local_m(nb_stride): the scans' candidate-list length
};

inline WsPtrs ws_ptrs(const TopkWorkspace& lay, void* ws_base) {
  char* base = reinterpret_cast<char*>(ws_base);
  WsPtrs ws;
  ws.scores = reinterpret_cast<int32_t*>(base + lay.off_scores);
  ws.keys = reinterpret_cast<uint64_t*>(base + lay.off_keys);
  ws.bitmap = reinterpret_cast<uint64_t*>(base + lay.off_bitmap);
  ws.keys2 = reinterpret_cast<uint64_t*>(base + lay.off_keys2);
  ws.hist = reinterpret_cast<uint32_t*>(base + lay.off_hist);
  ws.cinfo = reinterpret_cast<uint32_t*>(base + lay.off_cinfo);
  ws.gen = reinterpret_cast<uint32_t*>(base + lay.off_gen);
  ws.hist_stride = (size_t)lay.rows * kBins;
  ws.nb_stride = lay.nb_stride;
  ws.list_m = local_m(lay.nb_stride);
  return ws;
}

__device__ __forceinline__ int score_bin(int32_t s) {
  return (int)(((uint32_t)(s + (1 << 24))) >> kBinShift);
}

// 64-bit candidate key: larger key = higher score, then lower block index.
__device__ __forceinline__ uint64_t cand_key(int32_t score, uint32_t j) {
  return ((uint64_t)((uint32_t)score ^ 0x80000000u) << 32) | (uint64_t)(0xffffffffu - j);
}

__device__ __forceinline__ int32_t key_score(uint64_t key) {
  return (int32_t)((uint32_t)(key >> 32) ^ 0x80000000u);
}

// Block-wide exclusive prefix sum (blockDim.x threads, a multiple of 64).
// kReuse: end with a barrier, so that sh may be written again right away.
template <int NT, bool kReuse = true>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* sh /*[NT/64]*/) {
  const int l = lane_id(), w = threadIdx.x / 64;
  const uint32_t inc = wave_incl_scan(v);
  if (l == 63) sh[w] = inc;
  __syncthreads();
  uint32_t off = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) off += (i < w) ? sh[i] : 0u;
  if (kReuse) __syncthreads();
  return off + inc - v;
}

// Threshold bin from a histogram held as per-thread counts (thread t holds
// bins kBins-1-(kPer t + i), i.e. descending): the bin T with
// count(bins > T) < ks <= count(bins >= T).  Writes (T, count above T).
template <int NT>
__device__ __forceinline__ void threshold_from_counts(const uint32_t (&cnt)[kBins / NT], uint32_t ks,
                                                      uint32_t* sh, int32_t* s_T, uint32_t* s_above) {
  constexpr int kPer = kBins / NT;
  const int tid = threadIdx.x;
  uint32_t mine = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) mine += cnt[i];
  // sh is next written after the barrier below
  uint32_t above = block_excl_scan<NT, false>(mine, sh);
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    if (above < ks && above + cnt[i] >= ks) { *s_T = kBins - 1 - (kPer * tid + i); *s_above = above; }
    above += cnt[i];
  }
  __syncthreads();
}

template <int NT>
__device__ __forceinline__ void load_hist_desc(const uint32_t* h, uint32_t (&cnt)[kBins / NT]) {
  constexpr int kPer = kBins / NT;
#pragma unroll
  for (int i = 0; i < kPer; ++i) cnt[i] = h[kBins - 1 - (kPer * threadIdx.x + i)];
}

// The digit of an MSB-first radix select from one pass's 256-bin histogram:
// lane l owns digits 255-4l .. 252-4l (descending).  Picks the digit holding
// the rem-th largest key; returns the count in larger digits and in the digit.
__device__ __forceinline__ void radix_digit(const uint32_t* h, uint32_t rem, uint32_t& dsel, uint32_t& larger,
                                            uint32_t& cnt) {
  const int l = lane_id();
  const uint4 hv = *reinterpret_cast<const uint4*>(&h[252 - 4 * l]);
  const uint32_t cs[4] = {hv.w, hv.z, hv.y, hv.x};
  const uint32_t tot = cs[0] + cs[1] + cs[2] + cs[3];
  uint32_t acc = wave_incl_scan(tot) - tot;  // count in larger digits
  dsel = 0; larger = 0; cnt = 0;
  bool found = false;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (!found && acc < rem && acc + cs[i] >= rem) { found = true; dsel = 255 - 4 * l - i; larger = acc; cnt = cs[i]; }
    acc += cs[i];
  }
  const int src = __ffsll((long long)__ballot(found)) - 1;
  dsel = (uint32_t)__builtin_amdgcn_readlane((int)dsel, src);
  larger = (uint32_t)__builtin_amdgcn_readlane((int)larger, src);
  cnt = (uint32_t)__builtin_amdgcn_readlane((int)cnt, src);
}

// Selection of one row, by a workgroup of kFinThreads threads: the row's
// threshold bin T from its histogram; the chunks' candidate lists (one round
// of loads, issued before the row length is known) are classified: bin > T ->
// selected (bitmap), bin == T -> threshold candidates; the missing ones among
// those are picked by an MSB-first radix select, and the bitmap is emitted in
// ascending order.
constexpr int kFinThreads = 512;
constexpr int kCandLds = 4096;   // threshold candidates held in LDS (more: see below)
constexpr int kWordsLds = 4096;  // bitmap words held in LDS (rows up to 262,144 blocks)
constexpr int kRadixPasses = (32 + kBinShift + 7) / 8;  // 8-bit digits below the threshold bin

// kBmLds: the selection bitmap of every row fits the LDS (the host picks it
// from the workspace's row stride), so no mark or read of it branches on where
// it lives.
//
// Returns t, the workspace's count of scored calls (gen[0]): the scan left
// the row's histogram in histogram t & 1.  Both rows are loaded (the count, a
// vector load behind them, picks one: no dependent round trip); neither is
// written.  The caller clears the other histogram for the next scan
// (clear_next_hist) and publishes t as selected.
//
// One workgroup per row (the finalize kernel): the result goes to out (k
// entries); threshold candidates beyond kCandLds spill to the workspace.
template <bool kBmLds>
__device__ __forceinline__ uint32_t select_row(int s, const int32_t* __restrict__ sel_seq_len, int32_t k,
                                               int32_t max_seq_len, int32_t* __restrict__ out, const WsPtrs& ws) {
  constexpr int kPer = kBins / kFinThreads;
  __shared__ uint32_t sh[kFinThreads / 64];
  __shared__ __align__(16) uint32_t rhist[kRadixPasses][256];
  __shared__ uint64_t cand[kCandLds];
  __shared__ uint64_t bml[kBmLds ? kWordsLds : 1];
  __shared__ int32_t s_T;
  __shared__ uint32_t s_above, s_n, s_nfb;
  __shared__ uint16_t s_fb[kMaxChunksPerRow];  // chunks read again from their scores
  const int tid = threadIdx.x;
  const int nchunks_max = ws.nb_stride / kScoreChunk;
  const int tpc = chunk_threads(ws.nb_stride);     // threads per chunk in a round
  const int cpr = kFinThreads / tpc;               // chunks per round
  const int sub = tid % tpc;
  const uint32_t* ghist0 = ws.hist + (size_t)s * kBins;  // the row in histogram 0
  const uint32_t* cinfo = ws.cinfo + (size_t)s * nchunks_max;
  const uint64_t* ckeys = ws.keys + (size_t)s * ws.nb_stride;
  const int32_t* srow = ws.scores + (size_t)s * ws.nb_stride;
  uint64_t* gkeys = ws.keys2 + (size_t)s * ws.nb_stride;
  uint64_t* bm = ws.bitmap + (size_t)s * (ws.nb_stride / 64);

  // First round, before the row length is known (clamped in bounds, masked
  // below): the row histogram and, for the first cpr chunks, each chunk's
  // cinfo and the first tpc * kFinKeys keys of its list.
  uint32_t h0[kPer], h1[kPer];
  load_hist_desc<kFinThreads>(ghist0, h0);
  load_hist_desc<kFinThreads>(ghist0 + ws.hist_stride, h1);
  const int32_t Lv = vload_same(sel_seq_len + s);
  const int32_t tv = vload_same(reinterpret_cast<const int32_t*>(ws.gen));
  int cc = min(tid / tpc, nchunks_max - 1);
  uint32_t ci = cinfo[cc];
  uint64_t kk[kFinKeys];
#pragma unroll
  for (int e = 0; e < kFinKeys; ++e) kk[e] = ckeys[(size_t)cc * kScoreChunk + sub * kFinKeys + e];
  asm volatile("" ::: "memory");  // the loads go out here, not sunk to where they are used
  // the histogram, the length and the count before the length test below (the
  // keys and cinfo, loaded after them, are waited for only after the threshold)
  const int Lr = __builtin_amdgcn_readfirstlane(Lv);
  const uint32_t t = (uint32_t)__builtin_amdgcn_readfirstlane(tv);
  uint32_t hc[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) hc[i] = (t & 1u) ? h1[i] : h0[i];

  const int L = min(Lr, max_seq_len);
  const int nb = max(L, 0) >> 2;
  if (nb == 0) {  // nothing was scored: the histogram is untouched
    for (int i = tid; i < k; i += kFinThreads) out[i] = -1;
    return t;
  }
  const uint32_t ks = (uint32_t)min(k, nb);
  const int nchunks = (nb + kScoreChunk - 1) / kScoreChunk;
  const int nwords = (nb + 63) >> 6;
  constexpr bool bm_lds = kBmLds;  // then nwords <= nb_stride / 64 <= kWordsLds
  if (bm_lds) {
    for (int i = tid; i < nwords; i += kFinThreads) bml[i] = 0;
  } else {
    for (int i = tid; i < nwords; i += kFinThreads) bm[i] = 0;
  }
  for (int i = tid; i < kRadixPasses * 64; i += kFinThreads)
    reinterpret_cast<uint4*>(&rhist[0][0])[i] = uint4{0u, 0u, 0u, 0u};
  if (tid == 0) { s_n = 0; s_T = 0; s_above = 0; s_nfb = 0; }
  threshold_from_counts<kFinThreads>(hc, ks, sh, &s_T, &s_above);
  asm volatile("" ::"v"(ci));
#pragma unroll
  for (int e = 0; e < kFinKeys; ++e) asm volatile("" ::"v"(kk[e]));
  const int T = s_T;
  const uint32_t above = s_above;

  auto mark = [&](uint32_t j) {
    if (bm_lds) atomicOr(reinterpret_cast<unsigned long long*>(&bml[j >> 6]), 1ull << (j & 63));
    else atomicOr(reinterpret_cast<unsigned long long*>(&bm[j >> 6]), 1ull << (j & 63));
  };
  auto keep = [&](uint32_t i, uint64_t key) {
    if (i < (uint32_t)kCandLds) cand[i] = key;
    else gkeys[i] = key;
  };
  auto classify = [&](uint64_t key) {
    const int bin = score_bin(key_score(key));
    if (bin > T) {
      mark(0xffffffffu - (uint32_t)(key & 0xffffffffull));
    } else if (bin == T) {
      keep(atomicAdd(&s_n, 1u), key);
    }
  };
  for (int c0 = 0; c0 < nchunks; c0 += cpr) {
    const int c = c0 + tid / tpc;
    if (c0 > 0) {  // rows of more than cpr chunks: further rounds
      cc = min(c, nchunks_max - 1);
      ci = cinfo[cc];
#pragma unroll
      for (int e = 0; e < kFinKeys; ++e) kk[e] = ckeys[(size_t)cc * kScoreChunk + sub * kFinKeys + e];
    }
    uint32_t at_t = 0;  // which of this thread's first-round keys are threshold candidates
    if (c < nchunks) {
      const uint32_t cnt = ci >> 16;
      const int lb = (int)(ci & 0xffffu);
      if (lb <= T) {  // the list holds every block of this chunk with bin >= T
#pragma unroll
        for (int e = 0; e < kFinKeys; ++e) {
          const int bin = score_bin(key_score(kk[e]));
          const bool valid = (uint32_t)(sub * kFinKeys + e) < cnt;
          if (valid && bin > T) mark(0xffffffffu - (uint32_t)(kk[e] & 0xffffffffull));
          at_t |= (valid && bin == T) ? 1u << e : 0u;
        }
        for (uint32_t i = (uint32_t)(tpc * kFinKeys + sub); i < cnt; i += tpc)
          classify(ckeys[(size_t)c * kScoreChunk + i]);
      } else if (sub == 0) {  // local bin above T: bins [T, lb) are not listed; read the chunk's scores below
        s_fb[atomicAdd(&s_nfb, 1u)] = (uint16_t)c;
      }
    }
    // The first-round threshold candidates are appended with one slot
    // reservation per wave (a wave prefix sum of the per-thread counts), so no
    // returning atomic sits between a thread's keys.
    const uint32_t na = (uint32_t)__builtin_popcount(at_t);
    const uint32_t incl = wave_incl_scan(na);
    const uint32_t wtot = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
    if (wtot) {
      uint32_t base = 0;
      if (lane_id() == 0) base = atomicAdd(&s_n, wtot);
      base = (uint32_t)__builtin_amdgcn_readfirstlane((int)base);
      uint32_t pos = base + incl - na;
      if (base + wtot <= (uint32_t)kCandLds) {  // the usual case: all in LDS, no branch per key
#pragma unroll
        for (int e = 0; e < kFinKeys; ++e) {
          if (at_t & (1u << e)) cand[pos] = kk[e];
          pos += (at_t >> e) & 1u;
        }
      } else {
#pragma unroll
        for (int e = 0; e < kFinKeys; ++e) {
          if (at_t & (1u << e)) {
            keep(pos, kk[e]);
            ++pos;
          }
        }
      }
    }
  }
  __syncthreads();
  // Chunks whose list may be short, by the whole workgroup, up to kFbChunks at
  // a time: their scores are loaded in one round and classified.
  constexpr int kFbChunks = 4;
  constexpr int kFbIters = kScoreChunk / kFinThreads;
  const uint32_t nfb = s_nfb;
  for (uint32_t f0 = 0; f0 < nfb; f0 += kFbChunks) {
    int32_t fs[kFbChunks][kFbIters];
    int fc[kFbChunks];
#pragma unroll
    for (int q = 0; q < kFbChunks; ++q) {
      fc[q] = s_fb[min(f0 + q, nfb - 1)];  // past the list: the last chunk again, not classified
#pragma unroll
      for (int it = 0; it < kFbIters; ++it) fs[q][it] = srow[fc[q] * kScoreChunk + it * kFinThreads + tid];
    }
#pragma unroll
    for (int q = 0; q < kFbChunks; ++q) {
#pragma unroll
      for (int it = 0; it < kFbIters; ++it) {
        const int j = fc[q] * kScoreChunk + it * kFinThreads + tid;
        if (f0 + q < nfb && j < nb) classify(cand_key(fs[q][it], (uint32_t)j));
      }
    }
  }
  if (nfb) __syncthreads();
  const uint32_t n = s_n;
  const uint32_t need = ks - above;  // 1 <= need <= n
  auto key_at = [&](uint32_t i) -> uint64_t { return i < (uint32_t)kCandLds ? cand[i] : gkeys[i]; };

  // MSB-first radix select of the need-th largest threshold candidate by the
  // whole workgroup.  All candidates share the threshold bin, i.e. key bits
  // 32 + kBinShift and up, so the first digit is the 8 bits right below (with
  // ~300 candidates over 256 digits, one pass usually settles it), then 8 bits
  // at a time down to bit 0.  Each thread holds one candidate in a register
  // (any beyond the workgroup's size are read again per pass).  Every pass
  // counts into a histogram of its own, cleared with the bitmap above, so one
  // barrier per pass suffices: after it every wave reads the same counts and
  // finds the digit by itself.
  constexpr uint64_t kBinMask = ~((1ull << (32 + kBinShift)) - 1ull);
  const uint64_t mine = key_at(min((uint32_t)tid, n - 1));
  uint64_t prefix = 0, mask = 0;  // (mask 0 keeps every candidate)
  if (need < n) {
    mask = kBinMask;
    prefix = cand[0] & kBinMask;
    uint32_t rem = need;
    for (int p = 0, shift = 32 + kBinShift - 8;; ++p, shift = max(shift - 8, 0)) {
      uint32_t* h = rhist[p];
      if ((uint32_t)tid < n && (mine & mask) == prefix) atomicAdd(&h[(mine >> shift) & 0xff], 1u);
      for (uint32_t i = tid + kFinThreads; i < n; i += kFinThreads) {
        const uint64_t key = key_at(i);
        if ((key & mask) == prefix) atomicAdd(&h[(key >> shift) & 0xff], 1u);
      }
      __syncthreads();
      uint32_t dsel, larger, cnt;
      radix_digit(h, rem, dsel, larger, cnt);
      rem -= larger;
      prefix = (prefix & ~(0xffull << shift)) | ((uint64_t)dsel << shift);
      mask |= 0xffull << shift;
      if (cnt == rem || shift == 0) break;  // every remaining candidate with this prefix is kept
    }
  }
  if ((uint32_t)tid < n && (mine & mask) >= prefix) mark(0xffffffffu - (uint32_t)(mine & 0xffffffffull));
  for (uint32_t i = tid + kFinThreads; i < n; i += kFinThreads) {
    const uint64_t key = key_at(i);
    if ((key & mask) >= prefix) mark(0xffffffffu - (uint32_t)(key & 0xffffffffull));
  }
  __syncthreads();

  // emit ascending block ids: popcount prefix over the bitmap words
  const int per = (nwords + kFinThreads - 1) / kFinThreads;
  const int w0 = min(nwords, tid * per), w1 = min(nwords, w0 + per);
  uint32_t cntw = 0;
  for (int i = w0; i < w1; ++i) cntw += (uint32_t)__popcll(bm_lds ? bml[i] : bm[i]);
  uint32_t pos = block_excl_scan<kFinThreads, false>(cntw, sh);  // sh is not written again
  for (int i = w0; i < w1; ++i) {
    uint64_t m = bm_lds ? bml[i] : bm[i];
    while (m) {
      const int bit = __ffsll((long long)m) - 1;
      m &= m - 1;
      if (pos < (uint32_t)k) out[pos] = i * 64 + bit;
      ++pos;
    }
  }
  for (int i = (int)ks + tid; i < k; i += kFinThreads) out[i] = -1;
  return t;
}

// ---------------------------------------------------------------------------
// Selection for one split of a row (the fused selection + attention kernel).
//
// Split p of P owns the run [floor(p ks / P), floor((p+1) ks / P)) of the row's
// ks ascending selected blocks (a contiguous stretch of the context with a
// near-equal share of the selection).  Every workgroup serving the row finds
// the selection itself, as select_row does: the threshold bin T from the
// histogram, the chunks' lists classified against it (blocks above T marked in
// an LDS bitmap of the row, bin-T blocks listed as candidates), and the radix
// select of the bin-T winners, marked too.  emit_run() then lists only the
// workgroup's own run, ascending: a popcount prefix sum over the bitmap, with
// the bit walk confined to the words that hold the run.
struct RowLds {
  uint32_t sh[kFinThreads / 64];
  __align__(16) uint32_t rhist[kRadixPasses][256];
  uint64_t cand[kCandLds];
  uint64_t bm[kWordsLds];  // the row's selection (rows of up to kWordsLds * 64 blocks)
  uint32_t slot_sums[2][kFinThreads / 64];  // emission: per word slot, per wave
  int32_t T;
  uint32_t above, n, nfb;
  uint16_t fb[kMaxChunksPerRow];  // chunks read again from their scores
};

struct RowSelector {
  RowLds& L;
  int s;
  int32_t k;
  WsPtrs ws;
  // set by first()
  int nb = 0, nwords = 0, nchunks = 0, T = 0, tpc = 1, cpr = 1, sub = 0;
  int Lsel = 0;     // the row's length (clamped at 0), uniform
  uint32_t t = 0;   // the workspace's count of scored calls: the scan's histogram is t & 1
  uint32_t ks = 0, above = 0;

  __device__ __forceinline__ void mark(uint32_t j) {
    atomicOr(reinterpret_cast<unsigned long long*>(&L.bm[j >> 6]), 1ull << (j & 63));
  }

  // The loads, the threshold bin and the classification.  pre(): right after
  // the histogram loads (the caller's first loads of its own); hook(): once
  // the first round of loads is in flight (Lsel is then known); mid(): by all
  // threads right before the barrier that ends the classification.  The row
  // length and the count of scored calls are vector loads issued behind the
  // histogram, so that nothing waits for a scalar round trip before the
  // histogram goes out.
  // KK: keys per thread in the first round (fused_keys of the workspace).
  template <int KK, class Pre, class Hook, class Mid>
  __device__ __forceinline__ void first(const int32_t* __restrict__ sel_seq_len, int32_t max_seq_len, Pre&& pre,
                                        Hook&& hook, Mid&& mid) {
    constexpr int kPer = kBins / kFinThreads;
    static_assert(kPer == 4 && (KK == 4 || KK == 6 || KK == 8), "vector loads of the first round");
    const int tid = threadIdx.x;
    const int nchunks_max = ws.nb_stride / kScoreChunk;
    tpc = chunk_threads(ws.nb_stride);
    cpr = kFinThreads / tpc;
    sub = tid % tpc;
    const uint32_t* ghist0 = ws.hist + (size_t)s * kBins;
    const uint32_t* cinfo = ws.cinfo + (size_t)s * nchunks_max;
    const uint64_t* ckeys = ws.keys + (size_t)s * ws.nb_stride;
    const int32_t* srow = ws.scores + (size_t)s * ws.nb_stride;

    // First round, one 16-byte load per four histogram bins or two keys: both
    // histogram rows (bins 2047 - 4 tid - i, i < 4: descending), the chunk's
    // cinfo and the first KK keys of its list.
    const uint4 hv0 = *reinterpret_cast<const uint4*>(ghist0 + kBins - 4 - 4 * tid);
    const uint4 hv1 = *reinterpret_cast<const uint4*>(ghist0 + ws.hist_stride + kBins - 4 - 4 * tid);
    pre();
    const int32_t Lv = vload_same(sel_seq_len + s);
    const int32_t tv = vload_same(reinterpret_cast<const int32_t*>(ws.gen));
    int cc = min(tid / tpc, nchunks_max - 1);
    uint32_t ci = cinfo[cc];
    uint64_t kk[KK];
    auto load_keys = [&](int c) {
      const i32x4* kp = reinterpret_cast<const i32x4*>(ckeys + (size_t)c * kScoreChunk + sub * KK);
#pragma unroll
      for (int e = 0; e < KK / 2; ++e) {
        const i32x4 v = kp[e];
        kk[2 * e] = (uint64_t)(uint32_t)v[0] | ((uint64_t)(uint32_t)v[1] << 32);
        kk[2 * e + 1] = (uint64_t)(uint32_t)v[2] | ((uint64_t)(uint32_t)v[3] << 32);
      }
    };
    load_keys(cc);
    asm volatile("" ::: "memory");  // the loads go out here, not sunk to where they are used
    // (one wait covers the histogram, the row length and the count: the key
    // loads behind them are waited for only after the threshold)
    const int Lr = __builtin_amdgcn_readfirstlane(Lv);
    t = (uint32_t)__builtin_amdgcn_readfirstlane(tv);
    Lsel = max(Lr, 0);
    hook();
    uint32_t hc[kPer];
    {
      const uint4 h = (t & 1u) ? hv1 : hv0;
      hc[0] = h.w; hc[1] = h.z; hc[2] = h.y; hc[3] = h.x;
    }
    const int Lc = min(Lr, max_seq_len);
    nb = max(Lc, 0) >> 2;
    if (nb == 0) {  // nothing was scored: no blocks, the histogram is untouched
      mid();
      __syncthreads();
      return;
    }
    ks = (uint32_t)min(k, nb);
    nwords = (nb + 63) >> 6;  // <= kWordsLds (checked by the host)
    nchunks = (nb + kScoreChunk - 1) / kScoreChunk;
    for (int i = tid; i < nwords; i += kFinThreads) L.bm[i] = 0;
    for (int i = tid; i < kRadixPasses * 64; i += kFinThreads)
      reinterpret_cast<uint4*>(&L.rhist[0][0])[i] = uint4{0u, 0u, 0u, 0u};
    if (tid == 0) { L.n = 0; L.T = 0; L.above = 0; L.nfb = 0; }
    threshold_from_counts<kFinThreads>(hc, ks, L.sh, &L.T, &L.above);
    asm volatile("" ::"v"(ci));
#pragma unroll
    for (int e = 0; e < KK; ++e) asm volatile("" ::"v"(kk[e]));
    T = L.T;
    above = L.above;

    auto classify = [&](uint64_t key) {
      const int bin = score_bin(key_score(key));
      if (bin > T) {
        mark(0xffffffffu - (uint32_t)(key & 0xffffffffull));
      } else if (bin == T) {
        const uint32_t i = atomicAdd(&L.n, 1u);
        if (i < (uint32_t)kCandLds) L.cand[i] = key;
      }
    };
    // One round: the chunks c0 + tid / tpc, whose cinfo and first keys are in
    // ci and kk.  The first round is a call of its own, outside the loop, so
    // that its waits count only the loads issued before the hook's (a wait in
    // a loop body shared with later rounds would wait for every load).
    auto round = [&](int c0) {
      const int c = c0 + tid / tpc;
      uint32_t at_t = 0;
      if (c < nchunks) {
        const uint32_t cnt = ci >> 16;
        const int lb = (int)(ci & 0xffffu);
        if (lb <= T) {  // the list holds every block of this chunk with bin >= T
#pragma unroll
          for (int e = 0; e < KK; ++e) {
            const int bin = score_bin(key_score(kk[e]));
            const bool valid = (uint32_t)(sub * KK + e) < cnt;
            if (valid && bin > T) mark(0xffffffffu - (uint32_t)(kk[e] & 0xffffffffull));
            at_t |= (valid && bin == T) ? 1u << e : 0u;
          }
          for (uint32_t i = (uint32_t)(tpc * KK + sub); i < cnt; i += tpc)
            classify(ckeys[(size_t)c * kScoreChunk + i]);
        } else if (sub == 0) {  // local bin above T: bins [T, lb) are not listed
          L.fb[atomicAdd(&L.nfb, 1u)] = (uint16_t)c;
        }
      }
      const uint32_t na = (uint32_t)__builtin_popcount(at_t);
      const uint32_t incl = wave_incl_scan(na);
      const uint32_t wtot = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
      if (wtot) {
        uint32_t base = 0;
        if (lane_id() == 0) base = atomicAdd(&L.n, wtot);
        base = (uint32_t)__builtin_amdgcn_readfirstlane((int)base);
        uint32_t pos = base + incl - na;
#pragma unroll
        for (int e = 0; e < KK; ++e) {
          if ((at_t & (1u << e)) && pos < (uint32_t)kCandLds) L.cand[pos] = kk[e];
          pos += (at_t >> e) & 1u;
        }
      }
    };
    round(0);
    for (int c0 = cpr; c0 < nchunks; c0 += cpr) {
      cc = min(c0 + tid / tpc, nchunks_max - 1);
      ci = cinfo[cc];
      load_keys(cc);
      round(c0);
    }
    mid();
    __syncthreads();
    constexpr int kFbChunks = 4;
    constexpr int kFbIters = kScoreChunk / kFinThreads;
    const uint32_t nfb = L.nfb;
    for (uint32_t f0 = 0; f0 < nfb; f0 += kFbChunks) {
      int32_t fs[kFbChunks][kFbIters];
      int fc[kFbChunks];
#pragma unroll
      for (int q = 0; q < kFbChunks; ++q) {
        fc[q] = L.fb[min(f0 + q, nfb - 1)];
#pragma unroll
        for (int it = 0; it < kFbIters; ++it) fs[q][it] = srow[fc[q] * kScoreChunk + it * kFinThreads + tid];
      }
#pragma unroll
      for (int q = 0; q < kFbChunks; ++q) {
#pragma unroll
        for (int it = 0; it < kFbIters; ++it) {
          const int j = fc[q] * kScoreChunk + it * kFinThreads + tid;
          if (f0 + q < nfb && j < nb) classify(cand_key(fs[q][it], (uint32_t)j));
        }
      }
    }
    if (nfb) __syncthreads();
  }

  // The radix select of the bin-T winners (as in select_row), marked in the
  // bitmap; ends with a barrier.
  __device__ __forceinline__ void second() {
    const int tid = threadIdx.x;
    if (nb == 0) return;
    const int nchunks_max = ws.nb_stride / kScoreChunk;
    const uint32_t* cinfo = ws.cinfo + (size_t)s * nchunks_max;
    const uint64_t* ckeys = ws.keys + (size_t)s * ws.nb_stride;
    const int32_t* srow = ws.scores + (size_t)s * ws.nb_stride;
    const uint32_t n = L.n;
    const uint32_t need = ks - above;  // 1 <= need <= n
    constexpr uint64_t kBinMask = ~((1ull << (32 + kBinShift)) - 1ull);
    if (n <= (uint32_t)kCandLds) {
      const uint64_t mine = L.cand[min((uint32_t)tid, n - 1)];
      uint64_t prefix = 0, mask = 0;
      if (need < n) {
        mask = kBinMask;
        prefix = L.cand[0] & kBinMask;
        uint32_t rem = need;
        for (int pass = 0, shift = 32 + kBinShift - 8;; ++pass, shift = max(shift - 8, 0)) {
          uint32_t* h = L.rhist[pass];
          if ((uint32_t)tid < n && (mine & mask) == prefix) atomicAdd(&h[(mine >> shift) & 0xff], 1u);
          for (uint32_t i = tid + kFinThreads; i < n; i += kFinThreads) {
            const uint64_t key = L.cand[i];
            if ((key & mask) == prefix) atomicAdd(&h[(key >> shift) & 0xff], 1u);
          }
          __syncthreads();
          uint32_t dsel, larger, cnt;
          radix_digit(h, rem, dsel, larger, cnt);
          rem -= larger;
          prefix = (prefix & ~(0xffull << shift)) | ((uint64_t)dsel << shift);
          mask |= 0xffull << shift;
          if (cnt == rem || shift == 0) break;
        }
      }
      if ((uint32_t)tid < n && (mine & mask) >= prefix) mark(0xffffffffu - (uint32_t)(mine & 0xffffffffull));
      for (uint32_t i = tid + kFinThreads; i < n; i += kFinThreads) {
        const uint64_t key = L.cand[i];
        if ((key & mask) >= prefix) mark(0xffffffffu - (uint32_t)(key & 0xffffffffull));
      }
    } else {
      // More bin-T candidates than the LDS holds (massive ties): every pass
      // and the marking visit them where the classification found them.
      auto visit = [&](auto&& f) {
        for (int c0 = 0; c0 < nchunks; c0 += cpr) {
          const int c = c0 + tid / tpc;
          if (c >= nchunks) continue;
          const uint32_t cinf = cinfo[c];
          if ((int)(cinf & 0xffffu) <= T) {
            const uint32_t cnt = cinf >> 16;
            for (uint32_t i = sub; i < cnt; i += tpc) {
              const uint64_t key = ckeys[(size_t)c * kScoreChunk + i];
              if (score_bin(key_score(key)) == T) f(key);
            }
          } else {
            const int jn = min(kScoreChunk, nb - c * kScoreChunk);
            for (int i = sub; i < jn; i += tpc) {
              const uint32_t j = (uint32_t)(c * kScoreChunk + i);
              const uint64_t key = cand_key(srow[j], j);
              if (score_bin(key_score(key)) == T) f(key);
            }
          }
        }
      };
      uint64_t mask = kBinMask, prefix = L.cand[0] & kBinMask;
      uint32_t rem = need;
      for (int pass = 0, shift = 32 + kBinShift - 8;; ++pass, shift = max(shift - 8, 0)) {
        uint32_t* h = L.rhist[pass];
        visit([&](uint64_t key) {
          if ((key & mask) == prefix) atomicAdd(&h[(key >> shift) & 0xff], 1u);
        });
        __syncthreads();
        uint32_t dsel, larger, cnt;
        radix_digit(h, rem, dsel, larger, cnt);
        rem -= larger;
        prefix = (prefix & ~(0xffull << shift)) | ((uint64_t)dsel << shift);
        mask |= 0xffull << shift;
        if (cnt == rem || shift == 0) break;
      }
      visit([&](uint64_t key) {
        if ((key & mask) >= prefix) mark(0xffffffffu - (uint32_t)(key & 0xffffffffull));
      });
    }
    __syncthreads();
  }

  // The selected blocks at positions [i0, i1) of the row's ascending selection
  // into list[0, i1 - i0) (LDS); each(i, j) is called for list entry i = block
  // j.  Block-wide: ends with a barrier.
  template <class Each>
  __device__ __forceinline__ void emit_run(int i0, int i1, int32_t* list, Each&& each) {
    if (nb == 0) return;
    const int per = (nwords + kFinThreads - 1) / kFinThreads;  // <= kWordsLds / kFinThreads
    if (per <= 2) emit_words<2>(per, i0, i1, list, each);
    else emit_words_contiguous<kWordsLds / kFinThreads>(per, i0, i1, list, each);
  }

  // Rows of more than 1,024 words (over 256k tokens): each thread owns `per`
  // consecutive words (one block scan of the per-thread counts); with N slots
  // per thread the interleaved layout below would take N wave scans, which
  // cost more there than the walk it spreads.
  template <int N, class Each>
  __device__ __forceinline__ void emit_words_contiguous(int per, int i0, int i1, int32_t* list, Each&& each) {
    const int tid = threadIdx.x;
    const int w0 = min(nwords, tid * per), nw = min(nwords, w0 + per) - w0;
    uint64_t wv[N];
    uint32_t cntw = 0;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      wv[i] = (i < nw) ? L.bm[min(w0 + i, kWordsLds - 1)] : 0ull;
      cntw += (uint32_t)__popcll(wv[i]);
    }
    uint32_t pos = block_excl_scan<kFinThreads, false>(cntw, L.sh);
    if ((int)pos < i1 && (int)(pos + cntw) > i0) {  // this thread's words hold part of the run
#pragma unroll
      for (int i = 0; i < N; ++i) {
        uint64_t m = wv[i];
        const uint32_t c = (uint32_t)__popcll(m);
        if ((int)(pos + c) > i0 && (int)pos < i1) {
          while (m) {
            const int bit = __ffsll((long long)m) - 1;
            m &= m - 1;
            if ((int)pos >= i0 && (int)pos < i1) {
              list[pos - i0] = (w0 + i) * 64 + bit;
              each((int)pos - i0, (w0 + i) * 64 + bit);
            }
            ++pos;
          }
        } else {
          pos += c;
        }
      }
    }
    __syncthreads();
  }

  // emit_run for rows of up to N * 512 words, held in registers (read once
  // for the popcounts; the walk then runs from registers).  Word w is
  // thread w mod 512's slot w / 512: consecutive words sit in consecutive
  // threads, so the words of a run spread over many threads and waves instead
  // of being walked one after another by a few threads of one wave.  A word's
  // rank is the total of the slots before its own plus the prefix of its slot
  // over the threads before it (one wave scan per slot, one barrier).
  template <int N, class Each>
  __device__ __forceinline__ void emit_words(int per, int i0, int i1, int32_t* list, Each&& each) {
    static_assert(N <= 2, "slot_sums holds two slots");
    (void)per;
    const int tid = threadIdx.x, wave = tid >> 6;
    uint64_t wv[N];
    uint32_t c[N], inc[N];
#pragma unroll
    for (int k = 0; k < N; ++k) {
      const int w = k * kFinThreads + tid;
      wv[k] = (w < nwords) ? L.bm[min(w, kWordsLds - 1)] : 0ull;
      c[k] = (uint32_t)__popcll(wv[k]);
      inc[k] = wave_incl_scan(c[k]);
      if (lane_id() == 63) L.slot_sums[k][wave] = inc[k];
    }
    __syncthreads();
    uint32_t base = 0;
#pragma unroll
    for (int k = 0; k < N; ++k) {
      uint32_t before = 0, tot = 0;
#pragma unroll
      for (int x = 0; x < kFinThreads / 64; ++x) {
        const uint32_t v = L.slot_sums[k][x];
        tot += v;
        before += (x < wave) ? v : 0u;
      }
      uint32_t pos = base + before + inc[k] - c[k];
      base += tot;
      if ((int)pos < i1 && (int)(pos + c[k]) > i0) {  // this word holds part of the run
        uint64_t m = wv[k];
        const int w = k * kFinThreads + tid;
        while (m) {
          const int bit = __ffsll((long long)m) - 1;
          m &= m - 1;
          if ((int)pos >= i0 && (int)pos < i1) {
            list[pos - i0] = w * 64 + bit;
            each((int)pos - i0, w * 64 + bit);
          }
          ++pos;
        }
      }
    }
    __syncthreads();
  }
};

// After the selection of the call counted t: row s of the other histogram,
// the one the next scan adds into, back to zero (the workgroup's threads share
// it; the last call that used it finished before this call's scan began).
__device__ __forceinline__ void clear_next_hist(const WsPtrs& ws, int s, uint32_t t) {
  uint4* h = reinterpret_cast<uint4*>(ws.hist + (size_t)((t + 1u) & 1u) * ws.hist_stride + (size_t)s * kBins);
  for (int i = threadIdx.x; i < kBins / 4; i += blockDim.x) h[i] = uint4{0u, 0u, 0u, 0u};
}

}  // namespace

}  // namespace qsa
