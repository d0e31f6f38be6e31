// qsa_sparse_decode: attention over the selected uncompressed K/V, as split
// partials; qsa_merge_partials: their log-sum-exp merge.
//
// Method ("Qwen 4 QSA 迎来解码上下文并行" blog, section on what the pull request
// changes): the final softmax and value aggregation run over the uncompressed
// K and V at the positions of the kept micro-blocks; with decode context
// parallelism every partition of the context yields a partial result and the
// partials are merged at the end.  Here the partitions are P contiguous runs of
// the ascending selection on one GPU (the last one also owns the open tail
// block), and the merge is a separate kernel.
//
// One workgroup per (split, KV head, selecting row).  All query rows that share
// the selection and all query heads of the GQA group are processed together
// (NH = rows x heads-per-KV-head), so each K/V row is read from HBM once.
// Per tile of 16 token slots (four micro-blocks), per wave:
//   * QK^T:  v_mfma_f32_16x16x32_bf16, M = 16 slots, N = 16 heads; K rows go
//            straight from global memory into the A operand (16 B per lane).
//   * softmax: online, fp32, exp2 domain; per-head running max / sum.
//   * PV:    v_mfma_f32_16x16x16_bf16, M = 16 heads, N = 16 dims, K = 16 slots.
//            The QK accumulator layout is already the PV A-operand layout, so P
//            never leaves registers; it is split into two bf16 terms (hi + lo)
//            to keep ~16 mantissa bits.  The output dims are permuted: column
//            lc of PV chunk m is dim (D/16) lc + m, so lane lc loads D/16
//            consecutive dims of each of its four V rows in one load per row
//            (16 B for bf16 at d = 128) and builds the B operands with byte
//            permutes; the permutation is undone when the output is written.
// Block ids and page positions of a split are staged in LDS once; K/V loads
// run one tile ahead.  The waves (8, or 4 for large head groups) take
// interleaved tiles and are merged in LDS in a fixed order (deterministic).
// FP8 (OCP E4M3) K/V are widened exactly to bf16; the per-token K scale
// multiplies the logit and the V scale multiplies the probability.
#include "qsa_device.h"
#include "qsa_internal.h"
#include "qsa_select.h"

namespace qsa {

namespace {

// Waves per workgroup: 8 (one 16-slot tile each for a split of 32 blocks) when
// the grid has fewer workgroups than two per CU and the per-wave output
// staging fits the LDS; else 4, so that two workgroups share a CU and one's
// tail overlaps the other's loads.
constexpr int kDecodeWideMaxGroups = 512;
template <int NH>
constexpr bool decode_wide_ok() { return NH <= 16; }
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 8 fp8 E4M3 bytes -> 8 bf16 (exact: every E4M3 value is a bf16 value).
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(i32x2 w) {
  bf16x8 r;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(w[h], false);
    auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(w[h], true);
    r[4 * h + 0] = __builtin_bit_cast(__bf16, (uint16_t)(__float_as_uint(lo[0]) >> 16));
    r[4 * h + 1] = __builtin_bit_cast(__bf16, (uint16_t)(__float_as_uint(lo[1]) >> 16));
    r[4 * h + 2] = __builtin_bit_cast(__bf16, (uint16_t)(__float_as_uint(hi[0]) >> 16));
    r[4 * h + 3] = __builtin_bit_cast(__bf16, (uint16_t)(__float_as_uint(hi[1]) >> 16));
  }
  return r;
}

struct DecodeArgs {
  const uint16_t* q;
  const int32_t* row_sel;      // [R]: selecting row of each query row; NULL: row r is selecting row r
  const int32_t* row_seq_len;  // [R]
  const int32_t* sel_req;      // [S]
  const int32_t* sel_seq_len;  // [S]
  const int32_t* topk;         // [S, k] (decode_kernel)
  const int32_t* block_table;
  const void* k_cache;
  const void* v_cache;
  const float* k_scale;
  const float* v_scale;
  float* o_part;
  float* lse_part;
  int32_t k, max_pages, page_log2, Hq, Hkv, G, P, R, S;
  int32_t qps;          // most query rows per selecting row (rows ranked past it are not attended)
  int32_t qg, qpw, nh;  // row groups per (KV head, selecting row) (grid y = Hkv * qg), rows per group
                        // (qg * qpw >= qps), heads per workgroup (G * qpw)
  float scale_log2;     // softmax_scale * log2(e)
};

// Token-slot view of one split: slot u covers token 4*blk(u/4) + u%4, where
// blk(i) is the i-th selected block of the split, or a block of the tail.
constexpr int kRound = 512;  // blocks staged in LDS per round

template <int D, bool FP8>
struct TileLoad {
  static constexpr int KK = D / 32;
  static constexpr int VDW = (D / 16) * (FP8 ? 1 : 2) / 4;  // dwords of one V row slice per lane
  i32x4 k[FP8 ? 1 : KK];   // bf16: 16 B per k-step
  i32x2 k8[FP8 ? KK : 1];  // fp8: 8 B per k-step
  uint32_t v[4][VDW];      // V of slots 4*lg+e at dims (D/16) lc .. (D/16) lc + D/16 - 1
  int tok;                 // first token of the block of slots 4*lg..4*lg+3 (-1: none)
  f32x4 ks, vs;            // fp8 scales of those four slots
};

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ s16x4 pack4(uint32_t lo, uint32_t hi) {
  return __builtin_bit_cast(s16x4, i32x2{(int)lo, (int)hi});
}

// Reductions across the four 16-lane groups with the gfx950 lane swaps (VALU, no LDS).
__device__ __forceinline__ float max_lg(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_lg(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

constexpr int kMaxRowsPerGroup = 64;  // query rows one workgroup attends (heads of them <= 64)

// The query rows of selecting row s that row group g attends: ranks
// [g * qpw, (g+1) * qpw) among the rows r with row_sel[r] == s, in ascending r
// ([PR53896]: later draft tokens reuse the first token's selection).  Wave 0
// writes rows_lds[0, qpw) (row index, -1 where the row has fewer); the caller
// publishes them with a barrier.  rs0: row_sel[lane] (loaded early).
__device__ __forceinline__ void find_rows(const DecodeArgs& a, int s, int g, int rs0, int* rows_lds) {
  if (threadIdx.x >= 64) return;
  const int l = lane_id();
  if (a.row_sel == nullptr) {  // (then qg = qpw = 1)
    if (l == 0) rows_lds[0] = s;
    return;
  }
  const int want0 = g * a.qpw, want1 = want0 + a.qpw;
  int base = 0;
  for (int r0 = 0; r0 < a.R && base < want1; r0 += 64) {
    const int r = r0 + l;
    const int v = (r0 == 0) ? rs0 : (r < a.R ? a.row_sel[r] : -1);
    const bool m = r < a.R && v == s;
    const uint64_t bal = __ballot(m);
    const int rank = base + (int)lanes_below(bal);
    if (m && rank >= want0 && rank < want1 && rank < a.qps) rows_lds[rank - want0] = r;
    base += (int)__popcll(bal);
  }
  if (l < a.qpw && (want0 + l >= base || want0 + l >= a.qps)) rows_lds[l] = -1;
}

__device__ __forceinline__ int load_rs0(const DecodeArgs& a) {
  const int l = lane_id();
  return (a.row_sel != nullptr) ? a.row_sel[min(l, a.R - 1)] : -1;
}

// Page ids of the request: the first nbt entries from pg0 on may be staged in LDS.
struct BtView {
  const int32_t* lds;  // [nbt] (nullptr: none)
  int pg0, nbt;
};

// The attention of one workgroup: split p of selecting row s, KV head kvh,
// query rows rows_lds[0, qpw) (nh = G * qpw heads), over lists of the split's
// blocks (LDS) and, for the last split, the tail blocks from tail_lo up to the
// longest row.  Blocks come in batches; a batch is staged in LDS (first token
// and page position per block) in rounds of up to kRound blocks, and its first
// round may be staged and its first tiles issued before the caller does other
// work (so that the loads of one batch overlap the selection of the next).
// Writes o_part / lse_part of its heads.
template <int D, int NH, bool FP8, int W>
struct Attend {
  static constexpr int kWaves = W;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int NT = (NH + 15) / 16;  // MFMA tiles of 16 heads
  static constexpr int NHP = NT * 16;        // heads padded to whole tiles
  static constexpr int KK = D / 32;          // QK MFMA k steps over the head dim
  static constexpr int NPAIR = D / 32;       // PV: pairs of 16-wide d-chunks (bf16 dwords of a V slice)
  static constexpr int VDW = TileLoad<D, FP8>::VDW;
  static constexpr int NM = D / 16;          // PV MFMAs (16-wide d-chunks) per head tile

  // A batch of blocks: list[0, n) (ascending block ids), then ntail tail blocks.
  struct Batch {
    const int32_t* list;
    int n, tail_lo, ntail;
    int32_t* tok;  // LDS [kRound]: first token of each staged block (-1: none)
    int32_t* pos;  // LDS [kRound]: its position in the page pool
    int off;       // tile t of a round goes to wave (t + off) % W
    __device__ __forceinline__ int total() const { return n + ntail; }
  };

  bf16x8 bq[NT][KK];
  int rlen_[NT];   // context length of the row owning head nt*16+lc, as loaded
  bool real_[NT];  // head nt*16+lc is one of the group's (else padding: no token counts)
  float m_run[NT], l_run[NT];
  // O in the MFMA C layout: acc[nt][m][e] = O[head nt*16+4lg+e][d = (D/16) lc + m]
  f32x4 acc[NT][NM];

  __device__ __forceinline__ void init() {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      m_run[nt] = -INFINITY;
      l_run[nt] = 0.f;
#pragma unroll
      for (int m = 0; m < NM; ++m) acc[nt][m] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }

  // The context length of head nt*16+lc's row (-1: padding).  Padding is
  // applied here, where the lengths are used, so that nothing waits for the
  // loads of load_q before then.
  __device__ __forceinline__ int rlen(int nt) const { return real_[nt] ? rlen_[nt] : -1; }

  // Q as the QK MFMA B operand: lane (lc, lg) holds head n = nt*16+lc, dims
  // 32kk+8lg..+8.  Unconditional loads, used as loaded (padding heads read
  // the first row's first head; their tokens are all masked through rlen, so
  // their query values never count).  row_of_group(i): query row of the
  // group's i-th row (-1: none).
  template <class RowFn>
  __device__ __forceinline__ void load_q(const DecodeArgs& a, int kvh, RowFn&& row_of_group) {
    const int lc = lane_id() & 15, lg = lane_id() >> 4;
    const int r_first = max(row_of_group(0), 0);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int n = nt * 16 + lc;
      const int i0 = min(n, a.nh - 1) / a.G;
      const int rr = row_of_group(i0);
      const bool real = n < a.nh && rr >= 0;
      const int r = real ? rr : r_first;
      const int h = kvh * a.G + (real ? n - i0 * a.G : 0);
      const uint16_t* qrow = a.q + ((size_t)r * a.Hq + h) * D;
      rlen_[nt] = a.row_seq_len[r];
      real_[nt] = real;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) bq[nt][kk] = __builtin_bit_cast(bf16x8, ld16(qrow + 32 * kk + 8 * lg));
    }
  }

  // Tail blocks of the last split: up to the longest row of the group (every
  // real row owns some head n < nh); only that split waits for the row lengths.
  __device__ __forceinline__ int tail_blocks(const DecodeArgs& a, int p, int tail_lo) const {
    if (p != a.P - 1) return 0;
    int tail_hi = 0;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) tail_hi = max(tail_hi, rlen(nt));
    tail_hi = wave_max_i32(tail_hi);
    return (max(0, tail_hi - tail_lo) + 3) >> 2;
  }

  // Stages blocks [r0, r0 + kRound) of the batch (all threads; the caller
  // barriers before and after).  Page ids come from the LDS copy when it holds
  // them, else from the block table.  kLdsOnly: the caller knows the LDS copy
  // holds every page of the batch, and no global load is made (a global load
  // here, waited for at once, would also wait for every K/V load in flight).
  template <bool kLdsOnly = false>
  __device__ __forceinline__ void stage(const DecodeArgs& a, const Batch& bt_, int r0, const int32_t* bt,
                                        BtView btv) const {
    const int nr = min(kRound, bt_.total() - r0);
    const int page_size = 1 << a.page_log2;
    for (int i = threadIdx.x; i < nr; i += kThreads) {
      const int u = r0 + i;
      int tok = -1, pos = 0;
      if (u < bt_.n) {
        const int j = bt_.list[u];
        tok = (j >= 0) ? 4 * j : -1;
      } else {
        tok = bt_.tail_lo + 4 * (u - bt_.n);
      }
      if (tok >= 0) {
        const int pg = tok >> a.page_log2;
        // (two loads, not one through a selected pointer: that would be a
        // generic load, which waits for LDS and global memory alike)
        int pid;
        if (kLdsOnly) {
          pid = btv.lds[min(max(pg - btv.pg0, 0), max(btv.nbt - 1, 0))];
        } else if (btv.lds != nullptr) {
          const int rel = pg - btv.pg0;
          pid = btv.lds[min(max(rel, 0), max(btv.nbt - 1, 0))];
          asm volatile("" : "+v"(pid));  // keeps the two loads apart
          if (rel < 0 || rel >= btv.nbt) pid = bt[pg];
        } else {
          pid = bt[pg];
        }
        pos = (pid << a.page_log2) | (tok & (page_size - 1));
      }
      bt_.tok[i] = tok;
      bt_.pos[i] = pos;
    }
  }

  // Tile ti of a staged round = blocks 4ti..4ti+3.  The A operand (K) of lane
  // (lc, lg) is slot lc = token lc%4 of block 4ti + lc/4; its C-layout slots
  // 4lg..4lg+3 (scores, V rows, scales) are the four tokens of block 4ti + lg.
  // Slots without a token read row 0 of the cache (a valid address) and are masked.
  __device__ __forceinline__ void issue(const DecodeArgs& a, int kvh, const Batch& bt_, int nr, int ti,
                                        TileLoad<D, FP8>& tl) const {
    const int lc = lane_id() & 15, lg = lane_id() >> 4;
    const int page_size = 1 << a.page_log2;
    auto row_of = [&](int pos) {  // token row inside the cache for this KV head
      return (((pos >> a.page_log2) * a.Hkv + kvh) << a.page_log2) | (pos & (page_size - 1));
    };
    const char* kbase = reinterpret_cast<const char*>(a.k_cache);
    const char* vbase = reinterpret_cast<const char*>(a.v_cache);
    // (ti < 0: no tile; every slot reads row 0, masked)
    const int ba = 4 * ti + (lc >> 2), bc = 4 * ti + lg;
    const bool in_a = ti >= 0 && ba < nr, in_c = ti >= 0 && bc < nr;
    const int tok_a = in_a ? bt_.tok[max(ba, 0)] : -1;
    const int pos_a = in_a ? bt_.pos[max(ba, 0)] : 0;
    const int tok_c = in_c ? bt_.tok[max(bc, 0)] : -1;
    const int pos_c = in_c ? bt_.pos[max(bc, 0)] : 0;
    const int row_a = (tok_a >= 0) ? row_of(pos_a) + (lc & 3) : 0;
    const int row_c = (tok_c >= 0) ? row_of(pos_c) : 0;
    tl.tok = tok_c;
    if (FP8) {
      tl.ks = *reinterpret_cast<const f32x4*>(a.k_scale + (tok_c >= 0 ? pos_c : 0));
      tl.vs = *reinterpret_cast<const f32x4*>(a.v_scale + (tok_c >= 0 ? pos_c : 0));
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        tl.k8[kk] = *reinterpret_cast<const i32x2*>(kbase + (size_t)row_a * D + 32 * kk + 8 * lg);
    } else {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) tl.k[kk] = ld16(kbase + ((size_t)row_a * D + 32 * kk + 8 * lg) * 2);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const size_t el = (size_t)(row_c + (tok_c >= 0 ? e : 0)) * D + (D / 16) * lc;  // element index
      const char* src = vbase + el * (FP8 ? 1 : 2);
      if (VDW == 4) {
        const i32x4 x = ld16(src);
#pragma unroll
        for (int r = 0; r < 4; ++r) tl.v[e][r] = (uint32_t)x[r];
      } else if (VDW == 2) {
        const i32x2 x = *reinterpret_cast<const i32x2*>(src);
        tl.v[e][0] = (uint32_t)x[0];
        tl.v[e][VDW - 1] = (uint32_t)x[1];
      } else {
        tl.v[e][0] = *reinterpret_cast<const uint32_t*>(src);
      }
    }
  }

  // The online-softmax update of one loaded tile (alpha_w: the wave's LDS row).
  __device__ __forceinline__ void compute(const DecodeArgs& a, const TileLoad<D, FP8>& cur, float* alpha_w) {
    const int lc = lane_id() & 15, lg = lane_id() >> 4;
    // ---- S^T = K Q^T  (M = 16 token slots, N = 16 heads) ----
    bf16x8 ak[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      if (FP8) ak[kk] = fp8x8_to_bf16x8(cur.k8[kk]);
      else ak[kk] = __builtin_bit_cast(bf16x8, cur.k[kk]);
    }
    f32x4 c[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      c[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        c[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak[kk], bq[nt][kk], c[nt], 0, 0, 0);
    }
    // V operand (B: K = 16 slots, N = 16 dims): lane (lc, lg) holds slots 4lg..4lg+3
    // of dim 32q + 2lc + h for chunk m = 2q + h.
    // Chunk m = 2q + h is dim (D/16) lc + m: the low (h = 0) or high bf16 of
    // dword q of each slot's slice.
    s16x4 bv[NM];
    uint32_t vb[4][NPAIR];  // bf16 pairs: dims (D/16) lc + 2q, +1 of slot 4lg+e
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (FP8) {  // four e4m3 bytes -> four bf16 (exact): two dwords
#pragma unroll
        for (int r = 0; r < VDW; ++r) {
          auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)cur.v[e][r], false);
          auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)cur.v[e][r], true);
          vb[e][2 * r] = (__float_as_uint(lo[0]) >> 16) | (__float_as_uint(lo[1]) & 0xffff0000u);
          vb[e][2 * r + 1] = (__float_as_uint(hi[0]) >> 16) | (__float_as_uint(hi[1]) & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int r = 0; r < NPAIR; ++r) vb[e][r] = cur.v[e][r];
      }
    }
#pragma unroll
    for (int q = 0; q < NPAIR; ++q) {
      const uint32_t w0 = vb[0][q], w1 = vb[1][q], w2 = vb[2][q], w3 = vb[3][q];
      bv[2 * q + 0] = pack4(__builtin_amdgcn_perm(w1, w0, 0x05040100u), __builtin_amdgcn_perm(w3, w2, 0x05040100u));
      bv[2 * q + 1] = pack4(__builtin_amdgcn_perm(w1, w0, 0x07060302u), __builtin_amdgcn_perm(w3, w2, 0x07060302u));
    }
    float pe[NT][4];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float z[4];
      float mt = -INFINITY;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = cur.tok + e;
        const bool ok = cur.tok >= 0 && t < rlen(nt);
        float zz = c[nt][e] * a.scale_log2;
        if (FP8) zz *= cur.ks[e];
        z[e] = ok ? zz : -INFINITY;
        mt = fmaxf(mt, z[e]);
      }
      mt = max_lg(mt);
      const float m_new = fmaxf(m_run[nt], mt);
      float alpha, ps = 0.f;
      if (m_new == -INFINITY) {
        alpha = 1.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) pe[nt][e] = 0.f;
      } else {
        alpha = exp2f(m_run[nt] - m_new);
#pragma unroll
        for (int e = 0; e < 4; ++e) { pe[nt][e] = exp2f(z[e] - m_new); ps += pe[nt][e]; }
      }
      ps = sum_lg(ps);
      l_run[nt] = l_run[nt] * alpha + ps;
      m_run[nt] = m_new;
      if (lg == 0) alpha_w[nt * 16 + lc] = alpha;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      // P as the PV A operand (M = 16 heads, K = 16 slots): exactly this C layout.
      // Split p = hi + lo (two bf16) so the product keeps ~16 mantissa bits.
      uint32_t ph[2], pl[2];
#pragma unroll
      for (int e2 = 0; e2 < 2; ++e2) {
        float x0 = pe[nt][2 * e2], x1 = pe[nt][2 * e2 + 1];
        if (FP8) { x0 *= cur.vs[2 * e2]; x1 *= cur.vs[2 * e2 + 1]; }
        const __bf16 h0 = (__bf16)x0, h1 = (__bf16)x1;
        const __bf16 l0 = (__bf16)(x0 - (float)h0), l1 = (__bf16)(x1 - (float)h1);
        ph[e2] = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
        pl[e2] = (uint32_t)__builtin_bit_cast(uint16_t, l0) | ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
      }
      const s16x4 aph = pack4(ph[0], ph[1]), apl = pack4(pl[0], pl[1]);
      // rescale accumulator rows (heads 4lg+e) by their alpha
      const f32x4 al = *reinterpret_cast<const f32x4*>(&alpha_w[nt * 16 + 4 * lg]);
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        acc[nt][m] *= al;
        acc[nt][m] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(aph, bv[m], acc[nt][m], 0, 0, 0);
        acc[nt][m] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(apl, bv[m], acc[nt][m], 0, 0, 0);
      }
    }
  }

  // This wave's first tile of a batch's round (-1: none).
  __device__ __forceinline__ int first_tile(const Batch& bt_, int nr) const {
    const int w = threadIdx.x / 64;
    const int t0 = (w - bt_.off % W + W) % W;
    return t0 < ((nr + 3) >> 2) ? t0 : -1;
  }

  // Runs a batch whose first round was staged (and published) by the caller
  // and whose first tile this wave issued into cur (when first_tile >= 0) and,
  // with pre2, its second into nxt; later rounds are staged here (all threads
  // take part).
  __device__ __forceinline__ void run(const DecodeArgs& a, int kvh, const Batch& bt_, TileLoad<D, FP8>& cur,
                                      TileLoad<D, FP8>& nxt, bool pre2, const int32_t* bt, BtView btv,
                                      float* alpha_w) {
    const int nall = bt_.total();
    for (int r0 = 0; r0 < nall; r0 += kRound) {
      const int nr = min(kRound, nall - r0);
      int ti = first_tile(bt_, nr);
      bool have_next = r0 == 0 && pre2;
      if (r0 > 0) {
        __syncthreads();
        stage(a, bt_, r0, bt, btv);
        __syncthreads();
        if (ti >= 0) issue(a, kvh, bt_, nr, ti, cur);
      }
      const int ntiles = (nr + 3) >> 2;
      for (; ti >= 0 && ti < ntiles; ti += W) {
        if (ti + W < ntiles && !have_next) issue(a, kvh, bt_, nr, ti + W, nxt);
        have_next = false;
        compute(a, cur, alpha_w);
        cur = nxt;
      }
    }
  }

  // Merge the waves (fixed order => deterministic) and write the partials.
  __device__ __forceinline__ void finish(const DecodeArgs& a, int p, int kvh, const int* rows_lds) {
    __shared__ float ml_lds[kWaves][2][NHP];
    __shared__ float fac_lds[NHP][kWaves + 1];  // per-head wave factors, then 1/sum
    __shared__ float o_w[kWaves][NH][D];        // each wave's unnormalised output
    const int lc = lane_id() & 15, lg = lane_id() >> 4, w = threadIdx.x / 64;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      if (lg == 0) { ml_lds[w][0][nt * 16 + lc] = m_run[nt]; ml_lds[w][1][nt * 16 + lc] = l_run[nt]; }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int n = nt * 16 + 4 * lg + e;
        if (n < NH) {
#pragma unroll
          for (int m4 = 0; m4 < NM / 4; ++m4)
            *reinterpret_cast<f32x4*>(&o_w[w][n][(D / 16) * lc + 4 * m4]) =
                f32x4{acc[nt][4 * m4][e], acc[nt][4 * m4 + 1][e], acc[nt][4 * m4 + 2][e], acc[nt][4 * m4 + 3][e]};
        }
      }
    }
    __syncthreads();
    if (threadIdx.x < NHP) {
      const int n = threadIdx.x;
      float M = -INFINITY;
#pragma unroll
      for (int x = 0; x < kWaves; ++x) M = fmaxf(M, ml_lds[x][0][n]);
      float Ls = 0.f;
#pragma unroll
      for (int x = 0; x < kWaves; ++x) {
        const float mw = ml_lds[x][0][n];
        const float f = (mw == -INFINITY) ? 0.f : exp2f(mw - M);
        fac_lds[n][x] = f;
        Ls += ml_lds[x][1][n] * f;
      }
      fac_lds[n][kWaves] = (Ls > 0.f) ? 1.f / Ls : 0.f;
      if (n < a.nh) {
        const int r = rows_lds[n / a.G];
        const int h = kvh * a.G + n % a.G;
        if (r >= 0) a.lse_part[((size_t)p * a.R + r) * a.Hq + h] = (Ls > 0.f) ? (M + log2f(Ls)) * kLn2 : -INFINITY;
      }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < a.nh * D; idx += kThreads) {
      const int n = idx / D, d = idx % D;
      float v = 0.f;
#pragma unroll
      for (int x = 0; x < kWaves; ++x) v += o_w[x][n][d] * fac_lds[n][x];
      const int r = rows_lds[n / a.G];
      const int h = kvh * a.G + n % a.G;
      if (r >= 0) a.o_part[(((size_t)p * a.R + r) * a.Hq + h) * D + d] = v * fac_lds[n][kWaves];
    }
  }
};

// ---- attention over a stored selection (qsa_sparse_decode) ----
// One workgroup per (split, KV head x row group, selecting row).  The row's
// top-k (ascending, its first min(k, nb) entries valid) is staged in LDS in
// the first round of loads; split p takes the run [floor(p n / P),
// floor((p+1) n / P)) of those n entries.
template <int D, int NH, bool FP8, int W>
__global__ __launch_bounds__(W * 64) void decode_kernel(DecodeArgs a) {
  using At = Attend<D, NH, FP8, W>;
  constexpr int kThreads = W * 64;
  constexpr int kPer = 2048 / kThreads;
  __shared__ int32_t topk_lds[2048];
  __shared__ int rows_lds[kMaxRowsPerGroup];
  __shared__ int32_t blk_tok[kRound], blk_pos[kRound];
  __shared__ float alpha_lds[W][At::NHP];
  const int p = blockIdx.x, kvh = (int)blockIdx.y / a.qg, g = (int)blockIdx.y % a.qg, s = blockIdx.z;
  const int w = threadIdx.x / 64;
  const int b = a.sel_req[s];
  const int Lsel = max(a.sel_seq_len[s], 0);
  int tv[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) tv[i] = a.topk[(size_t)s * a.k + min((int)threadIdx.x + kThreads * i, a.k - 1)];
  const int rs0 = load_rs0(a);
  At at;
  at.init();
  const bool ident = a.row_sel == nullptr;  // row s is selecting row s: its q goes out with the first loads
  if (ident) at.load_q(a, kvh, [&](int i) { return i == 0 ? s : -1; });
  asm volatile("" ::"s"(b), "s"(Lsel));
  const int nb = Lsel >> 2;
  const int nsel = (Lsel >= 4) ? min(a.k, nb) : 0;
  const int i0 = (p * nsel) / a.P, i1 = ((p + 1) * nsel) / a.P;  // (p * nsel <= 64 * 2048)
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = (int)threadIdx.x + kThreads * i;
    if (e < a.k) topk_lds[e] = tv[i];
  }
  find_rows(a, s, g, rs0, rows_lds);
  __syncthreads();
  if (!ident) at.load_q(a, kvh, [&](int i) { return rows_lds[i]; });
  const int32_t* bt = a.block_table + (size_t)b * a.max_pages;
  const int tail_lo = 4 * nb;
  typename At::Batch batch{topk_lds + i0, i1 - i0, tail_lo, at.tail_blocks(a, p, tail_lo), blk_tok, blk_pos, 0};
  const BtView none{nullptr, 0, 0};
  TileLoad<D, FP8> cur, nxt;
  if (batch.total() > 0) {
    at.stage(a, batch, 0, bt, none);
    __syncthreads();
    const int t0 = at.first_tile(batch, min(kRound, batch.total()));
    if (t0 >= 0) at.issue(a, kvh, batch, min(kRound, batch.total()), t0, cur);
    at.run(a, kvh, batch, cur, nxt, false, bt, none, alpha_lds[w]);
  }
  at.finish(a, p, kvh, rows_lds);
}

// ---- selection + attention in one launch (qsa_select_sparse_decode) ----
// Every workgroup (split p, KV head x row group, selecting row s) finds the
// row's selection itself from the scored workspace (RowSelector: the finalize
// of select_row, into an LDS bitmap of the row) while the request's page-table
// row is staged in LDS, then lists its own run of the ascending selection,
// stages it for the attention (one block per thread) and attends it.  The row's top-k
// is never assembled in one place: the workgroups of row group 0 write their
// runs of topk while the K/V loads are in flight.  No workgroup waits for
// another: the row's histogram is only read (the workspace keeps two, and a
// selection clears the one the next call's scan adds into).
constexpr int kBtLds = 4096;         // page-table entries staged in LDS
constexpr int kFusedMaxTopk = 2048;  // k <= 2048 (checked by the API)

template <int D, int NH>
constexpr size_t decode_lds_bytes(int W) {
  constexpr int NHP = ((NH + 15) / 16) * 16;
  return (size_t)W * 2 * NHP * 4 + (size_t)W * NHP * 4 + (size_t)NHP * (W + 1) * 4 + (size_t)W * NH * D * 4 +
         2 * (size_t)kRound * 4;
}
template <int D, int NH>
constexpr bool select_decode_ok() {
  return NH <= 16 &&
         decode_lds_bytes<D, NH>(8) + sizeof(RowLds) + (kFusedMaxTopk + kBtLds) * 4 + 1024 <= 160 * 1024;
}
// the most heads one fused workgroup takes, by head dim
constexpr int kFusedHeads128 = 8, kFusedHeads64 = 16;
static_assert(select_decode_ok<128, kFusedHeads128>() && !select_decode_ok<128, 2 * kFusedHeads128>() &&
              select_decode_ok<64, kFusedHeads64>(), "fused head limits");

// kIdent: no row map (row_sel null; row s is selecting row s, qg = qpw = 1).
// A template parameter, not a branch: the hook then issues the same loads on
// every path, and the compiler's waits count exactly the loads before them.
// KK: list keys per thread in the selection's first round (fused_keys).
template <int D, int NH, bool FP8, bool kIdent, int KK>
__global__ __launch_bounds__(kFinThreads) void select_decode_kernel(DecodeArgs a, WsPtrs ws, int32_t max_seq_len,
                                                                     int32_t* __restrict__ topk_out) {
  static_assert(kFinThreads == 8 * 64, "the selection runs on the attention's 8 waves");
  using At = Attend<D, NH, FP8, 8>;
  constexpr int kBtPer = kBtLds / kFinThreads;
  __shared__ RowLds sl;
  __shared__ int32_t list_a[kFusedMaxTopk];
  __shared__ int32_t bt_lds[kBtLds];
  __shared__ int rows_lds[kMaxRowsPerGroup];
  __shared__ int32_t tok_a[kRound], pos_a[kRound];
  __shared__ float alpha_lds[8][At::NHP];
  // Work item f = p + P * (y + Hkv * qg * s), y = kvh * qg + g.  Workgroup i
  // of a launch runs on XCD i mod 8, and each XCD has an L2 of its own; the
  // workgroups of one selecting row read the same selection inputs and
  // page-table row, so consecutive work items go to one XCD (workgroups
  // i < 8 * (n / 8) take f = (i mod 8) * (n / 8) + i / 8): a row's workgroups
  // sit on as few XCDs as the grid allows, and each L2 fetches those inputs
  // once.  Any numbering is correct; this one only saves reads.
  const uint32_t nwg = gridDim.x, q8 = nwg >> 3, wi = blockIdx.x;
  const uint32_t f = (wi < 8u * q8) ? (wi & 7u) * q8 + (wi >> 3) : wi;
  const uint32_t yn = (uint32_t)(a.Hkv * a.qg), fy = f / (uint32_t)a.P;
  const int p = (int)(f % (uint32_t)a.P), y = (int)(fy % yn), s = (int)(fy / yn);
  const int kvh = y / a.qg, g = y % a.qg;
  const int w = threadIdx.x / 64;
  int bv = 0;  // the request id, loaded behind the histogram (vector load, see RowSelector::first)
  int b = 0, Lsel = 0;
  int btv[kBtPer];
  int nbt = 0, rs0 = -1;
  At at;
  at.init();
  constexpr bool ident = kIdent;
  RowSelector sel{sl, s, a.k, ws};
  auto pre = [&] { bv = vload_same(a.sel_req + s); };
  // Issued after the selection's first loads: the request's page-table row
  // (up to kBtLds entries, past them the attention reads the table itself),
  // the first 64 entries of row_sel, and q with the row lengths when the rows
  // are known without the row map (waited for only where the attention uses
  // them).
  auto hook = [&] {
    b = __builtin_amdgcn_readfirstlane(bv);
    Lsel = sel.Lsel;
    const int need = min((int)(((int64_t)Lsel + 8 + (1 << a.page_log2) - 1) >> a.page_log2), a.max_pages);
    nbt = min(need, kBtLds);
    const int32_t* btp = a.block_table + (size_t)b * a.max_pages;
#pragma unroll
    for (int i = 0; i < kBtPer; ++i) btv[i] = btp[min((int)threadIdx.x + kFinThreads * i, max(nbt - 1, 0))];
    if constexpr (ident) at.load_q(a, kvh, [&](int i) { return i == 0 ? s : -1; });
    else rs0 = load_rs0(a);
  };
  auto mid = [&] {
    find_rows(a, s, g, rs0, rows_lds);
#pragma unroll
    for (int i = 0; i < kBtPer; ++i) {
      const int e = (int)threadIdx.x + kFinThreads * i;
      if (e < nbt) bt_lds[e] = btv[i];
    }
  };
  sel.template first<KK>(a.sel_seq_len, max_seq_len, pre, hook, mid);
  // rows_lds and bt_lds were written before the classification's barrier: the
  // query rows of a row map go out now, waited for only at the first tile
  if constexpr (!ident) at.load_q(a, kvh, [&](int i) { return rows_lds[i]; });
  sel.second();
  const uint32_t t = sel.t;
  const int32_t* bt = a.block_table + (size_t)b * a.max_pages;
  const BtView btv_lds{bt_lds, 0, nbt};
  const int ks = (int)sel.ks;
  const int i0 = (p * ks) / a.P, i1 = ((p + 1) * ks) / a.P;  // (p * ks <= 64 * 2048)
  const int tail_lo = 4 * (Lsel >> 2);
  const int ntail = at.tail_blocks(a, p, tail_lo);
  typename At::Batch ba{list_a, i1 - i0, tail_lo, ntail, tok_a, pos_a, 0};
  // The run's blocks are listed (a barrier publishes the list), then staged
  // with the tail's blocks, one entry per thread: the page ids missing from
  // the LDS copy are then loaded all at once, not one after another.
  sel.emit_run(i0, i1, list_a, [](int, int) {});
  {
    const int page_mask = (1 << a.page_log2) - 1;
    const int nst = min(kRound, ba.total());
    for (int i = threadIdx.x; i < nst; i += kFinThreads) {
      const int tok = (i < ba.n) ? 4 * list_a[i] : tail_lo + 4 * (i - ba.n);
      const int pg = tok >> a.page_log2;
      int pid = bt_lds[min(pg, max(nbt - 1, 0))];
      asm volatile("" : "+v"(pid));  // keeps the two loads apart
      if (pg >= nbt) pid = bt[pg];
      tok_a[i] = tok;
      pos_a[i] = (pid << a.page_log2) | (tok & page_mask);
    }
  }
  __syncthreads();
  // The issue runs unconditionally (a wave without a tile loads a masked row):
  // a branch around it would make the compiler wait for these loads where the
  // paths join.
  const int nra = min(kRound, ba.total());
  TileLoad<D, FP8> cur, nxt;
  const int t0 = at.first_tile(ba, nra);
  at.issue(a, kvh, ba, nra, t0, cur);
  // While the loads are in flight (stores issued after them do not hold up
  // the waits for them): row group 0 writes its run of the row's top-k (the
  // last split pads it); workgroup (0, 0) of the row clears its row of the
  // next call's histogram; one workgroup publishes the count.
  if (y == 0) {
    int32_t* trow = topk_out + (size_t)s * a.k;
    for (int i = threadIdx.x; i < ba.n; i += kFinThreads) trow[i0 + i] = list_a[i];
    if (p == a.P - 1)
      for (int i = ks + (int)threadIdx.x; i < a.k; i += kFinThreads) trow[i] = -1;
    if (p == 0) {
      clear_next_hist(ws, s, t);
      if (s == 0 && threadIdx.x == 0) ws.gen[1] = t;
    }
  }
  at.run(a, kvh, ba, cur, nxt, false, bt, btv_lds, alpha_lds[w]);
  at.finish(a, p, kvh, rows_lds);
}

// ---- merge: one wave per (row, head) ----
// The partials' LSEs and outputs are loaded in one round (16 partials at a
// time), then reduced: lane p holds lse_p; the outputs are weighted by
// exp(lse_p - lse) broadcast from lane p.
template <int D, typename OutT>
__global__ __launch_bounds__(64) void merge_kernel(const float* __restrict__ o_part,
                                                    const float* __restrict__ lse_part,
                                                    OutT* __restrict__ out, float* __restrict__ lse,
                                                    int32_t P, int32_t RH) {
  constexpr int DPL = D / 64;
  constexpr int CH = 16;
  const int l = lane_id();
  const int rh = blockIdx.x;
  if (rh >= RH) return;
  const float lp_raw = lse_part[(size_t)min(l, P - 1) * RH + rh];
  const float lp = (l < P) ? lp_raw : -INFINITY;
  typedef float fvec __attribute__((ext_vector_type(DPL)));
  fvec v[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i)
    v[i] = *reinterpret_cast<const fvec*>(o_part + ((size_t)min(i, P - 1) * RH + rh) * D + l * DPL);
  const float M = wave_max_dpp(lp);
  float acc[DPL];
#pragma unroll
  for (int j = 0; j < DPL; ++j) acc[j] = 0.f;
  if (M == -INFINITY) {
    if (l == 0) lse[rh] = -INFINITY;
  } else {
    const float wgt = (lp == -INFINITY) ? 0.f : expf(lp - M);
    const float sum = wave_sum_dpp(wgt);
    if (l == 0) lse[rh] = M + logf(sum);
    const float inv = 1.f / sum;
    // empty partials have weight 0 and finite (zero) outputs
    // lane i's weight, read with readlane (i is uniform)
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const float wp = (i < P) ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wgt), i)) * inv : 0.f;
#pragma unroll
      for (int j = 0; j < DPL; ++j) acc[j] = fmaf(wp, v[i][j], acc[j]);
    }
    for (int p0 = CH; p0 < P; p0 += CH) {
#pragma unroll
      for (int i = 0; i < CH; ++i)
        v[i] = *reinterpret_cast<const fvec*>(o_part + ((size_t)min(p0 + i, P - 1) * RH + rh) * D + l * DPL);
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const float wp = (p0 + i < P) ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wgt), p0 + i)) * inv : 0.f;
#pragma unroll
        for (int j = 0; j < DPL; ++j) acc[j] = fmaf(wp, v[i][j], acc[j]);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < DPL; ++j) {
    if constexpr (sizeof(OutT) == 2) out[(size_t)rh * D + l * DPL + j] = f32_to_bf16_bits(acc[j]);
    else out[(size_t)rh * D + l * DPL + j] = acc[j];
  }
}

template <int D, int NH, bool FP8>
qsa_status launch_decode_t(dim3 grid, const DecodeArgs& a, hipStream_t stream) {
  const int64_t groups = (int64_t)grid.x * grid.y * grid.z;
  if constexpr (decode_wide_ok<NH>()) {
    if (groups < kDecodeWideMaxGroups) {
      hipLaunchKernelGGL((decode_kernel<D, NH, FP8, 8>), grid, dim3(8 * 64), 0, stream, a);
      return check_launch("qsa_sparse_decode");
    }
  }
  hipLaunchKernelGGL((decode_kernel<D, NH, FP8, 4>), grid, dim3(4 * 64), 0, stream, a);
  return check_launch("qsa_sparse_decode");
}

template <int D, bool FP8>
qsa_status launch_decode_nh(int nh, dim3 grid, DecodeArgs a, hipStream_t stream) {
  if (nh <= 4) return launch_decode_t<D, 4, FP8>(grid, a, stream);
  if (nh <= 8) return launch_decode_t<D, 8, FP8>(grid, a, stream);
  if (nh <= 16) return launch_decode_t<D, 16, FP8>(grid, a, stream);
  if (nh <= 32) return launch_decode_t<D, 32, FP8>(grid, a, stream);
  return launch_decode_t<D, 64, FP8>(grid, a, stream);
}

}  // namespace

namespace {

DecodeArgs decode_args(const qsa_config& c, int32_t R, int32_t S, int32_t qps, int32_t P, const void* q,
                       const int32_t* row_sel, const int32_t* row_seq_len, const int32_t* sel_req,
                       const int32_t* sel_seq_len, const int32_t* topk, const int32_t* block_table,
                       const void* k_cache, const void* v_cache, const float* k_scale, const float* v_scale,
                       float* o_part, float* lse_part) {
  DecodeArgs a;
  a.q = reinterpret_cast<const uint16_t*>(q);
  a.row_sel = row_sel;
  a.row_seq_len = row_seq_len;
  a.sel_req = sel_req;
  a.sel_seq_len = sel_seq_len;
  a.topk = topk;
  a.block_table = block_table;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.o_part = o_part;
  a.lse_part = lse_part;
  a.k = c.topk_blocks;
  a.max_pages = c.max_pages_per_req;
  a.page_log2 = __builtin_ctz((unsigned)c.page_size);
  a.Hq = c.num_q_heads;
  a.Hkv = c.num_kv_heads;
  a.G = c.num_q_heads / c.num_kv_heads;
  a.qps = qps;
  a.qg = 1;
  a.qpw = qps;
  a.nh = a.G * qps;
  a.P = P;
  a.R = R;
  a.S = S;
  a.scale_log2 = c.softmax_scale * kLog2e;
  return a;
}

// false: this shape has no fused kernel (the caller runs the two kernels)
template <int D, int NH, bool FP8>
bool launch_select_decode_t(dim3 grid, const DecodeArgs& a, const WsPtrs& ws, int32_t max_seq_len,
                            int32_t* topk, hipStream_t stream) {
  if constexpr (select_decode_ok<D, NH>()) {
    const int kk = fused_keys(ws.nb_stride);
    auto go = [&](auto kern) {
      hipLaunchKernelGGL(kern, grid, dim3(kFinThreads), 0, stream, a, ws, max_seq_len, topk);
    };
    if (a.row_sel == nullptr) {
      if (kk == 4) go(select_decode_kernel<D, NH, FP8, true, 4>);
      else if (kk == 6) go(select_decode_kernel<D, NH, FP8, true, 6>);
      else go(select_decode_kernel<D, NH, FP8, true, kFinKeys>);
    } else {
      if (kk == 4) go(select_decode_kernel<D, NH, FP8, false, 4>);
      else if (kk == 6) go(select_decode_kernel<D, NH, FP8, false, 6>);
      else go(select_decode_kernel<D, NH, FP8, false, kFinKeys>);
    }
    return true;
  } else {
    return false;
  }
}

template <int D, bool FP8>
bool launch_select_decode_nh(int nh, dim3 grid, const DecodeArgs& a, const WsPtrs& ws, int32_t max_seq_len,
                             int32_t* topk, hipStream_t stream) {
  if (nh <= 4) return launch_select_decode_t<D, 4, FP8>(grid, a, ws, max_seq_len, topk, stream);
  if (nh <= 8) return launch_select_decode_t<D, 8, FP8>(grid, a, ws, max_seq_len, topk, stream);
  if (nh <= 16) return launch_select_decode_t<D, 16, FP8>(grid, a, ws, max_seq_len, topk, stream);
  return false;
}

// Row groups of the fused kernel: the fewest groups qg whose rows' heads fit one
// workgroup (G * ceil(qps / qg) <= lim); 0 when not even one row fits.
int fused_row_groups(int G, int qps, int lim) {
  for (int g = 1; g <= qps; ++g)
    if (G * ((qps + g - 1) / g) <= lim) return g;
  return 0;
}

int fused_head_limit(int head_dim) { return head_dim == 128 ? kFusedHeads128 : kFusedHeads64; }

}  // namespace

int select_decode_launches(const qsa_config& c, int32_t S, int32_t qps, int32_t P, int32_t max_seq_len) {
  const int G = c.num_q_heads / c.num_kv_heads;
  const int qg = fused_row_groups(G, qps, fused_head_limit(c.head_dim));
  if (qg == 0) return 2;
  const int64_t groups = (int64_t)P * c.num_kv_heads * qg * S;
  // one launch when that grid has fewer than two workgroups per CU and the
  // rows' selection bitmaps fit the LDS
  const TopkWorkspace lay = topk_workspace_layout(S, max_seq_len);
  return (groups < kDecodeWideMaxGroups && lay.nb_stride / 64 <= kWordsLds) ? 1 : 2;
}

qsa_status launch_sparse_decode(const qsa_config& c, int32_t R, int32_t S, int32_t qps, int32_t P,
                                const void* q, const int32_t* row_sel, const int32_t* row_seq_len,
                                const int32_t* sel_req, const int32_t* sel_seq_len, const int32_t* topk,
                                const int32_t* block_table, const void* k_cache,
                                const void* v_cache, const float* k_scale, const float* v_scale,
                                float* o_part, float* lse_part, hipStream_t stream) {
  if (S == 0 || R == 0) return QSA_OK;
  const DecodeArgs a = decode_args(c, R, S, qps, P, q, row_sel, row_seq_len, sel_req, sel_seq_len, topk,
                                   block_table, k_cache, v_cache, k_scale, v_scale, o_part, lse_part);
  dim3 grid(P, c.num_kv_heads, S);
  const bool fp8 = c.kv_dtype == QSA_KV_FP8_E4M3;
  if (c.head_dim == 128)
    return fp8 ? launch_decode_nh<128, true>(a.nh, grid, a, stream)
               : launch_decode_nh<128, false>(a.nh, grid, a, stream);
  if (c.head_dim == 64)
    return fp8 ? launch_decode_nh<64, true>(a.nh, grid, a, stream)
               : launch_decode_nh<64, false>(a.nh, grid, a, stream);
  return fail(QSA_ERR_UNSUPPORTED, "head_dim %d not built", c.head_dim);
}

qsa_status launch_select_decode(const qsa_config& c, int32_t R, int32_t S, int32_t qps, int32_t P,
                                int32_t max_seq_len, const void* q, const int32_t* row_sel,
                                const int32_t* row_seq_len, const int32_t* sel_req, const int32_t* sel_seq_len,
                                const int32_t* block_table, const void* k_cache, const void* v_cache,
                                const float* k_scale, const float* v_scale, int32_t* topk, float* o_part,
                                float* lse_part, const TopkWorkspace& lay, void* ws_base, hipStream_t stream) {
  if (S == 0) return QSA_OK;
  if (c.head_dim != 64 && c.head_dim != 128) return fail(QSA_ERR_UNSUPPORTED, "head_dim %d not built", c.head_dim);
  if (select_decode_launches(c, S, qps, P, max_seq_len) == 1 && R > 0) {
    DecodeArgs a = decode_args(c, R, S, qps, P, q, row_sel, row_seq_len, sel_req, sel_seq_len, topk, block_table,
                               k_cache, v_cache, k_scale, v_scale, o_part, lse_part);
    // A selecting row with more query rows than one workgroup's heads hold is
    // spread over qg row groups per KV head (each selects the row itself and
    // attends its own query rows).
    a.qg = fused_row_groups(a.G, qps, fused_head_limit(c.head_dim));
    a.qpw = (qps + a.qg - 1) / a.qg;
    a.nh = a.G * a.qpw;
    const WsPtrs ws = ws_ptrs(lay, ws_base);
    dim3 grid((uint32_t)(P * c.num_kv_heads * a.qg * S));  // < kDecodeWideMaxGroups (checked above)
    const bool fp8 = c.kv_dtype == QSA_KV_FP8_E4M3;
    bool done;
    if (c.head_dim == 128)
      done = fp8 ? launch_select_decode_nh<128, true>(a.nh, grid, a, ws, max_seq_len, topk, stream)
                 : launch_select_decode_nh<128, false>(a.nh, grid, a, ws, max_seq_len, topk, stream);
    else
      done = fp8 ? launch_select_decode_nh<64, true>(a.nh, grid, a, ws, max_seq_len, topk, stream)
                 : launch_select_decode_nh<64, false>(a.nh, grid, a, ws, max_seq_len, topk, stream);
    if (!done) return fail(QSA_ERR_UNSUPPORTED, "qsa_select_sparse_decode: no fused kernel for %d heads", a.nh);
    return check_launch("qsa_select_sparse_decode");
  }
  qsa_status st = launch_finalize_ws(c, S, sel_seq_len, max_seq_len, topk, lay, ws_base, stream);
  if (st != QSA_OK) return st;
  return launch_sparse_decode(c, R, S, qps, P, q, row_sel, row_seq_len, sel_req, sel_seq_len, topk, block_table,
                              k_cache, v_cache, k_scale, v_scale, o_part, lse_part, stream);
}

qsa_status launch_merge(int32_t P, int32_t R, int32_t H, int32_t d, const float* o_part,
                        const float* lse_part, void* out, bool out_bf16, float* lse, hipStream_t stream) {
  const int RH = R * H;
  if (RH == 0) return QSA_OK;
  dim3 grid(RH);  // one wave per (row, head): the loads spread over more CUs
  uint16_t* ob = reinterpret_cast<uint16_t*>(out);
  float* of = reinterpret_cast<float*>(out);
  if (d == 128) {
    if (out_bf16) hipLaunchKernelGGL((merge_kernel<128, uint16_t>), grid, dim3(64), 0, stream, o_part, lse_part, ob, lse, P, RH);
    else hipLaunchKernelGGL((merge_kernel<128, float>), grid, dim3(64), 0, stream, o_part, lse_part, of, lse, P, RH);
  } else if (d == 64) {
    if (out_bf16) hipLaunchKernelGGL((merge_kernel<64, uint16_t>), grid, dim3(64), 0, stream, o_part, lse_part, ob, lse, P, RH);
    else hipLaunchKernelGGL((merge_kernel<64, float>), grid, dim3(64), 0, stream, o_part, lse_part, of, lse, P, RH);
  } else {
    return fail(QSA_ERR_UNSUPPORTED, "head_dim %d not built", d);
  }
  return check_launch("qsa_merge_partials");
}

}  // namespace qsa
