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
  const int32_t* row_seq_len;
  const int32_t* sel_req;
  const int32_t* sel_seq_len;
  const int32_t* topk;
  const int32_t* block_table;
  const void* k_cache;
  const void* v_cache;
  const float* k_scale;
  const float* v_scale;
  float* o_part;
  float* lse_part;
  int32_t k, max_pages, page_log2, Hq, Hkv, G, qps, nh, P, R;
  int32_t qg, qpw;  // query-row groups per KV head (grid y = Hkv * qg), rows per group (nh = G * qpw)
  float scale_log2;  // softmax_scale * log2(e)
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

constexpr int kBtLdsMax = 4096;  // page-table entries the fused kernel stages in LDS

// Where the fused kernel's selection lives (LDS), for decode_body.
struct SelView {
  const int32_t* sel;  // the row's k selected block ids (ascending, -1 padded)
  const int32_t* bt;   // the request's first nbt page-table entries
  int nbt;
};

// The attention of one workgroup (split p, KV head kvh, selecting row s,
// query rows q0 .. q0 + qpw - 1 of the row's qps).
// kFusedSel: the selection is not read from a.topk; select_fn(b, load_q)
// computes it, calls load_q() once its own first loads are in flight, and
// returns where the selection is.
template <int D, int NH, bool FP8, int W, bool kFusedSel, class SelectFn>
__device__ __forceinline__ void decode_body(const DecodeArgs& a, SelectFn&& select_fn) {
  constexpr int kWaves = W;
  constexpr int kThreads = kWaves * 64;
  constexpr int NT = (NH + 15) / 16;  // MFMA tiles of 16 heads
  constexpr int NHP = NT * 16;        // heads padded to whole tiles
  constexpr int KK = D / 32;          // QK MFMA k steps over the head dim
  constexpr int NPAIR = D / 32;       // PV: pairs of 16-wide d-chunks (bf16 dwords of a V slice)
  constexpr int VDW = TileLoad<D, FP8>::VDW;
  constexpr int NM = D / 16;          // PV MFMAs (16-wide d-chunks) per head tile

  __shared__ float ml_lds[kWaves][2][NHP];
  __shared__ float alpha_lds[kWaves][NHP];
  __shared__ float fac_lds[NHP][kWaves + 1];  // per-head wave factors, then 1/sum
  __shared__ float o_w[kWaves][NH][D];        // each wave's unnormalised output
  __shared__ int32_t blk_tok[kRound];         // first token of each staged block
  __shared__ int32_t blk_pos[kRound];         // its position in the page pool (page*page_size + slot)

  const int p = blockIdx.x, kvh = (int)blockIdx.y / a.qg, s = blockIdx.z;
  const int q0 = ((int)blockIdx.y - kvh * a.qg) * a.qpw;
  const int l = lane_id(), w = threadIdx.x / 64;
  const int lc = l & 15, lg = l >> 4;

  // The split's block ids for a row with at least k closed blocks (nsel = k,
  // the usual case at long context), loaded before the row's length is known:
  // one dependent round trip less.  Used when the row turns out to be that long
  // and the split fits the workgroup; otherwise they are loaded again below.
  // (p * k <= 64 * 2048: 32-bit products and quotients)
  const int lo_full = (p * a.k) / a.P;
  const int n_full = ((p + 1) * a.k) / a.P - lo_full;
  const int spec_blk =
      kFusedSel ? 0 : a.topk[(size_t)s * a.k + lo_full + min((int)threadIdx.x, max(n_full - 1, 0))];

  const int b = a.sel_req[s];
  const int Lsel = max(a.sel_seq_len[s], 0);
  // Q as the QK MFMA B operand: lane (lc, lg) holds head n = nt*16+lc, dims
  // 32kk+8lg..+8.  The loads are unconditional (padding heads read the group's
  // first head and are zeroed), so they all go out with the loads above (with
  // kFusedSel, after the selection's first loads: those are waited for first).
  bf16x8 bq[NT][KK];
  int rlen[NT];  // context length of the row owning head nt*16+lc
  auto load_q = [&] {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int n = nt * 16 + lc;
      const bool real = n < a.nh;
      const int nn = real ? n : 0;
      const int i0 = nn / a.G;
      const int i = q0 + i0;
      const int h = kvh * a.G + (nn - i0 * a.G);
      const uint16_t* qrow = a.q + ((size_t)(s * a.qps + i) * a.Hq + h) * D;
      const int rl = a.row_seq_len[s * a.qps + i];
      rlen[nt] = real ? rl : -1;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const i32x4 v = ld16(qrow + 32 * kk + 8 * lg);
        bq[nt][kk] = __builtin_bit_cast(bf16x8, real ? v : i32x4{0, 0, 0, 0});
      }
    }
  };
  SelView sv{nullptr, nullptr, 0};
  if constexpr (kFusedSel) {
    sv = select_fn(b, load_q);
  } else {
    load_q();
    // the request and the selecting row's length, fetched while the vector
    // loads above are in flight (the compiler would otherwise fetch them at
    // first use)
    asm volatile("" ::"s"(b), "s"(Lsel));
  }
  // longest row of the selection: every row owns some head n < nh
  int tail_hi = 0;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) tail_hi = max(tail_hi, rlen[nt]);
  tail_hi = wave_max_i32(tail_hi);
  const int nsel = (Lsel >= 4) ? min(a.k, Lsel >> 2) : 0;
  const int lo = (p * nsel) / a.P;
  const int hi = ((p + 1) * nsel) / a.P;
  const int nblk = hi - lo;
  const int tail_lo = 4 * (Lsel >> 2);
  const int ntailblk = (p == a.P - 1) ? (max(0, tail_hi - tail_lo) + 3) >> 2 : 0;
  const int nall = nblk + ntailblk;  // blocks of this split (selected, then tail)
  const int page_size = 1 << a.page_log2;
  const int32_t* bt = a.block_table + (size_t)b * a.max_pages;
  const int32_t* sel = kFusedSel ? sv.sel + lo : a.topk + (size_t)s * a.k + lo;

  float m_run[NT], l_run[NT];
  // O in the MFMA C layout: acc[nt][m][e] = O[head nt*16+4lg+e][d = (D/16) lc + m]
  f32x4 acc[NT][NM];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m_run[nt] = -INFINITY;
    l_run[nt] = 0.f;
#pragma unroll
    for (int m = 0; m < NM; ++m) acc[nt][m] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const char* kbase = reinterpret_cast<const char*>(a.k_cache);
  const char* vbase = reinterpret_cast<const char*>(a.v_cache);
  auto row_of = [&](int pos) {  // token row inside the cache for this KV head
    return (((pos >> a.page_log2) * a.Hkv + kvh) << a.page_log2) | (pos & (page_size - 1));
  };

  const bool use_spec = !kFusedSel && nsel == a.k && n_full <= kThreads;  // then lo == lo_full, nblk == n_full
  for (int r0 = 0; r0 < nall; r0 += kRound) {
    const int nr = min(kRound, nall - r0);
    // ---- stage block ids and page positions of this round in LDS ----
    __syncthreads();
    for (int i = threadIdx.x; i < nr; i += kThreads) {
      const int u = r0 + i;
      int tok = -1, pos = 0;
      if (u < nblk) {
        const int j = use_spec ? spec_blk : sel[u];  // use_spec: one round, u == threadIdx.x
        tok = (j >= 0) ? 4 * j : -1;
      } else {
        tok = tail_lo + 4 * (u - nblk);
      }
      if (tok >= 0) {
        const int pg = tok >> a.page_log2;
        // (two loads, not one through a selected pointer: that would be a
        // generic load, which waits for LDS and global memory alike)
        int pid;
        if constexpr (kFusedSel) {
          pid = sv.bt[min(pg, kBtLdsMax - 1)];
          asm volatile("" : "+v"(pid));  // keeps the two loads apart
          if (pg >= sv.nbt) pid = bt[pg];
        } else {
          pid = bt[pg];
        }
        pos = (pid << a.page_log2) | (tok & (page_size - 1));
      }
      blk_tok[i] = tok;
      blk_pos[i] = pos;
    }
    __syncthreads();
    const int ntiles = (nr + 3) >> 2;

    // Tile ti = blocks 4ti..4ti+3 of the round.  The A operand (K) of lane
    // (lc, lg) is slot lc = token lc%4 of block 4ti + lc/4; its C-layout slots
    // 4lg..4lg+3 (scores, V rows, scales) are the four tokens of block 4ti + lg.
    // Slots without a token read row 0 of the cache (a valid address) and are masked.
    auto issue = [&](int ti, TileLoad<D, FP8>& tl) {
      const int ba = 4 * ti + (lc >> 2), bc = 4 * ti + lg;
      const int tok_a = (ba < nr) ? blk_tok[ba] : -1;
      const int pos_a = (ba < nr) ? blk_pos[ba] : 0;
      const int tok_c = (bc < nr) ? blk_tok[bc] : -1;
      const int pos_c = (bc < nr) ? blk_pos[bc] : 0;
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
    };

    TileLoad<D, FP8> cur, nxt;
    int ti = w;
    if (ti < ntiles) issue(ti, cur);
    for (; ti < ntiles; ti += kWaves) {
      if (ti + kWaves < ntiles) issue(ti + kWaves, nxt);
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
          const bool ok = cur.tok >= 0 && t < rlen[nt];
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
        if (lg == 0) alpha_lds[w][nt * 16 + lc] = alpha;
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
        const f32x4 al = *reinterpret_cast<const f32x4*>(&alpha_lds[w][nt * 16 + 4 * lg]);
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          acc[nt][m] *= al;
          acc[nt][m] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(aph, bv[m], acc[nt][m], 0, 0, 0);
          acc[nt][m] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(apl, bv[m], acc[nt][m], 0, 0, 0);
        }
      }
      cur = nxt;
    }
  }

  // ---- merge the waves (fixed order => deterministic) ----
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
      const int r = s * a.qps + q0 + n / a.G;
      const int h = kvh * a.G + n % a.G;
      a.lse_part[((size_t)p * a.R + r) * a.Hq + h] = (Ls > 0.f) ? (M + log2f(Ls)) * kLn2 : -INFINITY;
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < a.nh * D; idx += kThreads) {
    const int n = idx / D, d = idx % D;
    float v = 0.f;
#pragma unroll
    for (int x = 0; x < kWaves; ++x) v += o_w[x][n][d] * fac_lds[n][x];
    const int r = s * a.qps + q0 + n / a.G;
    const int h = kvh * a.G + n % a.G;
    a.o_part[(((size_t)p * a.R + r) * a.Hq + h) * D + d] = v * fac_lds[n][kWaves];
  }
}

template <int D, int NH, bool FP8, int W>
__global__ __launch_bounds__(W * 64) void decode_kernel(DecodeArgs a) {
  decode_body<D, NH, FP8, W, false>(a, [](int, auto&&) { return SelView{nullptr, nullptr, 0}; });
}

// ---- selection + attention in one launch ----
// Every workgroup of selecting row s (all splits and KV heads) runs the
// row's selection (select_row: the finalize of the scored workspace) into its
// LDS, then attends.  The selection costs every workgroup the same few
// microseconds the finalize kernel would take, in parallel; what it saves is
// the launch boundary, the round trip that reads the selection back and the
// one that looks up the pages: the request's page-table row is loaded into
// LDS while the selection runs.  No workgroup waits for another: the row's
// histogram is only read (the workspace keeps two, and a selection clears the
// one the next call's scan adds into), and workgroup (0, 0) of each row writes
// the row's top-k.  One 8-wave workgroup per (split, KV head, row), as the
// decode.
constexpr int kBtLds = kBtLdsMax;   // page-table entries staged in LDS
constexpr int kFusedMaxTopk = 2048;  // k <= 2048 (checked by the API)

template <int D, int NH>
constexpr size_t decode_lds_bytes(int W) {
  constexpr int NHP = ((NH + 15) / 16) * 16;
  return (size_t)W * 2 * NHP * 4 + (size_t)W * NHP * 4 + (size_t)NHP * (W + 1) * 4 + (size_t)W * NH * D * 4 +
         2 * (size_t)kRound * 4;
}
constexpr size_t kSelectLdsBytes = (kFinThreads / 64) * 4 + kRadixPasses * 256 * 4 + kCandLds * 8 +
                                   kWordsLds * 8 + 16 + 32 + kMaxChunksPerRow * 2;
template <int D, int NH>
constexpr bool select_decode_ok() {
  return decode_wide_ok<NH>() &&
         decode_lds_bytes<D, NH>(8) + kSelectLdsBytes + (kFusedMaxTopk + kBtLds) * 4 + 1024 <= 160 * 1024;
}
// the most heads one fused workgroup takes, by head dim
constexpr int kFusedHeads128 = 8, kFusedHeads64 = 16;
static_assert(select_decode_ok<128, kFusedHeads128>() && !select_decode_ok<128, 2 * kFusedHeads128>() &&
              select_decode_ok<64, kFusedHeads64>(), "fused head limits");

template <int D, int NH, bool FP8>
__global__ __launch_bounds__(kFinThreads) void select_decode_kernel(DecodeArgs a, WsPtrs ws, int32_t max_seq_len,
                                                                     int32_t* __restrict__ topk_out) {
  static_assert(kFinThreads == 8 * 64, "the selection runs on the decode's 8 waves");
  __shared__ int32_t sel_lds[kFusedMaxTopk];
  __shared__ int32_t bt_lds[kBtLds];
  constexpr int kBtPer = kBtLds / kFinThreads;
  const int s = blockIdx.z;
  const uint32_t t = ws.gen[0];  // the scan's histogram: t & 1
  auto select = [&](int b, auto&& load_q) -> SelView {
    int nbt = 0;
    int btv[kBtPer];
    // issued after the selection's first loads, which wait for nothing (the
    // row length and the request are loaded by then; past nbt the loads
    // re-read a valid entry and are dropped); then the attention's own loads
    auto hook = [&] {
      const int Lsel = max(a.sel_seq_len[s], 0);
      const int need = min((int)(((int64_t)Lsel + (1 << a.page_log2) - 1) >> a.page_log2), a.max_pages);
      nbt = need <= kBtLds ? need : 0;  // longer rows look their pages up in global memory
      const int32_t* bt = a.block_table + (size_t)b * a.max_pages;
#pragma unroll
      for (int i = 0; i < kBtPer; ++i) btv[i] = bt[min((int)threadIdx.x + kFinThreads * i, max(nbt - 1, 0))];
      load_q();  // the attention's q and row lengths, needed only after the selection
    };
    select_row<true, true>(s, a.sel_seq_len, a.k, max_seq_len, nullptr, sel_lds, ws, t, hook);
#pragma unroll
    for (int i = 0; i < kBtPer; ++i) {
      const int e = (int)threadIdx.x + kFinThreads * i;
      if (e < nbt) bt_lds[e] = btv[i];
    }
    return SelView{sel_lds, bt_lds, nbt};  // (the decode's staging barrier publishes both)
  };
  decode_body<D, NH, FP8, 8, true>(a, select);
  // Global writes last: the decode's waits on global memory come in issue
  // order.  Workgroup (0, 0) of the row writes the row's top-k and clears its
  // row of the next call's histogram; one workgroup publishes the count.
  if (blockIdx.x == 0 && blockIdx.y == 0) {
    for (int i = threadIdx.x; i < a.k; i += kFinThreads) topk_out[(size_t)s * a.k + i] = sel_lds[i];
    clear_next_hist(ws, s, t);
    if (s == 0 && threadIdx.x == 0) ws.gen[1] = t;
  }
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

DecodeArgs decode_args(const qsa_config& c, int32_t S, int32_t q_per_sel, int32_t P, const void* q,
                       const int32_t* row_seq_len, const int32_t* sel_req, const int32_t* sel_seq_len,
                       const int32_t* topk, const int32_t* block_table, const void* k_cache, const void* v_cache,
                       const float* k_scale, const float* v_scale, float* o_part, float* lse_part) {
  DecodeArgs a;
  a.q = reinterpret_cast<const uint16_t*>(q);
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
  a.qps = q_per_sel;
  a.qg = 1;
  a.qpw = q_per_sel;
  a.nh = a.G * q_per_sel;
  a.P = P;
  a.R = S * q_per_sel;
  a.scale_log2 = c.softmax_scale * kLog2e;
  return a;
}

// false: this shape has no fused kernel (the caller runs the two kernels)
template <int D, int NH, bool FP8>
bool launch_select_decode_t(dim3 grid, const DecodeArgs& a, const WsPtrs& ws, int32_t max_seq_len,
                            int32_t* topk, hipStream_t stream) {
  if constexpr (select_decode_ok<D, NH>()) {
    hipLaunchKernelGGL((select_decode_kernel<D, NH, FP8>), grid, dim3(kFinThreads), 0, stream, a, ws, max_seq_len,
                       topk);
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

}  // namespace

qsa_status launch_sparse_decode(const qsa_config& c, int32_t S, int32_t q_per_sel, int32_t P,
                                const void* q, const int32_t* row_seq_len, const int32_t* sel_req,
                                const int32_t* sel_seq_len, const int32_t* topk,
                                const int32_t* block_table, const void* k_cache,
                                const void* v_cache, const float* k_scale, const float* v_scale,
                                float* o_part, float* lse_part, hipStream_t stream) {
  if (S == 0) return QSA_OK;
  const DecodeArgs a = decode_args(c, S, q_per_sel, P, q, row_seq_len, sel_req, sel_seq_len, topk, block_table,
                                   k_cache, v_cache, k_scale, v_scale, o_part, lse_part);
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

qsa_status launch_select_decode(const qsa_config& c, int32_t S, int32_t q_per_sel, int32_t P, int32_t max_seq_len,
                                const void* q, const int32_t* row_seq_len, const int32_t* sel_req,
                                const int32_t* sel_seq_len, const int32_t* block_table, const void* k_cache,
                                const void* v_cache, const float* k_scale, const float* v_scale, int32_t* topk,
                                float* o_part, float* lse_part, const TopkWorkspace& lay, void* ws_base,
                                hipStream_t stream) {
  if (S == 0) return QSA_OK;
  if (c.head_dim != 64 && c.head_dim != 128) return fail(QSA_ERR_UNSUPPORTED, "head_dim %d not built", c.head_dim);
  DecodeArgs a = decode_args(c, S, q_per_sel, P, q, row_seq_len, sel_req, sel_seq_len, topk, block_table,
                             k_cache, v_cache, k_scale, v_scale, o_part, lse_part);
  const WsPtrs ws = ws_ptrs(lay, ws_base);
  // The fused kernel holds up to kFusedHeads heads per workgroup: a selecting
  // row with more query rows than fit is spread over qg workgroups per KV
  // head (each selects the row itself and attends its own query rows).
  const int lim = c.head_dim == 128 ? kFusedHeads128 : kFusedHeads64;
  for (int g = 1; g <= q_per_sel; ++g) {
    if (q_per_sel % g == 0 && a.G * (q_per_sel / g) <= lim) {
      a.qg = g;
      a.qpw = q_per_sel / g;
      a.nh = a.G * a.qpw;
      break;
    }
  }
  dim3 grid(P, c.num_kv_heads * a.qg, S);
  // One launch when the decode would run 8-wave workgroups (fewer than two
  // per CU), the rows' bitmaps fit the LDS and the shape has a fused kernel;
  // otherwise the finalize and the decode, one after the other.
  const int64_t groups = (int64_t)P * c.num_kv_heads * a.qg * S;
  bool done = false;
  if (groups < kDecodeWideMaxGroups && lay.nb_stride / 64 <= kWordsLds) {
    const bool fp8 = c.kv_dtype == QSA_KV_FP8_E4M3;
    if (c.head_dim == 128)
      done = fp8 ? launch_select_decode_nh<128, true>(a.nh, grid, a, ws, max_seq_len, topk, stream)
                 : launch_select_decode_nh<128, false>(a.nh, grid, a, ws, max_seq_len, topk, stream);
    else
      done = fp8 ? launch_select_decode_nh<64, true>(a.nh, grid, a, ws, max_seq_len, topk, stream)
                 : launch_select_decode_nh<64, false>(a.nh, grid, a, ws, max_seq_len, topk, stream);
  }
  if (done) return check_launch("qsa_select_sparse_decode");
  qsa_status st = launch_finalize_ws(c, S, sel_seq_len, max_seq_len, topk, lay, ws_base, stream);
  if (st != QSA_OK) return st;
  return launch_sparse_decode(c, S, q_per_sel, P, q, row_seq_len, sel_req, sel_seq_len, topk, block_table, k_cache,
                              v_cache, k_scale, v_scale, o_part, lse_part, stream);
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
