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
// (NH = rows x heads-per-KV-head), so each K/V row is read from HBM once:
//   * QK^T:  v_mfma_f32_16x16x32_bf16 with the 16 tokens of a tile as M and the
//            NH heads as N (the group makes this dense); K goes straight from
//            global memory into the A operand (16 B per lane).
//   * softmax: online, fp32, exp2 domain; per-head running max / sum.
//   * PV:    VALU FMAs, lane = d-pair, all NH heads per lane, so every V row is
//            one coalesced 256 B wave load; p broadcast through LDS.
// Four waves take interleaved tiles of 16 tokens and are merged in LDS in a
// fixed order (deterministic).  FP8 (OCP E4M3) K/V are widened exactly to
// bf16 / fp32; the per-token K scale multiplies the logit and the V scale
// multiplies the probability.
#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

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
  float scale_log2;  // softmax_scale * log2(e)
};

// Token-slot view of one split: slot u covers token 4*blk(u/4) + u%4, where
// blk(i) is the i-th selected block of the split, or a block of the tail.
constexpr int kRound = 512;  // blocks staged in LDS per round

template <int D, bool FP8>
struct TileLoad {
  static constexpr int KK = D / 32;
  static constexpr int DPL = D / 64;
  i32x4 k[FP8 ? 1 : KK];   // bf16: 16 B per k-step
  i32x2 k8[FP8 ? KK : 1];  // fp8: 8 B per k-step
  uint32_t v[16];          // this lane's V bytes of each of the 16 slots
  int t;                   // token of slot lc (-1: none)
  float ks, vs;            // fp8 scales of slot lc
};

template <int D, int NH, bool FP8>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a) {
  constexpr int NT = (NH + 15) / 16;  // MFMA N tiles of 16 heads
  constexpr int KK = D / 32;          // MFMA k steps over the head dim
  constexpr int DPL = D / 64;         // head-dim values per lane in PV
  constexpr int ES = FP8 ? 1 : 2;     // bytes per K/V element

  __shared__ float p_lds[kWaves][16][NH];
  __shared__ float alpha_lds[kWaves][NH];
  __shared__ float ml_lds[kWaves][2][NH];
  __shared__ float o_sh[NH][D];
  __shared__ int32_t blk_tok[kRound];   // first token of each staged block
  __shared__ int32_t blk_pos[kRound];   // its position in the page pool (page*page_size + slot)

  const int p = blockIdx.x, kvh = blockIdx.y, s = blockIdx.z;
  const int l = lane_id(), w = threadIdx.x / 64;
  const int lc = l & 15, lg = l >> 4;

  const int b = a.sel_req[s];
  const int Lsel = max(a.sel_seq_len[s], 0);
  const int nsel = (Lsel >= 4) ? min(a.k, Lsel >> 2) : 0;
  const int lo = (int)(((int64_t)p * nsel) / a.P);
  const int hi = (int)(((int64_t)(p + 1) * nsel) / a.P);
  const int nblk = hi - lo;
  const int tail_lo = 4 * (Lsel >> 2);
  int tail_hi = 0;
  for (int i = 0; i < a.qps; ++i) tail_hi = max(tail_hi, a.row_seq_len[s * a.qps + i]);
  const int ntailblk = (p == a.P - 1) ? (max(0, tail_hi - tail_lo) + 3) >> 2 : 0;
  const int nall = nblk + ntailblk;  // blocks of this split (selected, then tail)
  const int page_size = 1 << a.page_log2;
  const int32_t* bt = a.block_table + (size_t)b * a.max_pages;
  const int32_t* sel = a.topk + (size_t)s * a.k + lo;

  // Q as the MFMA B operand: lane (lc, lg) holds head n = nt*16+lc, dims 32kk+8lg..+8.
  bf16x8 bq[NT][KK];
  int rlen[NT];  // context length of the row owning head n (C layout)
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int n = nt * 16 + lc;
    const bool real = n < a.nh;
    const int i = real ? n / a.G : 0;
    const int h = kvh * a.G + (real ? n % a.G : 0);
    const uint16_t* qrow = a.q + ((size_t)(s * a.qps + i) * a.Hq + h) * D;
    rlen[nt] = real ? a.row_seq_len[s * a.qps + i] : -1;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      i32x4 v = real ? ld16(qrow + 32 * kk + 8 * lg) : i32x4{0, 0, 0, 0};
      bq[nt][kk] = __builtin_bit_cast(bf16x8, v);
    }
  }

  float m_run[NT], l_run[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) { m_run[nt] = -INFINITY; l_run[nt] = 0.f; }
  float o[NH][DPL];
#pragma unroll
  for (int n = 0; n < NH; ++n)
#pragma unroll
    for (int j = 0; j < DPL; ++j) o[n][j] = 0.f;

  const char* kbase = reinterpret_cast<const char*>(a.k_cache);
  const char* vbase = reinterpret_cast<const char*>(a.v_cache);

  for (int r0 = 0; r0 < nall; r0 += kRound) {
    const int nr = min(kRound, nall - r0);
    // ---- stage block ids and page positions of this round in LDS ----
    __syncthreads();
    for (int i = threadIdx.x; i < nr; i += kThreads) {
      const int u = r0 + i;
      int tok = -1, pos = 0;
      if (u < nblk) {
        const int j = sel[u];
        tok = (j >= 0) ? 4 * j : -1;
      } else {
        tok = tail_lo + 4 * (u - nblk);
      }
      if (tok >= 0) pos = (bt[tok >> a.page_log2] << a.page_log2) | (tok & (page_size - 1));
      blk_tok[i] = tok;
      blk_pos[i] = pos;
    }
    __syncthreads();
    const int ntiles = (nr + 3) >> 2;

    // Slot lc of tile ti: block 4*ti + lc/4 of the round, token offset lc%4.
    auto issue = [&](int ti, TileLoad<D, FP8>& tl) {
      const int bi = 4 * ti + (lc >> 2);
      int t = -1, pos = 0;
      if (bi < nr) {
        const int tok = blk_tok[bi];
        if (tok >= 0) { t = tok + (lc & 3); pos = blk_pos[bi] + (lc & 3); }
      }
      // slots without a token read row 0 of the cache (a valid address) and are masked
      const int row = (t >= 0) ? ((((pos >> a.page_log2) * a.Hkv + kvh) << a.page_log2) | (pos & (page_size - 1))) : 0;
      tl.t = t;
      if (FP8) {
        tl.ks = a.k_scale[pos];
        tl.vs = a.v_scale[pos];
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
          tl.k8[kk] = *reinterpret_cast<const i32x2*>(kbase + (size_t)row * D + 32 * kk + 8 * lg);
      } else {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) tl.k[kk] = ld16(kbase + ((size_t)row * D + 32 * kk + 8 * lg) * 2);
      }
#pragma unroll
      for (int uu = 0; uu < 16; ++uu) {
        const int r = __builtin_amdgcn_readlane(row, uu);
        const char* vp = vbase + ((size_t)r * D + (size_t)l * DPL) * ES;
        if (ES * DPL == 4) tl.v[uu] = *reinterpret_cast<const uint32_t*>(vp);
        else if (ES * DPL == 2) tl.v[uu] = *reinterpret_cast<const uint16_t*>(vp);
        else tl.v[uu] = *reinterpret_cast<const uint8_t*>(vp);
      }
    };

    TileLoad<D, FP8> cur, nxt;
    int ti = w;
    if (ti < ntiles) issue(ti, cur);
    for (; ti < ntiles; ti += kWaves) {
      if (ti + kWaves < ntiles) issue(ti + kWaves, nxt);
      // ---- S^T = K Q^T ----
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
      // C layout: lane (lc, lg) holds slots 4*lg+e (e<4) for head nt*16+lc.
      int tc[4];
      float ksc[4], vsc[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        tc[e] = __shfl(cur.t, 4 * lg + e, 64);
        if (FP8) { ksc[e] = __shfl(cur.ks, 4 * lg + e, 64); vsc[e] = __shfl(cur.vs, 4 * lg + e, 64); }
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        float z[4];
        float mt = -INFINITY;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool ok = tc[e] >= 0 && tc[e] < rlen[nt];
          float zz = c[nt][e] * a.scale_log2;
          if (FP8) zz *= ksc[e];
          z[e] = ok ? zz : -INFINITY;
          mt = fmaxf(mt, z[e]);
        }
        mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
        mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
        const float m_new = fmaxf(m_run[nt], mt);
        float alpha, ps = 0.f;
        float pe[4];
        if (m_new == -INFINITY) {
          alpha = 1.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) pe[e] = 0.f;
        } else {
          alpha = exp2f(m_run[nt] - m_new);
#pragma unroll
          for (int e = 0; e < 4; ++e) { pe[e] = exp2f(z[e] - m_new); ps += pe[e]; }
        }
        ps += __shfl_xor(ps, 16, 64);
        ps += __shfl_xor(ps, 32, 64);
        l_run[nt] = l_run[nt] * alpha + ps;
        m_run[nt] = m_new;
        const int n = nt * 16 + lc;
        if (n < NH) {
#pragma unroll
          for (int e = 0; e < 4; ++e) p_lds[w][4 * lg + e][n] = FP8 ? pe[e] * vsc[e] : pe[e];
          if (lg == 0) alpha_lds[w][n] = alpha;
        }
      }
      wave_sync_lds();
      // ---- O = alpha O + P V ----
#pragma unroll
      for (int n = 0; n < NH; ++n) {
        const float al = alpha_lds[w][n];
#pragma unroll
        for (int j = 0; j < DPL; ++j) o[n][j] *= al;
      }
#pragma unroll
      for (int uu = 0; uu < 16; ++uu) {
        float vf[DPL];
        if (FP8) {
          auto f = __builtin_amdgcn_cvt_pk_f32_fp8((int)cur.v[uu], false);
#pragma unroll
          for (int j = 0; j < DPL; ++j) vf[j] = f[j];
        } else {
#pragma unroll
          for (int j = 0; j < DPL; ++j) vf[j] = bf16_bits_to_f32((cur.v[uu] >> (16 * j)) & 0xffffu);
        }
#pragma unroll
        for (int n = 0; n < NH; ++n) {
          const float pn = p_lds[w][uu][n];
#pragma unroll
          for (int j = 0; j < DPL; ++j) o[n][j] = fmaf(pn, vf[j], o[n][j]);
        }
      }
      wave_sync_lds();
      cur = nxt;
    }
  }

  // ---- merge the four waves (fixed order => deterministic) ----
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int n = nt * 16 + lc;
    if (n < NH && lg == 0) { ml_lds[w][0][n] = m_run[nt]; ml_lds[w][1][n] = l_run[nt]; }
  }
  __syncthreads();
  for (int ww = 0; ww < kWaves; ++ww) {
    if (w == ww) {
#pragma unroll
      for (int n = 0; n < NH; ++n) {
        float M = -INFINITY;
#pragma unroll
        for (int x = 0; x < kWaves; ++x) M = fmaxf(M, ml_lds[x][0][n]);
        const float mw = ml_lds[w][0][n];
        const float f = (mw == -INFINITY) ? 0.f : exp2f(mw - M);
#pragma unroll
        for (int j = 0; j < DPL; ++j) {
          const float val = o[n][j] * f;
          if (ww == 0) o_sh[n][l * DPL + j] = val;
          else o_sh[n][l * DPL + j] += val;
        }
      }
    }
    __syncthreads();
  }
  for (int idx = threadIdx.x; idx < a.nh * D; idx += kThreads) {
    const int n = idx / D, d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int x = 0; x < kWaves; ++x) M = fmaxf(M, ml_lds[x][0][n]);
    float Ls = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int x = 0; x < kWaves; ++x) {
        const float mw = ml_lds[x][0][n];
        Ls += (mw == -INFINITY) ? 0.f : ml_lds[x][1][n] * exp2f(mw - M);
      }
    }
    const int r = s * a.qps + n / a.G;
    const int h = kvh * a.G + n % a.G;
    const size_t orow = ((size_t)p * a.R + r) * a.Hq + h;
    a.o_part[orow * D + d] = (Ls > 0.f) ? o_sh[n][d] / Ls : 0.f;
    if (d == 0) a.lse_part[orow] = (Ls > 0.f) ? (M + log2f(Ls)) * kLn2 : -INFINITY;
  }
}

// ---- merge: one wave per (row, head) ----
template <int D, typename OutT>
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ o_part,
                                                    const float* __restrict__ lse_part,
                                                    OutT* __restrict__ out, float* __restrict__ lse,
                                                    int32_t P, int32_t RH) {
  constexpr int DPL = D / 64;
  const int l = lane_id();
  const int rh = blockIdx.x * 4 + threadIdx.x / 64;
  if (rh >= RH) return;
  float lp = (l < P) ? lse_part[(size_t)l * RH + rh] : -INFINITY;
  const float M = wave_max(lp);
  float acc[DPL];
#pragma unroll
  for (int j = 0; j < DPL; ++j) acc[j] = 0.f;
  if (M == -INFINITY) {
    if (l == 0) lse[rh] = -INFINITY;
  } else {
    const float wgt = (lp == -INFINITY) ? 0.f : expf(lp - M);
    const float sum = wave_sum(wgt);
    if (l == 0) lse[rh] = M + logf(sum);
    const float inv = 1.f / sum;
#pragma unroll 8
    for (int pp = 0; pp < P; ++pp) {
      // empty partials have weight 0 and finite (zero) outputs: no branch
      const float wp = __shfl(wgt, pp, 64) * inv;
      const float* src = o_part + ((size_t)pp * RH + rh) * D + l * DPL;
#pragma unroll
      for (int j = 0; j < DPL; ++j) acc[j] = fmaf(wp, src[j], acc[j]);
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
  hipLaunchKernelGGL((decode_kernel<D, NH, FP8>), grid, dim3(kThreads), 0, stream, a);
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

qsa_status launch_sparse_decode(const qsa_config& c, int32_t S, int32_t q_per_sel, int32_t P,
                                const void* q, const int32_t* row_seq_len, const int32_t* sel_req,
                                const int32_t* sel_seq_len, const int32_t* topk,
                                const int32_t* block_table, const void* k_cache,
                                const void* v_cache, const float* k_scale, const float* v_scale,
                                float* o_part, float* lse_part, hipStream_t stream) {
  if (S == 0) return QSA_OK;
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
  a.nh = a.G * q_per_sel;
  a.P = P;
  a.R = S * q_per_sel;
  a.scale_log2 = c.softmax_scale * kLog2e;
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

qsa_status launch_merge(int32_t P, int32_t R, int32_t H, int32_t d, const float* o_part,
                        const float* lse_part, void* out, bool out_bf16, float* lse, hipStream_t stream) {
  const int RH = R * H;
  if (RH == 0) return QSA_OK;
  dim3 grid((RH + 3) / 4);
  uint16_t* ob = reinterpret_cast<uint16_t*>(out);
  float* of = reinterpret_cast<float*>(out);
  if (d == 128) {
    if (out_bf16) hipLaunchKernelGGL((merge_kernel<128, uint16_t>), grid, dim3(256), 0, stream, o_part, lse_part, ob, lse, P, RH);
    else hipLaunchKernelGGL((merge_kernel<128, float>), grid, dim3(256), 0, stream, o_part, lse_part, of, lse, P, RH);
  } else if (d == 64) {
    if (out_bf16) hipLaunchKernelGGL((merge_kernel<64, uint16_t>), grid, dim3(256), 0, stream, o_part, lse_part, ob, lse, P, RH);
    else hipLaunchKernelGGL((merge_kernel<64, float>), grid, dim3(256), 0, stream, o_part, lse_part, of, lse, P, RH);
  } else {
    return fail(QSA_ERR_UNSUPPORTED, "head_dim %d not built", d);
  }
  return check_launch("qsa_merge_partials");
}

}  // namespace qsa
