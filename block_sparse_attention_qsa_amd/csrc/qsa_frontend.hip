// qsa_indexer_project: hidden states -> int8 indexer query and keys.
//
// Method ("PR #53896 完整报告", key source snippets, QSAIndexer): the indexer
// projects Q and K from the hidden states, normalises them with a Gemma-style
// RMSNorm and applies a rotary embedding, 1-D or MRoPE, before the keys enter
// the raw-key ring and the query selects.  Here, per token t at position p:
//   [q | k] = h_t W^T            W bf16 [2D, H] (q rows, then k rows), fp32 sums
//   x <- x / sqrt(mean(x^2) + 1e-6) * (1 + g)          (g_q for q, g_k for k)
//   (x_i, x_{i+D/2}) rotated by p * base^(-2i/D)       (after the norm)
//   int8 = clamp(round-half-even(x * scale), -127, 127)
// With MRoPE p has three components (temporal, height, width: positions
// [3, T]) and pair i takes the component of the contiguous section of the D/2
// frequencies it lies in (sections [0, sec1), [sec1, sec2), [sec2, D/2)); the
// 1-D call is the same kernel with one component (stride 0, sec1 = D/2).
//
// Two kernels.  project (grid: 64-token block x slice of H): each of the 4
// waves owns a quarter of the output columns for all 64 tokens (four MFMA
// M tiles) and runs v_mfma_f32_16x16x32_bf16 over its slice of H in steps of
// 32.  Lane l's A operand is 8 consecutive hidden values of token l%16 of a
// tile and its B operand 8 consecutive weights of output column l%16 (the
// weight's rows are contiguous over H): plain 16-byte loads, the A ones shared
// by the 4 waves through L1.
// The slices (about 256 workgroups in all, so that small token counts still
// spread over the chip) write fp32 partial sums to the workspace.  finish
// (grid: 16 tokens): sums the slices in a fixed order (deterministic), then
// 8 threads per (token, q or k) vector reduce the squares with lane swaps, and
// the rotation partner of a dim (i +- D/2) sits 4 threads away.  Angles are
// taken in double precision (positions reach 2^23, where an fp32 product would
// lose the angle).
#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {

namespace {

constexpr int kFeThreads = 256;
constexpr int kFeBlockRows = 64;   // tokens per project workgroup (16 per wave)
constexpr int kFeRows = 16;        // tokens per finish workgroup
constexpr int kFeSliceMin = 256;   // smallest slice of H per workgroup

template <int D>
__global__ __launch_bounds__(kFeThreads) void project_kernel(
    int32_t T, int32_t H, int32_t slice, const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ w,
    float* __restrict__ part, int32_t t_pad) {
  constexpr int kNT = 2 * D / 16 / 4;   // 16-column tiles per wave (a quarter of the outputs)
  constexpr int kMT = kFeBlockRows / 16; // 16-token tiles: all of the block's tokens in every wave
  constexpr int kU = (D >= 128) ? 4 : 8; // steps of 32 per load round
  const int l = lane_id(), wv = threadIdx.x >> 6;
  const int rb = blockIdx.x * kFeBlockRows;
  const int ks = blockIdx.y;
  const int kb = ks * slice, ke = min(H, kb + slice);
  const uint16_t* arow[kMT];
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt)  // tokens clamped: rows past T are computed and dropped
    arow[mt] = hidden + (size_t)min(rb + 16 * mt + (l & 15), T - 1) * H + 8 * (l >> 4);
  const uint16_t* bcol = w + (size_t)(wv * kNT * 16 + (l & 15)) * H + 8 * (l >> 4);
  f32x4 acc[kMT][kNT];
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // All loads of a round first (clamped in bounds; steps past the slice
  // multiply zeros), then the MFMAs.
  for (int k0 = kb; k0 < ke; k0 += 32 * kU) {
    i32x4 a[kU][kMT], b[kU][kNT];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int kk = min(k0 + 32 * u, H - 32);
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt) a[u][mt] = ld16(arow[mt] + kk);
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) b[u][nt] = ld16(bcol + (size_t)nt * 16 * H + kk);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const bool live = k0 + 32 * u < ke;
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) {
        const i32x4 bu = live ? b[u][nt] : i32x4{0, 0, 0, 0};
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[u][mt]),
                                                                __builtin_bit_cast(bf16x8, bu), acc[mt][nt], 0, 0, 0);
      }
    }
  }
  // C layout: acc[mt][nt][e] = out[token rb + 16mt + 4(l/16)+e][column (wv kNT + nt) 16 + l%16];
  // partials [slice][t_pad][2D]
  float* dst = part + ((size_t)ks * t_pad + rb) * (2 * D);
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        dst[(size_t)(16 * mt + 4 * (l >> 4) + e) * (2 * D) + (wv * kNT + nt) * 16 + (l & 15)] = acc[mt][nt][e];
}

template <int D>
__global__ __launch_bounds__(kFeThreads) void finish_kernel(
    int32_t T, int32_t nslices, const float* __restrict__ part, int32_t t_pad, const int32_t* __restrict__ positions,
    int32_t pos_stride, int32_t sec1, int32_t sec2, const float* __restrict__ g_q, const float* __restrict__ g_k, float base, float q_scale, float k_scale,
    int8_t* __restrict__ q_out, int8_t* __restrict__ k_out) {
  constexpr int kPer = D / 8;  // dims per thread
  __shared__ double inv_freq[D / 2];
  if (threadIdx.x < D / 2) inv_freq[threadIdx.x] = pow((double)base, -2.0 * (double)threadIdx.x / (double)D);
  // thread -> (token m, q or k, dims [kPer*part, kPer*part + kPer))
  const int v = threadIdx.x >> 3, part_i = threadIdx.x & 7;
  const int m = v >> 1, isk = v & 1;
  const int tok = blockIdx.x * kFeRows + m;
  const int tokc = min(tok, T - 1);
  const float* g = isk ? g_k : g_q;
  float x[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) x[e] = 0.f;
  // kSl slices per round, all loads first (clamped; slices past the last one add
  // nothing), summed in slice order: deterministic.
  constexpr int kSl = (D >= 128) ? 8 : 16;
  for (int k0 = 0; k0 < nslices; k0 += kSl) {
    f32x4 p4[kSl][kPer / 4];
#pragma unroll
    for (int u = 0; u < kSl; ++u) {
      const float* src = part + ((size_t)min(k0 + u, nslices - 1) * t_pad + tokc) * (2 * D) + isk * D + part_i * kPer;
#pragma unroll
      for (int e = 0; e < kPer / 4; ++e) p4[u][e] = *reinterpret_cast<const f32x4*>(src + 4 * e);
    }
#pragma unroll
    for (int u = 0; u < kSl; ++u) {
      if (k0 + u < nslices) {
#pragma unroll
        for (int e = 0; e < kPer / 4; ++e) {
          x[4 * e] += p4[u][e][0];
          x[4 * e + 1] += p4[u][e][1];
          x[4 * e + 2] += p4[u][e][2];
          x[4 * e + 3] += p4[u][e][3];
        }
      }
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < kPer; ++e) ss = fmaf(x[e], x[e], ss);
  ss += __shfl_xor(ss, 1, 64);
  ss += __shfl_xor(ss, 2, 64);
  ss += __shfl_xor(ss, 4, 64);
  const float inv = 1.0f / sqrtf(ss / (float)D + 1e-6f);
#pragma unroll
  for (int e = 0; e < kPer; ++e) x[e] = x[e] * inv * (1.0f + g[part_i * kPer + e]);
  __syncthreads();  // inv_freq
  // rotation: dims i < D/2 live in parts 0..3, their partners i + D/2 in parts 4..7
  // the token's three position components (one, read three times, for 1-D)
  const double pos0 = (double)positions[tokc];
  const double pos1 = (double)positions[(size_t)pos_stride + tokc];
  const double pos2 = (double)positions[2 * (size_t)pos_stride + tokc];
  const float sc = isk ? k_scale : q_scale;
  uint32_t packed[kPer / 4];
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const float other = __shfl_xor(x[e], 4, 64);
    const int i = (part_i & 3) * kPer + e;  // pair index < D/2
    // angle reduced to [-pi, pi] in double (exact enough for positions up to
    // 2^23), then the single-precision sine and cosine of the remainder
    const double pos = (i < sec1) ? pos0 : (i < sec2 ? pos1 : pos2);
    const double ang = pos * inv_freq[i];
    const double r = ang - 6.283185307179586 * rint(ang * 0.15915494309189535);
    float s, c;
    sincosf((float)r, &s, &c);
    const float y = (part_i < 4) ? fmaf(x[e], c, -other * s) : fmaf(x[e], c, other * s);
    const float qv = fminf(fmaxf(__builtin_rintf(y * sc), -127.f), 127.f);
    const uint32_t byte = (uint32_t)(uint8_t)(int8_t)(int)qv;
    if (e % 4 == 0) packed[e / 4] = 0;
    packed[e / 4] |= byte << (8 * (e % 4));
  }
  if (tok < T) {
    int8_t* dst = (isk ? k_out : q_out) + (size_t)tok * D + part_i * kPer;
#pragma unroll
    for (int u = 0; u < kPer / 4; ++u) reinterpret_cast<uint32_t*>(dst)[u] = packed[u];
  }
}

// Slices of H per token block: about 256 project workgroups in all, each
// slice a multiple of 32 and at least kFeSliceMin long.
void plan(int32_t T, int32_t H, int32_t* nslices, int32_t* slice, int32_t* t_pad) {
  const int blocks = (T + kFeBlockRows - 1) / kFeBlockRows;
  int ns = (256 + blocks - 1) / blocks;
  const int max_ns = (H + kFeSliceMin - 1) / kFeSliceMin;
  if (ns > max_ns) ns = max_ns;
  if (ns < 1) ns = 1;
  int sl = (H + ns - 1) / ns;
  sl = (sl + 31) / 32 * 32;
  ns = (H + sl - 1) / sl;
  *nslices = ns;
  *slice = sl;
  *t_pad = blocks * kFeBlockRows;
}

}  // namespace

size_t indexer_project_workspace_bytes(int32_t T, int32_t H, int32_t D) {
  int32_t ns, sl, tp;
  plan(T, H, &ns, &sl, &tp);
  return (size_t)ns * tp * 2 * D * sizeof(float);
}

qsa_status launch_indexer_project(int32_t T, int32_t H, int32_t D, const void* hidden, const int32_t* positions,
                                  int32_t pos_stride, int32_t sec1, int32_t sec2, const void* w_qk, const float* g_q, const float* g_k, float base, float q_scale,
                                  float k_scale, int8_t* q_index, int8_t* keys, float* ws, hipStream_t stream) {
  if (T == 0) return QSA_OK;
  int32_t ns, sl, tp;
  plan(T, H, &ns, &sl, &tp);
  dim3 pgrid(tp / kFeBlockRows, ns);
  dim3 fgrid((T + kFeRows - 1) / kFeRows);
  const uint16_t* h = reinterpret_cast<const uint16_t*>(hidden);
  const uint16_t* w = reinterpret_cast<const uint16_t*>(w_qk);
  switch (D) {
#define QSA_FE_CASE(DD)                                                                                      \
    case DD:                                                                                                 \
      hipLaunchKernelGGL(project_kernel<DD>, pgrid, dim3(kFeThreads), 0, stream, T, H, sl, h, w, ws, tp);   \
      if (check_launch("qsa_indexer_project(project)") != QSA_OK) return QSA_ERR_HIP;                       \
      hipLaunchKernelGGL(finish_kernel<DD>, fgrid, dim3(kFeThreads), 0, stream, T, ns, ws, tp, positions,   \
                         pos_stride, sec1, sec2, g_q, g_k, base, q_scale, k_scale, q_index, keys);           \
      break;
    QSA_FE_CASE(32)
    QSA_FE_CASE(64)
    QSA_FE_CASE(128)
#undef QSA_FE_CASE
    default:
      return fail(QSA_ERR_UNSUPPORTED, "index_dim %d not built", D);
  }
  return check_launch("qsa_indexer_project(finish)");
}

}  // namespace qsa
