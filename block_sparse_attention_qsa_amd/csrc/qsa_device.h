// Device-side helpers shared by the QSA kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qsa.h"

namespace qsa {

constexpr int kRatio = 4;   // tokens per micro-block
constexpr int kRing = 8;    // ring slots (slot t % 8): the last 8 tokens' raw keys

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// 16-byte global load (dwordx4).
__device__ __forceinline__ i32x4 ld16(const void* p) { return *reinterpret_cast<const i32x4*>(p); }

// A dword every lane reads from the same address, as a vector load: it joins
// the in-order queue of the wave's vector loads (waiting for it waits only for
// the loads issued before it), where a scalar load would be waited for with
// every other scalar load in flight.  The offset comes from an asm statement,
// so the compiler cannot turn the load into a scalar one.
__device__ __forceinline__ int32_t vload_same(const int32_t* p) {
  int32_t z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
  return p[z];
}

// Agent-scope relaxed atomic accessors for counters shared between workgroups.
__device__ __forceinline__ uint32_t ld_acq_u32(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_acq_u64(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_rel_u32(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wave-wide reductions over 64 lanes (xor butterfly through ds_swizzle/bpermute).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Inclusive prefix sum across the wave: DPP row shifts inside each 16-lane
// row, then the row totals (read from lanes 15, 31, 47) added to later rows.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, true);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, true);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, true);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, true);  // row_shr:8
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 15);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 31);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 47);
  const int row = lane_id() >> 4;
  return v + (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
}

// Number of set bits of a wave mask below this lane.
__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Maximum across the wave, uniform result: DPP row shifts give each 16-lane
// row's maximum in its last lane (a lane whose source is outside the row keeps
// its own value), then the four row maxima are read with readlane.
__device__ __forceinline__ int wave_max_i32(int v) {
  v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x111, 0xf, 0xf, false));  // row_shr:1
  v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x112, 0xf, 0xf, false));  // row_shr:2
  v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x114, 0xf, 0xf, false));  // row_shr:4
  v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x118, 0xf, 0xf, false));  // row_shr:8
  return max(max(__builtin_amdgcn_readlane(v, 15), __builtin_amdgcn_readlane(v, 31)),
             max(__builtin_amdgcn_readlane(v, 47), __builtin_amdgcn_readlane(v, 63)));
}

// fp32 maximum and sum across the wave, uniform results, by the same DPP row
// shifts plus readlane of the four row ends (no LDS).  The sum adds in a fixed
// order (rows, then the four row sums), so it is deterministic.
__device__ __forceinline__ float wave_max_dpp(float x) {
  int v = __float_as_int(x);
  v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(__builtin_amdgcn_update_dpp(v, v, 0x111, 0xf, 0xf, false))));
  v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(__builtin_amdgcn_update_dpp(v, v, 0x112, 0xf, 0xf, false))));
  v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(__builtin_amdgcn_update_dpp(v, v, 0x114, 0xf, 0xf, false))));
  v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(__builtin_amdgcn_update_dpp(v, v, 0x118, 0xf, 0xf, false))));
  return fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(v, 15)), __int_as_float(__builtin_amdgcn_readlane(v, 31))),
               fmaxf(__int_as_float(__builtin_amdgcn_readlane(v, 47)), __int_as_float(__builtin_amdgcn_readlane(v, 63))));
}
__device__ __forceinline__ float wave_sum_dpp(float x) {
  int v = __float_as_int(x);
  v = __float_as_int(__int_as_float(v) + __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true)));
  v = __float_as_int(__int_as_float(v) + __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true)));
  v = __float_as_int(__int_as_float(v) + __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true)));
  v = __float_as_int(__int_as_float(v) + __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true)));
  return (__int_as_float(__builtin_amdgcn_readlane(v, 15)) + __int_as_float(__builtin_amdgcn_readlane(v, 31))) +
         (__int_as_float(__builtin_amdgcn_readlane(v, 47)) + __int_as_float(__builtin_amdgcn_readlane(v, 63)));
}

// Round-to-nearest-even fp32 -> bf16 bits (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

}  // namespace qsa
