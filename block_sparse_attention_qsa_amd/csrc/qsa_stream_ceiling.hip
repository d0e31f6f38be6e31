// Read-only streaming kernel: the HBM read rate this part reaches with plain
// vector loads, reported next to the scan's rate as the achievable ceiling.
// Built into its own library (libqsa_ceiling.so); not part of the QSA path.
//
// Each workgroup streams one contiguous region; every thread keeps eight
// 16-byte non-temporal loads in flight per iteration, with no bounds branches
// (the region size is a whole number of iterations).  The loaded words are
// folded into one value per thread so the loads cannot be dropped.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 8;
constexpr int kBlocks = 2048;
constexpr size_t kIterBytes = (size_t)kThreads * kUnroll * 16;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const i32x4* buf, size_t iters_per_block,
                                                               uint32_t* sink) {
  const i32x4* p = buf + (size_t)blockIdx.x * iters_per_block * (kThreads * kUnroll) + threadIdx.x;
  i32x4 acc = {0, 0, 0, 0};
  for (size_t it = 0; it < iters_per_block; ++it) {
    i32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(p + u * kThreads);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
    p += kThreads * kUnroll;
  }
  sink[(size_t)blockIdx.x * kThreads + threadIdx.x] = (uint32_t)(acc.x ^ acc.y ^ acc.z ^ acc.w);
}

}  // namespace

extern "C" {

// Bytes of the sink buffer qsa_stream_read writes.
size_t qsa_stream_sink_bytes(void) { return (size_t)kBlocks * kThreads * 4; }

// Sizes qsa_stream_read accepts are multiples of this.
size_t qsa_stream_granule(void) { return kIterBytes * kBlocks; }

// Streams `bytes` (a multiple of qsa_stream_granule()) from device buffer
// `buf` (16-byte aligned) once.  Returns 0, 1 on a bad argument, 4 on a launch error.
int qsa_stream_read(const void* buf, size_t bytes, void* sink, hipStream_t stream) {
  if (!buf || !sink || bytes == 0 || bytes % (kIterBytes * kBlocks) != 0 ||
      (reinterpret_cast<uintptr_t>(buf) & 15) != 0)
    return 1;
  const size_t iters = bytes / (kIterBytes * kBlocks);
  hipLaunchKernelGGL(stream_read_kernel, dim3(kBlocks), dim3(kThreads), 0, stream,
                     reinterpret_cast<const i32x4*>(buf), iters, reinterpret_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

// One pass of the same loads over a shorter buffer: `bytes` (a multiple of
// qsa_stream_tile(), at most qsa_stream_granule()) from `buf`, one workgroup
// per qsa_stream_tile() bytes (eight 16-byte loads per thread), so that a
// transfer of a kernel's size is timed with the same launch ramp as that
// kernel.  Returns 0, 1 on a bad argument, 4 on a launch error.
size_t qsa_stream_tile(void) { return kIterBytes; }

int qsa_stream_read_once(const void* buf, size_t bytes, void* sink, hipStream_t stream) {
  if (!buf || !sink || bytes == 0 || bytes % kIterBytes != 0 || bytes > kIterBytes * kBlocks ||
      (reinterpret_cast<uintptr_t>(buf) & 15) != 0)
    return 1;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)(bytes / kIterBytes)), dim3(kThreads), 0, stream,
                     reinterpret_cast<const i32x4*>(buf), (size_t)1, reinterpret_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // extern "C"
