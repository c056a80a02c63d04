// Read-bandwidth probe: the rate at which this device streams a contiguous
// buffer from HBM with the load width (16 bytes per lane) and cache policy
// (non-temporal) of the tree-verify kernels' KV stream.  Measurement only:
// the verify step never calls it.  The benchmark reports the rate it reaches
// beside the verify kernel's own, as the practical ceiling for a read-only
// stream on the machine at hand.
#include "launch.h"

namespace ta {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;  // 4 KB blocks per workgroup iteration

// Workgroup w reads 32 KB contiguous per iteration (kProbeUnroll consecutive
// 4 KB blocks, one 16-byte load per lane each, all in flight before any is
// used), at iterations w, w + grid, ...; a remainder of 16-byte chunks past
// the last whole iteration is read grid-stride.  The loads are folded into an
// XOR so they stay live; one lane per wavefront folds its wavefront's value
// into *sink with a vector atomic.  One workgroup per CU (32 KB in flight per
// CU) streamed fastest in a sweep of 1-4 workgroups of 256 or 512 threads per
// CU with 1-8 blocks per iteration: 0.87 of 8 TB/s on a 1 GiB buffer, against
// 0.79 for four workgroups per CU with the same loads.
__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const u32x4* __restrict__ src,
                                                                    size_t n16,
                                                                    uint32_t* __restrict__ sink) {
  constexpr size_t kChunk = (size_t)kProbeUnroll * kProbeThreads;  // 16-byte units
  const size_t n_iter = n16 / kChunk;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (size_t it = blockIdx.x; it < n_iter; it += gridDim.x) {
    const u32x4* base = src + it * kChunk + threadIdx.x;
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(base + u * kProbeThreads);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u];
  }
  for (size_t i = n_iter * kChunk + (size_t)blockIdx.x * kProbeThreads + threadIdx.x; i < n16;
       i += (size_t)gridDim.x * kProbeThreads)
    acc ^= __builtin_nontemporal_load(src + i);
  uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x ^= __shfl_xor(x, off);
  if ((threadIdx.x & 63) == 0) atomicXor(sink, x);
}

}  // namespace

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int n_cu,
                              hipStream_t stream) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  // One workgroup per CU (32 KB in flight per CU), or fewer for a small buffer.
  const size_t want = (size_t)(n_cu > 0 ? n_cu : 256);
  const size_t need = (n16 + kProbeThreads - 1) / kProbeThreads;
  const unsigned grid = (unsigned)(need < want ? need : want);
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(kProbeThreads), 0, stream,
                     static_cast<const u32x4*>(src), n16, sink);
  return hipGetLastError();
}

}  // namespace ta
