// Greedy token of every tree node from the base model's logits (LMDeploy PR
// #1231: evaluate_posterior at LM-head temperature 0).
//
// One workgroup per (sequence, node) row streams the row's logits once with
// 16-byte loads, all in flight before any compare, and reduces (value, token)
// pairs: the larger value wins, the smaller token among equal values; NaN
// never wins, and a row with nothing comparable gives token 0.
//
// The acceptance that consumes the tokens runs as a second launch: making
// every row's token visible to one workgroup per sequence inside this launch
// takes a release per workgroup, which on gfx950 writes back the XCD's L2
// (measured: 47 us for the fused form against 16.6 + ~5 us for two launches
// on the 7B batch-16 shape).
#include "launch.h"
#include "mfma_tile.h"

namespace ta {
namespace {

constexpr int kArgThreads = 256;

struct Best {
  float v;
  int i;
};

// a is better than b: larger value, or equal value and smaller token.
__device__ __forceinline__ bool better(float av, int ai, float bv, int bi) {
  return av > bv || (av == bv && ai < bi);
}

__device__ __forceinline__ void take(Best& b, float v, int i) {
  if (better(v, i, b.v, b.i)) {
    b.v = v;
    b.i = i;
  }
}

// Row argmax over V values; every thread of the workgroup returns the result.
template <typename S>
__device__ __forceinline__ int row_argmax(const S* row, int V, int tid, float* s_v, int* s_i) {
  Best b{-INFINITY, 0x7FFFFFFF};
  constexpr int kPer = 16 / sizeof(S);  // values per 16-byte load
  const bool vec = (V % kPer) == 0 && (reinterpret_cast<uintptr_t>(row) & 15u) == 0;
  if (vec) {
    const int nchunks = V / kPer;
    const u32x4* src = reinterpret_cast<const u32x4*>(row);
    constexpr int kUnroll = 16;
    for (int c0 = 0; c0 < nchunks; c0 += kUnroll * kArgThreads) {
      u32x4 x[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int c = c0 + u * kArgThreads + tid;
        x[u] = c < nchunks ? src[c] : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int c = c0 + u * kArgThreads + tid;
        if (c < nchunks) {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            if (sizeof(S) == 2) {
              take(b, bf16_lo(x[u][w]), c * kPer + 2 * w);
              take(b, bf16_hi(x[u][w]), c * kPer + 2 * w + 1);
            } else {
              take(b, __uint_as_float(x[u][w]), c * kPer + w);
            }
          }
        }
      }
    }
  } else {
    for (int i = tid; i < V; i += kArgThreads) take(b, ld(row, i), i);
  }
  // wavefront, then workgroup
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float ov = __shfl_xor(b.v, off);
    const int oi = __shfl_xor(b.i, off);
    take(b, ov, oi);
  }
  const int lane = tid & 63, wv = tid >> 6;
  if (lane == 0) {
    s_v[wv] = b.v;
    s_i[wv] = b.i;
  }
  __syncthreads();
  Best r{s_v[0], s_i[0]};
#pragma unroll
  for (int w = 1; w < kArgThreads / 64; ++w) take(r, s_v[w], s_i[w]);
  return r.i == 0x7FFFFFFF ? 0 : r.i;
}

template <typename S>
__global__ __launch_bounds__(kArgThreads) void vocab_argmax_kernel(const S* __restrict__ logits,
                                                                   int V,
                                                                   int32_t* __restrict__ out) {
  __shared__ float s_v[kArgThreads / 64];
  __shared__ int s_i[kArgThreads / 64];
  const size_t row = blockIdx.x;
  const int tok = row_argmax(logits + row * V, V, threadIdx.x, s_v, s_i);
  if (threadIdx.x == 0) out[row] = tok;
}

}  // namespace

hipError_t launch_vocab_argmax(const void* logits, int dtype, int V, int rows, int32_t* out,
                               hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  if (dtype == TA_BF16)
    hipLaunchKernelGGL(vocab_argmax_kernel<uint16_t>, dim3(rows), dim3(kArgThreads), 0, stream,
                       static_cast<const uint16_t*>(logits), V, out);
  else
    hipLaunchKernelGGL(vocab_argmax_kernel<float>, dim3(rows), dim3(kArgThreads), 0, stream,
                       static_cast<const float*>(logits), V, out);
  return hipGetLastError();
}

}  // namespace ta
