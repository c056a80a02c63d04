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
#include "accept.h"
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

// ---------------------------------------------------------------------------
// Typical acceptance (the Medusa scheme vLLM issue #1171 names): with
// p = softmax(logits / temperature) after node n and H its entropy, child c
// of n passes iff p[cand_tokens[c]] > min(epsilon, delta * exp(-H)).
//
// Kernel 1, one workgroup per (sequence, node) row: a single pass over the
// row keeps, per thread and then merged over the workgroup, the running max
// m of y = x / temperature, z = sum e^(y - m) and s = sum e^(y - m) (y - m)
// (rescaled by e^(m - m') when the max moves to m'); then
// lse = m + ln z and H = ln z - s / z.  Kernel 2, one wavefront per
// sequence: each child gathers its token's logit from the parent's row and
// tests p = e^(x / temperature - lse) against the threshold; the path is then
// chosen as in greedy acceptance.
// ---------------------------------------------------------------------------
struct Lse {
  float m, z, s;
};

// Merge b into a (both over disjoint sets of values).
__device__ __forceinline__ void merge_lse(Lse& a, const Lse& b) {
  if (b.z == 0.f) return;
  if (a.z == 0.f) {
    a = b;
    return;
  }
  if (b.m > a.m) {
    const float f = __expf(a.m - b.m);
    a.s = f * (a.s + (a.m - b.m) * a.z) + b.s;
    a.z = f * a.z + b.z;
    a.m = b.m;
  } else {
    const float f = __expf(b.m - a.m);
    a.s += f * (b.s + (b.m - a.m) * b.z);
    a.z += f * b.z;
  }
}

template <int kN>
__device__ __forceinline__ void add_values(Lse& a, const float (&y)[kN], int n) {
  float mt = -INFINITY;
#pragma unroll
  for (int j = 0; j < kN; ++j)
    if (j < n) mt = fmaxf(mt, y[j]);
  if (mt == -INFINITY) return;  // nothing but -inf: no mass
  Lse t{mt, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < kN; ++j)
    if (j < n) {
      const float d = y[j] - mt;
      const float e = __expf(d);
      t.z += e;
      t.s += d == -INFINITY ? 0.f : e * d;
    }
  merge_lse(a, t);
}

template <typename S>
__global__ __launch_bounds__(kArgThreads) void row_entropy_kernel(const S* __restrict__ logits,
                                                                  int V, float inv_temp,
                                                                  float2* __restrict__ stats) {
  __shared__ Lse s_l[kArgThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const S* row = logits + (size_t)blockIdx.x * V;
  Lse a{-INFINITY, 0.f, 0.f};
  constexpr int kPer = 16 / sizeof(S);
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
        float y[kPer];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          if (sizeof(S) == 2) {
            y[2 * w] = bf16_lo(x[u][w]) * inv_temp;
            y[2 * w + 1] = bf16_hi(x[u][w]) * inv_temp;
          } else {
            y[w] = __uint_as_float(x[u][w]) * inv_temp;
          }
        }
        add_values(a, y, c < nchunks ? kPer : 0);
      }
    }
  } else {
    for (int i = tid; i < V; i += kArgThreads) {
      const float y[1] = {ld(row, i) * inv_temp};
      add_values(a, y, 1);
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const Lse o{__shfl_xor(a.m, off), __shfl_xor(a.z, off), __shfl_xor(a.s, off)};
    merge_lse(a, o);
  }
  if (lane == 0) s_l[wv] = a;
  __syncthreads();
  if (tid == 0) {
    Lse r = s_l[0];
#pragma unroll
    for (int w = 1; w < kArgThreads / 64; ++w) merge_lse(r, s_l[w]);
    const float lz = __logf(r.z);
    stats[blockIdx.x] = r.z > 0.f ? float2{r.m + lz, lz - r.s / r.z}
                                  : float2{-INFINITY, __builtin_nanf("")};
  }
}

template <typename S>
__global__ __launch_bounds__(64) void typical_accept_kernel(
    const S* __restrict__ logits, int V, int T, float inv_temp, float epsilon, float delta,
    const float2* __restrict__ stats, const int32_t* __restrict__ cand_tokens,
    const int32_t* __restrict__ tree_parent, int32_t* __restrict__ node_ok,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ accept_path) {
  const int b = blockIdx.x, i = threadIdx.x;
  const bool in_tree = i < T;
  const size_t row = (size_t)b * T;
  const int par = in_tree ? tree_parent[row + i] : kPadParent;
  const bool linked = (i == 0) ? (par == -1) : (par >= 0 && par < i);
  bool pass = false;
  if (linked && i > 0) {
    const int tok = cand_tokens[row + i];
    if (tok >= 0 && tok < V) {
      const float2 st = stats[row + par];
      const float p = __expf(ld(logits + (row + par) * V, tok) * inv_temp - st.x);
      const float thr = fminf(epsilon, delta * __expf(-st.y));
      pass = p > thr;
    }
  }
  const Acceptance a = select_path(par, pass, in_tree, i);
  write_acceptance(a, accept_len, accept_path, b, T, i);
  if (in_tree) node_ok[row + i] = (linked && (i == 0 || pass)) ? 1 : 0;
}

}  // namespace

hipError_t launch_typical_accept(const void* logits, int dtype, int V, int B, int T,
                                 float temperature, float epsilon, float delta,
                                 const int32_t* cand_tokens, const int32_t* tree_parent,
                                 float* node_stats, int32_t* node_ok, int32_t* accept_len,
                                 int32_t* accept_path, hipStream_t stream) {
  const float inv_temp = 1.0f / temperature;
  float2* stats = reinterpret_cast<float2*>(node_stats);
  if (dtype == TA_BF16) {
    hipLaunchKernelGGL(row_entropy_kernel<uint16_t>, dim3((unsigned)(B * T)), dim3(kArgThreads),
                       0, stream, static_cast<const uint16_t*>(logits), V, inv_temp, stats);
    hipLaunchKernelGGL(typical_accept_kernel<uint16_t>, dim3((unsigned)B), dim3(64), 0, stream,
                       static_cast<const uint16_t*>(logits), V, T, inv_temp, epsilon, delta,
                       stats, cand_tokens, tree_parent, node_ok, accept_len, accept_path);
  } else {
    hipLaunchKernelGGL(row_entropy_kernel<float>, dim3((unsigned)(B * T)), dim3(kArgThreads), 0,
                       stream, static_cast<const float*>(logits), V, inv_temp, stats);
    hipLaunchKernelGGL(typical_accept_kernel<float>, dim3((unsigned)B), dim3(64), 0, stream,
                       static_cast<const float*>(logits), V, T, inv_temp, epsilon, delta,
                       stats, cand_tokens, tree_parent, node_ok, accept_len, accept_path);
  }
  return hipGetLastError();
}

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
