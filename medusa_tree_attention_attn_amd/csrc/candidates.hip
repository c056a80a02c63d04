// Candidate tree from the Medusa heads (LMDeploy PR #1231:
// generate_candidates over a fixed "medusa choices" list).
//
// The choice list is static: the host validates it and numbers its nodes
// (root 0, then paths by length, then lexicographically) and passes the node
// table by value.  On the GPU, one workgroup per (Medusa head h, sequence b)
// takes the top-k tokens of the head's logits row and writes the candidate
// token of every node at depth h + 1 (rank r of the node's path -> the r-th
// best token).  No workgroup needs another's result, so one launch does it.
//
// Top-k: every thread keeps a sorted list of its best kMaxTopK values (larger
// logit first, smaller token among equals; NaN ranks as -inf) while it
// streams its share of the row with 16-byte loads; then k rounds of a
// workgroup argmax over the list heads pick the winners in order.
#include "launch.h"
#include "mfma_tile.h"

namespace ta {
namespace {

constexpr int kCandThreads = 256;

struct Entry {
  float v;
  int i;
};

__device__ __forceinline__ bool better(float av, int ai, float bv, int bi) {
  return av > bv || (av == bv && ai < bi);
}

// Insert (v, i) into the descending list L[0..kMaxTopK) (L[0] best).
__device__ __forceinline__ void insert(Entry (&L)[kMaxTopK], float v, int i) {
  v = v != v ? -INFINITY : v;  // NaN ranks as -inf
  if (!better(v, i, L[kMaxTopK - 1].v, L[kMaxTopK - 1].i)) return;
  Entry cur{v, i};
#pragma unroll
  for (int s = 0; s < kMaxTopK; ++s) {
    if (better(cur.v, cur.i, L[s].v, L[s].i)) {
      const Entry t = L[s];
      L[s] = cur;
      cur = t;
    }
  }
}

template <typename S>
__global__ __launch_bounds__(kCandThreads) void candidates_kernel(
    const S* __restrict__ head_logits, int V, int n_heads, int topk, CandTree tree,
    const int32_t* __restrict__ root_token, int32_t* __restrict__ cand,
    int32_t* __restrict__ parent, int32_t* __restrict__ depth, int T) {
  __shared__ float s_v[kCandThreads / 64];
  __shared__ int s_i[kCandThreads / 64];
  __shared__ int s_top[kMaxTopK];
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const S* row = head_logits + ((size_t)b * n_heads + h) * V;

  Entry L[kMaxTopK];
#pragma unroll
  for (int s = 0; s < kMaxTopK; ++s) L[s] = Entry{-INFINITY, 0x7FFFFFFF};
  constexpr int kPer = 16 / sizeof(S);
  const bool vec = (V % kPer) == 0 && (reinterpret_cast<uintptr_t>(row) & 15u) == 0;
  if (vec) {
    const int nchunks = V / kPer;
    const u32x4* src = reinterpret_cast<const u32x4*>(row);
    constexpr int kUnroll = 8;
    for (int c0 = 0; c0 < nchunks; c0 += kUnroll * kCandThreads) {
      u32x4 x[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int c = c0 + u * kCandThreads + tid;
        x[u] = c < nchunks ? src[c] : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int c = c0 + u * kCandThreads + tid;
        if (c < nchunks) {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            if (sizeof(S) == 2) {
              insert(L, bf16_lo(x[u][w]), c * kPer + 2 * w);
              insert(L, bf16_hi(x[u][w]), c * kPer + 2 * w + 1);
            } else {
              insert(L, __uint_as_float(x[u][w]), c * kPer + w);
            }
          }
        }
      }
    }
  } else {
    for (int i = tid; i < V; i += kCandThreads) insert(L, ld(row, i), i);
  }

  // k rounds: the best list head of the workgroup is the next token.
  for (int r = 0; r < topk; ++r) {
    float v = L[0].v;
    int i = L[0].i;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const float ov = __shfl_xor(v, off);
      const int oi = __shfl_xor(i, off);
      if (better(ov, oi, v, i)) {
        v = ov;
        i = oi;
      }
    }
    if (lane == 0) {
      s_v[wv] = v;
      s_i[wv] = i;
    }
    __syncthreads();
    float bv = s_v[0];
    int bi = s_i[0];
#pragma unroll
    for (int w = 1; w < kCandThreads / 64; ++w)
      if (better(s_v[w], s_i[w], bv, bi)) {
        bv = s_v[w];
        bi = s_i[w];
      }
    if (tid == 0) s_top[r] = bi;
    if (L[0].i == bi && L[0].v == bv) {  // this thread's head won: drop it
#pragma unroll
      for (int s = 0; s + 1 < kMaxTopK; ++s) L[s] = L[s + 1];
      L[kMaxTopK - 1] = Entry{-INFINITY, 0x7FFFFFFF};
    }
    __syncthreads();
  }

  // Nodes at depth h + 1 take their rank's token.
  const size_t base = (size_t)b * T;
  for (int n = tid; n < tree.n_nodes; n += kCandThreads) {
    if (n > 0 && tree.depth[n] == h + 1) {
      const int tok = s_top[tree.rank[n]];
      cand[base + n] = tok < V ? tok : 0;  // V < k: missing ranks give token 0
    }
  }
  if (h == 0) {
    for (int n = tid; n < T; n += kCandThreads) {
      if (n < tree.n_nodes) {
        parent[base + n] = tree.parent[n];
        depth[base + n] = tree.depth[n];
        if (n == 0) cand[base] = root_token[b];
      } else {
        parent[base + n] = kPadParent;
        depth[base + n] = 0;
        cand[base + n] = 0;
      }
    }
  }
}

}  // namespace

hipError_t launch_candidates(const void* head_logits, int dtype, int V, int n_heads, int topk,
                             const CandTree& tree, const int32_t* root_token, int32_t* cand,
                             int32_t* parent, int32_t* depth, int B, int T, hipStream_t stream) {
  const dim3 grid((unsigned)n_heads, (unsigned)B);
  if (dtype == TA_BF16)
    hipLaunchKernelGGL(candidates_kernel<uint16_t>, grid, dim3(kCandThreads), 0, stream,
                       static_cast<const uint16_t*>(head_logits), V, n_heads, topk, tree,
                       root_token, cand, parent, depth, T);
  else
    hipLaunchKernelGGL(candidates_kernel<float>, grid, dim3(kCandThreads), 0, stream,
                       static_cast<const float*>(head_logits), V, n_heads, topk, tree,
                       root_token, cand, parent, depth, T);
  return hipGetLastError();
}

}  // namespace ta
