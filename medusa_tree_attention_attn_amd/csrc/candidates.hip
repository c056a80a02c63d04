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
// Top-k without per-element sorting.  Every element (value, token) gets a
// 64-bit key whose unsigned order is the top-k order: the value's bits made
// monotone (NaN as -inf, -0 as +0) above the inverted token (smaller token
// first among equal values); key 0 is below every element.  The row is
// taken in segments of kSegChunks 16-byte chunks per thread, held in
// registers; elements past the row's end read as -inf and are excluded by
// index where -inf matters.  Per segment:
//   1. each thread finds its best element: the max value, then the smallest
//      token holding it;
//   2. each wavefront takes the k-th best of its 64 lanes' bests, and tau is
//      the largest of these.  The wavefront that gives tau has k lanes whose
//      bests are >= tau, so the segment's k best elements are all >= tau,
//      and in every wavefront only lanes among its k best can hold anything
//      >= tau;
//   3. the elements >= tau (at most k lanes per wavefront times the values
//      per lane) and the k winners of the previous segment go to an LDS
//      list;
//   4. the list's k best are ranked by counting, for each entry, the entries
//      above it (rounds of workgroup max when the list is long).
// Typical rows put a few dozen elements on the list; the bound holds for any
// data, ties and NaN included.
#include "launch.h"
#include "mfma_tile.h"

namespace ta {
namespace {

constexpr int kCandThreads = 1024;  // 16 wavefronts: four per SIMD
constexpr int kCandWaves = kCandThreads / 64;
constexpr int kSegChunks = 4;  // 16-byte chunks per thread per segment

__device__ __forceinline__ uint64_t elem_key(float v, int i) {
  uint32_t u = __float_as_uint(v != v ? -INFINITY : v);
  u = u == 0x80000000u ? 0u : u;                  // -0 as +0
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);  // monotone in v
  return ((uint64_t)u << 32) | (uint32_t)~(uint32_t)i;
}

__device__ __forceinline__ int key_token(uint64_t k) { return (int)~(uint32_t)k; }

// Value j of a chunk.
template <typename S>
__device__ __forceinline__ float chunk_value(const u32x4& x, int j) {
  if (sizeof(S) == 2) return (j & 1) ? bf16_hi(x[j >> 1]) : bf16_lo(x[j >> 1]);
  return __uint_as_float(x[j]);
}

// Chunk c of a row (values c * kPer ...); values at or past V read as -inf.
template <typename S>
__device__ __forceinline__ u32x4 load_chunk(const S* row, int V, int c, bool vec) {
  constexpr int kPer = 16 / sizeof(S);
  constexpr uint32_t kNegInf = sizeof(S) == 2 ? 0xFF80FF80u : 0xFF800000u;
  u32x4 x{kNegInf, kNegInf, kNegInf, kNegInf};
  const int i0 = c * kPer;
  if (i0 >= V) return x;
  if (vec) return reinterpret_cast<const u32x4*>(row)[c];
  if (sizeof(S) == 2) {
    const uint16_t* r = reinterpret_cast<const uint16_t*>(row);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t lo = i0 + 2 * w < V ? r[i0 + 2 * w] : 0xFF80u;
      const uint32_t hi = i0 + 2 * w + 1 < V ? r[i0 + 2 * w + 1] : 0xFF80u;
      x[w] = lo | (hi << 16);
    }
  } else {
    const uint32_t* r = reinterpret_cast<const uint32_t*>(row);
#pragma unroll
    for (int w = 0; w < 4; ++w) x[w] = i0 + w < V ? r[i0 + w] : kNegInf;
  }
  return x;
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int off) {
  const uint32_t lo = __shfl_xor((uint32_t)v, off), hi = __shfl_xor((uint32_t)(v >> 32), off);
  return ((uint64_t)hi << 32) | lo;
}

template <typename S>
__global__ __launch_bounds__(kCandThreads) void candidates_kernel(
    const S* __restrict__ head_logits, int V, int n_heads, int topk, CandTree tree,
    const int32_t* __restrict__ root_token, int32_t* __restrict__ cand,
    int32_t* __restrict__ parent, int32_t* __restrict__ depth, int T) {
  constexpr int kPer = 16 / sizeof(S);
  constexpr int kSegValues = kSegChunks * kPer;           // per thread
  constexpr int kCap = kMaxTopK * kCandWaves * kSegValues + kMaxTopK;  // list bound
  __shared__ __align__(16) uint64_t s_list[kCap];
  __shared__ __align__(16) uint64_t s_best[kCandThreads];
  __shared__ uint64_t s_red[kCandWaves];
  __shared__ uint64_t s_tauw[kCandWaves];
  __shared__ uint64_t s_win[kMaxTopK];
  __shared__ int s_n;
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const S* row = head_logits + ((size_t)b * n_heads + h) * V;
  const bool vec = (V % kPer) == 0 && (reinterpret_cast<uintptr_t>(row) & 15u) == 0;
  const int nchunks = (V + kPer - 1) / kPer;

  for (int c0 = 0, seg = 0; c0 < nchunks; c0 += kSegChunks * kCandThreads, ++seg) {
    u32x4 x[kSegChunks];
#pragma unroll
    for (int u = 0; u < kSegChunks; ++u)
      x[u] = load_chunk(row, V, c0 + u * kCandThreads + tid, vec);
    const int first = (c0 + tid) * kPer;  // this thread's smallest token here
    // 1. this thread's best element
    float m = -INFINITY;
#pragma unroll
    for (int u = 0; u < kSegChunks; ++u)
#pragma unroll
      for (int j = 0; j < kPer; ++j) m = fmaxf(m, chunk_value<S>(x[u], j));  // NaN ignored
    uint64_t best;
    if (m > -INFINITY) {
      int bi = 0;
#pragma unroll
      for (int u = kSegChunks - 1; u >= 0; --u)
#pragma unroll
        for (int j = kPer - 1; j >= 0; --j)
          if (chunk_value<S>(x[u], j) == m) bi = (c0 + u * kCandThreads + tid) * kPer + j;
      best = elem_key(m, bi);
    } else {
      // only -inf, NaN or nothing: all equal, the smallest token wins
      best = first < V ? elem_key(-INFINITY, first) : 0ull;
    }
    s_best[tid] = best;
    if (lane == 0) s_tauw[wv] = 0ull;
    if (tid == 0) s_n = 0;
    __syncthreads();
    // 2. tau_w: the best of this wavefront's lanes with exactly k - 1 above
    //    it (0 when fewer than k lanes have elements); tau = max over
    //    wavefronts.  The wavefront holding that max has k lanes whose bests
    //    are >= tau, so the segment's k best are all >= tau; in any
    //    wavefront, only lanes among its k best reach tau.
    int rank = 0;
    const ulonglong2* sb = reinterpret_cast<const ulonglong2*>(s_best + 64 * wv);
#pragma unroll 8
    for (int q = 0; q < 32; ++q) {
      const ulonglong2 e = sb[q];
      rank += (e.x > best ? 1 : 0) + (e.y > best ? 1 : 0);
    }
    if (rank == topk - 1 && best != 0ull) s_tauw[wv] = best;
    __syncthreads();
    uint64_t tau = 0ull;
#pragma unroll
    for (int w = 0; w < kCandWaves; ++w) tau = s_tauw[w] > tau ? s_tauw[w] : tau;
    // 3. the list: elements >= tau, then the previous segment's winners
    if (best >= tau) {  // this thread holds elements >= tau
      const float tv = __uint_as_float((uint32_t)(tau >> 32) & 0x80000000u
                                           ? (uint32_t)(tau >> 32) & 0x7FFFFFFFu
                                           : ~(uint32_t)(tau >> 32));
      const bool exact = !(tv > -INFINITY);  // tau is -inf or none: test keys
#pragma unroll
      for (int u = 0; u < kSegChunks; ++u) {
        const int i0 = (c0 + u * kCandThreads + tid) * kPer;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
          const float v = chunk_value<S>(x[u], j);
          if (exact || v >= tv) {
            const uint64_t k = elem_key(v, i0 + j);
            if (i0 + j < V && k >= tau) {
              const int slot = atomicAdd(&s_n, 1);
              if (slot < kCap) s_list[slot] = k;
            }
          }
        }
      }
    }
    if (seg > 0 && tid < topk) {
      const int slot = atomicAdd(&s_n, 1);
      if (slot < kCap) s_list[slot] = s_win[tid];
    }
    __syncthreads();
    // 4. the list's k best, in order
    const int n = min(s_n, kCap);
    if (n <= kCandThreads) {
      if (tid < n) {
        const uint64_t e = s_list[tid];
        int r = (n & 1) && s_list[n - 1] > e ? 1 : 0;
        const ulonglong2* sl = reinterpret_cast<const ulonglong2*>(s_list);
        for (int q = 0; q < n / 2; ++q) {
          const ulonglong2 p = sl[q];
          r += (p.x > e ? 1 : 0) + (p.y > e ? 1 : 0);
        }
        if (r < topk) s_win[r] = e;
      }
      __syncthreads();
    } else {
      uint64_t prev = ~0ull;  // above every element
      for (int r = 0; r < topk; ++r) {
        uint64_t w = 0ull;
        for (int q = tid; q < n; q += kCandThreads) {
          const uint64_t e = s_list[q];
          if (e < prev && e > w) w = e;
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
          const uint64_t o = shfl_xor_u64(w, off);
          w = o > w ? o : w;
        }
        if (lane == 0) s_red[wv] = w;
        __syncthreads();
        w = s_red[0];
#pragma unroll
        for (int q = 1; q < kCandWaves; ++q) w = s_red[q] > w ? s_red[q] : w;
        if (tid == 0) s_win[r] = w;
        prev = w;
        __syncthreads();
      }
    }
  }

  // Nodes at depth h + 1 take their rank's token.
  const size_t base = (size_t)b * T;
  for (int n = tid; n < tree.n_nodes; n += kCandThreads) {
    if (n > 0 && tree.depth[n] == h + 1) cand[base + n] = key_token(s_win[tree.rank[n]]);
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
