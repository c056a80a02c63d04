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
// index.  Per segment:
//   1. each thread takes the max value of its elements, each wavefront the
//      max of its lanes' (values only: no key is built for most elements);
//   2. tau is the k-th largest of the 16 wavefront maxima: at least k
//      elements have values >= tau, so the segment's k best all do;
//   3. the few threads whose max reaches tau stage their values in LDS, and
//      the whole workgroup, one staged value per thread, puts the k winners
//      of the previous segment and the elements >= tau on a list (slots
//      taken with one LDS atomic per wavefront);
//   4. the list's k best are ranked by counting, for each entry, the entries
//      above it (rounds of workgroup max when the list is long, and over
//      the staged values when it overflows its capacity).
// Typical rows put about 10-25 elements on the list; any data, ties and NaN
// included, gives the exact top-k.
#include "launch.h"
#include "mfma_tile.h"
#include "page_stream.h"

namespace ta {
namespace {

constexpr int kCandThreads = 1024;  // 16 wavefronts: four per SIMD
constexpr int kCandWaves = kCandThreads / 64;
constexpr int kSegChunks = 4;  // 16-byte chunks per thread per segment
constexpr int kListCap = 2048;  // list entries held in LDS
constexpr int kRankPad = 256;   // list entries cleared per segment
constexpr int kRankFast = 64;   // longest list ranked by eight threads per entry

__device__ __forceinline__ uint64_t elem_key(float v, int i) {
  uint32_t u = __float_as_uint(v != v ? -INFINITY : v);
  u = u == 0x80000000u ? 0u : u;                  // -0 as +0
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);  // monotone in v
  return ((uint64_t)u << 32) | (uint32_t)~(uint32_t)i;
}

__device__ __forceinline__ int key_token(uint64_t k) { return (int)~(uint32_t)k; }

// A float's bits as an unsigned integer in the float's order (for non-NaN).
__device__ __forceinline__ uint32_t mono_bits(float v) {
  const uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

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

// Max over the wavefront's lanes, with DPP moves within each row of 16 lanes
// (neighbours, pairs, half-row mirror, row mirror) and the four row maxima
// read from lanes 0, 16, 32, 48.
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_move<0xB1>(x));
  x = fmaxf(x, dpp_move<0x4E>(x));
  x = fmaxf(x, dpp_move<0x141>(x));
  x = fmaxf(x, dpp_move<0x140>(x));
  auto lane_f = [](float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
  };
  return fmaxf(fmaxf(lane_f(x, 0), lane_f(x, 16)), fmaxf(lane_f(x, 32), lane_f(x, 48)));
}

// Number of set bits of `mask` below this lane.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

template <typename S>
__global__ __launch_bounds__(kCandThreads) void candidates_kernel(
    const S* __restrict__ head_logits, int V, int n_heads, int topk, CandTree tree,
    const int32_t* __restrict__ root_token, int32_t* __restrict__ cand,
    int32_t* __restrict__ parent, int32_t* __restrict__ depth, int T) {
  constexpr int kPer = 16 / sizeof(S);
  constexpr int kSegValues = kSegChunks * kPer;  // per thread
  static_assert(kMaxTopK <= kCandWaves, "tau ranks the wavefront maxima");
  __shared__ __align__(16) u32x4 s_stage[kCandThreads][kSegChunks];  // candidate threads' values
  __shared__ __align__(16) uint64_t s_list[kListCap];
  __shared__ int s_ct[kCandThreads];  // thread of each staged slot
  __shared__ __align__(16) uint32_t s_wk[kCandWaves];
  __shared__ uint64_t s_red[kCandWaves];
  __shared__ uint64_t s_win[kMaxTopK];
  __shared__ int s_n, s_nct;
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const S* row = head_logits + ((size_t)b * n_heads + h) * V;
  const bool vec = (V % kPer) == 0 && (reinterpret_cast<uintptr_t>(row) & 15u) == 0;
  const int nchunks = (V + kPer - 1) / kPer;
  static_assert(kMaxTree <= kCandThreads, "node n is thread n's");
  // This thread's node (n = tid), read in the first segment right after
  // its row loads are issued, so that the reads' latency passes under the
  // row's and nothing delays the row's loads.  (Nothing combines them
  // before the end, so no wait for them comes before the wait for the row.)
  bool has_node = false;
  int nd_parent = 0, nd_depth = 0, nd_rank = 0;
  int32_t root = 0;
  for (int c0 = 0, seg = 0; c0 < nchunks; c0 += kSegChunks * kCandThreads, ++seg) {
    u32x4 x[kSegChunks];
#pragma unroll
    for (int u = 0; u < kSegChunks; ++u)
      x[u] = load_chunk(row, V, c0 + u * kCandThreads + tid, vec);
    if (seg == 0) {
      has_node = tid < tree.n_nodes;
      if (has_node) {
        nd_parent = tree.parent[tid];
        nd_depth = tree.depth[tid];
        nd_rank = tree.rank[tid];
      }
      // The root token through a vector load: a scalar load would be
      // waited for with the kernel arguments.
      int b_v = b;
      asm volatile("" : "+v"(b_v));
      if (h == 0 && tid == 0) root = root_token[b_v];
    }
    const int first = (c0 + tid) * kPer;  // this thread's smallest token here
    // 1. this thread's max value (NaN ignored) and its wavefront's
    float m = -INFINITY;
#pragma unroll
    for (int u = 0; u < kSegChunks; ++u)
#pragma unroll
      for (int j = 0; j < kPer; ++j) m = fmaxf(m, chunk_value<S>(x[u], j));
    const float wm = wave_max(m);  // never NaN
    if (lane == 0) s_wk[wv] = (mono_bits(wm) & ~0xFu) | (uint32_t)wv;
    // The previous segment's winners take list slots 0 .. k-1.
    const uint64_t prev_win = (seg > 0 && tid < topk) ? s_win[tid] : 0ull;
    if (tid == 0) {
      s_n = seg > 0 ? topk : 0;
      s_nct = 0;
    }
    if (tid < kRankPad) s_list[tid] = 0ull;  // entries past a short list read as 0
    __syncthreads();
    if (seg > 0 && tid < topk) s_list[tid] = prev_win;
    // 2. tau: the k-th largest of the 16 wavefront maxima, ranked on lanes
    //    0..15 as 32-bit keys: the value's monotone bits with the low four
    //    replaced by the wavefront's index (unique keys), read back with the
    //    low four cleared (never above any of the k values it stands for).
    //    At least k elements have values >= tau, so the segment's k best all
    //    do.  When tau is -inf (fewer than k wavefronts hold a finite value;
    //    its key then reads back as NaN) every element is a candidate.
    float tv;
    {
      const uint32_t mine = s_wk[lane & (kCandWaves - 1)];
      int above = 0;
#pragma unroll
      for (int w2 = 0; w2 < kCandWaves; ++w2) above += s_wk[w2] > mine ? 1 : 0;
      const uint64_t hit = __ballot(lane < kCandWaves && above == topk - 1);  // k <= 16: one lane
      const uint32_t t = hit ? __builtin_amdgcn_readlane(mine, __builtin_ctzll(hit)) & ~0xFu : 0u;
      tv = __uint_as_float((t & 0x80000000u) ? (t & 0x7FFFFFFFu) : ~t);
    }
    const bool all = !(tv > -INFINITY);
    // 3. candidate threads (max >= tau) stage their values in LDS, in slots
    //    taken with one LDS atomic per wavefront ...
    const bool is_cand = all ? first < V : m >= tv;
    const uint64_t cb = __ballot(is_cand);
    if (cb) {  // uniform
      int base = 0;
      if (lane == 0) base = atomicAdd(&s_nct, __popcll(cb));
      base = __builtin_amdgcn_readfirstlane(base);
      if (is_cand) {
        const int slot = base + lanes_below(cb);
        s_ct[slot] = tid;
#pragma unroll
        for (int u = 0; u < kSegChunks; ++u) s_stage[slot][u] = x[u];
      }
    }
    __syncthreads();
    //    ... and the workgroup, one staged value per thread, puts the
    //    elements >= tau on the list (again one atomic per wavefront).
    const int n_vals = s_nct * kSegValues;
    for (int e0 = wv * 64; e0 < n_vals; e0 += kCandThreads) {  // uniform per wavefront
      const int e = e0 + lane;
      const int slot = e / kSegValues, jj = e % kSegValues;
      float v = -INFINITY;
      int tok = V;
      if (e < n_vals) {
        const int u = jj / kPer, q = jj % kPer;
        v = chunk_value<S>(s_stage[slot][u], q);
        tok = (c0 + u * kCandThreads + s_ct[slot]) * kPer + q;
      }
      const bool ok = tok < V && (all || v >= tv);
      const uint64_t ob = __ballot(ok);
      if (ob) {
        int base = 0;
        if (lane == 0) base = atomicAdd(&s_n, __popcll(ob));
        base = __builtin_amdgcn_readfirstlane(base);
        const int at = base + lanes_below(ob);
        if (ok && at < kListCap) s_list[at] = elem_key(v, tok);
      }
    }
    __syncthreads();
    // 4. the k best, in order: by counting, for each list entry, the entries
    //    above it; rounds of workgroup max over a long list; and when the
    //    list overflowed (rows whose values crowd at the top, e.g. all
    //    equal), rounds of workgroup max over the staged values.
    const int n_all = s_n;
    auto wg_max = [&](uint64_t w) {
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
      return w;
    };
    if (n_all > kListCap) {
      // Overflow: rounds over the staged values, filtered as above.
      uint64_t prev = ~0ull;  // above every element
      for (int r = 0; r < topk; ++r) {
        uint64_t w = (seg > 0 && tid < topk && prev_win < prev) ? prev_win : 0ull;
        for (int e = tid; e < n_vals; e += kCandThreads) {
          const int slot = e / kSegValues, jj = e % kSegValues;
          const int u = jj / kPer, q = jj % kPer;
          const float v = chunk_value<S>(s_stage[slot][u], q);
          const int tok = (c0 + u * kCandThreads + s_ct[slot]) * kPer + q;
          if (tok < V && (all || v >= tv)) {
            const uint64_t k = elem_key(v, tok);
            if (k < prev && k > w) w = k;
          }
        }
        w = wg_max(w);
        if (tid == 0) s_win[r] = w;
        prev = w;
        __syncthreads();
      }
    } else if (n_all <= kRankFast) {
      // Eight threads per entry, each comparing it with every eighth entry
      // (entries n .. kRankPad - 1 are 0 and count for nothing); the eight
      // partial counts are summed with DPP moves within each half-row.
      const int i = tid >> 3, j0 = tid & 7;
      const uint64_t e = s_list[i];
      int r = 0;
#pragma unroll
      for (int m = 0; m < kRankFast / 8; ++m) r += s_list[j0 + 8 * m] > e ? 1 : 0;
      r += __builtin_amdgcn_mov_dpp(r, 0xB1, 0xF, 0xF, false);   // neighbours
      r += __builtin_amdgcn_mov_dpp(r, 0x4E, 0xF, 0xF, false);   // pairs
      r += __builtin_amdgcn_mov_dpp(r, 0x141, 0xF, 0xF, false);  // quads of a half-row
      if (j0 == 0 && i < n_all && r < topk) s_win[r] = e;
      __syncthreads();
    } else if (n_all <= kRankPad - 8) {
      // Eight entries per step: entries n .. kRankPad - 1 are 0 and count
      // for nothing.
      const int n = n_all;
      if (tid < n) {
        const uint64_t e = s_list[tid];
        int r = 0;
        const ulonglong2* sl = reinterpret_cast<const ulonglong2*>(s_list);
        for (int q = 0; q < n; q += 8) {
          ulonglong2 p[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) p[i] = sl[q / 2 + i];
#pragma unroll
          for (int i = 0; i < 4; ++i) r += (p[i].x > e ? 1 : 0) + (p[i].y > e ? 1 : 0);
        }
        if (r < topk) s_win[r] = e;
      }
      __syncthreads();
    } else if (n_all <= kCandThreads) {
      const int n = n_all;
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
      const int n = n_all;
      uint64_t prev = ~0ull;  // above every element
      for (int r = 0; r < topk; ++r) {
        uint64_t w = 0ull;
        for (int q = tid; q < n; q += kCandThreads) {
          const uint64_t e = s_list[q];
          if (e < prev && e > w) w = e;
        }
        w = wg_max(w);
        if (tid == 0) s_win[r] = w;
        prev = w;
        __syncthreads();
      }
    }
  }

  // Nodes at depth h + 1 take their rank's token.
  const size_t base = (size_t)b * T;
  if (has_node && tid > 0 && nd_depth == h + 1) cand[base + tid] = key_token(s_win[nd_rank]);
  if (h == 0) {
    for (int n = tid; n < T; n += kCandThreads) {
      if (n < tree.n_nodes) {  // n == tid
        parent[base + n] = nd_parent;
        depth[base + n] = nd_depth;
        if (n == 0) cand[base] = root;
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
