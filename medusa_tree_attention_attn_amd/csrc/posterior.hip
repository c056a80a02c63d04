// Greedy token of every tree node from the base model's logits (LMDeploy PR
// #1231: evaluate_posterior at LM-head temperature 0).
//
// One workgroup per (sequence, node) row streams the row's logits once with
// 16-byte loads (stream_row: the next chunk of every thread in flight while
// one is compared) and reduces (value, token) pairs: the larger value wins,
// the smaller token among equal values; NaN never wins, and a row with
// nothing comparable gives token 0.
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

constexpr int kArgThreads = 256;  // threads per logits row (argmax)
// Threads per logits row of the entropy pass (16 x 64 rows of 32000 bf16,
// with a running max and two chunks per batch: 18.5 us at 256 threads, 18.8
// at 512; with one chunk per batch 19.4, 20.1 and 23.5 at 256, 512 and
// 1024.  With a fixed reference: 17.0 us at 256 and at 512 threads, and the
// same with all of a thread's chunks in flight at once).
constexpr int kEntThreads = 256;

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

// Streams a row of nchunks 16-byte chunks through registers: thread tid
// takes chunks i * Op::kThreads + tid for i = 0, 1, ..., in increasing order,
// in batches of Op::kBatch, with the next batch in flight while one is
// consumed.  The loads are unconditional (an index past the row reads its
// last chunk, which the consumer ignores), so the compiler's wait counts
// cover them and a chunk is consumed as soon as its own load has arrived.
// The rows are read once: the loads carry the non-temporal hint.
// Op::batch(x, i0) consumes chunks i0 .. i0 + kBatch - 1 of the thread.
// (Measured on 16 x 64 rows of 32000 bf16: one or two chunks per batch beat
// four or eight, and 256 threads per row beat 512 or 1024.)
template <typename Op>
__device__ __forceinline__ void stream_row(const u32x4* __restrict__ src, int nchunks, int tid,
                                           Op& op) {
  constexpr int kB = Op::kBatch;
  constexpr int kT = Op::kThreads;  // threads streaming the row
  const int n = (nchunks + kT - 1) / kT;  // chunks per thread
  const int last = nchunks - 1;
  u32x4 ra[kB], rb[kB];
#pragma unroll
  for (int u = 0; u < kB; ++u) ra[u] = __builtin_nontemporal_load(&src[min(u * kT + tid, last)]);
  // Keep batch a's loads ahead of batch b's: the wait for a then leaves b in
  // flight, on the first pass as on every later one.
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int u = 0; u < kB; ++u)
    rb[u] = __builtin_nontemporal_load(&src[min((kB + u) * kT + tid, last)]);
  for (int i0 = 0; i0 < n; i0 += 2 * kB) {
    op.batch(ra, i0);
#pragma unroll
    for (int u = 0; u < kB; ++u)
      ra[u] = __builtin_nontemporal_load(&src[min((i0 + 2 * kB + u) * kT + tid, last)]);
    op.batch(rb, i0 + kB);
#pragma unroll
    for (int u = 0; u < kB; ++u)
      rb[u] = __builtin_nontemporal_load(&src[min((i0 + 3 * kB + u) * kT + tid, last)]);
  }
}

// Argmax consumer of stream_row.
template <typename S>
struct ArgmaxOp {
  static constexpr int kBatch = 1;
  static constexpr int kThreads = kArgThreads;
  Best b;
  int nchunks, tid;
  __device__ __forceinline__ void batch(const u32x4 (&x)[kBatch], int i0) {
    constexpr int kPer = 16 / sizeof(S);
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int c = (i0 + u) * kArgThreads + tid;
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
};

// Row argmax over V values; every thread of the workgroup returns the result.
template <typename S>
__device__ __forceinline__ int row_argmax(const S* row, int V, int tid, float* s_v, int* s_i) {
  Best b{-INFINITY, 0x7FFFFFFF};
  constexpr int kPer = 16 / sizeof(S);  // values per 16-byte load
  const bool vec = (V % kPer) == 0 && (reinterpret_cast<uintptr_t>(row) & 15u) == 0;
  if (vec) {
    ArgmaxOp<S> op{b, V / kPer, tid};
    stream_row(reinterpret_cast<const u32x4*>(row), V / kPer, tid, op);
    b = op.b;
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
// Kernel 1, one workgroup per (sequence, node) row, one pass over the row in
// base 2: with u = x * log2(e) / temperature, every thread keeps a
// reference m (a value of u it has seen), z = sum 2^(u - m) and
// s = sum 2^(u - m) (u - m), over batches of two 16-byte chunks per thread
// (stream_row); the threads' states are merged with rescales (2^(m - m')
// when the reference moves to m').  Since e^(y - m ln 2) = 2^(u - m) for
// y = x / temperature, whatever the reference,
//   lse = (m + log2 z) ln 2,   H = ln z - sum e^(y - m ln 2) (y - m ln 2) / z
//                                = (log2 z - s / z) ln 2.
// Kernel 2, one wavefront per sequence: each child gathers its token's logit
// from the parent's row and tests p = e^(x / temperature - lse) against the
// threshold; the path is then chosen as in greedy acceptance.
// Measured on 16 x 64 rows of 32000 bf16 (graph replay): 17.1 us for both
// launches; 14.5 us for kernel 1 alone, 12.4 us for kernel 1 with nothing
// but its loads (65.5 MB: 5.3 TB/s with the launch and first-load latency
// included), so the row pass is close to its read floor and the second
// launch (two dependent round trips) costs 2.7 us.
// ---------------------------------------------------------------------------
struct Lse {
  float m, z, s;  // base-2 running max, sum of 2^(u - m), sum of 2^(u - m) (u - m)
};

// Merge b into a (both over disjoint sets of values).
__device__ __forceinline__ void merge_lse(Lse& a, const Lse& b) {
  if (b.z == 0.f) return;
  if (a.z == 0.f) {
    a = b;
    return;
  }
  if (b.m > a.m) {
    const float d = a.m - b.m, f = __builtin_amdgcn_exp2f(d);
    a.s = f * (a.s + d * a.z) + b.s;
    a.z = f * a.z + b.z;
    a.m = b.m;
  } else {
    const float d = b.m - a.m, f = __builtin_amdgcn_exp2f(d);
    a.s += f * (b.s + d * b.z);
    a.z += f * b.z;
  }
}

// Adds 2^(u - m) and its weighted term for one value u = x * c, relative to
// the batch max m.  Values far below m (and -inf) add nothing: the
// difference is clamped where 2^d is already 0 in fp32, which also keeps
// 0 * (-inf) out of s.
__device__ __forceinline__ void add_term(Lse& t, float x, float c) {
  const float d = fmaxf(fmaf(x, c, -t.m), -256.f);
  const float e = __builtin_amdgcn_exp2f(d);
  t.z += e;
  t.s = fmaf(e, d, t.s);
}

// Entropy consumer of stream_row.  Each thread sums its terms against a
// reference it fixes once: the max of its first batch holding a finite
// value (c > 0, so the max of x gives the max of u = x c).  A batch then
// adds its sums to the running ones with no max pass and no rescale; the
// identities for lse and H hold for any reference.  A batch whose sum
// reaches 2^32 (a value 32 or more above the reference in base 2, or +inf)
// is redone against its own max and merged with a rescale, which moves the
// reference up; so terms stay below 2^32 and the reference within 32 of
// the values that carry the mass.  A batch with no finite max adds nothing
// (as a batch whose max is +inf gives no finite term).
template <typename S>
struct EntropyOp {
  static constexpr int kBatch = 2;
  static constexpr int kThreads = kEntThreads;
  Lse a;
  float c;
  int nchunks, tid;
  __device__ __forceinline__ float batch_max(const u32x4 (&x)[kBatch], int i0) const {
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if ((i0 + u) * kThreads + tid < nchunks) {
#pragma unroll
        for (int w = 0; w < 4; ++w)
          mx = sizeof(S) == 2 ? fmaxf(mx, fmaxf(bf16_lo(x[u][w]), bf16_hi(x[u][w])))
                              : fmaxf(mx, __uint_as_float(x[u][w]));
      }
    }
    return mx;
  }
  __device__ __forceinline__ void terms(Lse& t, const u32x4 (&x)[kBatch], int i0) const {
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if ((i0 + u) * kThreads + tid < nchunks) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          if (sizeof(S) == 2) {
            add_term(t, bf16_lo(x[u][w]), c);
            add_term(t, bf16_hi(x[u][w]), c);
          } else {
            add_term(t, __uint_as_float(x[u][w]), c);
          }
        }
      }
    }
  }
  __device__ __forceinline__ void batch(const u32x4 (&x)[kBatch], int i0) {
    if (a.z == 0.f) {  // no reference yet
      const float mx = batch_max(x, i0);
      if (!(fabsf(mx) < INFINITY)) return;
      a.m = mx * c;
    }
    Lse t{a.m, 0.f, 0.f};
    terms(t, x, i0);
    if (t.z < 0x1p32f) {
      a.z += t.z;
      a.s += t.s;
      return;
    }
    const float mx = batch_max(x, i0);
    Lse r{mx * c, 0.f, 0.f};
    terms(r, x, i0);
    merge_lse(a, r);
  }
};

template <typename S>
__global__ __launch_bounds__(kEntThreads) void row_entropy_kernel(const S* __restrict__ logits,
                                                                  int V, float c,
                                                                  float2* __restrict__ stats) {
  __shared__ Lse s_l[kEntThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const S* row = logits + (size_t)blockIdx.x * V;
  Lse a{-INFINITY, 0.f, 0.f};
  constexpr int kPer = 16 / sizeof(S);
  const bool vec = (V % kPer) == 0 && (reinterpret_cast<uintptr_t>(row) & 15u) == 0;
  if (vec) {
    EntropyOp<S> op{a, c, V / kPer, tid};
    stream_row(reinterpret_cast<const u32x4*>(row), V / kPer, tid, op);
    a = op.a;
  } else {
    for (int i = tid; i < V; i += kEntThreads) {
      const float x = ld(row, i);
      if (x == -INFINITY) continue;
      Lse t{x * c, 0.f, 0.f};
      add_term(t, x, c);
      merge_lse(a, t);
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
    for (int w = 1; w < kEntThreads / 64; ++w) merge_lse(r, s_l[w]);
    constexpr float kLn2 = 0.69314718055994531f;
    const float l2z = __log2f(r.z);
    stats[blockIdx.x] = r.z > 0.f ? float2{(r.m + l2z) * kLn2, (l2z - r.s / r.z) * kLn2}
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
  const float c = 1.4426950408889634f / temperature;  // log2(e) / temperature
  float2* stats = reinterpret_cast<float2*>(node_stats);
  if (dtype == TA_BF16) {
    hipLaunchKernelGGL(row_entropy_kernel<uint16_t>, dim3((unsigned)(B * T)), dim3(kEntThreads),
                       0, stream, static_cast<const uint16_t*>(logits), V, c, stats);
    hipLaunchKernelGGL(typical_accept_kernel<uint16_t>, dim3((unsigned)B), dim3(64), 0, stream,
                       static_cast<const uint16_t*>(logits), V, T, inv_temp, epsilon, delta,
                       stats, cand_tokens, tree_parent, node_ok, accept_len, accept_path);
  } else {
    hipLaunchKernelGGL(row_entropy_kernel<float>, dim3((unsigned)(B * T)), dim3(kEntThreads), 0,
                       stream, static_cast<const float*>(logits), V, c, stats);
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
