// Greedy acceptance, KV commit, RoPE table and workspace fill kernels.
#include <math.h>

#include "accept.h"
#include "launch.h"

namespace ta {
namespace {

// ---------------------------------------------------------------------------
// Greedy acceptance (LMDeploy PR #1231 evaluate_posterior at LM-head
// temperature 0): one wavefront per sequence, lane i = tree node i.
//   ok_i     = edge parent(i) -> i matches (the root is always ok)
//   M        = ballot(ok)
//   anc_i    = ancestor-or-self set of i, by pointer doubling over the lanes
//   accepted = every node on the root path is ok:  (anc_i & ~M) == 0
//   end      = argmax over accepted nodes of (depth, -index)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void accept_kernel(const int32_t* __restrict__ node_argmax,
                                                    const int32_t* __restrict__ cand_tokens,
                                                    const int32_t* __restrict__ tree_parent,
                                                    int32_t* __restrict__ accept_len,
                                                    int32_t* __restrict__ accept_path, int T) {
  const int b = blockIdx.x, i = threadIdx.x;
  const Acceptance a = accept_wave(node_argmax, cand_tokens, tree_parent, b, T, i);
  write_acceptance(a, accept_len, accept_path, b, T, i);
}

// ---------------------------------------------------------------------------
// KV commit (mlc-llm issue #2319 KV-cache update; vLLM issue #1171 block
// tables): slot i < accept_len takes node n = accept_path[i] to position
// p = ctx_len + i: page block_table[p / 16], row p % 16.  K is rotated at p
// with the fixed-order fp32 arithmetic and rounded to the pool type; V is
// copied bit for bit.  The 16-byte row helpers below serve the commit
// kernels further down.
// ---------------------------------------------------------------------------
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void load8(const uint16_t* p, float (&x)[8]) {
  const u32x4 u = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[2 * j] = bf16_to_f32((uint16_t)(u[j] & 0xFFFFu));
    x[2 * j + 1] = bf16_to_f32((uint16_t)(u[j] >> 16));
  }
}
__device__ __forceinline__ void load8(const float* p, float (&x)[8]) {
  const f32x4 a = reinterpret_cast<const f32x4*>(p)[0], b = reinterpret_cast<const f32x4*>(p)[1];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[j] = a[j];
    x[4 + j] = b[j];
  }
}
__device__ __forceinline__ void store8(uint16_t* p, const float (&y)[8]) {
  u32x4 u;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    u[j] = (uint32_t)f32_to_bf16_rne(y[2 * j]) | ((uint32_t)f32_to_bf16_rne(y[2 * j + 1]) << 16);
  *reinterpret_cast<u32x4*>(p) = u;
}
__device__ __forceinline__ void store8(float* p, const float (&y)[8]) {
  reinterpret_cast<f32x4*>(p)[0] = f32x4{y[0], y[1], y[2], y[3]};
  reinterpret_cast<f32x4*>(p)[1] = f32x4{y[4], y[5], y[6], y[7]};
}

// ---------------------------------------------------------------------------
// KV commit, one workgroup per (sequence b, group of kCommitHeads KV heads).
// The workgroup writes every accepted row of its heads: slot i < accept_len
// takes path node n_i to position p = ctx_len + i, page
// block_table[b][p / 16], row p % 16.  The rows of one head split into
// 16-byte tasks: d/16 K tasks (8 RoPE pairs each: x_k and x_{k+d/2}, rotated
// at p with the fixed-order fp32 arithmetic and rounded to the pool type) and
// d*sizeof(S)/16 V tasks (bit copies).  Thread t takes tasks t, t + 256, ...
// of the flattened (slot, head, task) list; with two heads of head_dim 128 in
// bf16 a slot holds 48 tasks, so a path of up to five rows is one task per
// thread.  Every load of a task (table entry, k_new or v_new row, (cos, sin)
// row) is issued before any is used, and the stores are skipped when the
// page id is out of range, so a task costs about one memory round trip.
// ---------------------------------------------------------------------------
constexpr int kCommitHeads = 2;
constexpr int kCommitThreads = 256;

// The accepted node at path slot i, given the path as a node bitmask: the
// nodes of a root path have increasing indices (every parent precedes its
// children), so the node at depth i is the i-th lowest set bit.
__device__ __forceinline__ int nth_set_bit(uint64_t m, int i) {
  for (int k = 0; k < i; ++k) m &= m - 1;
  return m ? __builtin_ctzll(m) : -1;
}

template <typename S>
__device__ __forceinline__ void commit_task(const CommitParams& p, int b, int ctx, int i, int n,
                                            int hk, int r, int groups) {
  const int D = p.D, half = D / 2;
  const int pos = ctx + i;
  const int lb = pos / kPage;
  const int blk = p.block_table[(size_t)b * p.max_blocks + min(lb, p.max_blocks - 1)];
  const bool ok_pos = lb < p.max_blocks && pos < p.rope_max_pos;
  S* pages = static_cast<S*>(p.kv_pages);
  const size_t row = ((size_t)b * p.T + n) * p.Hkv + hk;
  if (r < groups) {  // K: pairs k0 .. k0+7 and their partners
    const int k0 = r * 8;
    const S* kn = static_cast<const S*>(p.k_new) + row * D;
    const float* cs = p.rope + (size_t)min(pos, p.rope_max_pos - 1) * D + 2 * k0;
    float x1[8], x2[8], cc[8], ss[8], y1[8], y2[8];
    load8(kn + k0, x1);
    load8(kn + k0 + half, x2);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 t = reinterpret_cast<const f32x4*>(cs)[j];
      cc[2 * j] = t[0];
      ss[2 * j] = t[1];
      cc[2 * j + 1] = t[2];
      ss[2 * j + 1] = t[3];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) rope_pair_exact(x1[j], x2[j], cc[j], ss[j], y1[j], y2[j]);
    if (ok_pos && blk >= 0 && blk < p.num_blocks) {
      S* krow = pages + page_row(blk, 0, hk, pos % kPage, p.Hkv, D);
      store8(krow + k0, y1);
      store8(krow + k0 + half, y2);
    }
  } else {  // V: one 16-byte chunk, copied bit for bit
    constexpr int kPer16 = 16 / sizeof(S);
    const int off = (r - groups) * kPer16;
    const u32x4 v = *reinterpret_cast<const u32x4*>(static_cast<const S*>(p.v_new) + row * D + off);
    if (ok_pos && blk >= 0 && blk < p.num_blocks)
      *reinterpret_cast<u32x4*>(pages + page_row(blk, 1, hk, pos % kPage, p.Hkv, D) + off) = v;
  }
}

// The rows of path slots [0, len) for this workgroup's heads.  node_of(i)
// gives the node at slot i (-1 or >= T: nothing is written for that slot).
template <typename S, typename NodeOf>
__device__ __forceinline__ void commit_heads(const CommitParams& p, int b, int ctx, int len,
                                             NodeOf node_of) {
  const int h0 = blockIdx.x * kCommitHeads;
  const int nh = min(kCommitHeads, p.Hkv - h0);
  const int groups = p.D / 16;
  const int per_head = groups + p.D * (int)sizeof(S) / 16;
  const int per_slot = nh * per_head;
  for (int t = threadIdx.x; t < len * per_slot; t += kCommitThreads) {
    const int i = t / per_slot, rem = t - i * per_slot;
    const int hh = rem / per_head, r = rem - hh * per_head;
    const int n = node_of(i);
    if (n < 0 || n >= p.T) continue;
    commit_task<S>(p, b, ctx, i, n, h0 + hh, r, groups);
  }
}

template <typename S>
__global__ __launch_bounds__(kCommitThreads) void commit_kernel(CommitParams p) {
  const int b = blockIdx.y;
  const int len = p.accept_len[b];
  const int ctx = clampi(p.ctx_lens[b], 0, p.max_ctx);
  if (len <= 0 || len > p.T) return;  // uniform
  const int32_t* path = p.accept_path + (size_t)b * p.T;
  commit_heads<S>(p, b, ctx, len, [&](int i) { return path[i]; });
}

// Acceptance and commit in one launch: one workgroup per (sequence, group of
// KV heads).  Every wavefront evaluates the sequence's tree (each gets the
// same answer; no LDS or barrier is needed), the first workgroup of each
// sequence publishes accept_len / accept_path, and then every workgroup
// writes the accepted rows of its heads.  Same results as accept_kernel
// followed by commit_kernel.
template <typename S>
__global__ __launch_bounds__(kCommitThreads) void accept_commit_kernel(
    CommitParams p, const int32_t* __restrict__ node_argmax,
    const int32_t* __restrict__ cand_tokens, const int32_t* __restrict__ tree_parent,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ accept_path) {
  const int b = blockIdx.y, lane = threadIdx.x & 63;
  // One round trip: the tree rows and ctx_len.
  const AcceptRows rows = load_accept_rows(node_argmax, cand_tokens, tree_parent, b, p.T, lane);
  const int ctx = clampi(p.ctx_lens[b], 0, p.max_ctx);
  const Acceptance a = accept_rows(rows, p.T, lane);
  if (blockIdx.x == 0 && threadIdx.x < 64) write_acceptance(a, accept_len, accept_path, b, p.T, lane);
  commit_heads<S>(p, b, ctx, a.len, [&](int i) { return nth_set_bit(a.path, i); });
}

// (cos, sin) of pos * base^(-2k/d): angle in fp64, one rounding to fp32.
__global__ void rope_table_kernel(int head_dim, double base, int max_pos, float* table) {
  const int half = head_dim / 2;
  const size_t n = (size_t)max_pos * half;
  for (size_t idx = blockIdx.x * (size_t)blockDim.x + threadIdx.x; idx < n;
       idx += (size_t)gridDim.x * blockDim.x) {
    const int pos = (int)(idx / half), k = (int)(idx % half);
    const double inv = pow(base, -(2.0 * k) / (double)head_dim);
    const double ang = (double)pos * inv;
    table[2 * idx] = (float)cos(ang);
    table[2 * idx + 1] = (float)sin(ang);
  }
}

__global__ void fill_zero_kernel(uint32_t* p, size_t words) {
  for (size_t idx = blockIdx.x * (size_t)blockDim.x + threadIdx.x; idx < words;
       idx += (size_t)gridDim.x * blockDim.x)
    p[idx] = 0u;
}

}  // namespace

hipError_t launch_accept(const int32_t* node_argmax, const int32_t* cand_tokens,
                         const int32_t* tree_parent, int32_t* accept_len, int32_t* accept_path,
                         int B, int T, hipStream_t stream) {
  hipLaunchKernelGGL(accept_kernel, dim3(B), dim3(64), 0, stream, node_argmax, cand_tokens,
                     tree_parent, accept_len, accept_path, T);
  return hipGetLastError();
}

hipError_t launch_commit(const CommitParams& p, int dtype, hipStream_t stream) {
  dim3 grid((p.Hkv + kCommitHeads - 1) / kCommitHeads, p.B);
  if (dtype == TA_BF16)
    hipLaunchKernelGGL(commit_kernel<uint16_t>, grid, dim3(kCommitThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(commit_kernel<float>, grid, dim3(kCommitThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_accept_commit(const CommitParams& p, const int32_t* node_argmax,
                                const int32_t* cand_tokens, const int32_t* tree_parent,
                                int32_t* accept_len, int32_t* accept_path, int dtype,
                                hipStream_t stream) {
  dim3 grid((p.Hkv + kCommitHeads - 1) / kCommitHeads, p.B);
  if (dtype == TA_BF16)
    hipLaunchKernelGGL(accept_commit_kernel<uint16_t>, grid, dim3(kCommitThreads), 0, stream, p, node_argmax,
                       cand_tokens, tree_parent, accept_len, accept_path);
  else
    hipLaunchKernelGGL(accept_commit_kernel<float>, grid, dim3(kCommitThreads), 0, stream, p, node_argmax,
                       cand_tokens, tree_parent, accept_len, accept_path);
  return hipGetLastError();
}

hipError_t launch_rope_table(int head_dim, float base, int max_pos, float* table,
                             hipStream_t stream) {
  const size_t n = (size_t)max_pos * (head_dim / 2);
  const int blocks = (int)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
  hipLaunchKernelGGL(rope_table_kernel, dim3(blocks > 0 ? blocks : 1), dim3(256), 0, stream,
                     head_dim, (double)base, max_pos, table);
  return hipGetLastError();
}

hipError_t launch_fill_zero(void* ptr, size_t bytes, hipStream_t stream) {
  const size_t words = bytes / 4;
  if (words == 0) return hipSuccess;
  const int blocks = (int)((words + 255) / 256 < 4096 ? (words + 255) / 256 : 4096);
  hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks), dim3(256), 0, stream,
                     static_cast<uint32_t*>(ptr), words);
  return hipGetLastError();
}

}  // namespace ta
