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
// tables): one workgroup per (path slot i, sequence b).  Slot i < accept_len
// takes node n = accept_path[i] to position p = ctx_len + i: page
// block_table[p / 16], row p % 16.  K is rotated at p with the fixed-order
// fp32 arithmetic and rounded to the pool type; V is copied bit for bit.
// Each thread handles 8 consecutive RoPE pairs with 16-byte loads, all issued
// before any use, so a slot costs about one memory round trip.
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

// Where path slot i of sequence b goes: position ctx_len + i and the page
// holding it (block_table[b][pos / 16], row pos % 16).  Only ctx_len and the
// table are read, so callers look the page up while the acceptance is still
// being decided; the table index is clamped and the id is tested only where
// the rows are stored (commit_row), so nothing here waits on the lookup.
struct Dest {
  int pos, blk;
  bool in_table;  // pos has a table column and a RoPE row
};
__device__ __forceinline__ Dest commit_dest(const CommitParams& p, int b, int i, int ctx_raw) {
  const int pos = clampi(ctx_raw, 0, p.max_ctx) + i;
  const int lb = pos / kPage;
  const int blk = p.block_table[(size_t)b * p.max_blocks + min(lb, p.max_blocks - 1)];
  return Dest{pos, blk, lb < p.max_blocks && pos < p.rope_max_pos};
}

// Path slot at position d.pos holds node n: write its K/V rows there.  Every
// row load (k_new, v_new, the (cos, sin) row) is issued before the page id
// is tested, so the table lookup and the row loads share a round trip; the
// stores are skipped when the page is out of range.
template <typename S>
__device__ __forceinline__ void commit_row(const CommitParams& p, int b, int n, const Dest& d) {
  const bool ok = d.in_table && d.blk >= 0 && d.blk < p.num_blocks;
  const int slot = d.pos % kPage;
  const int D = p.D, half = p.D / 2, groups = half / 8;
  const S* kn = static_cast<const S*>(p.k_new) + ((size_t)b * p.T + n) * p.Hkv * D;
  const S* vn = static_cast<const S*>(p.v_new) + ((size_t)b * p.T + n) * p.Hkv * D;
  S* pages = static_cast<S*>(p.kv_pages);
  const float* cs = p.rope + (size_t)min(d.pos, p.rope_max_pos - 1) * D;
  for (int c = threadIdx.x; c < p.Hkv * groups; c += blockDim.x) {
    const int hk = c / groups, k0 = (c % groups) * 8;
    float x1[8], x2[8], cc[8], ss[8], y1[8], y2[8];
    load8(kn + (size_t)hk * D + k0, x1);
    load8(kn + (size_t)hk * D + k0 + half, x2);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 t = reinterpret_cast<const f32x4*>(cs + 2 * k0)[j];
      cc[2 * j] = t[0];
      ss[2 * j] = t[1];
      cc[2 * j + 1] = t[2];
      ss[2 * j + 1] = t[3];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) rope_pair_exact(x1[j], x2[j], cc[j], ss[j], y1[j], y2[j]);
    if (ok) {
      S* krow = pages + page_row(d.blk, 0, hk, slot, p.Hkv, D);
      store8(krow + k0, y1);
      store8(krow + k0 + half, y2);
    }
  }
  constexpr int kPer16 = 16 / sizeof(S);
  const int row_chunks = D / kPer16;
  for (int c = threadIdx.x; c < p.Hkv * row_chunks; c += blockDim.x) {
    const int hk = c / row_chunks, off = (c % row_chunks) * kPer16;
    const u32x4 v = *reinterpret_cast<const u32x4*>(vn + (size_t)hk * D + off);
    if (ok) *reinterpret_cast<u32x4*>(pages + page_row(d.blk, 1, hk, slot, p.Hkv, D) + off) = v;
  }
}

template <typename S>
__global__ __launch_bounds__(256) void commit_kernel(CommitParams p) {
  const int i = blockIdx.x, b = blockIdx.y;
  const int len = p.accept_len[b];
  const int n = p.accept_path[(size_t)b * p.T + i];
  const Dest d = commit_dest(p, b, i, p.ctx_lens[b]);
  if (i >= len || len > p.T || n < 0 || n >= p.T) return;
  commit_row<S>(p, b, n, d);
}

// Acceptance and commit in one launch: one workgroup per (path slot i,
// sequence b).  Every wavefront evaluates the sequence's tree (each gets the
// same answer; the tree rows are L2 hits after the first), so no LDS or
// barrier is needed; the slot's page is looked up meanwhile.  The workgroup
// of slot 0 publishes accept_len/accept_path, and each workgroup whose slot
// is on the accepted path writes that row.  Same results as accept_kernel
// followed by commit_kernel.
template <typename S>
__global__ __launch_bounds__(256) void accept_commit_kernel(CommitParams p,
                                                            const int32_t* __restrict__ node_argmax,
                                                            const int32_t* __restrict__ cand_tokens,
                                                            const int32_t* __restrict__ tree_parent,
                                                            int32_t* __restrict__ accept_len,
                                                            int32_t* __restrict__ accept_path) {
  const int i = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
  // Round trip 1: the tree rows and ctx_len; then the slot's table entry,
  // issued before the rows are used.
  const AcceptRows rows = load_accept_rows(node_argmax, cand_tokens, tree_parent, b, p.T, lane);
  const int ctx_raw = p.ctx_lens[b];
  __builtin_amdgcn_sched_barrier(0);
  const Dest d = commit_dest(p, b, i, ctx_raw);
  __builtin_amdgcn_sched_barrier(0);
  const Acceptance a = accept_rows(rows, p.T, lane);
  if (i == 0 && tid < 64) write_acceptance(a, accept_len, accept_path, b, p.T, lane);
  const uint64_t at_i = __ballot(a.in_tree && ((a.path >> lane) & 1ull) && a.depth == i);
  if (at_i != 0ull) commit_row<S>(p, b, __builtin_ctzll(at_i), d);
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
  dim3 grid(p.T, p.B);
  if (dtype == TA_BF16)
    hipLaunchKernelGGL(commit_kernel<uint16_t>, grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(commit_kernel<float>, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_accept_commit(const CommitParams& p, const int32_t* node_argmax,
                                const int32_t* cand_tokens, const int32_t* tree_parent,
                                int32_t* accept_len, int32_t* accept_path, int dtype,
                                hipStream_t stream) {
  dim3 grid(p.T, p.B);
  if (dtype == TA_BF16)
    hipLaunchKernelGGL(accept_commit_kernel<uint16_t>, grid, dim3(256), 0, stream, p, node_argmax,
                       cand_tokens, tree_parent, accept_len, accept_path);
  else
    hipLaunchKernelGGL(accept_commit_kernel<float>, grid, dim3(256), 0, stream, p, node_argmax,
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
