// Greedy acceptance, KV commit, RoPE table and workspace fill kernels.
#include <math.h>

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
  const int b = blockIdx.x;
  const int i = threadIdx.x;
  const bool in_tree = i < T;
  const size_t row = (size_t)b * T;
  const int par = in_tree ? tree_parent[row + i] : kPadParent;
  const bool linked = (i == 0) ? (par == -1) : (par >= 0 && par < i);
  const bool ok = linked && (i == 0 || cand_tokens[row + i] == node_argmax[row + par]);
  const uint64_t M = __ballot(ok);

  uint64_t anc = linked ? (1ull << i) : 0ull;
  int up = (linked && i > 0) ? par : i;  // the root (and unlinked lanes) point at themselves
#pragma unroll
  for (int r = 0; r < 6; ++r) {          // 2^6 - 1 >= 63 levels
    const uint64_t a_up = __shfl(anc, up);
    const int up_up = __shfl(up, up);
    anc |= a_up;
    up = up_up;
  }
  const bool rooted = (anc & 1ull) != 0ull;
  const bool accepted = linked && rooted && ((anc & ~M) == 0ull);
  const int depth = __popcll(anc) - 1;
  int key = accepted ? (depth << 6) | (63 - i) : -1;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) key = max(key, __shfl_xor(key, off));
  const int end = 63 - (key & 63);       // key >= 0: the root is always accepted
  const uint64_t anc_end = __shfl(anc, end);
  const int len = __popcll(anc_end);
  if (in_tree) {
    if ((anc_end >> i) & 1ull) accept_path[row + depth] = i;
    if (i >= len) accept_path[row + i] = -1;
  }
  if (i == 0) accept_len[b] = len;
}

// ---------------------------------------------------------------------------
// KV commit (mlc-llm issue #2319 KV-cache update; vLLM issue #1171 block
// tables): one workgroup per (path slot i, sequence b).  Slot i < accept_len
// takes node n = accept_path[i] to position p = ctx_len + i: page
// block_table[p / 16], row p % 16.  K is rotated at p with the fixed-order
// fp32 arithmetic and rounded to the pool type; V is copied bit for bit.
// ---------------------------------------------------------------------------
template <typename S>
__global__ __launch_bounds__(256) void commit_kernel(CommitParams p) {
  const int i = blockIdx.x, b = blockIdx.y;
  const int len = p.accept_len[b];
  if (i >= len || len > p.T) return;
  const int n = p.accept_path[(size_t)b * p.T + i];
  if (n < 0 || n >= p.T) return;
  const int pos = clampi(p.ctx_lens[b], 0, p.max_ctx) + i;
  const int lb = pos / kPage;
  if (lb >= p.max_blocks || pos >= p.rope_max_pos) return;
  const int blk = p.block_table[(size_t)b * p.max_blocks + lb];
  if (blk < 0 || blk >= p.num_blocks) return;
  const int slot = pos % kPage;
  const int D = p.D, half = p.D / 2;
  const S* kn = static_cast<const S*>(p.k_new) + ((size_t)b * p.T + n) * p.Hkv * D;
  const S* vn = static_cast<const S*>(p.v_new) + ((size_t)b * p.T + n) * p.Hkv * D;
  S* pages = static_cast<S*>(p.kv_pages);
  const float* cs = p.rope + (size_t)pos * D;
  for (int idx = threadIdx.x; idx < p.Hkv * half; idx += blockDim.x) {
    const int hk = idx / half, k = idx % half;
    float y1, y2;
    rope_pair_exact(ld(kn, (size_t)hk * D + k), ld(kn, (size_t)hk * D + k + half), cs[2 * k],
                    cs[2 * k + 1], y1, y2);
    S* krow = pages + page_row(blk, 0, hk, slot, p.Hkv, D);
    st(krow, k, y1);
    st(krow, k + half, y2);
  }
  for (int idx = threadIdx.x; idx < p.Hkv * D; idx += blockDim.x) {
    const int hk = idx / D, k = idx % D;
    pages[page_row(blk, 1, hk, slot, p.Hkv, D) + k] = vn[(size_t)hk * D + k];
  }
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
