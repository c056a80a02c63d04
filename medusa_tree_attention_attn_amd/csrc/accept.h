// Acceptance of one sequence's tree by one wavefront (LMDeploy PR #1231
// evaluate_posterior), shared by the kernels that end in an acceptance.
// Lane i = tree node i:
//   ok_i     = edge parent(i) -> i passes its test (the root is always ok):
//              greedy token match, or the typical-acceptance threshold
//   M        = ballot(ok)
//   anc_i    = ancestor-or-self set of i, by pointer doubling over the lanes
//   accepted = every node on the root path is ok:  (anc_i & ~M) == 0
//   end      = argmax over accepted nodes of (depth, -index)
#pragma once

#include "common.h"

namespace ta {

struct Acceptance {
  int len;          // accepted nodes, root included
  uint64_t path;    // bit k set iff node k is on the accepted path
  int depth;        // this lane's depth in the tree (meaningful on linked lanes)
  bool in_tree;     // lane < T
};

// The accepted path of one tree, given each lane's (node's) parent and
// whether its edge passed the test (`edge_ok`; the root's is ignored).
// Called by one full wavefront; lane i = node i (lanes >= T: in_tree false,
// parent kPadParent).
__device__ __forceinline__ Acceptance select_path(int par, bool edge_ok, bool in_tree, int i) {
  const bool linked = (i == 0) ? (par == -1) : (par >= 0 && par < i);
  const bool ok = linked && (i == 0 || edge_ok);
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
  return Acceptance{(int)__popcll(anc_end), anc_end, depth, in_tree};
}

// Greedy acceptance: edge parent(i) -> i passes iff cand_tokens[i] equals
// the base model's greedy token after the parent.  Each lane loads its own
// node's row entries (the index clamped into the tree, so the three loads
// are unconditional and travel in one round trip) and takes the parent's
// greedy token from the parent's lane.  Split in two so that a caller can
// issue other loads between the row loads and their use.
struct AcceptRows {
  int par_raw, cand, greedy;
};
__device__ __forceinline__ AcceptRows load_accept_rows(const int32_t* __restrict__ node_argmax,
                                                       const int32_t* __restrict__ cand_tokens,
                                                       const int32_t* __restrict__ tree_parent,
                                                       int b, int T, int i) {
  const size_t ri = (size_t)b * T + min(i, T - 1);
  return AcceptRows{tree_parent[ri], cand_tokens[ri], node_argmax[ri]};
}
__device__ __forceinline__ Acceptance accept_rows(const AcceptRows& r, int T, int i) {
  const bool in_tree = i < T;
  const int par = in_tree ? r.par_raw : kPadParent;
  const bool linked = (i == 0) ? (par == -1) : (par >= 0 && par < i);
  const int after_parent = __shfl(r.greedy, linked && i > 0 ? par : 0);  // parent < i < T
  const bool match = linked && i > 0 && r.cand == after_parent;
  return select_path(par, match, in_tree, i);
}
__device__ __forceinline__ Acceptance accept_wave(const int32_t* __restrict__ node_argmax,
                                                  const int32_t* __restrict__ cand_tokens,
                                                  const int32_t* __restrict__ tree_parent, int b,
                                                  int T, int i) {
  return accept_rows(load_accept_rows(node_argmax, cand_tokens, tree_parent, b, T, i), T, i);
}

__device__ __forceinline__ void write_acceptance(const Acceptance& a, int32_t* accept_len,
                                                 int32_t* accept_path, int b, int T, int i) {
  const size_t row = (size_t)b * T;
  if (a.in_tree) {
    if ((a.path >> i) & 1ull) accept_path[row + a.depth] = i;
    if (i >= a.len) accept_path[row + i] = -1;
  }
  if (i == 0) accept_len[b] = a.len;
}


}  // namespace ta
