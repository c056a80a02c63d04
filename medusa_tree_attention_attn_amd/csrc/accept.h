// Acceptance of one sequence's tree by one wavefront (LMDeploy PR #1231
// evaluate_posterior), shared by the kernels that end in an acceptance.
// Lane i = tree node i:
//   ok_i     = edge parent(i) -> i passes its test (the root is always ok)
//   accepted = i is the root, or ok_i and parent(i) is accepted; found one
//              tree level per step, each step one ballot over the lanes
//              (a node is tested against the bitmask of the level above)
//   end      = argmax over accepted nodes of (depth, -index): the lowest
//              node of the deepest level found
//   path     = end and its ancestors, read from the parent lanes
#pragma once

#include "common.h"

namespace ta {

struct Acceptance {
  int len;          // accepted nodes, root included
  uint64_t path;    // bit k set iff node k is on the accepted path
  int depth;        // this lane's depth in the tree (meaningful on accepted lanes)
  bool in_tree;     // lane < T
};

// The accepted path of one tree, given each lane's (node's) parent and
// whether its edge passed the test (`edge_ok`; the root's is ignored).
// Called by one full wavefront; lane i = node i (lanes >= T: in_tree false,
// parent kPadParent).  A node is linked when it is the root with parent -1
// or its parent precedes it; nodes that are not linked, or hang below one,
// are never accepted, and a root that is not linked accepts nothing (len 0).
// Everything but the parent's index stays in registers: the level loop
// takes one ballot per tree level (at most 63) and the path walk one lane
// read per level, where pointer doubling took six rounds of LDS permutes.
__device__ __forceinline__ Acceptance select_path(int par, bool edge_ok, bool in_tree, int i) {
  const bool linked = (i == 0) ? (par == -1) : (par >= 0 && par < i);
  const bool ok = linked && (i == 0 || edge_ok);
  const int up = (linked && i > 0) ? par : 0;
  uint64_t found = __ballot(i == 0 && ok);  // accepted so far: the root, if linked
  uint64_t level = found;                   // the deepest level found
  int depth = 0, d = 0;
  while (level != 0ull) {  // uniform
    const bool add = ok && i > 0 && ((level >> up) & 1ull) != 0ull;
    const uint64_t next = __ballot(add);
    if (next == 0ull) break;
    ++d;
    if (add) depth = d;
    found |= next;
    level = next;
  }
  uint64_t path = 0ull;
  if (found != 0ull) {  // uniform
    int n = __builtin_ctzll(level);
    for (int k = d; k >= 0; --k) {
      path |= 1ull << n;
      n = __builtin_amdgcn_readlane(up, n);
    }
  }
  return Acceptance{(int)__popcll(path), path, depth, in_tree};
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
