// Host-side launchers of the kernels behind the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace ta {

// One wavefront per (node, head, sequence), any head_dim in {64, 128},
// bf16 or fp32.  Plain and slow; no workspace.
hipError_t launch_verify_simple(const VerifyParams& p, int dtype, hipStream_t stream);

// MFMA kernels for bf16, head_dim 128: one workgroup per work item, or the
// persistent kernel (one workgroup per CU, work items taken from the
// counters at p.ws_ctr).  When a context can take more than one split, the
// split partials are merged by launch_split_combine afterwards.
hipError_t launch_verify_mfma(const VerifyParams& p, hipStream_t stream);
// One-node trees (T = 1): one workgroup per (sequence, head), no workspace.
hipError_t launch_verify_decode(const VerifyParams& p, hipStream_t stream);
hipError_t launch_verify_stream(const VerifyParams& p, hipStream_t stream);
hipError_t launch_split_combine(const VerifyParams& p, hipStream_t stream);

hipError_t launch_accept(const int32_t* node_argmax, const int32_t* cand_tokens,
                         const int32_t* tree_parent, int32_t* accept_len,
                         int32_t* accept_path, int B, int T, hipStream_t stream);

struct CommitParams {
  const void* k_new;
  const void* v_new;
  const int32_t* accept_len;
  const int32_t* accept_path;
  void* kv_pages;
  const int32_t* block_table;
  const int32_t* ctx_lens;
  const float* rope;
  int B, T, Hkv, D, max_blocks, num_blocks, max_ctx, rope_max_pos;
};
hipError_t launch_commit(const CommitParams& p, int dtype, hipStream_t stream);

// Greedy acceptance and KV commit in one launch (same results as
// launch_accept followed by launch_commit on its outputs).
hipError_t launch_accept_commit(const CommitParams& p, const int32_t* node_argmax,
                                const int32_t* cand_tokens, const int32_t* tree_parent,
                                int32_t* accept_len, int32_t* accept_path, int dtype,
                                hipStream_t stream);

// node_argmax[r] = argmax over V of row r of logits (rows x V, dtype TA_BF16
// or TA_F32), smallest token among equal maxima.
hipError_t launch_vocab_argmax(const void* logits, int dtype, int V, int rows, int32_t* out,
                               hipStream_t stream);
// Typical acceptance: per-node (log-sum-exp of logits / temperature,
// entropy) into node_stats [rows][2], then the threshold test and the path.
hipError_t launch_typical_accept(const void* logits, int dtype, int V, int B, int T,
                                 float temperature, float epsilon, float delta,
                                 const int32_t* cand_tokens, const int32_t* tree_parent,
                                 float* node_stats, int32_t* node_ok, int32_t* accept_len,
                                 int32_t* accept_path, hipStream_t stream);

// Candidate tree from the Medusa heads: the node table of a validated
// "medusa choices" list (root 0, then paths by length, then lexicographic),
// passed by value.  rank[n] = last rank of node n's path (its token is the
// rank-th best of head depth[n] - 1).
constexpr int kMaxTopK = 16;
struct CandTree {
  int32_t n_nodes;          // root + choices, <= kMaxTree
  int8_t parent[kMaxTree];
  int8_t depth[kMaxTree];
  int8_t rank[kMaxTree];
};
hipError_t launch_candidates(const void* head_logits, int dtype, int V, int n_heads, int topk,
                             const CandTree& tree, const int32_t* root_token, int32_t* cand,
                             int32_t* parent, int32_t* depth, int B, int T, hipStream_t stream);

hipError_t launch_rope_table(int head_dim, float base, int max_pos, float* table,
                             hipStream_t stream);

hipError_t launch_fill_zero(void* ptr, size_t bytes, hipStream_t stream);

// Read-bandwidth probe: streams bytes (a multiple of 16 is read; the rest is
// ignored) from src with 16-byte non-temporal loads and XORs them into
// *sink.  Measurement only.
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int n_cu,
                              hipStream_t stream);

}  // namespace ta
