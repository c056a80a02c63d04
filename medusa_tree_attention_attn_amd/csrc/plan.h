// Host-side split plan and workspace layout of tree_attn_verify.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "tree_attn.h"

namespace ta {

// Split-KV sizing of the MFMA kernels.  A (sequence, head) whose context fits
// in one split is one work item and writes `out` directly; longer contexts
// are cut into splits of `chunk` tokens (a multiple of the 64-token tile)
// whose partials a second kernel merges.  Each work item pays a prologue
// (tree rows, q and tree k/v rows, RoPE rows, first tile) before it streams,
// and each split costs a partial write and read plus a merge launch, so the
// plan splits a context only while the work items still fit the CUs'
// resident slots (two per CU, kTargetItems): (sequence, head) pairs times
// splits <= kTargetItems, never below kMinChunk tokens (batch 1, 32 heads,
// 1024 tokens: 17.0 us with 128-token splits, 17.8 with 256, 19.7 with
// 384).  Overshooting the slots makes a second round of workgroups, which
// costs more than the balance it buys (13B-shaped, 320 pairs of 4096
// tokens: 136 us unsplit against 170 us with two splits).
constexpr int kTargetItems = 512;
constexpr int kMinChunk = 128;
constexpr int kTileTokens = 64;
constexpr int kMaxSplitTokens = 8192;   // the kernels keep a split's page ids in LDS

struct Plan {
  bool mfma;         // MFMA kernels (bf16, head_dim 128) or the plain kernel
  bool decode;       // the one-node (T = 1) kernel: whole contexts, no workspace
  bool stream;       // persistent MFMA kernel may run (workspace has its counters)
  int chunk;         // tokens per split
  int splits;        // max splits per (sequence, head)
  size_t off_ctr;    // uint32 [2] work counters of the persistent kernel
  size_t off_ml;     // float2 [B][H][splits][T] (running max, running sum)
  size_t off_o;      // float [B][H][splits][T][128] un-normalised partial O
  size_t bytes;      // total workspace
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Persistent kernel or one workgroup per work item.  The grid kernel (two
// co-resident workgroups per CU, the hardware dispatching later workgroups
// as slots free up, longest items first) measured faster on every shape
// tried, many work items per CU included (stress batch 64: 683 against 734
// us; batch 128 x 32 heads: 449 against 619 us; batch 32: 107 against 152
// us), so the persistent kernel runs only when the caller forces it.
inline bool use_stream_kernel(const tree_attn_desc& d) {
  return (d.flags & TA_FLAG_PERSISTENT_KERNEL) && !(d.flags & TA_FLAG_GRID_KERNEL);
}

// One-node trees (t_max == 1): the decode kernel below this context bound,
// the grid kernel (whose small-tree path streams the context on the vector
// ALU) above it.  Measured, batch 64: contexts 128..512 decode kernel 73.5
// against 77.9 us; 128..8192 624 against 637 us for the grid kernel; batch
// 256, contexts 128..2048: 706 against 746 us.
constexpr int kDecodeMaxCtx = 1024;

inline Plan make_plan(const tree_attn_desc& d) {
  Plan p{};
  p.mfma = d.dtype == TA_BF16 && d.head_dim == 128 && !(d.flags & TA_FLAG_SIMPLE_KERNEL);
  const bool forced = d.flags & (TA_FLAG_GRID_KERNEL | TA_FLAG_PERSISTENT_KERNEL);
  p.decode = p.mfma && d.t_max == 1 &&
             ((d.flags & TA_FLAG_DECODE_KERNEL) || (!forced && d.max_ctx_len <= kDecodeMaxCtx));
  p.stream = p.mfma && !p.decode;
  const int max_ctx = d.max_ctx_len > 0 ? d.max_ctx_len : 1;
  if (p.decode) {  // one workgroup streams a whole context; nothing to merge
    p.chunk = max_ctx;
    p.splits = 1;
    return p;
  }
  int chunk;
  if (d.split_tokens > 0) {
    chunk = d.split_tokens;
  } else {
    const long long bh = (long long)d.batch * d.num_heads;
    const long long want = kTargetItems / bh;  // splits per pair that fit the slots
    const int splits = (int)(want < 1 ? 1 : (want > max_ctx ? max_ctx : want));
    chunk = (max_ctx + splits - 1) / splits;
    if (chunk < kMinChunk) chunk = kMinChunk;
  }
  chunk = (chunk + kTileTokens - 1) / kTileTokens * kTileTokens;
  if (chunk > kMaxSplitTokens) chunk = kMaxSplitTokens;
  p.chunk = chunk;
  p.splits = (max_ctx + chunk - 1) / chunk;
  if (!p.mfma) return p;  // the plain kernel needs no workspace
  // The persistent kernel's work counters (kept zero between calls).
  p.off_ctr = 0;
  size_t off = 256;
  if (p.splits > 1) {
    const size_t bh = (size_t)d.batch * d.num_heads;
    const size_t rows = bh * (size_t)p.splits * d.t_max;
    p.off_ml = off;
    p.off_o = p.off_ml + align256(rows * 8);
    off = p.off_o + align256(rows * (size_t)d.head_dim * sizeof(float));
  }
  p.bytes = off;
  return p;
}

}  // namespace ta
