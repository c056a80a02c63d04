// Host-side split plan and workspace layout of tree_attn_verify.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "tree_attn.h"

namespace ta {

// Context tokens per split work item of the MFMA kernel.  Long contexts are
// cut into chunks of this many tokens so that every CU gets similar work;
// a (sequence, head) whose context fits in one chunk writes `out` directly
// and touches no workspace.
constexpr int kChunkTokens = 512;

// Set once the MFMA kernel is in place; until then every call takes the
// plain kernel.
constexpr bool kMfmaKernelReady = false;

struct Plan {
  bool mfma;         // MFMA kernel (bf16, head_dim 128) or the plain kernel
  int chunk;         // tokens per split
  int splits;        // max splits per (sequence, head)
  size_t off_count;  // int32 [B][H] arrival counters
  size_t off_ml;     // float2 [B][H][splits][T] (running max, running sum)
  size_t off_o;      // float [B][H][splits][T][128] un-normalised partial O
  size_t bytes;      // total workspace
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline Plan make_plan(const tree_attn_desc& d) {
  Plan p{};
  p.mfma = kMfmaKernelReady && d.dtype == TA_BF16 && d.head_dim == 128 && !(d.flags & TA_FLAG_SIMPLE_KERNEL);
  p.chunk = kChunkTokens;
  p.splits = d.max_ctx_len <= 0 ? 1 : (d.max_ctx_len + kChunkTokens - 1) / kChunkTokens;
  if (!p.mfma) return p;
  const size_t bh = (size_t)d.batch * d.num_heads;
  const size_t rows = bh * (size_t)p.splits * d.t_max;
  p.off_count = 0;
  p.off_ml = align256(bh * sizeof(int32_t));
  p.off_o = p.off_ml + align256(rows * 8);
  p.bytes = p.off_o + align256(rows * (size_t)d.head_dim * sizeof(float));
  return p;
}

}  // namespace ta
