// Vector-ALU building blocks for attention with a handful of queries per
// (sequence, head): the one-node decode kernel and the small-tree path of
// the grid verify kernel (gfx950, bf16, head_dim 128).
//
// Lane layout of a streamed KV row block: lane l = 16 g + dc holds dims
// 8 dc .. 8 dc + 7 of one token per lane group g, so a score is a dot2 sum
// over the lane's 8 dims followed by a sum over the 16 lanes of its group.
// Each lane group keeps its own online-softmax state per query (base 2: the
// queries are pre-scaled by scale * log2 e), so a token needs no exchange
// between groups; the states are merged once at the end.
#pragma once

#include "mfma_tile.h"

namespace ta {

typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

// 8-dim bf16 dot product added to acc.  (The words are copied out first:
// hipcc lowers a bit cast taken straight from a vector element to element 0
// for every index.)
__device__ __forceinline__ float dot8(const u32x4& a, const u32x4& b, float acc) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t aw = a[w], bw = b[w];
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, aw),
                                          __builtin_bit_cast(bf16x2v, bw), acc, false);
  }
  return acc;
}

// Sum over the 16 lanes of a lane group (a DPP row), with DPP moves, which
// stay in the vector ALU (a lane shuffle goes through the LDS crossbar):
// swap neighbours, swap pairs (every lane then holds its quad's sum), mirror
// each half-row (lane i of a half with lane 7 - i: quad with quad), mirror
// the row (lane i with lane 15 - i: half with half).
template <int kCtrl>
__device__ __forceinline__ float dpp_move(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), kCtrl,
                                                            0xF, 0xF, false));
}
__device__ __forceinline__ float group_sum(float x) {
  constexpr int kSwapNeighbours = 0xB1;  // quad_perm [1, 0, 3, 2]
  constexpr int kSwapPairs = 0x4E;       // quad_perm [2, 3, 0, 1]
  constexpr int kHalfRowMirror = 0x141;
  constexpr int kRowMirror = 0x140;
  x += dpp_move<kSwapNeighbours>(x);
  x += dpp_move<kSwapPairs>(x);
  x += dpp_move<kHalfRowMirror>(x);
  x += dpp_move<kRowMirror>(x);
  return x;
}

// One query's online-softmax state in one lane group: running max and sum
// (base 2) and the lane's 8 dims of the un-normalised output.
struct State {
  float m, l;
  float o[8];
};

__device__ __forceinline__ void reset(State& st) {
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) st.o[i] = 0.f;
}

// Adds up to four tokens (scores s[i], the lane's 8 dims of their values
// v[i]) to the state; tokens with s = -inf add nothing (their value rows
// must be finite: 0 * NaN would still poison the sum).
__device__ __forceinline__ void add_tokens(State& st, const float (&s)[4], const u32x4 (&v)[4]) {
  const float mp = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
  const float mn = fmaxf(st.m, mp);
  if (mn == -INFINITY) return;  // nothing valid yet
  const float alpha = __builtin_amdgcn_exp2f(st.m - mn);  // st.m = -inf -> 0
  float p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(s[i] - mn);
  st.l = st.l * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    float a0 = st.o[2 * w] * alpha, a1 = st.o[2 * w + 1] * alpha;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a0 = fmaf(p[i], bf16_lo(v[i][w]), a0);
      a1 = fmaf(p[i], bf16_hi(v[i][w]), a1);
    }
    st.o[2 * w] = a0;
    st.o[2 * w + 1] = a1;
  }
  st.m = mn;
}

}  // namespace ta
