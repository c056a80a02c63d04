// Device-side helpers shared by the tree-verify kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tree_attn.h"

namespace ta {

constexpr int kPage = 16;         // tokens per KV page
constexpr int kPadParent = -2;    // tree_parent value of a padding node
constexpr int kMaxTree = 64;      // one wavefront lane per tree node

// Everything a verify kernel needs, passed by value.
struct VerifyParams {
  const void* q;
  const void* k_new;
  const void* v_new;
  const void* kv_pages;
  const int32_t* block_table;
  const int32_t* ctx_lens;
  const int32_t* tree_parent;
  const int32_t* tree_depth;
  void* out;
  const float* rope;       // [rope_max_pos][d/2][2]
  float* ws_o;             // split partials: O  [B][H][splits][T][d]
  float2* ws_ml;           // split partials: (m, l) [B][H][splits][T]
  uint32_t* ws_ctr;        // work counters of the persistent kernel (2 words, kept zero between launches)
  int B, T, H, Hkv, D;
  int max_blocks, num_blocks, max_ctx, rope_max_pos;
  int chunk;               // context tokens per split work item
  int splits;              // max splits per (b, h) = ceil(max_ctx / chunk)
  int n_cu;                // compute units of the device (work-item ordering)
  float scale;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round to nearest, ties to even (quiet NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  return static_cast<uint16_t>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ float ld(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
__device__ __forceinline__ float ld(const float* p, size_t i) { return p[i]; }
__device__ __forceinline__ void st(uint16_t* p, size_t i, float v) { p[i] = f32_to_bf16_rne(v); }
__device__ __forceinline__ void st(float* p, size_t i, float v) { p[i] = v; }

// Value after a round trip through the storage type.
__device__ __forceinline__ float to_storage(const uint16_t*, float v) {
  return bf16_to_f32(f32_to_bf16_rne(v));
}
__device__ __forceinline__ float to_storage(const float*, float v) { return v; }

// Rotate-half RoPE of one pair with a fixed operation order: every product
// and sum rounded to fp32 separately, never fused into an FMA, so the result
// is reproducible bit for bit on any IEEE fp32 implementation.
// (hipcc contracts a*b - c*d into an FMA by default, and the _rn intrinsics
// do not stop it, hence the pragma.)
__device__ __forceinline__ void rope_pair_exact(float x1, float x2, float c, float s,
                                                float& y1, float& y2) {
#pragma clang fp contract(off)
  const float a = x1 * c;
  const float b = x2 * s;
  const float e = x2 * c;
  const float f = x1 * s;
  y1 = a - b;
  y2 = e + f;
}

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return min(max(x, lo), hi); }

// Offset (in elements) of row `slot` of page `blk`, kv plane `kv` (0 = K, 1 = V),
// head `hk`, in kv_pages[num_blocks][2][Hkv][16][D].
__device__ __forceinline__ size_t page_row(int blk, int kv, int hk, int slot, int Hkv, int D) {
  return ((((size_t)blk * 2 + kv) * Hkv + hk) * kPage + slot) * (size_t)D;
}

}  // namespace ta
