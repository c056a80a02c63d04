// Verify with one node per sequence (T = 1): plain paged decode, the step a
// Medusa server falls back to when speculation is off (vLLM issue #1171
// measures the batch sizes where that happens).  The node is the root at
// position ctx_len; it attends to the whole cached context and to itself.
//
// At T = 1 a KV byte carries two multiply-adds, so nothing here needs the
// matrix cores; what bounds the step is how many bytes each CU keeps in
// flight.  One workgroup of kDecWaves wavefronts per (sequence, head), launched
// longest context first.  Wavefront w streams pages w, w+kDecWaves, ... of
// the context on its own, with kDepth pages (K and V, 8 KB each) in flight in
// registers while it computes the oldest; at ~100 VGPRs several workgroups
// share a CU, far more bytes in flight than the tree kernels can afford.
//
// Page layout in the registers: load i of a 4 KB page plane is 1 KB, tokens
// 4i .. 4i+3, and lane l takes its 16 bytes at 16 l: token 4i + l/16, dims
// 8 (l%16) .. +7.  So every load instruction is one contiguous 1 KB, and a
// lane holds the same 8 dims of K and of V for tokens g, g+4, g+8, g+12
// (g = l/16).  A score is a dot2 over the lane's 8 dims, summed over the 16
// lanes of the group.  Each of the four lane groups keeps its own online
// softmax state (base 2; q is pre-scaled by scale * log2 e) over its tokens,
// so a page needs no exchange between groups; the 4 x 4 states of the
// workgroup are merged once at the end.  The node's own key (rotated with
// the commit's fixed-order arithmetic and rounded to bf16, as the commit
// will store it) joins wavefront 0's group 0 after the context.
#include "launch.h"
#include "page_stream.h"

namespace ta {
namespace {

// Wavefronts per workgroup and pages in flight per wavefront.
#ifndef TA_DECODE_WAVES
#define TA_DECODE_WAVES 4
#endif
#ifndef TA_DECODE_DEPTH
#define TA_DECODE_DEPTH 3
#endif
constexpr int kDecWaves = TA_DECODE_WAVES;
constexpr int kDecThreads = 64 * kDecWaves;
constexpr int kDepth = TA_DECODE_DEPTH;
constexpr int kWinPages = 2048;  // block ids staged in LDS at a time

struct Page {
  u32x4 k[4];
  u32x4 v[4];
};

// The pages are read once: the loads carry the non-temporal hint (batch 64,
// contexts 128..8192: 639 against 698 us per launch).
__device__ __forceinline__ void load_page(Page& P, const uint16_t* kbase, size_t v_plane,
                                          int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    P.k[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kbase + 512 * i + 8 * lane));
    P.v[i] = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4*>(kbase + v_plane + 512 * i + 8 * lane));
  }
}

// (b, h) of launch slot `slot`: with at most 64 sequences, sequences are
// ranked by context length (longest first) so the longest streams start
// first and the short ones fill the tail; otherwise natural order.
__device__ __forceinline__ void decode_item(const VerifyParams& p, int slot, int lane, int& b,
                                           int& h) {
  h = slot % p.H;
  const int r = slot / p.H;
  if (p.B > 64) {
    b = r;
    return;
  }
  const int ctx_l = lane < p.B ? p.ctx_lens[lane] : -1;
  int rank = 0;
  for (int j = 0; j < p.B; ++j) {
    const int cj = __shfl(ctx_l, j);
    rank += (cj > ctx_l) || (cj == ctx_l && j < lane);
  }
  b = __builtin_ctzll(__ballot(lane < p.B && rank == r));
}

__global__ __launch_bounds__(kDecThreads) void verify_decode_kernel(VerifyParams p) {
  __shared__ float s_o[kDecWaves][4][kD];
  __shared__ float s_ml[kDecWaves][4][2];
  __shared__ int s_ids[kWinPages];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int g = lane >> 4, dc = lane & 15;
  int b, h;
  decode_item(p, blockIdx.x, lane, b, h);
  const int hk = h / (p.H / p.Hkv);
  uint16_t* out = static_cast<uint16_t*>(p.out) + ((size_t)b * p.H + h) * kD;

  const int par = p.tree_parent[b];
  if (par == kPadParent) {  // a padding row: zeros
    if (wv == 0 && lane < 16) *reinterpret_cast<u32x4*>(out + 8 * lane) = u32x4{0u, 0u, 0u, 0u};
    return;
  }
  const int ctx = clampi(p.ctx_lens[b], 0, p.max_ctx);
  const int pos = ctx;  // depth 0 (the only node of a one-node tree)

  // q: dims 8 dc .. +7 of the rotated, pre-scaled row, as bf16 pairs.  Dims
  // d and d + 64 are RoPE partners: lanes dc and dc ^ 8 swap their raw dims.
  u32x4 qf;
  {
    const u32x4 raw = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(p.q) +
                                                      ((size_t)b * p.H + h) * kD + 8 * dc);
    u32x4 oth;
#pragma unroll
    for (int w = 0; w < 4; ++w) oth[w] = __shfl_xor(raw[w], 8);
    const f32x4* cs = reinterpret_cast<const f32x4*>(p.rope + (size_t)pos * kD + 16 * (dc & 7));
    const float qs = p.scale * kLog2e;
    const bool first = dc < 8;  // dims < 64: y = x c - x' s; else y = x c + x' s
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const f32x4 t = cs[w];  // (cos, sin) of k = 8 (dc & 7) + 2w and + 1
      const float x0 = bf16_lo(raw[w]), x1 = bf16_hi(raw[w]);
      const float y0 = bf16_lo(oth[w]), y1 = bf16_hi(oth[w]);
      const float r0 = first ? x0 * t[0] - y0 * t[1] : x0 * t[0] + y0 * t[1];
      const float r1 = first ? x1 * t[2] - y1 * t[3] : x1 * t[2] + y1 * t[3];
      qf[w] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{r0 * qs, r1 * qs},
                                                                     bf16x2));
    }
  }

  State st;
  reset(st);

  // The context in windows of kWinPages pages whose block ids (checked)
  // are first copied to LDS, so that no page address waits on a vector
  // load (the vector memory counter is in order: such a wait would also
  // wait for every page in flight).  Wavefront w streams pages w,
  // w + kDecWaves, ... of each window.
  const int n_pages = (ctx + kPage - 1) / kPage;
  const int32_t* table = p.block_table + (size_t)b * p.max_blocks;
  const uint16_t* pages = static_cast<const uint16_t*>(p.kv_pages);
  const size_t v_plane = (size_t)p.Hkv * kPage * kD;
  const size_t head_off = page_row(0, 0, hk, 0, p.Hkv, kD);
  const int wvu = __builtin_amdgcn_readfirstlane(wv);
  for (int p0 = 0; p0 < n_pages; p0 += kWinPages) {
    const int np = min(kWinPages, n_pages - p0);
    __syncthreads();  // the previous window's ids are no longer read
    // All of the window's table loads are issued, unconditionally, before
    // any is stored: one memory round trip, not one per pass, and no branch
    // for the compiler's wait counts to merge over.  Indices are clamped into
    // the window (n_pages <= max_blocks, since ctx <= max_ctx <= 16 *
    // max_blocks); a clamped duplicate is an L2 hit and is not stored.
    constexpr int kIdPasses = kWinPages / kDecThreads;
    static_assert(kWinPages % kDecThreads == 0, "whole passes");
    int raw[kIdPasses];
#pragma unroll
    for (int k = 0; k < kIdPasses; ++k) raw[k] = table[p0 + min(k * kDecThreads + tid, np - 1)];
#pragma unroll
    for (int k = 0; k < kIdPasses; ++k) {
      const int i = k * kDecThreads + tid;
      if (i < np) s_ids[i] = (raw[k] >= 0 && raw[k] < p.num_blocks) ? raw[k] : -1;
    }
    __syncthreads();
    const int my_pages = np > wvu ? (np - wvu + kDecWaves - 1) / kDecWaves : 0;
    if (my_pages == 0) continue;
    // Every ring load is unconditional, so the compiler can count the loads
    // in flight and wait only for the oldest page: an absent page reads
    // pool page 0 and is masked; past the end the last page is read again
    // (an L2 hit) and not used.
    auto page_id = [&](int j) {  // j-th page of this wavefront, clamped
      return __builtin_amdgcn_readfirstlane(s_ids[wvu + kDecWaves * min(j, my_pages - 1)]);
    };
    auto page_base = [&](int blk) {
      return pages + (size_t)max(blk, 0) * 2 * v_plane + head_off;
    };
    Page ring[kDepth];
    int ids[kDepth];
#pragma unroll
    for (int u = 0; u < kDepth; ++u) {
      ids[u] = page_id(u);
      load_page(ring[u], page_base(ids[u]), v_plane, lane);
    }
    for (int j0 = 0; j0 < my_pages; j0 += kDepth) {
#pragma unroll
      for (int u = 0; u < kDepth; ++u) {
        const int j = j0 + u;
        if (j < my_pages && ids[u] >= 0) {
          const int tok0 = (p0 + wvu + kDecWaves * j) * kPage;
          if (tok0 + kPage > ctx) {  // the context's last page: rows past its end
#pragma unroll                         // are masked, and zeroed so a NaN there
            for (int i = 0; i < 4; ++i)  // cannot reach 0 * V
              if (tok0 + 4 * i + g >= ctx) ring[u].v[i] = u32x4{0u, 0u, 0u, 0u};
          }
          float s[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float d = group_sum(dot8(qf, ring[u].k[i], 0.f));
            s[i] = tok0 + 4 * i + g < ctx ? d : -INFINITY;
          }
          add_tokens(st, s, ring[u].v);
        }
        ids[u] = page_id(j + kDepth);
        load_page(ring[u], page_base(ids[u]), v_plane, lane);
      }
    }
  }

  // The node's own key and value (a linked root only), in wavefront 0's
  // group 0: rotated with the commit's arithmetic, rounded to bf16.
  if (wv == 0 && par == -1) {
    const size_t row = ((size_t)b * p.Hkv + hk) * kD;
    const u32x4 kr = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(p.k_new) +
                                                     row + 8 * dc);
    const u32x4 vr = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(p.v_new) +
                                                     row + 8 * dc);
    u32x4 ko;
#pragma unroll
    for (int w = 0; w < 4; ++w) ko[w] = __shfl_xor(kr[w], 8);
    const f32x4* cs = reinterpret_cast<const f32x4*>(p.rope + (size_t)pos * kD + 16 * (dc & 7));
    const bool first = dc < 8;
    u32x4 kk;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const f32x4 t = cs[w];
      float a0, b0, a1, b1;
      // first half: (x1, x2) = (mine, partner) -> keep y1; second: keep y2
      if (first) {
        rope_pair_exact(bf16_lo(kr[w]), bf16_lo(ko[w]), t[0], t[1], a0, b0);
        rope_pair_exact(bf16_hi(kr[w]), bf16_hi(ko[w]), t[2], t[3], a1, b1);
      } else {
        rope_pair_exact(bf16_lo(ko[w]), bf16_lo(kr[w]), t[0], t[1], b0, a0);
        rope_pair_exact(bf16_hi(ko[w]), bf16_hi(kr[w]), t[2], t[3], b1, a1);
      }
      kk[w] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a0, a1}, bf16x2));
    }
    const float d = group_sum(dot8(qf, kk, 0.f));
    const float s[4] = {g == 0 ? d : -INFINITY, -INFINITY, -INFINITY, -INFINITY};
    const u32x4 vv[4] = {vr, vr, vr, vr};
    add_tokens(st, s, vv);
  }

  // Merge: the four groups of each wavefront, then the wavefronts.
  if (dc == 0) {
    s_ml[wv][g][0] = st.m;
    s_ml[wv][g][1] = st.l;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) s_o[wv][g][8 * dc + i] = st.o[i];
  __syncthreads();
  if (wv == 0) {
    // lane handles dims 2 lane, 2 lane + 1 over all 16 states
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w)
#pragma unroll
      for (int q = 0; q < 4; ++q) M = fmaxf(M, s_ml[w][q][0]);
    float L = 0.f, o0 = 0.f, o1 = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kDecWaves; ++w)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float f = __builtin_amdgcn_exp2f(s_ml[w][q][0] - M);  // -inf -> 0
          L = fmaf(s_ml[w][q][1], f, L);
          o0 = fmaf(s_o[w][q][2 * lane], f, o0);
          o1 = fmaf(s_o[w][q][2 * lane + 1], f, o1);
        }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    reinterpret_cast<uint32_t*>(out)[lane] =
        __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{o0 * inv, o1 * inv}, bf16x2));
  }
}

}  // namespace

hipError_t launch_verify_decode(const VerifyParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(verify_decode_kernel, dim3((unsigned)(p.B * p.H)), dim3(kDecThreads), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace ta
