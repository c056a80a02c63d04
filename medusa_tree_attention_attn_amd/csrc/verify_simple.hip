// Plain tree-verify kernel: one wavefront per (node, head, sequence).
//
// Every lane walks a strided share of the keys (cached context first, then
// the tree nodes that are ancestors of the node or the node itself), keeps a
// private online-softmax state, and the 64 states are merged at the end.
// It re-reads the KV cache once per node, so it is only meant for the cases
// the MFMA kernel does not take (fp32 data, head_dim 64) and as a second,
// independent GPU formulation in the tests.
//
// Semantics: vLLM issue #1171 (several new tokens over a paged KV cache with
// a tree mask), TensorRT-LLM issue #1946 (RoPE at ctx_len + depth).
#include "launch.h"

namespace ta {
namespace {

template <typename S, int D>
__global__ __launch_bounds__(64) void verify_simple_kernel(VerifyParams p) {
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const int T = p.T, Hkv = p.Hkv;
  const int hk = h / (p.H / Hkv);
  const int32_t* par = p.tree_parent + (size_t)b * T;
  const int32_t* dep = p.tree_depth + (size_t)b * T;
  S* out = static_cast<S*>(p.out) + (((size_t)b * T + i) * p.H + h) * D;

  if (par[i] == kPadParent) {
    for (int k = lane; k < D; k += 64) st(out, k, 0.f);
    return;
  }
  // ancestor-or-self set of node i (bit j = node j); stops on malformed links
  uint64_t anc = 0;
  for (int j = i, s = 0; j >= 0 && s < kMaxTree; ++s) {
    anc |= 1ull << j;
    const int pj = par[j];
    if (pj >= j) break;
    j = pj;
  }
  const int ctx = clampi(p.ctx_lens[b], 0, p.max_ctx);
  const int pos_i = ctx + clampi(dep[i], 0, T - 1);

  __shared__ float qs[D];
  __shared__ float red[64][D + 1];
  __shared__ float lane_m[64], lane_l[64];

  const S* q = static_cast<const S*>(p.q) + (((size_t)b * T + i) * p.H + h) * D;
  const float* cs_i = p.rope + (size_t)pos_i * D;
  for (int k = lane; k < D / 2; k += 64) {
    const float x1 = ld(q, k), x2 = ld(q, k + D / 2);
    const float c = cs_i[2 * k], s = cs_i[2 * k + 1];
    qs[k] = (x1 * c - x2 * s) * p.scale;
    qs[k + D / 2] = (x2 * c + x1 * s) * p.scale;
  }
  __syncthreads();

  const S* pages = static_cast<const S*>(p.kv_pages);
  const S* kn_all = static_cast<const S*>(p.k_new);
  const S* vn_all = static_cast<const S*>(p.v_new);
  float m = -INFINITY, l = 0.f;
  float o[D];
#pragma unroll
  for (int k = 0; k < D; ++k) o[k] = 0.f;

  for (int t = lane; t < ctx + T; t += 64) {
    float sc = 0.f;
    const S* vrow;
    if (t < ctx) {
      const int lb = t / kPage;
      if (lb >= p.max_blocks) continue;
      const int blk = p.block_table[(size_t)b * p.max_blocks + lb];
      if (blk < 0 || blk >= p.num_blocks) continue;
      const S* krow = pages + page_row(blk, 0, hk, t % kPage, Hkv, D);
      vrow = pages + page_row(blk, 1, hk, t % kPage, Hkv, D);
#pragma unroll 8
      for (int k = 0; k < D; ++k) sc += qs[k] * ld(krow, k);
    } else {
      const int j = t - ctx;
      if (!((anc >> j) & 1ull)) continue;
      const int pos_j = ctx + clampi(dep[j], 0, T - 1);
      const S* krow = kn_all + (((size_t)b * T + j) * Hkv + hk) * D;
      vrow = vn_all + (((size_t)b * T + j) * Hkv + hk) * D;
      const float* cs_j = p.rope + (size_t)pos_j * D;
#pragma unroll 8
      for (int k = 0; k < D / 2; ++k) {
        float y1, y2;
        rope_pair_exact(ld(krow, k), ld(krow, k + D / 2), cs_j[2 * k], cs_j[2 * k + 1], y1, y2);
        // the key as it will be stored by the commit
        sc += qs[k] * to_storage(krow, y1) + qs[k + D / 2] * to_storage(krow, y2);
      }
    }
    const float mn = fmaxf(m, sc);
    const float a = (m == -INFINITY) ? 0.f : expf(m - mn);
    const float e = expf(sc - mn);
    l = l * a + e;
#pragma unroll
    for (int k = 0; k < D; ++k) o[k] = o[k] * a + e * ld(vrow, k);
    m = mn;
  }

  // merge the 64 lane states
  lane_m[lane] = m;
  __syncthreads();
  float M = -INFINITY;
  for (int r = 0; r < 64; ++r) M = fmaxf(M, lane_m[r]);
  const float f = (m == -INFINITY) ? 0.f : expf(m - M);
  lane_l[lane] = l * f;
#pragma unroll
  for (int k = 0; k < D; ++k) red[lane][k] = o[k] * f;
  __syncthreads();
  float L = 0.f;
  for (int r = 0; r < 64; ++r) L += lane_l[r];
  for (int k = lane; k < D; k += 64) {
    float acc = 0.f;
    for (int r = 0; r < 64; ++r) acc += red[r][k];
    st(out, k, acc / L);
  }
}

template <typename S>
hipError_t launch_typed(const VerifyParams& p, hipStream_t stream) {
  dim3 grid(p.T, p.H, p.B);
  if (p.D == 128)
    hipLaunchKernelGGL((verify_simple_kernel<S, 128>), grid, dim3(64), 0, stream, p);
  else
    hipLaunchKernelGGL((verify_simple_kernel<S, 64>), grid, dim3(64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_verify_simple(const VerifyParams& p, int dtype, hipStream_t stream) {
  return dtype == TA_BF16 ? launch_typed<uint16_t>(p, stream) : launch_typed<float>(p, stream);
}

}  // namespace ta
