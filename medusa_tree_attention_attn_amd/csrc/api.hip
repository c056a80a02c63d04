// C ABI of the tree-verify library: host-side validation, split planning and
// dispatch.  No allocation and no device->host synchronisation.  The only
// global state is the static device workspace of tree_attn_verify_noalloc
// and its per-device address.
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <map>
#include <mutex>
#include <vector>

#include "launch.h"
#include "plan.h"

using namespace ta;

// Workspace of tree_attn_verify_noalloc: one file-scope device array, which
// every GPU the library runs on holds (at its own address) until the process
// ends.  In host code `scratch` only names the symbol: its device address on
// a given device comes from hipGetSymbolAddress (scratch_on_current_device
// below), and only that address is ever passed to a kernel.
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;

int check_common(const tree_attn_desc* d) {
  if (!d) return TA_ERR_NULL_POINTER;
  if (d->batch <= 0 || d->t_max <= 0 || d->num_heads <= 0 || d->num_kv_heads <= 0 ||
      d->max_blocks_per_seq <= 0 || d->num_blocks <= 0 || d->max_ctx_len < 0)
    return TA_ERR_BAD_DIMS;
  if (d->t_max > kMaxTree) return TA_ERR_TREE_TOO_LARGE;
  if (d->dtype != TA_BF16 && d->dtype != TA_F32) return TA_ERR_DTYPE;
  if (d->head_dim != 64 && d->head_dim != 128) return TA_ERR_HEAD_DIM;
  if (d->num_heads % d->num_kv_heads != 0) return TA_ERR_HEADS;
  if (d->block_size != kPage) return TA_ERR_BLOCK_SIZE;
  if (d->batch > 65535) return TA_ERR_BAD_DIMS;
  if ((int64_t)d->max_blocks_per_seq * kPage < (int64_t)d->max_ctx_len) return TA_ERR_CAPACITY;
  if (!d->rope_cos_sin || (int64_t)d->rope_max_pos < (int64_t)d->max_ctx_len + d->t_max)
    return TA_ERR_ROPE_TABLE;
  return TA_OK;
}

int status_of(hipError_t e) { return e == hipSuccess ? TA_OK : TA_ERR_LAUNCH; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Compute units of the current device (0 when the query fails).
int device_cu_count() {
  int dev = 0, n_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  return n_cu;
}

}  // namespace

extern "C" {

size_t tree_attn_workspace_size(const tree_attn_desc* d) {
  if (check_common(d) != TA_OK) return 0;
  return make_plan(*d).bytes;
}

int tree_attn_plan_info(const tree_attn_desc* d, int32_t* kernel, int32_t* splits,
                        int32_t* split_tokens) {
  const int rc = check_common(d);
  if (rc != TA_OK) return rc;
  const Plan plan = make_plan(*d);
  int k = TA_KERNEL_SIMPLE;
  if (plan.decode) {
    k = TA_KERNEL_DECODE;
  } else if (plan.mfma) {
    k = use_stream_kernel(*d) ? TA_KERNEL_PERSISTENT : TA_KERNEL_GRID;
  }
  if (kernel) *kernel = k;
  if (splits) *splits = plan.splits;
  if (split_tokens) *split_tokens = plan.chunk;
  return TA_OK;
}

int tree_attn_workspace_init(const tree_attn_desc* d) {
  if (!d) return TA_ERR_NULL_POINTER;
  if (d->workspace_bytes == 0) return TA_OK;
  if (!d->workspace) return TA_ERR_NULL_POINTER;
  return status_of(launch_fill_zero(d->workspace, d->workspace_bytes,
                                    static_cast<hipStream_t>(d->stream)));
}

}  // extern "C"

namespace {

// tree_attn_verify with its workspace passed separately: desc->workspace and
// desc->workspace_bytes for the ABI call, the static scratch array for
// tree_attn_verify_noalloc.
int verify_with_workspace(const tree_attn_desc* d, void* workspace, size_t workspace_bytes,
                          const void* q, const void* k_new, const void* v_new,
                          const void* kv_pages, const int32_t* block_table,
                          const int32_t* ctx_lens, const int32_t* tree_parent,
                          const int32_t* tree_depth, void* out) {
  const int rc = check_common(d);
  if (rc != TA_OK) return rc;
  if (!q || !k_new || !v_new || !kv_pages || !block_table || !ctx_lens || !tree_parent ||
      !tree_depth || !out)
    return TA_ERR_NULL_POINTER;
  const Plan plan = make_plan(*d);
  if (plan.bytes > 0 && (!workspace || workspace_bytes < plan.bytes)) return TA_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(kv_pages) ||
      !aligned16(out) || !aligned16(d->rope_cos_sin) ||
      (plan.bytes > 0 && !aligned16(workspace)))
    return TA_ERR_ALIGNMENT;

  VerifyParams p{};
  p.q = q;
  p.k_new = k_new;
  p.v_new = v_new;
  p.kv_pages = kv_pages;
  p.block_table = block_table;
  p.ctx_lens = ctx_lens;
  p.tree_parent = tree_parent;
  p.tree_depth = tree_depth;
  p.out = out;
  p.rope = d->rope_cos_sin;
  p.B = d->batch;
  p.T = d->t_max;
  p.H = d->num_heads;
  p.Hkv = d->num_kv_heads;
  p.D = d->head_dim;
  p.max_blocks = d->max_blocks_per_seq;
  p.num_blocks = d->num_blocks;
  p.max_ctx = d->max_ctx_len;
  p.rope_max_pos = d->rope_max_pos;
  p.scale = d->scale > 0.f ? d->scale : 1.0f / sqrtf((float)d->head_dim);
  p.chunk = plan.chunk;
  p.splits = plan.splits;
  hipStream_t stream = static_cast<hipStream_t>(d->stream);
  const int n_cu = device_cu_count();
  p.n_cu = n_cu;
  if (plan.decode) return status_of(launch_verify_decode(p, stream));
  if (plan.mfma) {
    char* ws = static_cast<char*>(workspace);
    if (plan.splits > 1) {
      p.ws_ml = reinterpret_cast<float2*>(ws + plan.off_ml);
      p.ws_o = reinterpret_cast<float*>(ws + plan.off_o);
    }
    hipError_t e;
    if (use_stream_kernel(*d)) {
      if (n_cu <= 0) return TA_ERR_LAUNCH;
      p.ws_ctr = reinterpret_cast<uint32_t*>(ws + plan.off_ctr);
      e = launch_verify_stream(p, stream);
    } else {
      e = launch_verify_mfma(p, stream);
    }
    if (e == hipSuccess && plan.splits > 1) e = launch_split_combine(p, stream);
    return status_of(e);
  }
  return status_of(launch_verify_simple(p, d->dtype, stream));
}

// Device address of `scratch` (defined at file scope above) on the current
// device, set up on first use there: the address is taken with that device
// current and kept per device, and the first 256 bytes (the persistent
// kernel's work counters) are zeroed by a fill kernel on `stream`, ahead of
// the caller's verify on the same stream.  nullptr if the device or the
// symbol cannot be resolved or the fill cannot be enqueued.
std::mutex scratch_mutex;
std::atomic<void*> scratch_ptr[kMaxDevices];

void* scratch_on_current_device(hipStream_t stream) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* ptr = scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr) return ptr;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  ptr = scratch_ptr[dev].load(std::memory_order_relaxed);
  if (ptr) return ptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
  if (launch_fill_zero(ptr, 256, stream) != hipSuccess) return nullptr;
  scratch_ptr[dev].store(ptr, std::memory_order_release);
  return ptr;
}

}  // namespace

extern "C" {

int tree_attn_verify(const tree_attn_desc* d, const void* q, const void* k_new,
                     const void* v_new, const void* kv_pages, const int32_t* block_table,
                     const int32_t* ctx_lens, const int32_t* tree_parent,
                     const int32_t* tree_depth, void* out) {
  if (!d) return TA_ERR_NULL_POINTER;
  return verify_with_workspace(d, d->workspace, d->workspace_bytes, q, k_new, v_new, kv_pages,
                               block_table, ctx_lens, tree_parent, tree_depth, out);
}

int tree_attn_verify_noalloc(const tree_attn_desc* d, const void* q, const void* k_new,
                             const void* v_new, const void* kv_pages,
                             const int32_t* block_table, const int32_t* ctx_lens,
                             const int32_t* tree_parent, const int32_t* tree_depth, void* out) {
  const int rc = check_common(d);
  if (rc != TA_OK) return rc;
  if (make_plan(*d).bytes > kScratchBytes) return TA_ERR_WORKSPACE;
  void* ws = scratch_on_current_device(static_cast<hipStream_t>(d->stream));
  if (!ws) return TA_ERR_LAUNCH;
  return verify_with_workspace(d, ws, kScratchBytes, q, k_new, v_new, kv_pages, block_table,
                               ctx_lens, tree_parent, tree_depth, out);
}

int tree_accept_greedy(const tree_attn_desc* d, const int32_t* node_argmax,
                       const int32_t* cand_tokens, const int32_t* tree_parent,
                       int32_t* accept_len, int32_t* accept_path) {
  if (!d) return TA_ERR_NULL_POINTER;
  if (d->batch <= 0 || d->t_max <= 0 || d->batch > (1 << 30)) return TA_ERR_BAD_DIMS;
  if (d->t_max > kMaxTree) return TA_ERR_TREE_TOO_LARGE;
  if (!node_argmax || !cand_tokens || !tree_parent || !accept_len || !accept_path)
    return TA_ERR_NULL_POINTER;
  return status_of(launch_accept(node_argmax, cand_tokens, tree_parent, accept_len,
                                 accept_path, d->batch, d->t_max,
                                 static_cast<hipStream_t>(d->stream)));
}

namespace {
int commit_params(const tree_attn_desc* d, const void* k_new, const void* v_new,
                  const int32_t* accept_len, const int32_t* accept_path, void* kv_pages,
                  const int32_t* block_table, const int32_t* ctx_lens, CommitParams& p) {
  const int rc = check_common(d);
  if (rc != TA_OK) return rc;
  if (!k_new || !v_new || !accept_len || !accept_path || !kv_pages || !block_table ||
      !ctx_lens)
    return TA_ERR_NULL_POINTER;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(kv_pages) ||
      !aligned16(d->rope_cos_sin))
    return TA_ERR_ALIGNMENT;
  p = CommitParams{};
  p.k_new = k_new;
  p.v_new = v_new;
  p.accept_len = accept_len;
  p.accept_path = accept_path;
  p.kv_pages = kv_pages;
  p.block_table = block_table;
  p.ctx_lens = ctx_lens;
  p.rope = d->rope_cos_sin;
  p.B = d->batch;
  p.T = d->t_max;
  p.Hkv = d->num_kv_heads;
  p.D = d->head_dim;
  p.max_blocks = d->max_blocks_per_seq;
  p.num_blocks = d->num_blocks;
  p.max_ctx = d->max_ctx_len;
  p.rope_max_pos = d->rope_max_pos;
  return TA_OK;
}
}  // namespace

int kv_commit_path(const tree_attn_desc* d, const void* k_new, const void* v_new,
                   const int32_t* accept_len, const int32_t* accept_path, void* kv_pages,
                   const int32_t* block_table, const int32_t* ctx_lens) {
  CommitParams p;
  const int rc = commit_params(d, k_new, v_new, accept_len, accept_path, kv_pages, block_table,
                               ctx_lens, p);
  if (rc != TA_OK) return rc;
  return status_of(launch_commit(p, d->dtype, static_cast<hipStream_t>(d->stream)));
}

int tree_accept_commit(const tree_attn_desc* d, const int32_t* node_argmax,
                       const int32_t* cand_tokens, const int32_t* tree_parent,
                       int32_t* accept_len, int32_t* accept_path, const void* k_new,
                       const void* v_new, void* kv_pages, const int32_t* block_table,
                       const int32_t* ctx_lens) {
  if (!node_argmax || !cand_tokens || !tree_parent) return TA_ERR_NULL_POINTER;
  CommitParams p;
  const int rc = commit_params(d, k_new, v_new, accept_len, accept_path, kv_pages, block_table,
                               ctx_lens, p);
  if (rc != TA_OK) return rc;
  return status_of(launch_accept_commit(p, node_argmax, cand_tokens, tree_parent, accept_len,
                                        accept_path, d->dtype,
                                        static_cast<hipStream_t>(d->stream)));
}

int tree_vocab_argmax(const tree_attn_desc* d, const void* logits, int32_t logits_dtype,
                      int32_t vocab, int32_t* node_argmax) {
  if (!d) return TA_ERR_NULL_POINTER;
  if (d->batch <= 0 || d->t_max <= 0 || d->batch > 65535) return TA_ERR_BAD_DIMS;
  if (d->t_max > kMaxTree) return TA_ERR_TREE_TOO_LARGE;
  if (logits_dtype != TA_BF16 && logits_dtype != TA_F32) return TA_ERR_DTYPE;
  if (vocab <= 0) return TA_ERR_BAD_DIMS;
  if (!logits || !node_argmax) return TA_ERR_NULL_POINTER;
  return status_of(launch_vocab_argmax(logits, logits_dtype, vocab, d->batch * d->t_max,
                                       node_argmax, static_cast<hipStream_t>(d->stream)));
}

int tree_argmax_accept(const tree_attn_desc* d, const void* logits, int32_t logits_dtype,
                       int32_t vocab, const int32_t* cand_tokens, const int32_t* tree_parent,
                       int32_t* node_argmax, int32_t* accept_len, int32_t* accept_path) {
  if (!d) return TA_ERR_NULL_POINTER;
  if (d->batch <= 0 || d->t_max <= 0 || d->batch > 65535) return TA_ERR_BAD_DIMS;
  if (d->t_max > kMaxTree) return TA_ERR_TREE_TOO_LARGE;
  if (logits_dtype != TA_BF16 && logits_dtype != TA_F32) return TA_ERR_DTYPE;
  if (vocab <= 0) return TA_ERR_BAD_DIMS;
  if (!logits || !cand_tokens || !tree_parent || !node_argmax || !accept_len || !accept_path)
    return TA_ERR_NULL_POINTER;
  hipStream_t stream = static_cast<hipStream_t>(d->stream);
  hipError_t e = launch_vocab_argmax(logits, logits_dtype, vocab, d->batch * d->t_max,
                                     node_argmax, stream);
  if (e == hipSuccess)
    e = launch_accept(node_argmax, cand_tokens, tree_parent, accept_len, accept_path, d->batch,
                      d->t_max, stream);
  return status_of(e);
}

int tree_accept_typical(const tree_attn_desc* d, const void* logits, int32_t logits_dtype,
                        int32_t vocab, const int32_t* cand_tokens, const int32_t* tree_parent,
                        float temperature, float epsilon, float delta, float* node_stats,
                        int32_t* node_ok, int32_t* accept_len, int32_t* accept_path) {
  if (!d) return TA_ERR_NULL_POINTER;
  if (d->batch <= 0 || d->t_max <= 0 || d->batch > 65535) return TA_ERR_BAD_DIMS;
  if (d->t_max > kMaxTree) return TA_ERR_TREE_TOO_LARGE;
  if (logits_dtype != TA_BF16 && logits_dtype != TA_F32) return TA_ERR_DTYPE;
  if (vocab <= 0) return TA_ERR_BAD_DIMS;
  if (!(temperature > 0.f) || !std::isfinite(temperature) || !std::isfinite(epsilon) ||
      !std::isfinite(delta))
    return TA_ERR_BAD_DIMS;
  if (!logits || !cand_tokens || !tree_parent || !node_stats || !node_ok || !accept_len ||
      !accept_path)
    return TA_ERR_NULL_POINTER;
  if ((reinterpret_cast<uintptr_t>(node_stats) & 7u) != 0) return TA_ERR_ALIGNMENT;
  return status_of(launch_typical_accept(logits, logits_dtype, vocab, d->batch, d->t_max,
                                         temperature, epsilon, delta, cand_tokens, tree_parent,
                                         node_stats, node_ok, accept_len, accept_path,
                                         static_cast<hipStream_t>(d->stream)));
}

int tree_medusa_tree(const int32_t* choices, int32_t n_choices, int32_t max_len, int32_t topk,
                     int32_t num_medusa_heads, int32_t* node_table, int32_t* n_nodes) {
  if (!node_table || !n_nodes || (n_choices > 0 && !choices)) return TA_ERR_NULL_POINTER;
  if (num_medusa_heads <= 0 || topk <= 0 || topk > kMaxTopK || n_choices < 0 || max_len <= 0)
    return TA_ERR_BAD_DIMS;
  if (n_choices + 1 > kMaxTree) return TA_ERR_TREE_TOO_LARGE;
  // Paths, validated, then numbered: root 0, then by length, then
  // lexicographically.
  std::vector<std::vector<int>> paths(n_choices);
  for (int c = 0; c < n_choices; ++c) {
    for (int j = 0; j < max_len; ++j) {
      const int r = choices[(size_t)c * max_len + j];
      if (r < 0) break;
      if (r >= topk) return TA_ERR_CHOICES;
      paths[c].push_back(r);
    }
    if (paths[c].empty() || (int)paths[c].size() > num_medusa_heads) return TA_ERR_CHOICES;
    for (int j = (int)paths[c].size(); j < max_len; ++j)
      if (choices[(size_t)c * max_len + j] >= 0) return TA_ERR_CHOICES;  // gap in a path
  }
  std::sort(paths.begin(), paths.end(), [](const std::vector<int>& a, const std::vector<int>& b) {
    return a.size() != b.size() ? a.size() < b.size() : a < b;
  });
  const int n = n_choices + 1;
  std::vector<int32_t> table(3 * (size_t)n, 0);
  std::map<std::vector<int>, int> node_of;
  node_of[{}] = 0;
  table[0] = -1;
  for (int c = 0; c < n_choices; ++c) {
    const std::vector<int>& p = paths[c];
    if (node_of.count(p)) return TA_ERR_CHOICES;  // duplicate
    const std::vector<int> up(p.begin(), p.end() - 1);
    const auto it = node_of.find(up);
    if (it == node_of.end()) return TA_ERR_CHOICES;  // prefix missing
    node_of[p] = c + 1;
    table[c + 1] = it->second;
    table[n + c + 1] = (int32_t)p.size();
    table[2 * n + c + 1] = p.back();
  }
  std::copy(table.begin(), table.end(), node_table);
  *n_nodes = n;
  return TA_OK;
}

int tree_medusa_candidates(const tree_attn_desc* d, const int32_t* node_table, int32_t n_nodes,
                           const void* head_logits, int32_t head_dtype, int32_t num_medusa_heads,
                           int32_t vocab, int32_t topk, const int32_t* root_token,
                           int32_t* cand_tokens, int32_t* tree_parent, int32_t* tree_depth) {
  if (!d) return TA_ERR_NULL_POINTER;
  if (d->batch <= 0 || d->t_max <= 0 || d->batch > 65535) return TA_ERR_BAD_DIMS;
  if (d->t_max > kMaxTree) return TA_ERR_TREE_TOO_LARGE;
  if (head_dtype != TA_BF16 && head_dtype != TA_F32) return TA_ERR_DTYPE;
  if (!node_table || !head_logits || !root_token || !cand_tokens || !tree_parent || !tree_depth)
    return TA_ERR_NULL_POINTER;
  if (num_medusa_heads <= 0 || num_medusa_heads > 65535 || vocab <= 0 || topk <= 0 ||
      topk > kMaxTopK || topk > vocab || n_nodes <= 0)
    return TA_ERR_BAD_DIMS;
  if (n_nodes > d->t_max) return TA_ERR_TREE_TOO_LARGE;
  // O(n) check of the table: root first, parents before children, depth one
  // below the parent's and within the heads, ranks below topk, no two
  // children of a node with the same rank.
  const int32_t* par = node_table;
  const int32_t* dep = node_table + n_nodes;
  const int32_t* rnk = node_table + 2 * (size_t)n_nodes;
  if (par[0] != -1 || dep[0] != 0) return TA_ERR_CHOICES;
  CandTree tree{};
  tree.n_nodes = n_nodes;
  tree.parent[0] = -1;
  uint32_t used[kMaxTree] = {};
  for (int n = 1; n < n_nodes; ++n) {
    const int p = par[n];
    if (p < 0 || p >= n || dep[n] != dep[p] + 1 || dep[n] > num_medusa_heads || rnk[n] < 0 ||
        rnk[n] >= topk || (used[p] >> rnk[n]) & 1u)
      return TA_ERR_CHOICES;
    used[p] |= 1u << rnk[n];
    tree.parent[n] = (int8_t)p;
    tree.depth[n] = (int8_t)dep[n];
    tree.rank[n] = (int8_t)rnk[n];
  }
  return status_of(launch_candidates(head_logits, head_dtype, vocab, num_medusa_heads, topk, tree,
                                     root_token, cand_tokens, tree_parent, tree_depth, d->batch,
                                     d->t_max, static_cast<hipStream_t>(d->stream)));
}

int tree_attn_rope_table(int32_t head_dim, float base, int32_t max_pos, float* table,
                         void* stream) {
  if (!table) return TA_ERR_NULL_POINTER;
  if (head_dim != 64 && head_dim != 128) return TA_ERR_HEAD_DIM;
  if (max_pos <= 0 || !(base > 1.0f)) return TA_ERR_BAD_DIMS;
  return status_of(launch_rope_table(head_dim, base, max_pos, table,
                                     static_cast<hipStream_t>(stream)));
}

int tree_attn_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (!src || !sink) return TA_ERR_NULL_POINTER;
  if (!aligned16(src) || (reinterpret_cast<uintptr_t>(sink) & 3u) != 0) return TA_ERR_ALIGNMENT;
  return status_of(launch_stream_read(src, bytes, sink, device_cu_count(),
                                      static_cast<hipStream_t>(stream)));
}

const char* tree_attn_strerror(int status) {
  switch (status) {
    case TA_OK: return "ok";
    case TA_ERR_NULL_POINTER: return "a required pointer is NULL";
    case TA_ERR_BAD_DIMS: return "invalid dimensions in the descriptor";
    case TA_ERR_DTYPE: return "unsupported dtype (TA_BF16 or TA_F32)";
    case TA_ERR_TREE_TOO_LARGE: return "t_max exceeds 64 nodes";
    case TA_ERR_HEAD_DIM: return "head_dim must be 64 or 128";
    case TA_ERR_HEADS: return "num_heads must be a multiple of num_kv_heads";
    case TA_ERR_BLOCK_SIZE: return "block_size must be 16";
    case TA_ERR_WORKSPACE: return "workspace missing or smaller than tree_attn_workspace_size";
    case TA_ERR_ROPE_TABLE: return "rope table missing or rope_max_pos < max_ctx_len + t_max";
    case TA_ERR_CAPACITY: return "max_blocks_per_seq * 16 < max_ctx_len";
    case TA_ERR_LAUNCH: return "kernel launch failed";
    case TA_ERR_ALIGNMENT: return "a tensor pointer is not aligned as the call requires";
    case TA_ERR_CHOICES: return "the medusa choices list is not a valid tree";
    default: return "unknown status";
  }
}

}  // extern "C"
