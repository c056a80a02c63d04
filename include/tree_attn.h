/*
 * tree_attn.h - C ABI of the Medusa tree-verify step on MI355X (gfx950).
 *
 * One verify step of Medusa speculative decoding, for a batch of sequences
 * that each submit a tree of up to 64 candidate tokens:
 *
 *   tree_attn_verify    every tree node attends to the sequence's paged KV
 *                       cache plus its own ancestors (and itself) in the tree,
 *                       with RoPE applied at position ctx_len + depth;
 *   tree_accept_greedy  greedy acceptance of the longest root-to-node path
 *                       whose candidate tokens equal the base model's greedy
 *                       predictions;
 *   kv_commit_path      writes the accepted path's K/V rows into the pages.
 *
 * Sources: vLLM issue #1171 "[Discussion] Will vLLM consider using
 * Speculative Sampling to accelerating LLM decoding?" (decode with several new
 * tokens over an existing paged KV cache; a tree mask inside the cached-KV
 * attention; block-table update on acceptance), TensorRT-LLM issue #1946
 * "How to use Medusa to support non llama models?" (position offsets fed to
 * RoPE for the Medusa tokens), LMDeploy PR #1231 "[WIP] support Medusa"
 * (evaluate_posterior at LM-head temperature 0; TreeMask on Flash Decoding),
 * mlc-llm issue #2319 "[Feature Request] Medusa support" (tree attention and
 * the KV-cache update as the two hard parts).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - All tensor pointers are DEVICE pointers owned by the caller, row-major,
 *    contiguous, 16-byte aligned (the kernels move 16-byte vectors).  The
 *    library allocates nothing, keeps no global state besides the static
 *    device workspace of tree_attn_verify_noalloc, never synchronises the
 *    device with the host, and enqueues all work on desc->stream (a
 *    hipStream_t; NULL = the default stream).
 *  - Element type of q, k_new, v_new, kv_pages and out is desc->dtype
 *    (TA_BF16 or TA_F32); index tensors are int32.
 *  - Layouts (B = batch, T = t_max, H = num_heads, Hkv = num_kv_heads,
 *    d = head_dim, P = block_size = 16):
 *        q, out            [B][T][H][d]
 *        k_new, v_new      [B][T][Hkv][d]      (k_new not yet rotated)
 *        kv_pages          [num_blocks][2][Hkv][P][d]   (index 0 = K, 1 = V;
 *                                               cached K is stored rotated)
 *        block_table       [B][max_blocks_per_seq]      physical block ids
 *        ctx_lens          [B]     committed tokens per sequence
 *        tree_parent       [B][T]  -1 for the root (node 0); parent[i] < i
 *                                  for real nodes; -2 for padding nodes,
 *                                  which must form a suffix
 *        tree_depth        [B][T]  depth of each node (root 0)
 *        node_argmax       [B][T]  base model's greedy token after node i
 *        cand_tokens       [B][T]  candidate token carried by node i
 *        accept_len        [B]     accepted nodes including the root
 *        accept_path       [B][T]  accepted node ids by depth, -1 beyond
 *        rope_cos_sin      [rope_max_pos][d/2][2] fp32 (cos, sin) of
 *                                  pos * base^(-2k/d), see tree_attn_rope_table
 *  - Token t of sequence b lives in page block_table[b][t / 16], slot t % 16.
 *  - RoPE is rotate-half: pairs (x_k, x_{k+d/2}), y_k = x_k*c - x_{k+d/2}*s,
 *    y_{k+d/2} = x_{k+d/2}*c + x_k*s, at position ctx_len[b] + depth.
 *  - Return value: TA_OK (0) or a negative TA_ERR_* code.  Every check that
 *    can be made on the host is made before anything is enqueued; nothing
 *    aborts and no exception crosses the ABI.  Device-resident values
 *    (ctx_lens, block ids, tree structure, accepted paths) are bounds-checked
 *    inside the kernels: an out-of-range value never causes an out-of-bounds
 *    access, but the affected outputs are unspecified (ctx_len is clamped to
 *    [0, max_ctx_len]; an out-of-range page id is never used as an address:
 *    its tokens are skipped or read from page 0).
 *  - Calls are asynchronous; a launch failure is reported as TA_ERR_LAUNCH.
 *    Two calls that share a workspace must not run concurrently.
 */
#ifndef TREE_ATTN_H
#define TREE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum ta_dtype { TA_BF16 = 0, TA_F32 = 1 };

/* desc->flags bits */
enum ta_flags {
  TA_FLAG_SIMPLE_KERNEL = 1,  /* verify with the plain one-wavefront-per-node  */
                              /* kernel even where the MFMA kernels apply      */
  TA_FLAG_GRID_KERNEL = 2,    /* MFMA verify: one workgroup per work item      */
  TA_FLAG_PERSISTENT_KERNEL = 4, /* MFMA verify: one resident workgroup per CU  */
                              /* taking work items from a counter.             */
  TA_FLAG_DECODE_KERNEL = 8   /* t_max == 1 (bf16, head_dim 128): the decode   */
                              /* kernel, one workgroup per (sequence, head).   */
                              /* Without a flag the library takes the decode   */
                              /* kernel when t_max == 1 and max_ctx_len <=     */
                              /* 1024, else the grid kernel, which sends work  */
                              /* items whose tree has at most 2 real nodes     */
                              /* (sequences of at most 64 work-item groups) to */
                              /* its vector-ALU small-tree path.               */
};

enum ta_status {
  TA_OK = 0,
  TA_ERR_NULL_POINTER = -1,   /* a required pointer is NULL                  */
  TA_ERR_BAD_DIMS = -2,       /* batch/t_max/heads/blocks not positive, etc. */
  TA_ERR_DTYPE = -3,          /* dtype not TA_BF16 / TA_F32                  */
  TA_ERR_TREE_TOO_LARGE = -4, /* t_max > 64                                  */
  TA_ERR_HEAD_DIM = -5,       /* head_dim not 64 or 128                      */
  TA_ERR_HEADS = -6,          /* num_heads not a multiple of num_kv_heads    */
  TA_ERR_BLOCK_SIZE = -7,     /* block_size != 16                            */
  TA_ERR_WORKSPACE = -8,      /* workspace NULL or smaller than required     */
  TA_ERR_ROPE_TABLE = -9,     /* rope table missing or rope_max_pos too small*/
  TA_ERR_CAPACITY = -10,      /* max_blocks_per_seq*16 < max_ctx_len         */
  TA_ERR_LAUNCH = -11,        /* the HIP runtime rejected a launch           */
  TA_ERR_ALIGNMENT = -12,     /* a pointer is not aligned as the call needs  */
  TA_ERR_CHOICES = -13        /* a medusa choices list is not a valid tree   */
};

typedef struct tree_attn_desc {
  int32_t batch;              /* B                                            */
  int32_t t_max;              /* T, nodes per tree incl. padding, 1..64       */
  int32_t num_heads;          /* H query heads                                */
  int32_t num_kv_heads;       /* Hkv KV heads, H % Hkv == 0                   */
  int32_t head_dim;           /* d, 64 or 128                                 */
  int32_t block_size;         /* tokens per page, must be 16                  */
  int32_t max_blocks_per_seq; /* columns of block_table                       */
  int32_t num_blocks;         /* pages in kv_pages                            */
  int32_t max_ctx_len;        /* host-known upper bound on every ctx_lens[b]; */
                              /* sizes the launch grid, never read back       */
  int32_t dtype;              /* enum ta_dtype                                */
  float scale;                /* softmax scale; <= 0 selects 1/sqrt(d)        */
  const float* rope_cos_sin;  /* device fp32 table, see layout above          */
  int32_t rope_max_pos;       /* rows of rope_cos_sin, >= max_ctx_len + t_max */
  void* workspace;            /* device scratch owned by the caller           */
  size_t workspace_bytes;     /* its size, >= tree_attn_workspace_size(desc)  */
  void* stream;               /* hipStream_t                                  */
  int32_t flags;              /* enum ta_flags, 0 by default                  */
  int32_t split_tokens;       /* context tokens per split-KV work item of the */
                              /* MFMA kernel, rounded up to a multiple of 64  */
                              /* and capped at 8192; 0 = chosen from batch,   */
                              /* heads and max_ctx_len (never below 128)      */
} tree_attn_desc;

/* Tree attention (vLLM #1171: several new tokens over a paged KV cache under
 * a tree mask; TensorRT-LLM #1946: RoPE position offsets; LMDeploy #1231:
 * TreeMask over split-KV Flash Decoding).
 * For every real node i of sequence b and query head h (kv head
 * h / (H/Hkv)):
 *   keys   = cached K of tokens 0..ctx_len[b]-1 (as stored), then the tree
 *            keys RoPE(k_new[b][j], ctx_len[b] + depth[j]) for the nodes j
 *            that are ancestors of i or i itself;
 *   values = cached V, then v_new[b][j] for the same j;
 *   out[b][i][h] = softmax(scale * RoPE(q[b][i][h], ctx_len[b] + depth[i])
 *                  . keys) . values, accumulated in fp32 and rounded to
 *                  dtype (round to nearest even).
 * Padding rows of out are written as zeros.  kv_pages is only read.
 * Needs desc->workspace of tree_attn_workspace_size(desc) bytes.  For the
 * MFMA kernels (bf16, head_dim 128) its first 256 bytes hold the persistent
 * kernel's work counters: zero-fill the workspace once with
 * tree_attn_workspace_init before its first verify; every verify leaves
 * them at zero again.  The rest holds split-KV partials between the kernels
 * of one call and needs no initialisation.  The current device must be the
 * one desc->stream belongs to.  Errors: every TA_ERR_* code. */
int tree_attn_verify(const tree_attn_desc* desc, const void* q, const void* k_new,
                     const void* v_new, const void* kv_pages,
                     const int32_t* block_table, const int32_t* ctx_lens,
                     const int32_t* tree_parent, const int32_t* tree_depth,
                     void* out);

/* Allocation-free tree_attn_verify, for callers that cannot allocate device
 * memory or hand the library a workspace: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same arguments,
 * results and kernels as tree_attn_verify, except that desc->workspace and
 * desc->workspace_bytes are ignored: the split-KV partials and the
 * persistent kernel's work counters live in a static device array of 32 MiB
 * that the library holds on every device it runs on until the process ends.
 * The first call on a device resolves the array's address there and zeroes
 * its 256 bytes of counters with a fill kernel on desc->stream; every call
 * leaves the counters at zero again.  No call allocates (no hipMalloc,
 * hipFree or allocating library routine).  All calls on one device share its
 * array, which keeps the last call's contents: calls that overlap on one
 * device (concurrent streams or host threads) race and must not be issued.
 * Errors: those of tree_attn_verify; TA_ERR_WORKSPACE when the plan for the
 * descriptor needs more than 32 MiB (tree_attn_workspace_size(desc) > 32 MiB:
 * long contexts cut into many splits); TA_ERR_LAUNCH when the array cannot
 * be resolved on the current device. */
int tree_attn_verify_noalloc(const tree_attn_desc* desc, const void* q, const void* k_new,
                             const void* v_new, const void* kv_pages,
                             const int32_t* block_table, const int32_t* ctx_lens,
                             const int32_t* tree_parent, const int32_t* tree_depth,
                             void* out);

/* Greedy acceptance (LMDeploy #1231 evaluate_posterior at temperature 0).
 * Node c (c >= 1) matches iff cand_tokens[b][c] == node_argmax[b][parent(c)];
 * a node is accepted iff every edge on its root path matches.  The end node
 * is the deepest accepted node, the smallest index among equals;
 * accept_len[b] = depth(end) + 1 and accept_path[b][k] = the accepted node at
 * depth k for k < accept_len[b], -1 after.  The root's own candidate token is
 * never checked.  The bonus token of the step is
 * node_argmax[b][accept_path[b][accept_len[b]-1]].
 * Uses batch, t_max and stream of desc; other fields are not read.  Output
 * is bit-exact: integer work only. */
int tree_accept_greedy(const tree_attn_desc* desc, const int32_t* node_argmax,
                       const int32_t* cand_tokens, const int32_t* tree_parent,
                       int32_t* accept_len, int32_t* accept_path);

/* KV commit (mlc-llm #2319 KV-cache update; vLLM #1171 block-table update).
 * For i < accept_len[b], node n = accept_path[b][i], position
 * p = ctx_len[b] + i: page block_table[b][p/16], slot p%16 receives
 *   K = RoPE(k_new[b][n], p) computed in fp32 from rope_cos_sin[p] as
 *       (x1*c) - (x2*s) and (x2*c) + (x1*s), each operation rounded, no fused
 *       multiply-add, then rounded to dtype (nearest even);
 *   V = v_new[b][n], bit for bit.
 * No other byte of kv_pages changes; ctx_lens is not modified (the caller
 * adds accept_len).  The caller reserves pages so that ctx_len + accept_len
 * fits in max_blocks_per_seq*16 and frees unused pages itself. */
int kv_commit_path(const tree_attn_desc* desc, const void* k_new, const void* v_new,
                   const int32_t* accept_len, const int32_t* accept_path,
                   void* kv_pages, const int32_t* block_table,
                   const int32_t* ctx_lens);

/* Greedy acceptance followed by the KV commit of the accepted path, in one
 * launch (LMDeploy #1231 evaluate_posterior; mlc-llm #2319 KV-cache update).
 * Writes accept_len and accept_path exactly as tree_accept_greedy does and
 * kv_pages exactly as kv_commit_path would from those outputs; the checks and
 * error codes are those of kv_commit_path plus a null test of the three
 * acceptance inputs.  accept_len/accept_path are outputs here.  It saves one
 * launch and one dependent memory round trip per step. */
int tree_accept_commit(const tree_attn_desc* desc, const int32_t* node_argmax,
                       const int32_t* cand_tokens, const int32_t* tree_parent,
                       int32_t* accept_len, int32_t* accept_path, const void* k_new,
                       const void* v_new, void* kv_pages, const int32_t* block_table,
                       const int32_t* ctx_lens);

/* Greedy token of the base model after every tree node (LMDeploy #1231
 * evaluate_posterior at LM-head temperature 0):
 *   node_argmax[b][i] = the smallest v < vocab with
 *                       logits[b][i][v] == max over v' of logits[b][i][v']
 * for all B * t_max rows (padding rows included).  logits is a device
 * tensor [B][t_max][vocab] of logits_dtype (TA_BF16 or TA_F32), compared as
 * exact values; NaN never wins and a row with no comparable value gives 0.
 * Uses batch, t_max and stream of desc.  Errors: TA_ERR_NULL_POINTER,
 * TA_ERR_BAD_DIMS, TA_ERR_TREE_TOO_LARGE, TA_ERR_DTYPE, TA_ERR_LAUNCH. */
int tree_vocab_argmax(const tree_attn_desc* desc, const void* logits, int32_t logits_dtype,
                      int32_t vocab, int32_t* node_argmax);

/* tree_vocab_argmax followed by tree_accept_greedy on its result, in one
 * call (two kernels on desc->stream; the kernel boundary publishes
 * node_argmax to the acceptance).  Writes node_argmax, accept_len and
 * accept_path exactly as the two calls would.  Errors: those of
 * tree_vocab_argmax. */
int tree_argmax_accept(const tree_attn_desc* desc, const void* logits, int32_t logits_dtype,
                       int32_t vocab, const int32_t* cand_tokens, const int32_t* tree_parent,
                       int32_t* node_argmax, int32_t* accept_len, int32_t* accept_path);

/* Typical acceptance (the Medusa scheme vLLM issue #1171 names as one of the
 * two non-standard parts of Medusa serving; the rule is the Medusa paper's).
 * For every node row r = (b, i), with y = logits[b][i][.] / temperature:
 *   node_stats[r][0] = lse = log sum_v exp(y_v)           (natural log)
 *   node_stats[r][1] = H   = -sum_v p_v log p_v,  p = softmax(y)
 * (all B * t_max rows, padding included).  Child c of node n passes iff
 *   exp(logits[b][n][cand_tokens[b][c]] / temperature - lse_n)
 *       > min(epsilon, delta * exp(-H_n));
 * node_ok[b][i] = 1 for the root and for every in-tree child that passes,
 * 0 otherwise (padding, unlinked nodes, tokens outside [0, vocab)).  The
 * accepted path is the deepest node whose whole root path passes (smallest
 * index among equals), written to accept_len / accept_path with the
 * conventions of tree_accept_greedy.  Arithmetic is fp32 (exp/log on the
 * hardware units): a child whose probability lies within a few ulps of the
 * threshold may go either way.  logits is a device tensor
 * [B][t_max][vocab] of logits_dtype (TA_BF16 or TA_F32); node_stats is a
 * device float [B][t_max][2], 8-byte aligned.  Two kernels on desc->stream.
 * Errors: TA_ERR_NULL_POINTER, TA_ERR_BAD_DIMS (also temperature <= 0 or a
 * non-finite temperature, epsilon or delta), TA_ERR_TREE_TOO_LARGE,
 * TA_ERR_DTYPE, TA_ERR_ALIGNMENT, TA_ERR_LAUNCH. */
int tree_accept_typical(const tree_attn_desc* desc, const void* logits, int32_t logits_dtype,
                        int32_t vocab, const int32_t* cand_tokens, const int32_t* tree_parent,
                        float temperature, float epsilon, float delta, float* node_stats,
                        int32_t* node_ok, int32_t* accept_len, int32_t* accept_path);

/* Node table of a fixed "medusa choices" list (LMDeploy #1231: the tree
 * buffers built once from the list), on the host; no GPU work.
 *   choices     HOST int32 [n_choices][max_len]: each row a path of top-k
 *               ranks (r_1, ..., r_d), -1 after its end.  The list must be
 *               prefix-closed (every proper prefix is also a row), without
 *               duplicates, with d <= num_medusa_heads and r < topk.
 *   node_table  HOST int32 [3][n_choices + 1], written: row 0 the parent,
 *               row 1 the depth, row 2 the rank r_d of every node (root:
 *               -1, 0, 0).  Nodes are numbered root 0, then the paths by
 *               length, then lexicographically (node = 1 + position).
 *   n_nodes     HOST int32, written: n_choices + 1.
 * Errors: TA_ERR_NULL_POINTER, TA_ERR_BAD_DIMS (topk outside [1, 16],
 * num_medusa_heads <= 0, n_choices < 0, max_len <= 0),
 * TA_ERR_TREE_TOO_LARGE (more than 64 nodes), TA_ERR_CHOICES (an invalid
 * list); node_table and n_nodes are untouched on error. */
int tree_medusa_tree(const int32_t* choices, int32_t n_choices, int32_t max_len, int32_t topk,
                     int32_t num_medusa_heads, int32_t* node_table, int32_t* n_nodes);

/* Candidate tree from the Medusa heads (LMDeploy #1231 generate_candidates),
 * laid out by a node table (tree_medusa_tree's, or any table of that
 * layout whose parents precede their children).
 *   node_table   HOST int32 [3][n_nodes] (parent, depth, rank rows).
 *   head_logits  device [B][num_medusa_heads][vocab] of head_dtype (TA_BF16
 *                or TA_F32); head h predicts the token at depth h + 1.
 *   root_token   device int32 [B]: the token decided by the previous step.
 * Writes, for every sequence:
 *   cand_tokens[b][n]  root_token[b] for n = 0; otherwise the rank[n]-th
 *                      best token of head depth[n] - 1 (logit descending,
 *                      smaller token among equal logits, NaN ranks as -inf);
 *   tree_parent[b][n]  parent[n];   tree_depth[b][n]  depth[n];
 * and padding (parent -2, depth 0, token 0) for n_nodes <= n < t_max.
 * Uses batch, t_max and stream of desc.  topk <= 16 and <= vocab;
 * n_nodes <= t_max.  The table is checked in O(n_nodes) (root -1/0, every
 * parent earlier, depth = parent's + 1 <= num_medusa_heads, 0 <= rank <
 * topk, siblings of distinct ranks): TA_ERR_CHOICES before anything is
 * enqueued; other errors as tree_vocab_argmax. */
int tree_medusa_candidates(const tree_attn_desc* desc, const int32_t* node_table,
                           int32_t n_nodes, const void* head_logits, int32_t head_dtype,
                           int32_t num_medusa_heads, int32_t vocab, int32_t topk,
                           const int32_t* root_token, int32_t* cand_tokens, int32_t* tree_parent,
                           int32_t* tree_depth);

/* Bytes of workspace tree_attn_verify needs for this descriptor (0 if the
 * descriptor is invalid or takes the plain or the decode kernel): for the
 * MFMA kernels, 256 bytes of work counters plus split-KV partials when the
 * plan splits contexts.  Pure host computation. */
size_t tree_attn_workspace_size(const tree_attn_desc* desc);

/* Kernels tree_attn_verify launches for this descriptor on the current
 * device: *kernel = TA_KERNEL_SIMPLE, TA_KERNEL_GRID, TA_KERNEL_PERSISTENT or
 * TA_KERNEL_DECODE (t_max == 1 with bf16 and head_dim 128, and either
 * TA_FLAG_DECODE_KERNEL or max_ctx_len <= 1024 without an MFMA flag: one
 * workgroup per (sequence, head) streams its whole context, no splits, no
 * workspace); *splits = context splits per (sequence, head) (a
 * merge kernel follows when it is > 1); *split_tokens = context tokens per
 * split.  Output pointers may be NULL.  Host-only query; errors as
 * tree_attn_verify's descriptor checks. */
enum ta_kernel {
  TA_KERNEL_SIMPLE = 0,
  TA_KERNEL_GRID = 1,
  TA_KERNEL_PERSISTENT = 2,
  TA_KERNEL_DECODE = 3
};
int tree_attn_plan_info(const tree_attn_desc* desc, int32_t* kernel, int32_t* splits,
                        int32_t* split_tokens);

/* Zero-fills desc->workspace (desc->workspace_bytes bytes) on desc->stream
 * with a fill kernel.  Required once before a workspace's first
 * tree_attn_verify when tree_attn_workspace_size is non-zero (the persistent
 * kernel's work counters must start at zero). */
int tree_attn_workspace_init(const tree_attn_desc* desc);

/* Fills table[pos][k][0..1] = (cos, sin)(pos * base^(-2k/head_dim)) for
 * pos < max_pos, k < head_dim/2: the angle is formed in fp64 and each value
 * rounded once to fp32 (TensorRT-LLM #1946 position offsets; neox-style
 * RoPE).  table is a device buffer of max_pos*head_dim floats. */
int tree_attn_rope_table(int32_t head_dim, float base, int32_t max_pos, float* table,
                         void* stream);

/* Read-bandwidth probe (measurement only; no step of the method calls it).
 * Streams the first bytes/16*16 bytes of the device buffer src with the load
 * width (16 bytes per lane) and cache policy (non-temporal) of the
 * tree-verify kernels' KV stream, and XORs every 32-bit word it reads into
 * the device word *sink (4-byte aligned): *sink ^= the XOR of those words,
 * which keeps the loads live and shows that each word was read once.
 * Timing this call on a buffer larger than the 256 MB Infinity Cache gives
 * the rate at which the device at hand streams a read-only buffer: the
 * practical ceiling beside the 8 TB/s nominal peak.  src 16-byte aligned.
 * Errors: TA_ERR_NULL_POINTER, TA_ERR_ALIGNMENT, TA_ERR_LAUNCH. */
int tree_attn_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

/* Static description of a status code. */
const char* tree_attn_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* TREE_ATTN_H */
