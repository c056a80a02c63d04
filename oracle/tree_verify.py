"""Plain CPU reference of the Medusa tree-verify step (test infrastructure).

Sources (the pages the method is described on):
  [vLLM-1171]  vLLM issue #1171 "[Discussion] Will vLLM consider using
               Speculative Sampling to accelerating LLM decoding?" -
               void-main's list of required changes (tree mask through a custom
               attention mask inside the cached-KV decode kernel; block-table
               update on acceptance; forward returning a list of tokens) and
               zhaoyang-star's description of decode with more than one new
               token on top of an existing paged KV cache.
  [TRT-1946]   TensorRT-LLM issue #1946 "How to use Medusa to support non
               llama models?" - rakib-hasan's answer: a position-offset tensor
               is passed so RoPE is applied correctly to the Medusa tokens;
               the neox-style RoPE type is named there.
  [LMD-1231]   LMDeploy PR #1231 "[WIP] support Medusa" - generate_candidates
               / evaluate_posterior with LM-head temperature 0 (greedy) over
               64 medusa choices; a TreeMask version built on Flash Decoding.
  [MLC-2319]   mlc-llm issue #2319 "[Feature Request] Medusa support" - the
               two hard parts: tree-based attention and the KV-cache update.

Readings where the pages are silent (each listed in the design notes):
  * node 0 is the root, at position ctx_len (depth 0), always committed;
  * every node sees the whole committed context, its ancestors and itself;
  * RoPE is rotate-half (neox) with base 10000, pairs (x_k, x_{k+d/2});
  * cached K is stored after RoPE; V is never rotated;
  * child c is accepted iff cand_tokens[c] == node_argmax[parent(c)];
  * the accepted end node is the deepest matched node, ties -> smallest index;
  * the committed K is rotated in fp32 with a fixed operation order and no
    fused multiply-add, from an fp32 cos/sin table whose angles are formed in
    fp64, then rounded to the pool's dtype with round-to-nearest-even.
"""
from __future__ import annotations

import numpy as np

PAD_PARENT = -2
ROPE_BASE = 10000.0
BLOCK = 16


def _np(x):
    """torch tensor or array -> numpy (bf16 tensors are widened exactly)."""
    if hasattr(x, "detach"):
        import torch
        x = x.detach().cpu()
        if x.dtype == torch.bfloat16:
            x = x.to(torch.float32)
        return x.numpy()
    return np.asarray(x)


# ------------------------------------------------------------------ RoPE ---
# [TRT-1946]: the Medusa tokens get RoPE at an offset position; the position
# of tree node i of sequence b is ctx_len[b] + depth[b][i].

def inv_freq(head_dim: int, base: float = ROPE_BASE) -> np.ndarray:
    """theta_k = base^(-2k/d), k < d/2, in fp64."""
    k = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(np.float64(base), -(2.0 * k) / head_dim)


def rope_exact(x: np.ndarray, pos, base: float = ROPE_BASE) -> np.ndarray:
    """Rotate-half RoPE in fp64.  x[..., d]; pos broadcasts against x[..., 0]."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv_freq(d, base)
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def rope_table(head_dim: int, max_pos: int, base: float = ROPE_BASE) -> np.ndarray:
    """fp32 table [max_pos][d/2][2] of (cos, sin) of pos*theta_k; the angle is
    formed in fp64 and each value is rounded once to fp32."""
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv_freq(head_dim, base)
    tab = np.empty((max_pos, head_dim // 2, 2), dtype=np.float32)
    tab[..., 0] = np.cos(ang).astype(np.float32)
    tab[..., 1] = np.sin(ang).astype(np.float32)
    return tab


def rope_pinned(x32: np.ndarray, cos32: np.ndarray, sin32: np.ndarray) -> np.ndarray:
    """Rotate-half in fp32, one rounding per operation, no fused multiply-add:
    y1 = (x1*c) - (x2*s);  y2 = (x2*c) + (x1*s).  NumPy float32 elementwise
    operations round each result to fp32 (round-to-nearest-even)."""
    x32 = np.asarray(x32, dtype=np.float32)
    d = x32.shape[-1]
    x1, x2 = x32[..., : d // 2], x32[..., d // 2:]
    c = np.asarray(cos32, dtype=np.float32)
    s = np.asarray(sin32, dtype=np.float32)
    a = x1 * c
    b = x2 * s
    e = x2 * c
    f = x1 * s
    return np.concatenate([a - b, e + f], axis=-1).astype(np.float32)


# ------------------------------------------------------------- bf16 bits ---

def f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest, ties to even."""
    u = np.asarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    r = np.where(nan, (u >> 16) | 0x40, r)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------- tree helpers ---

def ancestors(parent_row) -> list:
    """Ancestor-or-self node sets of one tree, as Python int bitmasks
    (bit j set = node j is an ancestor of, or equal to, node i).  Padding
    nodes get 0."""
    parent_row = [int(p) for p in parent_row]
    out = []
    for i, p in enumerate(parent_row):
        if p == PAD_PARENT:
            out.append(0)
            continue
        m, j = 0, i
        while j >= 0:
            m |= 1 << j
            j = parent_row[j]
        out.append(m)
    return out


def _depth(parent_row, i) -> int:
    d = 0
    while int(parent_row[i]) >= 0:
        i = int(parent_row[i])
        d += 1
    return d


def gather_context(kv_pages, block_table_row, ctx: int, kv_head: int):
    """Cached K and V of one sequence/head, token order, through the block
    table: token t lives in page block_table[t // 16] at slot t % 16.
    [vLLM-1171]: the cache is paged in fixed-size blocks."""
    pages = kv_pages
    t = np.arange(ctx)
    blk = np.asarray(block_table_row)[t // BLOCK]
    K = pages[blk, 0, kv_head, t % BLOCK, :].astype(np.float64)
    V = pages[blk, 1, kv_head, t % BLOCK, :].astype(np.float64)
    return K, V


# ---------------------------------------------------------------- verify ---

def verify_head(q, k_new, v_new, kv_pages, block_table, ctx_lens, tree_parent,
                tree_depth, b: int, h: int, scale=None, base=ROPE_BASE):
    """Attention output of every node of sequence b, query head h: [T][d] fp64
    (padding rows zero).  Inputs must already be numpy arrays (see verify)."""
    T = tree_parent.shape[1]
    H = q.shape[2]
    Hkv = k_new.shape[2]
    d = q.shape[3]
    hk = h // (H // Hkv)
    sc = 1.0 / np.sqrt(d) if scale is None else float(scale)
    ctx = int(ctx_lens[b])
    par = tree_parent[b]
    real = [i for i in range(T) if int(par[i]) != PAD_PARENT]
    anc = ancestors(par)
    K, V = gather_context(kv_pages, block_table[b], ctx, hk)
    pos = ctx + tree_depth[b].astype(np.int64)
    kt = rope_exact(k_new[b, :, hk, :], pos, base)        # tree keys [T][d]
    vt = v_new[b, :, hk, :].astype(np.float64)
    out = np.zeros((T, d), dtype=np.float64)
    for i in real:
        qi = rope_exact(q[b, i, h, :], pos[i], base)
        s_ctx = sc * (K @ qi)
        s_tree = sc * (kt @ qi)
        allowed = np.array([(anc[i] >> j) & 1 == 1 for j in range(T)])
        s_tree = np.where(allowed, s_tree, -np.inf)
        s = np.concatenate([s_ctx, s_tree])
        m = s.max()
        p = np.exp(s - m)
        p[np.isinf(s)] = 0.0
        out[i] = (p[:ctx] @ V + p[ctx:] @ vt) / p.sum()
    return out


def verify(q, k_new, v_new, kv_pages, block_table, ctx_lens, tree_parent,
           tree_depth, scale=None, base=ROPE_BASE):
    """Tree attention of every (sequence, head, node): out [B][T][H][d] fp64.

    For node i of sequence b and query head h the keys are the cached keys of
    the first ctx_len[b] tokens (stored already rotated) followed by the tree
    keys RoPE(k_new[j], ctx+depth[j]); scores are scale*RoPE(q_i, ctx+depth_i)
    . key, tree columns outside ancestor-or-self(i) are -inf, and the output is
    the max-subtracted softmax of the whole row times the values.
    [vLLM-1171] (tree mask over cached context + new tokens), [TRT-1946]
    (position offsets), [LMD-1231] (TreeMask over a paged decode)."""
    q, k_new, v_new, kv_pages = (_np(x) for x in (q, k_new, v_new, kv_pages))
    block_table, ctx_lens = _np(block_table), _np(ctx_lens)
    tree_parent, tree_depth = _np(tree_parent), _np(tree_depth)
    B, T, H, d = q.shape
    out = np.zeros((B, T, H, d), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            out[b, :, h, :] = verify_head(q, k_new, v_new, kv_pages, block_table,
                                          ctx_lens, tree_parent, tree_depth,
                                          b, h, scale, base)
    return out


# ---------------------------------------------------------------- accept ---

def accept_greedy(node_argmax, cand_tokens, tree_parent):
    """Greedy acceptance ([LMD-1231] evaluate_posterior at temperature 0).

    Walk the nodes in index order (parent[i] < i): the root is matched; node
    i is matched iff its parent is matched and cand_tokens[i] equals the base
    model's greedy token after its parent.  The end node is the deepest
    matched node, the smallest index among equals.  Returns accept_len [B]
    (= depth(end)+1, root counted) and accept_path [B][T] (node ids by depth,
    -1 beyond accept_len)."""
    node_argmax, cand_tokens = _np(node_argmax), _np(cand_tokens)
    tree_parent = _np(tree_parent)
    B, T = tree_parent.shape
    acc_len = np.zeros(B, dtype=np.int32)
    acc_path = np.full((B, T), -1, dtype=np.int32)
    for b in range(B):
        par = tree_parent[b]
        matched = [False] * T
        depth = [0] * T
        matched[0] = True
        best = 0
        for i in range(1, T):
            p = int(par[i])
            if p == PAD_PARENT:
                continue
            depth[i] = depth[p] + 1
            matched[i] = matched[p] and int(cand_tokens[b, i]) == int(node_argmax[b, p])
            if matched[i] and depth[i] > depth[best]:
                best = i
        path = []
        j = best
        while j >= 0:
            path.append(j)
            j = int(par[j])
        path.reverse()
        acc_len[b] = len(path)
        acc_path[b, : len(path)] = path
    return acc_len, acc_path


# ---------------------------------------------------------------- commit ---

def commit(k_new, v_new, accept_len, accept_path, kv_pages, block_table,
           ctx_lens, rope_tab):
    """KV commit ([MLC-2319] "KV cache update", [vLLM-1171] block tables).

    Returns a new pool (same dtype / bits as the input): for i < accept_len[b],
    node n = accept_path[b][i] at position p = ctx_len[b] + i lands in page
    block_table[b][p // 16], slot p % 16.  K is rope_pinned(k_new[b, n], p)
    rounded to the pool dtype; V is copied bit for bit.  No other byte
    changes.  Accepts torch tensors (bf16 or fp32) or numpy arrays."""
    import torch
    pool_t = kv_pages
    is_bf16 = hasattr(pool_t, "dtype") and pool_t.dtype == torch.bfloat16
    if is_bf16:
        pool = pool_t.detach().cpu().view(torch.int16).numpy().view(np.uint16).copy()
        kn = bf16_bits_to_f32(k_new.detach().cpu().view(torch.int16).numpy().view(np.uint16))
        vn = v_new.detach().cpu().view(torch.int16).numpy().view(np.uint16)
    else:
        pool = _np(pool_t).astype(np.float32).copy()
        kn = _np(k_new).astype(np.float32)
        vn = _np(v_new).astype(np.float32)
    accept_len, accept_path = _np(accept_len), _np(accept_path)
    block_table, ctx_lens = _np(block_table), _np(ctx_lens)
    B = accept_len.shape[0]
    for b in range(B):
        for i in range(int(accept_len[b])):
            n = int(accept_path[b, i])
            p = int(ctx_lens[b]) + i
            blk = int(block_table[b, p // BLOCK])
            slot = p % BLOCK
            k32 = rope_pinned(kn[b, n], rope_tab[p, :, 0], rope_tab[p, :, 1])
            if is_bf16:
                pool[blk, 0, :, slot, :] = f32_to_bf16_bits(k32)
            else:
                pool[blk, 0, :, slot, :] = k32
            pool[blk, 1, :, slot, :] = vn[b, n]
    if is_bf16:
        return torch.from_numpy(pool.view(np.int16)).view(torch.bfloat16)
    return torch.from_numpy(pool)
