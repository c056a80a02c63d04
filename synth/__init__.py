"""Seeded synthetic workloads for the Medusa tree-verify step.

This module only draws random inputs: trees, candidate tokens, the base
model's greedy predictions, context lengths, block tables and the dense
q / k_new / v_new / KV-pool tensors.  It holds none of the step's arithmetic
(no RoPE, no attention, no acceptance rule), so both the CPU oracle and the
GPU path can consume its output without sharing any of the method.

Workload shapes follow the decoding shapes the Medusa discussions revolve
around (Vicuna-7B/13B head geometry, trees of up to 64 candidates, depth 4-5,
paged KV with 16-token blocks).  None of the Spec-Bench / MT-Bench items is
reproduced: everything is drawn from seeded generators.

Tree recipe (the pages give none): node 0 is the root (the token already
decided by the previous step, depth 0).  Each further node picks its parent
uniformly among the nodes created so far whose depth is below the depth cap;
the nodes are then relabelled in breadth-first order (children visited in
creation order), so parent[i] < i.  Candidate tokens are distinct among
siblings, like the top-k of one Medusa head.  The base model's greedy
prediction after an internal node equals the token of a uniformly chosen
child with probability p, and is otherwise uniform over the tokens that match
no child; after a leaf it is uniform.  Padding nodes of a tree shorter than
t_max carry parent -2.
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import math
import os
from typing import Dict, Optional

import numpy as np
import torch

BLOCK_SIZE = 16
PAD_PARENT = -2


@dataclasses.dataclass(frozen=True)
class WorkloadSpec:
    name: str
    batch: int
    heads: int
    kv_heads: int
    head_dim: int
    dtype: str                 # "bf16" or "f32": q, k_new, v_new, KV pool and out
    ctx_range: tuple           # inclusive (lo, hi) context length per sequence
    tree_sizes: tuple          # T_b is drawn uniformly from this tuple
    max_depth: int             # depth cap of the random trees
    vocab: int
    p_match: float
    t_max: int = 64
    full_binary: bool = False  # the tiny case uses a fixed full binary tree


SPECS: Dict[str, WorkloadSpec] = {
    # batch 1, one head, d=64, fp32; full binary tree of depth 2 (7 nodes)
    "tiny": WorkloadSpec("tiny", 1, 1, 1, 64, "f32", (128, 128), (7,), 2,
                         1000, 0.5, t_max=7, full_binary=True),
    # Vicuna-7B geometry at batch 1
    "vicuna7b_bs1": WorkloadSpec("vicuna7b_bs1", 1, 32, 32, 128, "bf16",
                                 (1024, 1024), (64,), 4, 32000, 0.4),
    # Vicuna-7B geometry, batch 16, ragged contexts
    "vicuna7b_b16": WorkloadSpec("vicuna7b_b16", 16, 32, 32, 128, "bf16",
                                 (256, 2048), (64,), 4, 32000, 0.3),
    # Vicuna-13B geometry, batch 8, 4k context
    "vicuna13b_b8": WorkloadSpec("vicuna13b_b8", 8, 40, 40, 128, "bf16",
                                 (4096, 4096), (64,), 5, 32000, 0.35),
    # large-batch stress with mixed tree sizes (1 = plain decode)
    "stress_b64": WorkloadSpec("stress_b64", 64, 32, 32, 128, "bf16",
                               (128, 8192), (1, 8, 26, 64), 4, 32000, 0.25),
    # the plain-decode rows of the stress shape on their own: every sequence
    # has only its root (T = 1)
    "decode_b64": WorkloadSpec("decode_b64", 64, 32, 32, 128, "bf16",
                               (128, 8192), (1,), 0, 32000, 0.25, t_max=1),
    # the 7B batch-16 shape with grouped query heads: 32 query heads sharing
    # 8 KV heads (4 per KV head)
    "gqa_b16": WorkloadSpec("gqa_b16", 16, 32, 8, 128, "bf16",
                            (256, 2048), (64,), 4, 32000, 0.3),
}


@dataclasses.dataclass
class Workload:
    spec: WorkloadSpec
    seed: int
    ctx_lens: np.ndarray       # int32 [B]
    tree_sizes: np.ndarray     # int32 [B]  real nodes per sequence
    tree_parent: np.ndarray    # int32 [B][t_max]  -1 root, -2 padding
    tree_depth: np.ndarray     # int32 [B][t_max]
    cand_tokens: np.ndarray    # int32 [B][t_max]
    node_argmax: np.ndarray    # int32 [B][t_max]
    block_table: np.ndarray    # int32 [B][max_blocks]  -1 where unused
    num_blocks: int
    max_ctx_len: int           # host-side upper bound on ctx_lens
    q: torch.Tensor            # [B][t_max][H][d]
    k_new: torch.Tensor        # [B][t_max][Hkv][d]
    v_new: torch.Tensor        # [B][t_max][Hkv][d]
    kv_pages: torch.Tensor     # [num_blocks][2][Hkv][16][d]

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.spec.dtype == "bf16" else torch.float32

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def tree_tokens(self) -> int:
        return int(self.tree_sizes.sum())

    @property
    def max_depth(self) -> int:
        real = self.tree_parent != PAD_PARENT
        return int(self.tree_depth[real].max())


# ----------------------------------------------------------------- trees ---

def full_binary_tree(depth: int):
    """Parents of the full binary tree of the given depth, in BFS order."""
    n = 2 ** (depth + 1) - 1
    parent = np.full(n, -1, dtype=np.int32)
    for i in range(1, n):
        parent[i] = (i - 1) // 2
    return parent


def random_tree(rng: np.random.Generator, n: int, max_depth: int):
    """Random tree of n nodes, depth <= max_depth, relabelled in BFS order."""
    cap = min(max_depth, n - 1)
    par = [-1]
    dep = [0]
    for _ in range(1, n):
        open_nodes = [j for j in range(len(par)) if dep[j] < cap]
        p = open_nodes[int(rng.integers(len(open_nodes)))]
        par.append(p)
        dep.append(dep[p] + 1)
    children = [[] for _ in range(n)]
    for j in range(1, n):
        children[par[j]].append(j)          # creation order
    order = [0]
    head = 0
    while head < len(order):
        order.extend(children[order[head]])
        head += 1
    new_id = {old: new for new, old in enumerate(order)}
    parent = np.full(n, -1, dtype=np.int32)
    for old in range(1, n):
        parent[new_id[old]] = new_id[par[old]]
    return parent


def depths_of(parent: np.ndarray) -> np.ndarray:
    """Depth of each node from a BFS-ordered parent array (-1 root, -2 pad)."""
    d = np.zeros(len(parent), dtype=np.int32)
    for i in range(len(parent)):
        if parent[i] >= 0:
            d[i] = d[parent[i]] + 1
    return d


def draw_tokens(rng: np.random.Generator, parent: np.ndarray, vocab: int,
                p_match: float):
    """Candidate tokens (distinct among siblings) and planted greedy argmax."""
    n = len(parent)
    children = [[] for _ in range(n)]
    for i in range(1, n):
        children[parent[i]].append(i)
    cand = np.zeros(n, dtype=np.int32)
    cand[0] = int(rng.integers(vocab))
    for u in range(n):
        ch = children[u]
        if ch:
            toks = rng.choice(vocab, size=len(ch), replace=False)
            for c, t in zip(ch, toks):
                cand[c] = int(t)
    argmax = np.zeros(n, dtype=np.int32)
    for u in range(n):
        ch = children[u]
        if ch and rng.random() < p_match:
            argmax[u] = cand[ch[int(rng.integers(len(ch)))]]
        else:
            taken = {int(cand[c]) for c in ch}
            while True:
                t = int(rng.integers(vocab))
                if t not in taken:
                    break
            argmax[u] = t
    return cand, argmax


# ----------------------------------------------------------- dense data ---

def _normal(seed_seq: np.random.SeedSequence, shape, dtype: torch.dtype,
            chunk_elems: int = 1 << 24) -> torch.Tensor:
    """N(0,1) drawn in fp32, then rounded (RNE) to `dtype`.  The tensor is cut
    into fixed-size chunks, each drawn from its own spawned PCG64 stream, so
    the values do not depend on how many threads fill it."""
    out = torch.empty(shape, dtype=dtype)
    flat = out.view(-1)
    n = flat.numel()
    starts = list(range(0, n, chunk_elems))
    seqs = seed_seq.spawn(len(starts))

    def fill(k):
        s = starts[k]
        e = min(n, s + chunk_elems)
        g = np.random.Generator(np.random.PCG64(seqs[k]))
        x = g.standard_normal(e - s, dtype=np.float32)
        flat[s:e] = torch.from_numpy(x).to(dtype)

    workers = max(1, min(16, len(os.sched_getaffinity(0)), len(starts)))
    if workers == 1:
        for k in range(len(starts)):
            fill(k)
    else:
        with concurrent.futures.ThreadPoolExecutor(workers) as ex:
            list(ex.map(fill, range(len(starts))))
    return out


def make_workload(name: str, seed: int = 0, *, batch: Optional[int] = None,
                  ctx_range: Optional[tuple] = None,
                  tree_sizes: Optional[tuple] = None,
                  max_depth: Optional[int] = None,
                  heads: Optional[int] = None,
                  kv_heads: Optional[int] = None,
                  head_dim: Optional[int] = None,
                  chain: bool = False,
                  extra_pool_blocks: int = 0) -> Workload:
    """Build a seeded workload.  Keyword overrides shrink or reshape a preset
    (for parity tests at sizes the oracle finishes quickly); `chain` makes
    every tree a single path (list decoding)."""
    spec = SPECS[name]
    repl = {}
    if batch is not None:
        repl["batch"] = batch
    if ctx_range is not None:
        repl["ctx_range"] = tuple(ctx_range)
    if tree_sizes is not None:
        repl["tree_sizes"] = tuple(tree_sizes)
        repl["t_max"] = max(max(tree_sizes), 1) if spec.full_binary else max(
            spec.t_max, max(tree_sizes))
    if max_depth is not None:
        repl["max_depth"] = max_depth
    if heads is not None:
        repl["heads"] = heads
        repl["kv_heads"] = heads
    if kv_heads is not None:
        repl["kv_heads"] = kv_heads
    if head_dim is not None:
        repl["head_dim"] = head_dim
    if repl:
        spec = dataclasses.replace(spec, **repl)
    ss = np.random.SeedSequence([seed, 0x6D656475])
    s_meta, s_q, s_k, s_v, s_pool = ss.spawn(5)
    r_meta = np.random.Generator(np.random.PCG64(s_meta))
    B, T = spec.batch, spec.t_max
    lo, hi = spec.ctx_range
    ctx = r_meta.integers(lo, hi + 1, size=B).astype(np.int32)
    sizes = np.array([spec.tree_sizes[int(r_meta.integers(len(spec.tree_sizes)))]
                      for _ in range(B)], dtype=np.int32)
    parent = np.full((B, T), PAD_PARENT, dtype=np.int32)
    cand = np.zeros((B, T), dtype=np.int32)
    amax = np.zeros((B, T), dtype=np.int32)
    for b in range(B):
        n = int(sizes[b])
        if spec.full_binary and not chain:
            d = spec.max_depth  # deep enough for n nodes (a size override may ask for more)
            while 2 ** (d + 1) - 1 < n:
                d += 1
            pb = full_binary_tree(d)[:n]
        elif chain:
            pb = np.arange(-1, n - 1, dtype=np.int32)
        else:
            pb = random_tree(r_meta, n, spec.max_depth)
        parent[b, :n] = pb
        c, a = draw_tokens(r_meta, pb, spec.vocab, spec.p_match)
        cand[b, :n] = c
        amax[b, :n] = a
    depth = np.stack([depths_of(parent[b]) for b in range(B)]).astype(np.int32)
    dmax = int(depth.max())
    per_seq = [math.ceil((int(ctx[b]) + dmax + 1) / BLOCK_SIZE) for b in range(B)]
    # table columns cover the context bound plus one accepted path
    max_blocks = max(max(per_seq), math.ceil((hi + dmax + 1) / BLOCK_SIZE))
    nblocks = sum(per_seq) + extra_pool_blocks
    perm = r_meta.permutation(nblocks).astype(np.int32)
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        table[b, :per_seq[b]] = perm[off:off + per_seq[b]]
        off += per_seq[b]
    tdt = torch.bfloat16 if spec.dtype == "bf16" else torch.float32
    H, Hkv, d = spec.heads, spec.kv_heads, spec.head_dim
    q = _normal(s_q, (B, T, H, d), tdt)
    k_new = _normal(s_k, (B, T, Hkv, d), tdt)
    v_new = _normal(s_v, (B, T, Hkv, d), tdt)
    pool = _normal(s_pool, (nblocks, 2, Hkv, BLOCK_SIZE, d), tdt)
    return Workload(spec=spec, seed=seed, ctx_lens=ctx, tree_sizes=sizes,
                    tree_parent=parent, tree_depth=depth, cand_tokens=cand,
                    node_argmax=amax, block_table=table, num_blocks=nblocks,
                    max_ctx_len=int(hi), q=q, k_new=k_new, v_new=v_new,
                    kv_pages=pool)


def make_logits(wl: Workload, seed: int = 0, *, vocab: Optional[int] = None,
                dtype: torch.dtype = torch.bfloat16, scale: float = 2.0,
                planted_margin: float = 4.0, ties: int = 0) -> torch.Tensor:
    """Base-model logits after every tree node, [B][T][vocab] on the CPU.

    Values are scale * N(0,1) (drawn in fp32, rounded to `dtype`); in each row
    the token wl.node_argmax[b][i] is then raised to the row's largest value
    plus `planted_margin`, so the rows' greedy tokens are the workload's
    planted ones (and acceptance sees the workload's match rate).  With
    ties > 0, that many other random tokens of each row are set to the same
    value, so equal maxima occur (the greedy token is then the smallest id
    among them, no longer necessarily the planted one)."""
    B, T = wl.node_argmax.shape
    V = vocab or wl.spec.vocab
    rng = np.random.default_rng(np.random.SeedSequence([seed, 0x10C175]))
    x = _normal(np.random.SeedSequence([seed, 0x10C176]), (B, T, V), torch.float32) * scale
    top = x.max(dim=-1).values + planted_margin            # [B][T]
    tok = torch.from_numpy(np.asarray(wl.node_argmax, dtype=np.int64) % V)
    x.scatter_(-1, tok.unsqueeze(-1), top.unsqueeze(-1))
    if ties > 0:
        extra = torch.from_numpy(rng.integers(0, V, size=(B, T, ties)))
        x.scatter_(-1, extra, top.unsqueeze(-1).expand(B, T, ties))
    return x.to(dtype)


def make_choices(seed: int = 0, n: int = 63, max_depth: int = 4, topk: int = 10):
    """A synthetic "medusa choices" list: n distinct paths of top-k ranks,
    prefix-closed (every path's prefixes are in the list), at most max_depth
    long.  Grown from the root: a random existing node (the root or a path
    shorter than max_depth, shallower ones more likely) gets its next child
    rank (0, 1, 2, ... up to topk - 1), as lists tuned for an acceptance rate
    favour the heads' best ranks."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 0xC401CE]))
    children = {(): 0}
    paths = []
    while len(paths) < n:
        open_nodes = [p for p in children if len(p) < max_depth and children[p] < topk]
        w = np.array([0.5 ** len(p) for p in open_nodes])
        p = open_nodes[int(rng.choice(len(open_nodes), p=w / w.sum()))]
        c = p + (children[p],)
        children[p] += 1
        children[c] = 0
        paths.append(c)
    return paths


def make_head_logits(batch: int, heads: int, vocab: int, seed: int = 0,
                     dtype: torch.dtype = torch.bfloat16, ties: int = 0) -> torch.Tensor:
    """Medusa head logits [batch][heads][vocab]: 2 * N(0,1) drawn in fp32 and
    rounded to `dtype`; with ties > 0, each row's maximum is copied to that
    many random other tokens (equal logits among the top)."""
    x = _normal(np.random.SeedSequence([seed, 0x4EAD5]), (batch, heads, vocab),
                torch.float32) * 2.0
    if ties > 0:
        rng = np.random.default_rng(np.random.SeedSequence([seed, 0x4EAD6]))
        top = x.max(dim=-1).values
        extra = torch.from_numpy(rng.integers(0, vocab, size=(batch, heads, ties)))
        x.scatter_(-1, extra, top.unsqueeze(-1).expand(batch, heads, ties))
    return x.to(dtype)
