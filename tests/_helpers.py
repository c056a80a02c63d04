"""Plumbing shared by the GPU parity tests: device copies of a workload,
compact sub-problems for sampled oracle checks, and the oracle calls."""
from __future__ import annotations

import numpy as np
import torch

import oracle


def dev(wl, device="cuda"):
    """Device tensors of a workload (inputs only; nothing computed)."""
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)
    return dict(
        q=wl.q.to(device), k_new=wl.k_new.to(device), v_new=wl.v_new.to(device),
        kv_pages=wl.kv_pages.to(device), block_table=i32(wl.block_table),
        ctx_lens=i32(wl.ctx_lens), tree_parent=i32(wl.tree_parent),
        tree_depth=i32(wl.tree_depth), node_argmax=i32(wl.node_argmax),
        cand_tokens=i32(wl.cand_tokens))


def verifier(wl, flags=0, device="cuda", max_ctx_len=None, split_tokens=0):
    from medusa_tree_attention_attn_amd import TreeVerifier
    s = wl.spec
    return TreeVerifier(batch=s.batch, t_max=s.t_max, num_heads=s.heads,
                        num_kv_heads=s.kv_heads, head_dim=s.head_dim,
                        max_blocks_per_seq=wl.max_blocks, num_blocks=wl.num_blocks,
                        max_ctx_len=wl.max_ctx_len if max_ctx_len is None else max_ctx_len,
                        dtype=wl.torch_dtype, device=device, flags=flags,
                        split_tokens=split_tokens)


def sub_problem(wl, seqs):
    """Sequences `seqs` with only the pages they reference, renumbered: the
    oracle then needs no copy of the whole pool."""
    seqs = list(seqs)
    table = wl.block_table[seqs]
    used = np.unique(table[table >= 0])
    remap = -np.ones(wl.num_blocks, dtype=np.int64)
    remap[used] = np.arange(len(used))
    new_table = np.where(table >= 0, remap[np.maximum(table, 0)], -1).astype(np.int32)
    pool = wl.kv_pages.index_select(0, torch.from_numpy(used))
    return dict(q=wl.q[seqs], k_new=wl.k_new[seqs], v_new=wl.v_new[seqs], kv_pages=pool,
                block_table=new_table, ctx_lens=wl.ctx_lens[seqs],
                tree_parent=wl.tree_parent[seqs], tree_depth=wl.tree_depth[seqs])


def oracle_verify_rows(wl, seqs, heads=None):
    """Oracle output [len(seqs)][T][len(heads)][d] for the sampled rows."""
    sp = sub_problem(wl, seqs)
    f = lambda t: t.to(torch.float32).numpy()
    q, kn, vn, pool = f(sp["q"]), f(sp["k_new"]), f(sp["v_new"]), f(sp["kv_pages"])
    heads = list(range(wl.spec.heads)) if heads is None else list(heads)
    T, d = wl.spec.t_max, wl.spec.head_dim
    out = np.zeros((len(seqs), T, len(heads), d))
    for bi in range(len(seqs)):
        for hi, h in enumerate(heads):
            out[bi, :, hi] = oracle.verify_head(q, kn, vn, pool, sp["block_table"],
                                                sp["ctx_lens"], sp["tree_parent"],
                                                sp["tree_depth"], bi, h)
    return out


def pool_bits(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)
