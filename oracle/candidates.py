"""Plain CPU reference of Medusa candidate assembly (test infrastructure).

Source: LMDeploy PR #1231 "[WIP] support Medusa" - generate_candidates: the
candidate tokens of the tree come from the Medusa heads' top-k predictions,
laid out by a fixed list of "medusa choices" (64 nodes in the PR's tests).

Readings where the pages are silent (each listed in the design notes):
  * a choice is a path (r_1, ..., r_d) of top-k ranks: the node it names sits
    at depth d, carries the r_d-th best token of Medusa head d-1 (head h
    predicts the token at depth h+1), and its parent is the node named by
    (r_1, ..., r_{d-1}) (the root for d = 1);
  * nodes are numbered root 0, then the choices sorted by length and, within a
    length, lexicographically (node = 1 + position), which puts every parent
    before its children;
  * the root carries the token the previous step decided (its input here);
  * top-k orders tokens by logit, larger first, the smaller token id first
    among equal logits (NaN is never ranked above a number);
  * tree rows beyond the last node are padding (parent -2, depth 0, token 0).
"""
from __future__ import annotations

import numpy as np

from .tree_verify import PAD_PARENT, _np


def topk_tokens(logits, k: int) -> np.ndarray:
    """[..., V] -> int32 [..., k]: the k best tokens of each row."""
    x = _np(logits).astype(np.float64)
    x = np.where(np.isnan(x), -np.inf, x)
    V = x.shape[-1]
    ids = np.broadcast_to(np.arange(V), x.shape)
    # lexsort: last key is primary -> primary -value, secondary token id
    flat_x = x.reshape(-1, V)
    out = np.empty((flat_x.shape[0], k), dtype=np.int32)
    for r in range(flat_x.shape[0]):
        order = np.lexsort((ids.reshape(-1, V)[r], -flat_x[r]))
        out[r] = order[:k]
    return out.reshape(*x.shape[:-1], k)


def choice_tree(choices):
    """choices: list of tuples of ranks.  Returns (paths in node order,
    parent [n+1], depth [n+1]); node 0 is the root (parent -1, depth 0)."""
    paths = sorted((tuple(c) for c in choices), key=lambda c: (len(c), c))
    if len(set(paths)) != len(paths):
        raise ValueError("duplicate choice")
    index = {(): 0}
    for n, c in enumerate(paths):
        index[c] = n + 1
    parent = [-1]
    depth = [0]
    for c in paths:
        if len(c) == 0:
            raise ValueError("empty choice")
        if c[:-1] not in index:
            raise ValueError(f"choice {c} has no parent in the list")
        parent.append(index[c[:-1]])
        depth.append(len(c))
    return paths, np.array(parent, dtype=np.int32), np.array(depth, dtype=np.int32)


def assemble_candidates(head_logits, choices, root_token, t_max: int, k: int):
    """head_logits [B][H_medusa][V], root_token [B] -> (cand_tokens,
    tree_parent, tree_depth), each int32 [B][t_max]."""
    paths, parent, depth = choice_tree(choices)
    top = topk_tokens(head_logits, k)                       # [B][H][k]
    root = np.asarray(root_token)
    B = top.shape[0]
    n = len(paths) + 1
    if n > t_max:
        raise ValueError("more nodes than t_max")
    cand = np.zeros((B, t_max), dtype=np.int32)
    par = np.full((B, t_max), PAD_PARENT, dtype=np.int32)
    dep = np.zeros((B, t_max), dtype=np.int32)
    for b in range(B):
        cand[b, 0] = root[b]
        for i, c in enumerate(paths, start=1):
            cand[b, i] = top[b, len(c) - 1, c[-1]]
        par[b, :n] = parent
        dep[b, :n] = depth
    return cand, par, dep
