"""Plain CPU reference of the steps around acceptance (test infrastructure).

Sources:
  [LMD-1231]  LMDeploy PR #1231 "[WIP] support Medusa" - evaluate_posterior
              at LM-head temperature 0: the base model's greedy token after
              each tree node, compared with the node's children.
  [vLLM-1171] vLLM issue #1171 - the typical acceptance scheme named as one
              of the two non-standard parts of Medusa serving.

Readings where the pages are silent (each listed in the design notes):
  * the greedy token of a node is the argmax of its logits row over the
    vocabulary, the smallest token id among equal maxima; a row with no
    comparable value (all NaN) gives token 0;
  * typical acceptance (the rule of the Medusa paper, which the pages only
    name): with p = softmax(logits / temperature) after node n and
    H = -sum p log p its entropy, child c of n is accepted iff
    p[cand_tokens[c]] > min(epsilon, delta * exp(-H)); the accepted path is
    then chosen as in greedy acceptance (deepest, smallest index).
"""
from __future__ import annotations

import numpy as np

from .tree_verify import PAD_PARENT, _np


def vocab_argmax(logits) -> np.ndarray:
    """[..., V] -> int32 [...]: smallest v with logits[..., v] equal to the row
    maximum ([LMD-1231] greedy token at temperature 0).  The comparison is
    exact: bf16 and fp32 values are compared as the real numbers they are."""
    x = _np(logits).astype(np.float64)
    comparable = ~np.isnan(x)
    m = np.where(comparable, x, -np.inf).max(axis=-1, keepdims=True)
    hit = comparable & (x == m)
    # first hit along the vocabulary; rows with no hit (all NaN) -> 0
    idx = np.argmax(hit, axis=-1)
    return idx.astype(np.int32)


def softmax_stats(logits, temperature: float = 1.0):
    """Per row: probabilities p = softmax(logits / temperature) and entropy
    H = -sum p log p (natural log), in fp64."""
    x = _np(logits).astype(np.float64) / float(temperature)
    m = x.max(axis=-1, keepdims=True)
    e = np.exp(x - m)
    z = e.sum(axis=-1, keepdims=True)
    p = e / z
    with np.errstate(divide="ignore", invalid="ignore"):
        plogp = np.where(p > 0, p * np.log(p), 0.0)
    return p, -plogp.sum(axis=-1)


def typical_accept(logits, cand_tokens, tree_parent, temperature: float = 1.0,
                   epsilon: float = 0.09, delta: float = 0.3):
    """Typical acceptance ([vLLM-1171] names the scheme; rule as in the
    module docstring).  Returns (accept_len [B], accept_path [B][T]) with the
    same conventions as accept_greedy, and the per-node acceptance test
    ok [B][T] (root always true) for inspection."""
    par = np.asarray(tree_parent)
    cand = np.asarray(cand_tokens)
    B, T = par.shape
    p, H = softmax_stats(logits, temperature)           # p [B][T][V], H [B][T]
    thresh = np.minimum(epsilon, delta * np.exp(-H))    # [B][T]
    ok = np.zeros((B, T), dtype=bool)
    for b in range(B):
        for i in range(T):
            if par[b, i] == PAD_PARENT:
                break
            if i == 0:
                ok[b, i] = True
            else:
                n = int(par[b, i])
                ok[b, i] = p[b, n, int(cand[b, i])] > thresh[b, n]
    return (*_longest_path(ok, par), ok)


def _longest_path(ok, par):
    """Deepest node whose whole root path passes `ok` (smallest index among
    equals); path by depth, -1 after (the walk accept_greedy performs)."""
    B, T = par.shape
    accept_len = np.zeros(B, dtype=np.int32)
    accept_path = -np.ones((B, T), dtype=np.int32)
    for b in range(B):
        matched = np.zeros(T, dtype=bool)
        depth = np.zeros(T, dtype=np.int64)
        best = 0
        for i in range(T):
            if par[b, i] == PAD_PARENT:
                break
            if i == 0:
                matched[0] = True
                continue
            n = int(par[b, i])
            matched[i] = matched[n] and ok[b, i]
            depth[i] = depth[n] + 1
            if matched[i] and depth[i] > depth[best]:
                best = i
        path = []
        n = best
        while True:
            path.append(n)
            if n == 0:
                break
            n = int(par[b, n])
        path.reverse()
        accept_len[b] = len(path)
        accept_path[b, :len(path)] = path
    return accept_len, accept_path
