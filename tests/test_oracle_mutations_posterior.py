"""The pins of the posterior and candidate oracles catch plausible mistakes.

As in test_oracle_mutations.py: each case plants one mistake in the oracle on
the CPU (monkeypatching one function, in the oracle module and in the test
modules that imported it by name) and checks that at least one pin of
test_oracle_posterior.py / test_oracle_candidates.py then fails.
"""
import functools
import json
import os

import numpy as np
import pytest

import oracle.candidates as oc
import oracle.posterior as op
import tests.test_oracle_candidates as pc
import tests.test_oracle_posterior as pp
from oracle.tree_verify import PAD_PARENT, _np

_orig_softmax_stats = op.softmax_stats
_orig_topk = oc.topk_tokens


# ------------------------------------------------------------- argmax ----

def _argmax_tie_largest(logits):
    x = _np(logits).astype(np.float64)
    x = np.where(np.isnan(x), -np.inf, x)
    m = x.max(axis=-1, keepdims=True)
    hit = x == m
    V = x.shape[-1]
    return (V - 1 - np.argmax(hit[..., ::-1], axis=-1)).astype(np.int32)


def _argmax_nan_wins(logits):
    x = _np(logits).astype(np.float64)
    return np.argmax(np.where(np.isnan(x), np.inf, x), axis=-1).astype(np.int32)


# ------------------------------------------------------- softmax stats ----

def _stats_no_temperature(logits, temperature=1.0):
    return _orig_softmax_stats(logits, 1.0)


def _stats_log2_entropy(logits, temperature=1.0):
    p, H = _orig_softmax_stats(logits, temperature)
    return p, H / np.log(2.0)


# ------------------------------------------------- typical acceptance ----

def _typical(logits, cand_tokens, tree_parent, temperature=1.0, epsilon=0.09, delta=0.3,
             combine=np.minimum, own_row=False):
    par = np.asarray(tree_parent)
    cand = np.asarray(cand_tokens)
    B, T = par.shape
    p, H = op.softmax_stats(logits, temperature)
    thresh = combine(epsilon, delta * np.exp(-H))
    ok = np.zeros((B, T), dtype=bool)
    for b in range(B):
        for i in range(T):
            if par[b, i] == PAD_PARENT:
                break
            if i == 0:
                ok[b, i] = True
            else:
                n = i if own_row else int(par[b, i])
                v = p[b, n, int(cand[b, i])]
                ok[b, i] = v > thresh[b, n]
    return (*op._longest_path(ok, par), ok)


_typical_max = functools.partial(_typical, combine=np.maximum)
_typical_own_row = functools.partial(_typical, own_row=True)


def _longest_path_ignores_ancestors(ok, par):
    """Deepest passing node, whether or not its ancestors passed."""
    B, T = par.shape
    L = np.zeros(B, dtype=np.int32)
    P = -np.ones((B, T), dtype=np.int32)
    for b in range(B):
        depth = np.zeros(T, dtype=np.int64)
        best = 0
        for i in range(1, T):
            if par[b, i] == PAD_PARENT:
                break
            depth[i] = depth[int(par[b, i])] + 1
            if ok[b, i] and depth[i] > depth[best]:
                best = i
        path, n = [], best
        while True:
            path.append(n)
            if n == 0:
                break
            n = int(par[b, n])
        path.reverse()
        L[b] = len(path)
        P[b, :len(path)] = path
    return L, P


# ----------------------------------------------------------- candidates ----

def _topk_tie_largest(logits, k):
    x = _np(logits).astype(np.float64)
    x = np.where(np.isnan(x), -np.inf, x)
    V = x.shape[-1]
    flat = x.reshape(-1, V)
    out = np.empty((flat.shape[0], k), dtype=np.int32)
    for r in range(flat.shape[0]):
        out[r] = np.lexsort((-np.arange(V), -flat[r]))[:k]
    return out.reshape(*x.shape[:-1], k)


def _topk_nan_first(logits, k):
    x = _np(logits).astype(np.float64)
    x = np.where(np.isnan(x), np.inf, x)
    return _orig_topk(x, k)


def _choice_tree_lex_only(choices):
    paths = sorted(tuple(c) for c in choices)
    index = {(): 0}
    for n, c in enumerate(paths):
        index[c] = n + 1
    parent, depth = [-1], [0]
    for c in paths:
        if c[:-1] not in index:
            raise ValueError("missing prefix")
        parent.append(index[c[:-1]])
        depth.append(len(c))
    return paths, np.array(parent, dtype=np.int32), np.array(depth, dtype=np.int32)


def _assemble(head_logits, choices, root_token, t_max, k, head_of=lambda c: len(c) - 1,
              rank_of=lambda c: c[-1]):
    paths, parent, depth = oc.choice_tree(choices)
    top = oc.topk_tokens(head_logits, k)
    root = np.asarray(root_token)
    B = top.shape[0]
    n = len(paths) + 1
    cand = np.zeros((B, t_max), dtype=np.int32)
    par = np.full((B, t_max), PAD_PARENT, dtype=np.int32)
    dep = np.zeros((B, t_max), dtype=np.int32)
    for b in range(B):
        cand[b, 0] = root[b]
        for i, c in enumerate(paths, start=1):
            cand[b, i] = top[b, head_of(c), rank_of(c)]
        par[b, :n] = parent
        dep[b, :n] = depth
    return cand, par, dep


_assemble_head_off = functools.partial(_assemble, head_of=lambda c: len(c) % 2)
_assemble_rank_first = functools.partial(_assemble, rank_of=lambda c: c[0])


MUTATIONS = {
    "argmax_tie_largest": ("vocab_argmax", _argmax_tie_largest),
    "argmax_nan_wins": ("vocab_argmax", _argmax_nan_wins),
    "stats_no_temperature": ("softmax_stats", _stats_no_temperature),
    "stats_log2_entropy": ("softmax_stats", _stats_log2_entropy),
    "typical_threshold_max": ("typical_accept", _typical_max),
    "typical_child_row": ("typical_accept", _typical_own_row),
    "typical_path_ignores_ancestors": ("_longest_path", _longest_path_ignores_ancestors),
    "topk_tie_largest": ("topk_tokens", _topk_tie_largest),
    "topk_nan_first": ("topk_tokens", _topk_nan_first),
    "choices_lexicographic_only": ("choice_tree", _choice_tree_lex_only),
    "candidates_wrong_head": ("assemble_candidates", _assemble_head_off),
    "candidates_first_rank": ("assemble_candidates", _assemble_rank_first),
}

_GOLDEN_TYPICAL = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                              "typical_tiny.json")))["cases"]

PINS = [
    pp.test_argmax_brute_force_with_many_ties,
    pp.test_argmax_matches_numpy_on_finite_rows,
    pp.test_argmax_special_rows,
    pp.test_argmax_of_bf16_tensor_uses_exact_values,
    pp.test_softmax_stats_against_scipy,
    pp.test_entropy_closed_forms,
    *[functools.partial(pp.test_typical_golden, c) for c in _GOLDEN_TYPICAL],
    pp.test_typical_reduces_to_greedy_on_peaked_rows,
    pp.test_typical_flat_rows_accept_everything,
    pc.test_topk_brute_force_with_ties,
    pc.test_topk_brute_force_with_nan_and_infinities,
    pc.test_topk_matches_stable_sort,
    pc.test_golden_tree_and_candidates,
    functools.partial(pc.test_synthetic_choice_lists_are_trees, 0, 63, 4),
    pc.test_assembly_brute_force,
]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_some_pin_fails_under_mutation(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    for mod in (op, oc, pp, pc):
        if hasattr(mod, attr):
            monkeypatch.setattr(mod, attr, fn)
    failed = []
    for pin in PINS:
        try:
            pin()
        except (AssertionError, IndexError, ValueError):
            failed.append(getattr(pin, "__name__", getattr(pin, "func", pin).__name__))
    assert failed, f"no pin caught mutation {name}"


def test_pins_pass_without_mutation():
    for pin in PINS:
        pin()
