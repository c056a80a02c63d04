"""Pins of the oracle's greedy acceptance.

* Exhaustive enumeration: every tree shape with T <= 7 nodes (every parent
  array with parent[i] < i) and every one of the 2^(T-1) edge-match patterns,
  checked against a brute force that lists every root-to-node path, keeps the
  paths whose every edge matches, and takes the longest (smallest end index
  among equals).  Patterns where several siblings match realise duplicate
  sibling tokens, the tie-break's adversarial case.
* Closed forms: all edges match -> D+1; none -> (1, [0]); chain -> 1 + the
  matching prefix.
* Hand-worked example (tests/golden/accept_tiny.json).
* Generator statistics: E[accept_len] from the recursion
  E[L(n)] = 1 + p * mean_{c child of n} E[L(c)], E[L(leaf)] = 1, which gives
  1.75 for the full binary tree of depth 2 at p = 0.5.

Greedy acceptance at LM-head temperature 0 over the candidate tree follows
LMDeploy PR "[WIP] support Medusa" (evaluate_posterior) and the greedy-only
remark in vLLM issue #1171.
"""
import itertools
import json
import os

import numpy as np

import oracle
from synth import make_workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _all_parent_arrays(T):
    ranges = [range(i) for i in range(1, T)]
    for ps in itertools.product(*ranges):
        yield [-1] + list(ps)


def _brute(parent, match_edge):
    """match_edge[i] for i >= 1: edge parent[i] -> i matches."""
    T = len(parent)
    best = None
    for end in range(T):
        path = []
        j = end
        while j >= 0:
            path.append(j)
            j = parent[j]
        path.reverse()
        if all(match_edge[k] for k in path[1:]):
            if best is None or len(path) > len(best):
                best = path
    return best


def _realise(parent, pattern, rng):
    """Tokens / argmax that make exactly the edges in `pattern` match."""
    T = len(parent)
    argmax = rng.integers(100, 200, size=T)
    cand = np.zeros(T, dtype=np.int64)
    for i in range(1, T):
        if pattern[i]:
            cand[i] = argmax[parent[i]]
        else:
            cand[i] = argmax[parent[i]] + 1000 + i
    return cand, argmax


def test_exhaustive_small_trees():
    rng = np.random.default_rng(0)
    n_cases = 0
    for T in range(1, 8):
        shapes = list(_all_parent_arrays(T))
        pats = list(itertools.product([False, True], repeat=T - 1))
        # batch many (shape, pattern) cases into one oracle call
        rows_p, rows_c, rows_a, expect = [], [], [], []
        for par in shapes:
            for pat in pats:
                pattern = [True] + list(pat)
                cand, amax = _realise(par, pattern, rng)
                rows_p.append(par)
                rows_c.append(cand)
                rows_a.append(amax)
                expect.append(_brute(par, pattern))
        P = np.array(rows_p, dtype=np.int32)
        C = np.array(rows_c, dtype=np.int32)
        A = np.array(rows_a, dtype=np.int32)
        L, path = oracle.accept_greedy(A, C, P)
        for r, exp in enumerate(expect):
            assert L[r] == len(exp)
            assert list(path[r, : L[r]]) == exp
            assert np.all(path[r, L[r]:] == -1)
        n_cases += len(expect)
    assert n_cases == sum(
        int(np.prod(range(1, T))) * 2 ** (T - 1) for T in range(1, 8))


def test_closed_forms_random_trees():
    for seed in range(20):
        wl = make_workload("vicuna7b_bs1", seed, batch=4, heads=1, ctx_range=(1, 1),
                           tree_sizes=(64,))
        par = wl.tree_parent
        dep = wl.tree_depth
        B, T = par.shape
        # all edges match
        amax = np.zeros((B, T), dtype=np.int32) + 7
        cand = np.zeros((B, T), dtype=np.int32) + 7
        L, path = oracle.accept_greedy(amax, cand, par)
        for b in range(B):
            D = int(dep[b].max())
            assert L[b] == D + 1
            end = int(np.flatnonzero(dep[b] == D)[0])
            assert path[b, L[b] - 1] == end
        # nothing matches
        cand = cand + 1
        L, path = oracle.accept_greedy(amax, cand, par)
        assert np.all(L == 1) and np.all(path[:, 0] == 0) and np.all(path[:, 1:] == -1)


def test_chain_closed_form():
    rng = np.random.default_rng(3)
    for _ in range(200):
        T = int(rng.integers(1, 65))
        par = np.arange(-1, T - 1, dtype=np.int32)[None]
        amax = rng.integers(0, 3, size=(1, T)).astype(np.int32)
        cand = rng.integers(0, 3, size=(1, T)).astype(np.int32)
        k = 0
        while k + 1 < T and cand[0, k + 1] == amax[0, k]:
            k += 1
        L, path = oracle.accept_greedy(amax, cand, par)
        assert L[0] == k + 1
        assert list(path[0, : k + 1]) == list(range(k + 1))


def test_padding_nodes_never_match():
    par = np.array([[-1, 0, 0, 1, -2, -2]], dtype=np.int32)
    amax = np.array([[5, 6, 0, 0, 9, 9]], dtype=np.int32)
    cand = np.array([[0, 5, 5, 6, 6, 6]], dtype=np.int32)
    L, path = oracle.accept_greedy(amax, cand, par)
    assert L[0] == 3 and list(path[0]) == [0, 1, 3, -1, -1, -1]


def test_hand_worked_examples():
    with open(os.path.join(GOLDEN, "accept_tiny.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        L, path = oracle.accept_greedy(np.array([c["node_argmax"]], dtype=np.int32),
                                       np.array([c["cand_tokens"]], dtype=np.int32),
                                       np.array([c["tree_parent"]], dtype=np.int32))
        assert int(L[0]) == c["accept_len"], c["why"]
        assert list(path[0]) == c["accept_path"], c["why"]


def _expected_len(parent, p):
    T = len(parent)
    kids = [[] for _ in range(T)]
    for i in range(1, T):
        if parent[i] >= 0:
            kids[parent[i]].append(i)
    e = [1.0] * T
    for n in reversed(range(T)):
        if kids[n]:
            e[n] = 1.0 + p * np.mean([e[c] for c in kids[n]])
    return e[0]


def test_generator_statistics_tiny():
    """Full binary tree of depth 2, p = 0.5: E[accept_len] = 1.75."""
    assert abs(_expected_len([-1, 0, 0, 1, 1, 2, 2], 0.5) - 1.75) < 1e-12
    Ls = []
    for seed in range(3000):
        wl = make_workload("tiny", seed)
        L, _ = oracle.accept_greedy(wl.node_argmax, wl.cand_tokens, wl.tree_parent)
        Ls.append(int(L[0]))
    m = np.mean(Ls)
    se = np.std(Ls) / np.sqrt(len(Ls))
    assert abs(m - 1.75) < 4 * se, (m, se)


def test_generator_statistics_random_trees():
    diffs, ses = [], []
    Ls, Es = [], []
    for seed in range(60):
        wl = make_workload("vicuna7b_b16", seed, heads=1, ctx_range=(1, 1))
        L, _ = oracle.accept_greedy(wl.node_argmax, wl.cand_tokens, wl.tree_parent)
        for b in range(wl.spec.batch):
            Ls.append(int(L[b]))
            Es.append(_expected_len(list(wl.tree_parent[b]), wl.spec.p_match))
    m, e = np.mean(Ls), np.mean(Es)
    se = np.std(np.array(Ls) - np.array(Es)) / np.sqrt(len(Ls))
    assert abs(m - e) < 4 * se, (m, e, se)
