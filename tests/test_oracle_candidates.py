"""Pins of the oracle's candidate assembly: brute force, numpy's stable
sort, a hand-worked fixture and tree invariants on synthetic choice lists."""
import json
import os

import numpy as np
import pytest

import oracle
from oracle.candidates import assemble_candidates, choice_tree, topk_tokens
from synth import make_choices, make_head_logits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_topk_brute_force_with_ties():
    rng = np.random.default_rng(0)
    x = rng.integers(-2, 3, size=(30, 4, 23)).astype(np.float32)
    got = topk_tokens(x, 7)
    for idx in np.ndindex(x.shape[:-1]):
        row = list(x[idx])
        ref = sorted(range(len(row)), key=lambda i: (-row[i], i))[:7]
        assert got[idx].tolist() == ref


def test_topk_brute_force_with_nan_and_infinities():
    """NaN ranks as -inf (after every number, among the -inf entries by
    token); +inf ranks first."""
    import math
    rng = np.random.default_rng(2)
    x = rng.integers(-2, 3, size=(20, 3, 19)).astype(np.float32)
    x[rng.random(x.shape) < 0.2] = np.nan
    x[rng.random(x.shape) < 0.1] = -np.inf
    x[rng.random(x.shape) < 0.05] = np.inf
    got = topk_tokens(x, 12)
    for idx in np.ndindex(x.shape[:-1]):
        row = [(-math.inf if math.isnan(v) else float(v)) for v in x[idx]]
        ref = sorted(range(len(row)), key=lambda i: (-row[i], i))[:12]
        assert got[idx].tolist() == ref


def test_topk_matches_stable_sort():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((8, 5, 2000)).astype(np.float32)
    ref = np.argsort(-x, axis=-1, kind="stable")[..., :10]
    assert np.array_equal(topk_tokens(x, 10), ref)


def test_golden_tree_and_candidates():
    g = json.load(open(os.path.join(GOLDEN, "choices_tiny.json")))
    paths, par, dep = choice_tree([tuple(c) for c in g["choices"]])
    assert [list(p) for p in paths] == g["node_paths"][1:]
    assert par.tolist() == g["tree_parent"] and dep.tolist() == g["tree_depth"]
    logits = np.array(g["head_logits"], dtype=np.float32)
    assert topk_tokens(logits, 2).tolist() == g["topk_2"]
    cand, p2, d2 = assemble_candidates(logits, [tuple(c) for c in g["choices"]],
                                       g["root_token"], g["t_max"], 2)
    assert cand.tolist() == g["cand_tokens"]
    assert p2.tolist() == g["padded_parent"] and d2.tolist() == g["padded_depth"]


@pytest.mark.parametrize("seed,n,depth", [(0, 63, 4), (1, 63, 5), (2, 7, 2), (3, 1, 1)])
def test_synthetic_choice_lists_are_trees(seed, n, depth):
    choices = make_choices(seed, n=n, max_depth=depth)
    paths, par, dep = choice_tree(choices)
    assert len(paths) == n == len(set(paths))
    assert max(len(p) for p in paths) <= depth
    for i in range(1, n + 1):
        assert 0 <= par[i] < i and dep[i] == dep[par[i]] + 1
        p = paths[i - 1]
        assert (paths[par[i] - 1] if par[i] > 0 else ()) == p[:-1]
    # node order: by length, then lexicographic
    assert paths == sorted(paths, key=lambda c: (len(c), c))


def test_assembly_brute_force():
    choices = make_choices(4, n=40, max_depth=4, topk=6)
    B, H, V = 5, 4, 300
    logits = make_head_logits(B, H, V, seed=4, ties=2)
    root = np.arange(B, dtype=np.int32) * 11
    cand, par, dep = assemble_candidates(logits, choices, root, 64, 6)
    x = logits.float().numpy()
    paths = sorted(choices, key=lambda c: (len(c), c))
    for b in range(B):
        assert cand[b, 0] == root[b]
        for i, c in enumerate(paths, start=1):
            row = list(x[b, len(c) - 1])
            ranked = sorted(range(V), key=lambda t: (-row[t], t))
            assert cand[b, i] == ranked[c[-1]]
        assert np.all(par[b, len(paths) + 1:] == oracle.PAD_PARENT)


def test_invalid_choice_lists_rejected():
    with pytest.raises(ValueError):
        choice_tree([(0,), (0,)])           # duplicate
    with pytest.raises(ValueError):
        choice_tree([(0,), (1, 0)])         # (1,) missing
