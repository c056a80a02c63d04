"""Pins of the oracle's greedy-token argmax and typical acceptance against
things other than themselves: brute force, library routines (numpy argmax,
scipy softmax and entropy), closed forms and hand-worked fixtures.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle.posterior import softmax_stats, typical_accept, vocab_argmax

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------- argmax ----

def _argmax_brute(row):
    best, best_i = None, 0
    for i, x in enumerate(row):
        if math.isnan(x):
            continue
        if best is None or x > best:
            best, best_i = x, i
    return best_i


def test_argmax_brute_force_with_many_ties():
    rng = np.random.default_rng(0)
    x = rng.integers(-3, 4, size=(40, 9, 57)).astype(np.float32)  # lots of equal maxima
    got = vocab_argmax(x)
    for idx in np.ndindex(x.shape[:-1]):
        assert got[idx] == _argmax_brute(list(x[idx])), idx


def test_argmax_matches_numpy_on_finite_rows():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((16, 64, 1000)).astype(np.float32)
    assert np.array_equal(vocab_argmax(x), np.argmax(x, axis=-1))


def test_argmax_special_rows():
    ninf, nan = -np.inf, np.nan
    x = np.array([[ninf, ninf, ninf],          # all -inf: first
                  [nan, nan, nan],             # nothing comparable: 0
                  [nan, 1.0, 1.0],             # NaN skipped, first max
                  [2.0, np.inf, np.inf],       # +inf wins, first one
                  [-0.0, 0.0, -1.0]],          # -0 == +0: first
                 dtype=np.float32)
    assert vocab_argmax(x).tolist() == [0, 0, 1, 1, 0]


def test_argmax_of_bf16_tensor_uses_exact_values():
    import torch
    v = torch.tensor([[1.0, 1.00390625, 1.0078125, 1.00390625]], dtype=torch.bfloat16)
    assert vocab_argmax(v).tolist() == [2]


# ------------------------------------------------------- softmax stats ----

def test_softmax_stats_against_scipy():
    from scipy.special import softmax
    from scipy.stats import entropy
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 7, 300)) * 3
    for t in (1.0, 0.7, 2.5):
        p, H = softmax_stats(x, t)
        assert np.allclose(p, softmax(x / t, axis=-1), rtol=1e-12, atol=1e-15)
        assert np.allclose(H, entropy(softmax(x / t, axis=-1), axis=-1), rtol=1e-10)


def test_entropy_closed_forms():
    V = 32000
    p, H = softmax_stats(np.zeros((1, V)))
    assert np.allclose(p, 1.0 / V) and math.isclose(H[0], math.log(V), rel_tol=1e-12)
    # two-point distribution q, 1-q
    q = 0.3
    _, H2 = softmax_stats(np.array([[math.log(q), math.log(1 - q)]]))
    assert math.isclose(H2[0], -(q * math.log(q) + (1 - q) * math.log(1 - q)), rel_tol=1e-12)


# ------------------------------------------------- typical acceptance ----

@pytest.mark.parametrize("case", json.load(open(os.path.join(GOLDEN, "typical_tiny.json")))["cases"],
                         ids=lambda c: c["name"])
def test_typical_golden(case):
    logits = np.log(np.array(case["logits_log_weights"], dtype=np.float64))
    par = np.array(case["tree_parent"], dtype=np.int32)
    cand = np.array(case["cand_tokens"], dtype=np.int32)
    L, P, ok = typical_accept(logits, cand, par, case["temperature"], case["epsilon"],
                              case["delta"])
    _, H = softmax_stats(logits, case["temperature"])
    thr = np.minimum(case["epsilon"], case["delta"] * np.exp(-H))
    assert np.allclose(thr, case["threshold"], atol=5e-6)
    assert ok.tolist() == case["ok"]
    assert L.tolist() == case["accept_len"] and P.tolist() == case["accept_path"]


def test_typical_reduces_to_greedy_on_peaked_rows():
    """With one token far above the rest (p ~ 1, H ~ 0, threshold = epsilon),
    a child passes iff it carries that token: greedy acceptance."""
    from synth import make_workload
    wl = make_workload("vicuna7b_b16", 3, batch=6, heads=1, ctx_range=(16, 16))
    B, T = wl.tree_parent.shape
    V = 64
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((B, T, V))
    amax = rng.integers(0, V, size=(B, T))
    logits[np.arange(B)[:, None], np.arange(T)[None, :], amax] = 60.0
    cand = np.where(rng.random((B, T)) < 0.5, amax[np.arange(B)[:, None], np.maximum(wl.tree_parent, 0)],
                    rng.integers(0, V, size=(B, T))).astype(np.int32)
    L, P, _ = typical_accept(logits, cand, wl.tree_parent)
    Lg, Pg = oracle.accept_greedy(amax.astype(np.int32), cand, wl.tree_parent)
    assert np.array_equal(L, Lg) and np.array_equal(P, Pg)


def test_typical_flat_rows_accept_everything():
    """Uniform rows: p = 1/V > delta/V = threshold, so every node passes and
    the deepest node (smallest index among equals) ends the path."""
    from synth import make_workload
    wl = make_workload("vicuna7b_b16", 4, batch=5, heads=1, ctx_range=(16, 16))
    B, T = wl.tree_parent.shape
    L, P, ok = typical_accept(np.zeros((B, T, 100)), wl.cand_tokens % 100, wl.tree_parent)
    real = wl.tree_parent != oracle.PAD_PARENT
    assert np.all(ok[real])
    dmax = np.where(real, wl.tree_depth, -1).max(axis=1)
    assert np.array_equal(L, dmax + 1)
