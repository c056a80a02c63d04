"""The pins catch plausible oracle mistakes.

Each case plants one mistake in the oracle (on the CPU, by monkeypatching one
of its functions) and checks that at least one pin from the oracle test files
then fails.  A pin set that let any of these through would not be pinning the
oracle to the pages.
"""
import numpy as np
import pytest

import oracle
import oracle.tree_verify as tv
import tests.test_oracle_accept as pa
import tests.test_oracle_attention as pt
import tests.test_oracle_commit as pc

_orig_rope_exact = tv.rope_exact
_orig_rope_pinned = tv.rope_pinned
_orig_ancestors = tv.ancestors
_orig_accept = tv.accept_greedy


def _rope_sign(x, pos, base=tv.ROPE_BASE):
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    ang = np.asarray(pos, dtype=np.float64)[..., None] * tv.inv_freq(d, base)
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([x1 * c + x2 * s, x2 * c - x1 * s], axis=-1)


def _rope_interleaved(x, pos, base=tv.ROPE_BASE):
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    ang = np.asarray(pos, dtype=np.float64)[..., None] * tv.inv_freq(d, base)
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., 0::2], x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2] = x1 * c - x2 * s
    y[..., 1::2] = x2 * c + x1 * s
    return y


def _rope_pos_plus_one(x, pos, base=tv.ROPE_BASE):
    return _orig_rope_exact(x, np.asarray(pos) + 1, base)


def _anc_no_self(parent_row):
    return [m & ~(1 << i) if m else 0 for i, m in enumerate(_orig_ancestors(parent_row))]


def _anc_all(parent_row):
    full = sum(1 << j for j, p in enumerate(parent_row) if int(p) != tv.PAD_PARENT)
    return [full if m else 0 for m in _orig_ancestors(parent_row)]


def _anc_parent_only(parent_row):
    out = []
    for i, p in enumerate(parent_row):
        p = int(p)
        if p == tv.PAD_PARENT:
            out.append(0)
        else:
            out.append((1 << i) | ((1 << p) if p >= 0 else 0))
    return out


def _rope_pinned_fma(x32, cos32, sin32):
    x = np.asarray(x32, dtype=np.float64)
    d = x.shape[-1]
    c = np.asarray(cos32, dtype=np.float64)
    s = np.asarray(sin32, dtype=np.float64)
    x1, x2 = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1).astype(np.float32)


def _accept_largest_tie(node_argmax, cand_tokens, tree_parent):
    """Tie-break by the largest index instead of the smallest."""
    node_argmax, cand_tokens = np.asarray(node_argmax), np.asarray(cand_tokens)
    tree_parent = np.asarray(tree_parent)
    B, T = tree_parent.shape
    L = np.zeros(B, dtype=np.int32)
    P = np.full((B, T), -1, dtype=np.int32)
    for b in range(B):
        par = tree_parent[b]
        ok, dep, best = [False] * T, [0] * T, 0
        ok[0] = True
        for i in range(1, T):
            p = int(par[i])
            if p == tv.PAD_PARENT:
                continue
            dep[i] = dep[p] + 1
            ok[i] = ok[p] and cand_tokens[b, i] == node_argmax[b, p]
            if ok[i] and dep[i] >= dep[best]:
                best = i
        path, j = [], best
        while j >= 0:
            path.append(j)
            j = int(par[j])
        L[b] = len(path)
        P[b, : len(path)] = path[::-1]
    return L, P


def _accept_ignores_parent(node_argmax, cand_tokens, tree_parent):
    """Accept an edge even when its parent was rejected."""
    ones = np.array(node_argmax)
    L, P = _orig_accept(node_argmax, cand_tokens, tree_parent)
    B, T = np.asarray(tree_parent).shape
    for b in range(B):
        par = np.asarray(tree_parent)[b]
        best, bd = 0, 0
        for i in range(1, T):
            p = int(par[i])
            if p == tv.PAD_PARENT:
                continue
            d, j = 1, p
            while int(par[j]) >= 0:
                j = int(par[j])
                d += 1
            if cand_tokens[b][i] == ones[b][p] and d > bd:
                best, bd = i, d
        path, j = [], best
        while j >= 0:
            path.append(j)
            j = int(par[j])
        L[b] = len(path)
        P[b] = -1
        P[b, : len(path)] = path[::-1]
    return L, P


MUTATIONS = {
    "rope_sign": ("rope_exact", _rope_sign),
    "rope_interleaved": ("rope_exact", _rope_interleaved),
    "rope_position_off_by_one": ("rope_exact", _rope_pos_plus_one),
    "mask_without_self": ("ancestors", _anc_no_self),
    "mask_whole_tree": ("ancestors", _anc_all),
    "mask_parent_only": ("ancestors", _anc_parent_only),
    "commit_rotation_fused": ("rope_pinned", _rope_pinned_fma),
    "accept_tie_largest": ("accept_greedy", _accept_largest_tie),
    "accept_ignores_parent": ("accept_greedy", _accept_ignores_parent),
}

PINS = [
    pt.test_chain_tree_equals_causal_attention,
    pt.test_every_node_equals_its_own_path,
    pt.test_single_node_tree_is_decode_attention,
    pt.test_non_ancestor_independence,
    pt.test_one_hot_values_give_probabilities,
    pa.test_exhaustive_small_trees,
    pa.test_hand_worked_examples,
    pc.test_pinned_rotation_matches_emulation,
    pc.test_commit_bf16_slots_and_bits,
    pc.test_two_steps_resume_equals_causal_attention,
]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_some_pin_fails_under_mutation(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(tv, attr, fn)
    monkeypatch.setattr(oracle, attr, fn)
    failed = []
    for pin in PINS:
        try:
            pin()
        except (AssertionError, IndexError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught mutation {name}"
