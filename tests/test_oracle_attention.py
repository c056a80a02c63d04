"""Pins of the oracle's tree attention against things other than itself.

* RoPE: transformers' Llama rotary embedding (rotate-half, base 10000) - a
  library routine for the neox-style rotation; relative-position property;
  position 0 is the identity.
* Attention: torch's scaled_dot_product_attention in fp64 with an explicit
  boolean mask on the de-paged sequence (pages concatenated block by block):
  - a chain tree equals ordinary causal attention with a KV cache (list
    decoding, mlc-llm issue "[Feature Request] Medusa support");
  - every node equals causal attention over ctx + its own root-to-node path
    (verifying each path as its own sequence, the "multi-batch" alternative
    of LMDeploy PR "[WIP] support Medusa");
  - T = 1 equals single-query decode (vLLM issue #1171, paged_attention).
* Invariants: block-table permutation, non-ancestor independence, V = 1,
  one-hot V gives probabilities that sum to one.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from synth import make_workload


def _arrays(wl):
    f = lambda t: t.to(torch.float32).numpy() if t.dtype == torch.bfloat16 else t.numpy()
    return (f(wl.q), f(wl.k_new), f(wl.v_new), f(wl.kv_pages), wl.block_table,
            wl.ctx_lens, wl.tree_parent, wl.tree_depth)


def _hf_rope(x64: torch.Tensor, pos: torch.Tensor, d: int):
    """transformers' Llama RoPE on x [n][d] at integer positions pos [n]."""
    from transformers import LlamaConfig
    from transformers.models.llama.modeling_llama import (LlamaRotaryEmbedding,
                                                          apply_rotary_pos_emb)
    cfg = LlamaConfig(hidden_size=d * 2, num_attention_heads=2, head_dim=d,
                      rope_theta=10000.0)
    emb = LlamaRotaryEmbedding(cfg)
    cos, sin = emb(x64.float()[None], pos[None])
    xr, _ = apply_rotary_pos_emb(x64[None, None], x64[None, None],
                                 cos.double(), sin.double())
    return xr[0, 0]


def _depaged(pool, table_row, ctx, hk):
    """Concatenate whole pages in logical-block order, then cut to ctx."""
    nb = (ctx + 15) // 16
    K = np.concatenate([pool[table_row[j], 0, hk] for j in range(nb)], axis=0)[:ctx]
    V = np.concatenate([pool[table_row[j], 1, hk] for j in range(nb)], axis=0)[:ctx]
    return K.astype(np.float64), V.astype(np.float64)


def _sdpa(qr, K, V, mask, scale):
    q = torch.from_numpy(np.ascontiguousarray(qr))[None, None]
    k = torch.from_numpy(np.ascontiguousarray(K))[None, None]
    v = torch.from_numpy(np.ascontiguousarray(V))[None, None]
    m = torch.from_numpy(mask)[None, None]
    return F.scaled_dot_product_attention(q, k, v, attn_mask=m, scale=scale)[0, 0].numpy()


# ------------------------------------------------------------------- RoPE --

@pytest.mark.parametrize("d", [64, 128])
def test_rope_matches_transformers_llama(d):
    rng = np.random.default_rng(1)
    x = rng.standard_normal((40, d))
    pos = rng.integers(0, 300, size=40)
    ours = oracle.rope_exact(x, pos)
    ref = _hf_rope(torch.from_numpy(x), torch.from_numpy(pos), d).numpy()
    # transformers forms the angle in fp32: ~pos*2^-24 rad of slack
    assert np.max(np.abs(ours - ref)) < 2e-4


def test_rope_relative_position_and_identity():
    rng = np.random.default_rng(2)
    d = 128
    q = rng.standard_normal(d)
    k = rng.standard_normal(d)
    assert np.array_equal(oracle.rope_exact(q, 0), q)
    for m, n, shift in [(5, 3, 100), (1000, 990, 57), (17, 40, 4000)]:
        a = oracle.rope_exact(q, m) @ oracle.rope_exact(k, n)
        b = oracle.rope_exact(q, m + shift) @ oracle.rope_exact(k, n + shift)
        assert abs(a - b) < 1e-9
    # rotation: norms preserved, and it is not the interleaved (GPT-J) pairing
    assert abs(np.linalg.norm(oracle.rope_exact(q, 123)) - np.linalg.norm(q)) < 1e-12
    e0 = np.zeros(d)
    e0[0] = 1.0
    r = oracle.rope_exact(e0, 1)
    assert abs(r[0] - np.cos(1.0)) < 1e-15 and abs(r[d // 2] - np.sin(1.0)) < 1e-15
    assert r[1] == 0.0


def test_rope_table_matches_exact():
    tab = oracle.rope_table(128, 9000)
    x = np.zeros(128)
    x[:64] = 1.0
    for p in [0, 1, 777, 8999]:
        r = oracle.rope_exact(x, p)
        assert np.max(np.abs(r[:64] - tab[p, :, 0])) < 1e-7
        assert np.max(np.abs(r[64:] - tab[p, :, 1])) < 1e-7


# -------------------------------------------------------------- attention --

def test_chain_tree_equals_causal_attention():
    wl = make_workload("vicuna7b_bs1", 3, batch=2, heads=2, ctx_range=(35, 70),
                       tree_sizes=(9,), chain=True)
    q, kn, vn, pool, table, ctx, par, dep = _arrays(wl)
    out = oracle.verify(q, kn, vn, pool, table, ctx, par, dep)
    d = q.shape[-1]
    for b in range(2):
        c = int(ctx[b])
        T = int(wl.tree_sizes[b])
        pos = torch.arange(c, c + T)
        for h in range(2):
            Kc, Vc = _depaged(pool, table[b], c, h)
            kt = _hf_rope(torch.from_numpy(kn[b, :T, h].astype(np.float64)), pos, d).numpy()
            qt = _hf_rope(torch.from_numpy(q[b, :T, h].astype(np.float64)), pos, d).numpy()
            K = np.concatenate([Kc, kt])
            V = np.concatenate([Vc, vn[b, :T, h].astype(np.float64)])
            mask = np.tril(np.ones((T, c + T), dtype=bool), k=c)
            ref = _sdpa(qt, K, V, mask, 1.0 / np.sqrt(d))
            assert np.max(np.abs(out[b, :T, h] - ref)) < 2e-4


def test_every_node_equals_its_own_path():
    wl = make_workload("vicuna7b_bs1", 4, batch=2, heads=2, ctx_range=(20, 50),
                       tree_sizes=(24,))
    q, kn, vn, pool, table, ctx, par, dep = _arrays(wl)
    out = oracle.verify(q, kn, vn, pool, table, ctx, par, dep)
    d = q.shape[-1]
    for b in range(2):
        c = int(ctx[b])
        for h in range(2):
            Kc, Vc = _depaged(pool, table[b], c, h)
            for i in range(int(wl.tree_sizes[b])):
                path = []
                j = i
                while j >= 0:
                    path.append(j)
                    j = int(par[b, j])
                path = path[::-1]                       # root ... i
                pos = torch.arange(c, c + len(path))
                kt = _hf_rope(torch.from_numpy(kn[b, path, h].astype(np.float64)), pos, d).numpy()
                qi = _hf_rope(torch.from_numpy(q[b, [i], h].astype(np.float64)),
                              pos[-1:], d).numpy()
                K = np.concatenate([Kc, kt])
                V = np.concatenate([Vc, vn[b, path, h].astype(np.float64)])
                mask = np.ones((1, len(K)), dtype=bool)
                ref = _sdpa(qi, K, V, mask, 1.0 / np.sqrt(d))[0]
                assert np.max(np.abs(out[b, i, h] - ref)) < 2e-4


def test_single_node_tree_is_decode_attention():
    wl = make_workload("stress_b64", 5, batch=3, heads=2, ctx_range=(1, 90),
                       tree_sizes=(1,))
    q, kn, vn, pool, table, ctx, par, dep = _arrays(wl)
    out = oracle.verify(q, kn, vn, pool, table, ctx, par, dep)
    d = q.shape[-1]
    for b in range(3):
        c = int(ctx[b])
        for h in range(2):
            Kc, Vc = _depaged(pool, table[b], c, h)
            pos = torch.tensor([c])
            k0 = _hf_rope(torch.from_numpy(kn[b, [0], h].astype(np.float64)), pos, d).numpy()
            q0 = _hf_rope(torch.from_numpy(q[b, [0], h].astype(np.float64)), pos, d).numpy()
            K = np.concatenate([Kc, k0])
            V = np.concatenate([Vc, vn[b, [0], h].astype(np.float64)])
            ref = _sdpa(q0, K, V, np.ones((1, len(K)), dtype=bool), 1.0 / np.sqrt(d))[0]
            assert np.max(np.abs(out[b, 0, h] - ref)) < 2e-4


def test_empty_context_root_sees_only_itself():
    wl = make_workload("vicuna7b_bs1", 6, batch=1, heads=1, ctx_range=(0, 0),
                       tree_sizes=(5,))
    q, kn, vn, pool, table, ctx, par, dep = _arrays(wl)
    out = oracle.verify(q, kn, vn, pool, table, ctx, par, dep)
    assert np.array_equal(out[0, 0, 0], vn[0, 0, 0].astype(np.float64))


def test_block_table_permutation_invariance():
    wl = make_workload("vicuna7b_bs1", 7, batch=2, heads=2, ctx_range=(40, 80),
                       tree_sizes=(10,))
    q, kn, vn, pool, table, ctx, par, dep = _arrays(wl)
    out = oracle.verify(q, kn, vn, pool, table, ctx, par, dep)
    rng = np.random.default_rng(0)
    perm = rng.permutation(pool.shape[0])          # physical -> new physical
    pool2 = np.empty_like(pool)
    pool2[perm] = pool
    table2 = np.where(table >= 0, perm[np.maximum(table, 0)], -1)
    out2 = oracle.verify(q, kn, vn, pool2, table2, ctx, par, dep)
    assert np.array_equal(out, out2)


def test_non_ancestor_independence():
    wl = make_workload("vicuna7b_bs1", 8, batch=1, heads=2, ctx_range=(30, 30),
                       tree_sizes=(20,))
    q, kn, vn, pool, table, ctx, par, dep = _arrays(wl)
    out = oracle.verify(q, kn, vn, pool, table, ctx, par, dep)
    anc = oracle.ancestors(par[0])
    i = 19
    others = [j for j in range(20) if not (anc[i] >> j) & 1]
    assert others
    kn2, vn2, q2 = kn.copy(), vn.copy(), q.copy()
    kn2[0, others] += 3.0
    vn2[0, others] -= 5.0
    q2[0, others] *= -1.0
    out2 = oracle.verify(q2, kn2, vn2, pool, table, ctx, par, dep)
    assert np.array_equal(out[0, i], out2[0, i])
    assert not np.array_equal(out[0, others[0]], out2[0, others[0]])


def test_unit_values_give_unit_output():
    wl = make_workload("vicuna7b_bs1", 9, batch=2, heads=2, ctx_range=(10, 60),
                       tree_sizes=(16,))
    q, kn, vn, pool, table, ctx, par, dep = _arrays(wl)
    pool = pool.copy()
    pool[:, 1] = 1.0
    vn = np.ones_like(vn)
    out = oracle.verify(q, kn, vn, pool, table, ctx, par, dep)
    real = par != oracle.PAD_PARENT
    assert np.max(np.abs(out[real] - 1.0)) < 1e-12


def test_one_hot_values_give_probabilities():
    """With V rows = basis vectors, out = the attention probabilities of each
    key; they sum to 1, vanish on masked tree keys, and match an independent
    softmax of the scores."""
    d = 128
    wl = make_workload("vicuna7b_bs1", 10, batch=1, heads=1, ctx_range=(40, 40),
                       tree_sizes=(12,))
    q, kn, vn, pool, table, ctx, par, dep = _arrays(wl)
    c = 40
    pool = pool.copy()
    vn = np.zeros_like(vn)
    for t in range(c):
        blk, slot = table[0, t // 16], t % 16
        pool[blk, 1, 0, slot] = 0.0
        pool[blk, 1, 0, slot, t] = 1.0
    for j in range(12):
        vn[0, j, 0, c + j] = 1.0
    out = oracle.verify(q, kn, vn, pool, table, ctx, par, dep)
    anc = oracle.ancestors(par[0])
    Kc, _ = _depaged(pool, table[0], c, 0)
    for i in range(12):
        p = out[0, i, 0]
        assert abs(p.sum() - 1.0) < 1e-12
        for j in range(12):
            if not (anc[i] >> j) & 1:
                assert p[c + j] == 0.0
        cols = [j for j in range(12) if (anc[i] >> j) & 1]
        pos = torch.tensor([c + int(dep[0, j]) for j in cols])
        kt = _hf_rope(torch.from_numpy(kn[0, cols, 0].astype(np.float64)), pos, d).numpy()
        qi = _hf_rope(torch.from_numpy(q[0, [i], 0].astype(np.float64)),
                      torch.tensor([c + int(dep[0, i])]), d).numpy()[0]
        s = np.concatenate([Kc @ qi, kt @ qi]) / np.sqrt(d)
        ref = torch.softmax(torch.from_numpy(s), 0).numpy()
        got = np.concatenate([p[:c], p[[c + j for j in cols]]])
        assert np.max(np.abs(got - ref)) < 1e-4
