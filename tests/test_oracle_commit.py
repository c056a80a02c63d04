"""Pins of the oracle's KV commit and of the bit-level arithmetic it fixes.

* fp32 rotation with one rounding per operation and no fused multiply-add:
  checked against a pure-Python emulation (each product / sum formed in
  Python's binary64 and rounded once to binary32 with struct, which is exact
  for a product of two binary32 values and innocuous double rounding for a
  sum).
* fp32 -> bf16 round-to-nearest-even: checked against an exact rational
  rounding (fractions) and against torch's float -> bfloat16 conversion.
* Commit: the changed bytes are exactly the closed-form slots
  p = ctx_len + i -> (block_table[p // 16], p % 16); V bytes equal v_new
  bytes; K bytes equal the emulated rotation; every other byte is unchanged.
* Resume: verify -> accept -> commit, then a second verify at
  ctx_len + accept_len equals causal attention over the whole sequence
  (the KV-cache update of mlc-llm issue "[Feature Request] Medusa support"
  and the block-table update of vLLM issue #1171).
"""
import math
import struct
from fractions import Fraction

import numpy as np
import torch
import torch.nn.functional as F

import oracle
from synth import make_workload


def _f32(x: float) -> float:
    return struct.unpack("<f", struct.pack("<f", x))[0]


def _bits32(x: float) -> int:
    return struct.unpack("<I", struct.pack("<f", x))[0]


def _emulated_rot(x1, x2, c, s):
    y1 = _f32(_f32(x1 * c) - _f32(x2 * s))
    y2 = _f32(_f32(x2 * c) + _f32(x1 * s))
    return y1, y2


def _bf16_exact(y: float) -> int:
    """bf16 bits of the binary32 value y, nearest with ties to even, by exact
    rational arithmetic."""
    if y == 0.0:
        return _bits32(y) >> 16
    sign = 0x8000 if y < 0 else 0
    a = Fraction(abs(y))
    e = math.frexp(abs(y))[1]                 # |y| = m * 2^e, m in [0.5, 1)
    ulp_exp = max(e - 8, -133)                # 8 significant bits; subnormal floor
    ulp = Fraction(2) ** ulp_exp
    qn = round(a / ulp)                       # Fraction round: half to even
    val = qn * ulp
    return sign | (_bits32(float(val)) >> 16)


def test_pinned_rotation_matches_emulation():
    rng = np.random.default_rng(0)
    tab = oracle.rope_table(128, 4200)
    x = rng.standard_normal((300, 128)).astype(np.float32)
    pos = rng.integers(0, 4200, size=300)
    y = oracle.rope_pinned(x, tab[pos, :, 0], tab[pos, :, 1])
    for r in range(300):
        for k in range(0, 64, 7):
            c, s = float(tab[pos[r], k, 0]), float(tab[pos[r], k, 1])
            e1, e2 = _emulated_rot(float(x[r, k]), float(x[r, k + 64]), c, s)
            assert _bits32(float(y[r, k])) == _bits32(e1)
            assert _bits32(float(y[r, k + 64])) == _bits32(e2)


def test_bf16_rounding_exact_and_matches_torch():
    rng = np.random.default_rng(1)
    vals = list(rng.standard_normal(3000).astype(np.float32))
    # exact ties: low 16 bits == 0x8000, with even and odd kept bits
    for hi in (0x3F80, 0x3F81, 0xBF80, 0xBF81, 0x4049, 0x0001):
        vals.append(np.uint32((hi << 16) | 0x8000).view(np.float32))
    vals += [np.float32(v) for v in (0.0, -0.0, 1e-40, -3.0e-39, 65504.0, 3.3895e38)]
    arr = np.array(vals, dtype=np.float32)
    ours = oracle.f32_to_bf16_bits(arr)
    torch_bits = torch.from_numpy(arr).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, torch_bits)
    for v, o in zip(arr, ours):
        assert int(o) == _bf16_exact(float(v)), float(v)


def _pool_bits(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).reshape(-1)
    return t.numpy().view(np.uint32).reshape(-1)


def _check_commit(wl, L, path, new_pool, tab):
    old = _pool_bits(wl.kv_pages)
    new = _pool_bits(new_pool)
    Hkv, d = wl.spec.kv_heads, wl.spec.head_dim
    bf16 = wl.kv_pages.dtype == torch.bfloat16
    kf = wl.k_new.to(torch.float32).numpy()
    vbits = _pool_bits(wl.v_new).reshape(wl.v_new.shape)
    touched = np.zeros(old.shape, dtype=bool)
    n_rows = 0
    for b in range(wl.spec.batch):
        for i in range(int(L[b])):
            n = int(path[b, i])
            p = int(wl.ctx_lens[b]) + i
            blk = int(wl.block_table[b, p // 16])
            slot = p % 16
            n_rows += 1
            for h in range(Hkv):
                for kv in (0, 1):
                    base = (((blk * 2 + kv) * Hkv + h) * 16 + slot) * d
                    touched[base:base + d] = True
                    if kv == 1:
                        assert np.array_equal(new[base:base + d], vbits[b, n, h])
                        continue
                    for k in range(d // 2):
                        c, s = float(tab[p, k, 0]), float(tab[p, k, 1])
                        y1, y2 = _emulated_rot(float(kf[b, n, h, k]),
                                               float(kf[b, n, h, k + d // 2]), c, s)
                        if bf16:
                            e1, e2 = _bf16_exact(y1), _bf16_exact(y2)
                        else:
                            e1, e2 = _bits32(y1), _bits32(y2)
                        assert int(new[base + k]) == e1
                        assert int(new[base + k + d // 2]) == e2
    assert n_rows > wl.spec.batch          # some path longer than the root
    assert np.array_equal(new[~touched], old[~touched])


def test_commit_bf16_slots_and_bits():
    wl = make_workload("vicuna7b_bs1", 11, batch=3, heads=2, ctx_range=(5, 60),
                       tree_sizes=(20,))
    amax = np.full_like(wl.node_argmax, 7)
    cand = np.full_like(wl.cand_tokens, 7)           # every edge matches
    L, path = oracle.accept_greedy(amax, cand, wl.tree_parent)
    tab = oracle.rope_table(128, 200)
    new = oracle.commit(wl.k_new, wl.v_new, L, path, wl.kv_pages, wl.block_table,
                        wl.ctx_lens, tab)
    _check_commit(wl, L, path, new, tab)


def test_commit_f32_slots_and_bits():
    wl = make_workload("tiny", 12, batch=2, ctx_range=(14, 47))
    L, path = oracle.accept_greedy(np.full_like(wl.node_argmax, 3),
                                   np.full_like(wl.cand_tokens, 3), wl.tree_parent)
    tab = oracle.rope_table(64, 100)
    new = oracle.commit(wl.k_new, wl.v_new, L, path, wl.kv_pages, wl.block_table,
                        wl.ctx_lens, tab)
    _check_commit(wl, L, path, new, tab)


def test_two_steps_resume_equals_causal_attention():
    from transformers.models.llama.modeling_llama import apply_rotary_pos_emb
    d = 64
    wl = make_workload("tiny", 13, heads=2, ctx_range=(20, 40), tree_sizes=(12,),
                       chain=True)
    par = wl.tree_parent.copy()
    par[:, 6:] = oracle.PAD_PARENT                      # step 1 uses 6 nodes
    dep = np.where(par == oracle.PAD_PARENT, 0, wl.tree_depth)
    amax = np.arange(12, dtype=np.int32)[None] + 100
    cand = np.concatenate([[0], amax[0, :-1]])[None].astype(np.int32)
    cand[0, 4] = 1                                      # edge 3 -> 4 fails
    L, path = oracle.accept_greedy(amax, cand, par)
    assert L[0] == 4
    c0 = int(wl.ctx_lens[0])
    tab = oracle.rope_table(d, c0 + 20)
    pool1 = oracle.commit(wl.k_new, wl.v_new, L, path, wl.kv_pages, wl.block_table,
                          wl.ctx_lens, tab)
    # step 2: a fresh chain of 5 nodes on top of ctx + 4
    rng = np.random.default_rng(5)
    q2 = rng.standard_normal((1, 12, 2, d)).astype(np.float32)
    k2 = rng.standard_normal((1, 12, 2, d)).astype(np.float32)
    v2 = rng.standard_normal((1, 12, 2, d)).astype(np.float32)
    par2 = np.full((1, 12), oracle.PAD_PARENT, dtype=np.int32)
    par2[0, :5] = [-1, 0, 1, 2, 3]
    dep2 = np.zeros((1, 12), dtype=np.int32)
    dep2[0, :5] = range(5)
    c1 = np.array([c0 + 4], dtype=np.int32)
    out = oracle.verify(q2, k2, v2, pool1.numpy(), wl.block_table, c1, par2, dep2)

    def rope(x, pos):
        x = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))
        inv = 1.0 / (10000.0 ** (torch.arange(0, d, 2, dtype=torch.float64) / d))
        ang = torch.tensor(pos, dtype=torch.float64)[:, None] * inv[None]
        emb = torch.cat([ang, ang], dim=-1)
        r, _ = apply_rotary_pos_emb(x[None, None], x[None, None], emb.cos()[None],
                                    emb.sin()[None])
        return r[0, 0].numpy()

    pool0 = wl.kv_pages.numpy()
    for h in range(2):
        nb = (c0 + 15) // 16
        Kc = np.concatenate([pool0[wl.block_table[0, j], 0, h] for j in range(nb)])[:c0]
        Vc = np.concatenate([pool0[wl.block_table[0, j], 1, h] for j in range(nb)])[:c0]
        acc = list(path[0, :4])
        K1 = rope(wl.k_new[0, acc, h].numpy(), list(range(c0, c0 + 4)))
        V1 = wl.v_new[0, acc, h].numpy()
        pos2 = list(range(c0 + 4, c0 + 9))
        K2 = rope(k2[0, :5, h], pos2)
        Q2 = rope(q2[0, :5, h], pos2)
        K = np.concatenate([Kc, K1, K2]).astype(np.float64)
        V = np.concatenate([Vc, V1, v2[0, :5, h]]).astype(np.float64)
        mask = np.tril(np.ones((5, c0 + 9), dtype=bool), k=c0 + 4)
        ref = F.scaled_dot_product_attention(
            torch.from_numpy(Q2)[None, None], torch.from_numpy(K)[None, None],
            torch.from_numpy(V)[None, None], attn_mask=torch.from_numpy(mask)[None, None],
            scale=1.0 / math.sqrt(d))[0, 0].numpy()
        assert np.max(np.abs(out[0, :5, h] - ref)) < 1e-5
