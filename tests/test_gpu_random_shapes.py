"""Parity over seeded random shapes: each case draws its configuration from a
generator seeded by the case number, so a failure names a reproducible
shape.  Verify (every kernel the library routes to: grid, persistent,
plain, decode; splits; grouped query heads; bf16 and fp32; head_dim 64 and
128; empty, sub-page and long contexts; mixed tree sizes) against the
oracle on sampled rows; greedy acceptance and the KV commit, separate and
fused, bit-exact over the whole pool; vocabulary argmax, argmax +
acceptance and candidate assembly bit-exact.  The fixed-shape tests cover
each feature on purpose; these cover their combinations."""
import random

import numpy as np
import pytest
import torch

import oracle
from oracle.candidates import assemble_candidates
from oracle.posterior import vocab_argmax
from synth import make_choices, make_head_logits, make_logits, make_workload
from tests._helpers import check_attention_rows, dev, oracle_verify_rows, pool_bits, verifier

pytestmark = pytest.mark.gpu

TREE_SIZES = [1, 2, 3, 4, 5, 8, 16, 26, 40, 63, 64]


def _verify_case(rng):
    preset = rng.choice(["vicuna7b_b16", "vicuna7b_b16", "stress_b64", "tiny", "gqa_b16"])
    heads = rng.choice([1, 2, 4, 8, 16, 32])
    kv = heads // rng.choice([d for d in (1, 2, 4, 8) if heads % d == 0])
    lo = rng.choice([0, 1, 16, 63, 64, 100, 500, 1000])
    kw = dict(batch=rng.randint(1, 20), heads=heads, kv_heads=kv,
              ctx_range=(lo, lo + rng.choice([0, 1, 15, 64, 300, 1000, 2500])),
              tree_sizes=tuple(sorted(rng.sample(TREE_SIZES, rng.randint(1, 3)))))
    if preset == "tiny":  # fp32, head_dim 64, one KV head per query head
        kw.pop("kv_heads")
    split = rng.choice([0, 0, 64, 128, 256, 1024])
    flags = rng.choice([0, 0, 2, 4, 1])  # default, grid, persistent, plain
    if max(kw["tree_sizes"]) == 1 and rng.random() < 0.5:
        flags = 8  # decode
    return preset, rng.randint(0, 10**6), kw, split, flags


@pytest.mark.parametrize("case", range(40))
def test_verify_random_shapes(case):
    rng = random.Random(1000 + case)
    preset, seed, kw, split, flags = _verify_case(rng)
    print(f"random verify {case}: {preset} seed {seed} {kw} split {split} flags {flags}",
          flush=True)
    wl = make_workload(preset, seed, **kw)
    d = dev(wl)
    tv = verifier(wl, flags=flags, split_tokens=split)
    out = tv.verify(d["q"], d["k_new"], d["v_new"], d["kv_pages"], d["block_table"],
                    d["ctx_lens"], d["tree_parent"], d["tree_depth"])
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    seqs = sorted(rng.sample(range(wl.spec.batch), min(3, wl.spec.batch)))
    heads = sorted(rng.sample(range(wl.spec.heads), min(4, wl.spec.heads)))
    ref = oracle_verify_rows(wl, seqs, heads=heads)
    check_attention_rows(got[seqs][:, :, heads], ref, wl, seqs)


@pytest.mark.parametrize("case", range(40))
def test_accept_commit_random_shapes(case):
    rng = random.Random(2000 + case)
    preset = rng.choice(["vicuna7b_b16", "stress_b64", "tiny", "gqa_b16"])
    heads = rng.choice([1, 2, 4, 8])
    lo = rng.choice([0, 1, 15, 16, 63, 100, 500])
    kw = dict(batch=rng.randint(1, 12), heads=heads,
              kv_heads=heads // rng.choice([d for d in (1, 2, 4) if heads % d == 0]),
              ctx_range=(lo, lo + rng.choice([0, 1, 15, 64, 300, 1000])),
              tree_sizes=tuple(sorted(rng.sample(TREE_SIZES, rng.randint(1, 3)))),
              chain=rng.random() < 0.2)
    if preset == "tiny":
        kw.pop("kv_heads")
    seed = rng.randint(0, 10**6)
    print(f"random accept/commit {case}: {preset} seed {seed} {kw}", flush=True)
    wl = make_workload(preset, seed, **kw)
    Lr, Pr = oracle.accept_greedy(wl.node_argmax, wl.cand_tokens, wl.tree_parent)
    rope = oracle.rope_table(wl.spec.head_dim, wl.max_ctx_len + wl.spec.t_max)
    ref = oracle.commit(wl.k_new, wl.v_new, Lr, Pr, wl.kv_pages, wl.block_table, wl.ctx_lens,
                        rope)
    tv = verifier(wl)
    d = dev(wl)  # separate calls
    L, P = tv.accept(d["node_argmax"], d["cand_tokens"], d["tree_parent"])
    tv.commit(d["k_new"], d["v_new"], L, P, d["kv_pages"], d["block_table"], d["ctx_lens"])
    torch.cuda.synchronize()
    assert np.array_equal(L.cpu().numpy(), Lr) and np.array_equal(P.cpu().numpy(), Pr)
    assert int((pool_bits(d["kv_pages"].cpu()) != pool_bits(ref)).sum()) == 0
    d = dev(wl)  # one launch
    L2, P2 = tv.accept_commit(d["node_argmax"], d["cand_tokens"], d["tree_parent"], d["k_new"],
                              d["v_new"], d["kv_pages"], d["block_table"], d["ctx_lens"])
    torch.cuda.synchronize()
    assert np.array_equal(L2.cpu().numpy(), Lr) and np.array_equal(P2.cpu().numpy(), Pr)
    assert int((pool_bits(d["kv_pages"].cpu()) != pool_bits(ref)).sum()) == 0


@pytest.mark.parametrize("case", range(40))
def test_posterior_random_shapes(case):
    rng = random.Random(3000 + case)
    B = rng.randint(1, 8)
    sizes = tuple(sorted(rng.sample(TREE_SIZES, rng.randint(1, 3))))
    V = rng.choice([2, 7, 8, 64, 1000, 1001, 4096, 32000, 50257])
    dtype = rng.choice([torch.bfloat16, torch.float32])
    ties = rng.choice([0, 0, 1, 3])
    seed = rng.randint(0, 10**6)
    topk = rng.randint(1, min(16, V))
    depth = rng.randint(1, 5)
    n_choices = min(rng.choice([0, 1, 5, 20, 63]), sum(topk ** k for k in range(1, depth + 1)))
    n_heads = rng.randint(depth, 5)
    print(f"random posterior {case}: seed {seed} B {B} trees {sizes} V {V} {dtype} ties {ties} "
          f"top-{topk} {n_choices} choices of depth <= {depth}, {n_heads} heads", flush=True)
    wl = make_workload("vicuna7b_b16", seed, batch=B, heads=1, ctx_range=(16, 16),
                       tree_sizes=sizes)
    tv = verifier(wl)
    d = dev(wl)
    logits = make_logits(wl, seed, vocab=V, dtype=dtype, ties=ties)
    A = tv.vocab_argmax(logits.cuda())
    A2, L, P = tv.argmax_accept(logits.cuda(), d["cand_tokens"], d["tree_parent"])
    torch.cuda.synchronize()
    Ar = vocab_argmax(logits)
    assert np.array_equal(A.cpu().numpy(), Ar) and np.array_equal(A2.cpu().numpy(), Ar)
    Lr, Pr = oracle.accept_greedy(Ar, wl.cand_tokens, wl.tree_parent)
    assert np.array_equal(L.cpu().numpy(), Lr) and np.array_equal(P.cpu().numpy(), Pr)
    choices = make_choices(seed, n=n_choices, max_depth=depth, topk=topk) if n_choices else []
    head_logits = make_head_logits(B, n_heads, V, seed=seed, dtype=dtype, ties=ties)
    root = torch.from_numpy(np.random.default_rng(seed).integers(0, V, B).astype(np.int32))
    C, Pp, D = tv.candidates(choices, head_logits.cuda(), topk, root.cuda())
    torch.cuda.synchronize()
    Cr, Ppr, Dr = assemble_candidates(head_logits, choices, root.numpy(), wl.spec.t_max, topk)
    assert np.array_equal(Pp.cpu().numpy(), Ppr) and np.array_equal(D.cpu().numpy(), Dr)
    assert np.array_equal(C.cpu().numpy(), Cr)
