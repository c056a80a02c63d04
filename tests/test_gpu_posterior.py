"""GPU parity of the greedy-token argmax and the fused argmax + acceptance
against the CPU oracle (bit-exact: integer results of exact comparisons).

Cases: the 7B batch-16 shape at full size (vocabulary 32000, bf16 logits),
fp32 logits, equal maxima (ties go to the smallest token), rows of -inf and
NaN, vocabularies that are not a multiple of the 16-byte vector (scalar
path), small trees and one-node trees; the argmax-then-acceptance call is
repeated and compared with the two separate calls.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle.posterior import vocab_argmax
from synth import make_logits, make_workload
from tests._helpers import dev, verifier

pytestmark = pytest.mark.gpu


def _argmax_gpu(wl, logits):
    tv = verifier(wl)
    out = tv.vocab_argmax(logits.cuda())
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("name,seed,kw,vocab,dtype,ties", [
    ("vicuna7b_b16", 0, {}, None, torch.bfloat16, 0),
    ("vicuna7b_b16", 1, dict(batch=4), None, torch.bfloat16, 3),
    ("vicuna7b_b16", 2, dict(batch=3), 32000, torch.float32, 2),
    ("tiny", 0, {}, 1000, torch.float32, 1),
    ("stress_b64", 1, dict(batch=6), 1001, torch.bfloat16, 2),     # scalar path (odd vocab)
    ("stress_b64", 2, dict(batch=5), 12, torch.bfloat16, 4),       # tiny vocab, many ties
    ("vicuna7b_bs1", 3, {}, 250007, torch.bfloat16, 1),            # long rows, odd size
    ("vicuna7b_b16", 4, dict(batch=2), 6144, torch.bfloat16, 2),   # 3 chunks per thread
])
def test_vocab_argmax_bit_exact(name, seed, kw, vocab, dtype, ties):
    wl = make_workload(name, seed, heads=1, ctx_range=(16, 16), **kw)
    logits = make_logits(wl, seed, vocab=vocab, dtype=dtype, ties=ties)
    print(f"argmax {name} seed={seed} V={logits.shape[-1]} {dtype} ties={ties}", flush=True)
    got = _argmax_gpu(wl, logits)
    assert np.array_equal(got, vocab_argmax(logits))


def test_vocab_argmax_special_rows():
    wl = make_workload("vicuna7b_b16", 5, batch=2, heads=1, ctx_range=(16, 16))
    logits = make_logits(wl, 5, vocab=4096, dtype=torch.float32)
    logits[0, 0] = -float("inf")                      # all -inf: token 0
    logits[0, 1] = float("nan")                       # nothing comparable: token 0
    logits[0, 2, ::2] = float("nan")                  # NaN ignored
    logits[0, 3, 100] = float("inf")                  # +inf wins
    logits[0, 3, 50] = float("inf")                   # ... the first one
    logits[0, 4] = 0.0
    logits[0, 4, 7] = -0.0                            # -0 == +0: token 0
    logits[0, 5] = -float("inf")
    logits[0, 5, :10] = float("nan")                  # first comparable value is -inf: 10
    logits[0, 6] = -float("inf")
    logits[0, 6, 1000:] = float("nan")
    logits[0, 6, 3000] = -1e30                        # the only finite value: 3000
    got = _argmax_gpu(wl, logits)
    ref = vocab_argmax(logits)
    assert got[0, :7].tolist() == [0, 0, ref[0, 2], 50, 0, 10, 3000]
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("name,seed,kw,dtype", [
    ("vicuna7b_b16", 0, {}, torch.bfloat16),
    ("tiny", 1, {}, torch.float32),
    ("stress_b64", 3, dict(batch=12), torch.bfloat16),
    ("vicuna13b_b8", 2, {}, torch.bfloat16),
])
def test_argmax_accept_fused_bit_exact(name, seed, kw, dtype):
    wl = make_workload(name, seed, heads=1, ctx_range=(16, 16), **kw)
    logits = make_logits(wl, seed, dtype=dtype, ties=1).cuda()
    d = dev(wl)
    tv = verifier(wl)
    ref_amax = vocab_argmax(logits)
    Lr, Pr = oracle.accept_greedy(ref_amax, wl.cand_tokens, wl.tree_parent)
    for rep in range(3):
        A, L, P = tv.argmax_accept(logits, d["cand_tokens"], d["tree_parent"])
        torch.cuda.synchronize()
        assert np.array_equal(A.cpu().numpy(), ref_amax), rep
        assert np.array_equal(L.cpu().numpy(), Lr), rep
        assert np.array_equal(P.cpu().numpy(), Pr), rep


def test_argmax_accept_matches_separate_calls():
    wl = make_workload("stress_b64", 4, batch=9, heads=1, ctx_range=(16, 16))
    logits = make_logits(wl, 4, ties=2).cuda()
    d = dev(wl)
    tv = verifier(wl)
    A1 = tv.vocab_argmax(logits)
    L1, P1 = tv.accept(A1, d["cand_tokens"], d["tree_parent"])
    A2, L2, P2 = tv.argmax_accept(logits, d["cand_tokens"], d["tree_parent"])
    torch.cuda.synchronize()
    assert torch.equal(A1, A2) and torch.equal(L1, L2) and torch.equal(P1, P2)
