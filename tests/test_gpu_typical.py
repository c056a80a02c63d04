"""GPU parity of typical acceptance against the CPU oracle.

The per-node statistics (log-sum-exp of logits / temperature, entropy) are
compared with fp64 values within a tolerance; the per-child test is compared
exactly except for children whose probability lies within a relative 1e-4 of
the threshold (fp32 exp/log may put those on either side); the accepted path
must be exactly the one the oracle's path rule picks from the GPU's own
per-child results, and the oracle's path wherever no child of the sequence is
that close.

Cases: the 7B batch-16 shape at full vocabulary (bf16), fp32 logits,
temperatures below and above 1, peaked and flat rows, small vocabularies
(where non-greedy candidates often pass), masked (-inf) vocabulary tails,
odd vocabularies (scalar loads), long rows, and one-node trees.
"""
import numpy as np
import pytest
import torch
from scipy.special import logsumexp

from oracle.posterior import _longest_path, softmax_stats, typical_accept
from synth import make_logits, make_workload
from tests._helpers import dev, verifier

pytestmark = pytest.mark.gpu

# fp32 statistics of a row of up to 250k values: the sum of exponentials
# carries a relative error of a few 1e-6 (one rounding per add over ~1000
# terms per thread, plus the exp units' few ulps), so lse and H are good to
# ~1e-5 absolute; 1e-4 leaves a margin.
STAT_ATOL = 1e-4
STAT_RTOL = 1e-5
BAND = 1e-4


def _inputs(name, seed, kw, vocab, dtype, scale, margin, mask_tail=0):
    wl = make_workload(name, seed, heads=1, ctx_range=(16, 16), **kw)
    logits = make_logits(wl, seed, vocab=vocab, dtype=dtype, scale=scale,
                         planted_margin=margin)
    V = logits.shape[-1]
    if mask_tail:
        logits[..., V - mask_tail:] = -float("inf")
    cand = np.asarray(wl.cand_tokens, dtype=np.int64) % (V - mask_tail)
    return wl, logits, cand.astype(np.int32)


def _check(wl, logits, cand, temperature, epsilon, delta):
    tv = verifier(wl)
    d = dev(wl)
    cand_d = torch.from_numpy(cand).cuda()
    S, OK, L, P = tv.accept_typical(logits.cuda(), cand_d, d["tree_parent"],
                                    temperature=temperature, epsilon=epsilon, delta=delta)
    torch.cuda.synchronize()
    S, OK, L, P = S.cpu().numpy(), OK.cpu().numpy(), L.cpu().numpy(), P.cpu().numpy()
    par = np.asarray(wl.tree_parent)
    B, T = par.shape

    x = logits.to(torch.float64).numpy() / temperature
    lse = logsumexp(x, axis=-1)
    p, H = softmax_stats(logits, temperature)
    assert np.allclose(S[..., 0], lse, atol=STAT_ATOL, rtol=STAT_RTOL)
    assert np.allclose(S[..., 1], H, atol=STAT_ATOL, rtol=STAT_RTOL)

    Lr, Pr, okr = typical_accept(logits, cand, par, temperature, epsilon, delta)
    thr = np.minimum(epsilon, delta * np.exp(-H))
    near = np.zeros((B, T), dtype=bool)
    for b in range(B):
        for i in range(1, T):
            n = par[b, i]
            if n >= 0:
                near[b, i] = abs(p[b, n, cand[b, i]] - thr[b, n]) <= BAND * thr[b, n]
    assert np.array_equal(OK[~near], okr[~near].astype(np.int32))
    # the path rule applied to the GPU's own per-child results
    Lg, Pg = _longest_path(OK.astype(bool), par)
    assert np.array_equal(L, Lg) and np.array_equal(P, Pg)
    clean = ~near.any(axis=1)
    assert np.array_equal(L[clean], Lr[clean]) and np.array_equal(P[clean], Pr[clean])
    return okr, near


@pytest.mark.parametrize("name,seed,kw,vocab,dtype,scale,margin,temp", [
    ("vicuna7b_b16", 0, {}, None, torch.bfloat16, 2.0, 4.0, 1.0),
    ("vicuna7b_b16", 1, dict(batch=4), None, torch.bfloat16, 2.0, 4.0, 0.7),
    ("vicuna7b_b16", 2, dict(batch=3), 32000, torch.float32, 3.0, 2.0, 1.5),
    ("tiny", 0, {}, 64, torch.float32, 3.0, 0.0, 1.0),              # many non-greedy passes
    ("stress_b64", 1, dict(batch=6), 1001, torch.bfloat16, 2.0, 1.0, 1.0),  # scalar loads
    ("stress_b64", 2, dict(batch=5), 12, torch.bfloat16, 1.0, 0.0, 2.0),    # tiny vocab
    ("vicuna7b_bs1", 3, {}, 250007, torch.bfloat16, 2.0, 6.0, 1.0),         # long rows
    ("vicuna13b_b8", 4, {}, None, torch.bfloat16, 0.5, 0.0, 1.0),           # flat rows
])
def test_typical_accept_parity(name, seed, kw, vocab, dtype, scale, margin, temp):
    wl, logits, cand = _inputs(name, seed, kw, vocab, dtype, scale, margin)
    print(f"typical {name} seed={seed} V={logits.shape[-1]} {dtype} T={temp}", flush=True)
    okr, near = _check(wl, logits, cand, temp, 0.09, 0.3)
    assert near.sum() <= 2          # the band is rare, or the test says nothing


def test_typical_accept_mixes_outcomes():
    """A case where children pass and fail for reasons other than being the
    greedy token (so the threshold, not the argmax, decides)."""
    wl, logits, cand = _inputs("tiny", 5, dict(batch=8), 64, torch.float32, 3.0, 0.0)
    okr, _ = _check(wl, logits, cand, 1.0, 0.09, 0.3)
    par = np.asarray(wl.tree_parent)
    child = par >= 0
    amax = logits.argmax(-1).numpy()
    greedy = np.zeros_like(child)
    for b in range(par.shape[0]):
        for i in range(par.shape[1]):
            if child[b, i]:
                greedy[b, i] = cand[b, i] == amax[b, par[b, i]]
    assert (okr & child & ~greedy).any() and (~okr & child).any()


def test_typical_accept_masked_tail_and_thresholds():
    wl, logits, cand = _inputs("stress_b64", 6, dict(batch=7), 4096, torch.bfloat16, 2.0,
                               2.0, mask_tail=1000)
    for eps, delta in ((0.09, 0.3), (0.5, 0.5), (1e-4, 0.05), (1.0, 1.0)):
        _check(wl, logits, cand, 1.0, eps, delta)


def test_typical_accept_one_node_trees():
    wl, logits, cand = _inputs("vicuna7b_b16", 7, dict(batch=5, tree_sizes=(1, 1)), 512,
                               torch.float32, 2.0, 4.0)
    tv = verifier(wl)
    d = dev(wl)
    S, OK, L, P = tv.accept_typical(logits.cuda(), torch.from_numpy(cand).cuda(),
                                    d["tree_parent"])
    torch.cuda.synchronize()
    assert L.cpu().tolist() == [1] * 5
    assert P.cpu()[:, 0].tolist() == [0] * 5
    assert OK.cpu()[:, 0].tolist() == [1] * 5


@pytest.mark.parametrize("case", range(24))
def test_typical_accept_random_shapes(case):
    """Seeded random combinations of batch, tree sizes, vocabulary, dtype,
    temperature, thresholds, logit scale and masked tails."""
    import random
    rng = random.Random(4000 + case)
    vocab = rng.choice([12, 64, 1001, 4096, 32000, 50257])
    mask = rng.choice([0, 0, vocab // 4])
    kw = dict(batch=rng.randint(1, 8),
              tree_sizes=tuple(sorted(rng.sample([1, 2, 3, 5, 8, 16, 26, 40, 63, 64],
                                                 rng.randint(1, 3)))))
    dtype = rng.choice([torch.bfloat16, torch.float32])
    scale = rng.choice([0.5, 1.0, 2.0, 3.0])
    margin = rng.choice([0.0, 1.0, 4.0])
    temp = rng.choice([0.5, 0.7, 1.0, 1.5, 2.0])
    eps, delta = rng.choice([(0.09, 0.3), (0.5, 0.5), (1e-3, 0.1), (0.2, 0.9)])
    seed = rng.randint(0, 10**6)
    print(f"random typical {case}: seed {seed} {kw} V {vocab} masked {mask} {dtype} "
          f"scale {scale} margin {margin} T {temp} eps {eps} delta {delta}", flush=True)
    wl, logits, cand = _inputs("vicuna7b_b16", seed, kw, vocab, dtype, scale, margin,
                               mask_tail=mask)
    _check(wl, logits, cand, temp, eps, delta)
