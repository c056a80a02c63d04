"""GPU parity of the candidate tree built from Medusa head logits and a
medusa-choices list, against the CPU oracle (bit-exact integers), and the
tree it builds driving a verify step."""
import numpy as np
import pytest
import torch

import oracle
from oracle.candidates import assemble_candidates
from synth import make_choices, make_head_logits, make_workload
from tests._helpers import dev, oracle_verify_rows, verifier

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("B,H,V,topk,n,depth,dtype,ties,seed", [
    (16, 4, 32000, 10, 63, 4, torch.bfloat16, 0, 0),
    (16, 5, 32000, 10, 63, 5, torch.bfloat16, 3, 1),
    (4, 4, 32000, 16, 40, 4, torch.float32, 2, 2),
    (3, 3, 1001, 8, 20, 3, torch.bfloat16, 2, 3),        # odd vocabulary: scalar path
    (2, 2, 12, 12, 10, 2, torch.float32, 4, 4),          # topk == vocab
    (5, 1, 500, 3, 3, 1, torch.bfloat16, 1, 5),          # one head, a root with 3 children
    (1, 4, 32000, 10, 0, 4, torch.bfloat16, 0, 6),       # no choices: root only
])
def test_candidates_bit_exact(B, H, V, topk, n, depth, dtype, ties, seed):
    choices = make_choices(seed, n=n, max_depth=depth, topk=topk) if n else []
    logits = make_head_logits(B, H, V, seed=seed, dtype=dtype, ties=ties)
    root = torch.arange(B, dtype=torch.int32) * 7 + 3
    wl = make_workload("vicuna7b_b16", seed, batch=B, heads=1, ctx_range=(16, 16))
    tv = verifier(wl)
    print(f"candidates B={B} H={H} V={V} k={topk} n={n} {dtype} ties={ties}", flush=True)
    C, P, D = tv.candidates(choices, logits.cuda(), topk, root.cuda())
    torch.cuda.synchronize()
    Cr, Pr, Dr = assemble_candidates(logits, choices, root.numpy(), wl.spec.t_max, topk)
    assert np.array_equal(P.cpu().numpy(), Pr) and np.array_equal(D.cpu().numpy(), Dr)
    assert np.array_equal(C.cpu().numpy(), Cr)


def test_candidate_tree_drives_verify_and_accept():
    """The assembled tree (63 choices + root) as verify's and acceptance's
    tree: both agree with the oracle run on the oracle's own assembly."""
    B, H, V, topk = 3, 4, 32000, 10
    choices = make_choices(7, n=63, max_depth=4, topk=topk)
    logits = make_head_logits(B, H, V, seed=7)
    root = torch.tensor([5, 6, 7], dtype=torch.int32)
    wl = make_workload("vicuna7b_b16", 7, batch=B, heads=4, ctx_range=(200, 900))
    tv = verifier(wl)
    C, P, D = tv.candidates(choices, logits.cuda(), topk, root.cuda())
    Cr, Pr, Dr = assemble_candidates(logits, choices, root.numpy(), wl.spec.t_max, topk)
    import dataclasses
    wl2 = dataclasses.replace(wl, cand_tokens=Cr, tree_parent=Pr, tree_depth=Dr)
    d = dev(wl2)
    out = tv.verify(d["q"], d["k_new"], d["v_new"], d["kv_pages"], d["block_table"],
                    d["ctx_lens"], P, D)
    L, path = tv.accept(d["node_argmax"], C, P)
    torch.cuda.synchronize()
    ref = oracle_verify_rows(wl2, range(B))
    assert np.abs(out.float().cpu().numpy() - ref).max() <= 1e-2
    Lr, Pathr = oracle.accept_greedy(wl.node_argmax, Cr, Pr)
    assert np.array_equal(L.cpu().numpy(), Lr) and np.array_equal(path.cpu().numpy(), Pathr)
