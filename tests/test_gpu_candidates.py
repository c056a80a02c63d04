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
    (2, 2, 100000, 10, 20, 2, torch.bfloat16, 1, 8),     # several segments per row
    (2, 3, 150001, 16, 30, 3, torch.bfloat16, 2, 7),     # several segments, scalar path
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


def test_prepared_table_reused_across_calls():
    """A node table built once drives repeated calls on new head logits;
    each call equals the oracle's assembly (and the list form's output)."""
    B, H, V, topk = 4, 4, 32000, 10
    choices = make_choices(11, n=63, max_depth=4, topk=topk)
    wl = make_workload("vicuna7b_b16", 11, batch=B, heads=1, ctx_range=(16, 16))
    tv = verifier(wl)
    table = tv.medusa_tree(choices, topk, H)
    for rep in range(3):
        logits = make_head_logits(B, H, V, seed=100 + rep, ties=rep)
        root = torch.arange(B, dtype=torch.int32) + rep
        C, P, D = tv.candidates(table, logits.cuda(), topk, root.cuda())
        C2, P2, D2 = tv.candidates(choices, logits.cuda(), topk, root.cuda())
        torch.cuda.synchronize()
        Cr, Pr, Dr = assemble_candidates(logits, choices, root.numpy(), wl.spec.t_max, topk)
        assert np.array_equal(C.cpu().numpy(), Cr), rep
        assert np.array_equal(P.cpu().numpy(), Pr) and np.array_equal(D.cpu().numpy(), Dr)
        assert torch.equal(C, C2) and torch.equal(P, P2) and torch.equal(D, D2)


def test_candidates_adversarial_rows():
    """Rows whose best values all sit in a few threads' share of the row (a
    list of hundreds), all-equal rows (ties decided by token; the list
    overflows and the staged values are searched), rows of -inf and NaN with
    one +inf (tau is -inf: every element is a candidate), and rows whose
    wavefront maxima are all equal (lists longer than the workgroup)."""
    B, H, V, topk = 1, 4, 32000, 16
    choices = make_choices(9, n=60, max_depth=4, topk=topk)
    x = make_head_logits(B, H, V, seed=9, dtype=torch.float32)
    idx = torch.arange(V)
    chunk = idx // 8                                      # 16-byte bf16 chunks
    crowd = (chunk % 256) < 3                             # three threads' share
    x[0, 0] = torch.where(crowd, 100.0 + (idx % 97).float() / 8, x[0, 0])
    x[0, 1] = 1.5                                         # all equal
    x[0, 2] = -float("inf")
    x[0, 2, 31999] = float("nan")
    x[0, 2, 7] = float("inf")
    x[0, 3, ::3] = float("nan")
    logits = x.to(torch.bfloat16)
    # A second sequence: the 16-byte chunk c = token // 8 goes to thread
    # c % 1024, lane = thread % 64.  Head 3: lanes 0..15 of every wavefront
    # hold 100 + lane, so every wavefront's max is 115 and the list holds the
    # ~500 elements at 115.  Head 2: lanes 0..2 hold 100, so the list holds
    # ~1500 equal elements (longer than the workgroup: rounds over the list).
    y = make_head_logits(1, H, V, seed=19, dtype=torch.float32)
    lane_of = (idx // 8) % 1024 % 64
    y[0, 3] = torch.where(lane_of < 16, 100.0 + lane_of.float(), y[0, 3])
    y[0, 2] = torch.where(lane_of < 3, torch.full_like(y[0, 2], 100.0), y[0, 2])
    logits = torch.cat([logits, y.to(torch.bfloat16)], dim=0)
    B = 2
    root = torch.tensor([4, 9], dtype=torch.int32)
    wl = make_workload("vicuna7b_b16", 9, batch=B, heads=1, ctx_range=(16, 16))
    tv = verifier(wl)
    C, P, D = tv.candidates(choices, logits.cuda(), topk, root.cuda())
    torch.cuda.synchronize()
    Cr, Pr, Dr = assemble_candidates(logits, choices, root.numpy(), wl.spec.t_max, topk)
    assert np.array_equal(C.cpu().numpy(), Cr)
    assert np.array_equal(P.cpu().numpy(), Pr) and np.array_equal(D.cpu().numpy(), Dr)
