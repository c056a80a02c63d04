"""The library's calls captured into a HIP graph (torch.cuda.CUDAGraph) and
replayed, as a serving loop would run them: every replay must reproduce the
eager results bit for bit.  Between replays the outputs are cleared and the
KV pool restored by ordinary eager work, so each replay is checked on its
own.  The library records no memset into a graph (work counters and
scratch are cleared by kernels), which is what makes replays safe.

Cases: a verify + argmax-acceptance + commit step with the one-workgroup-
per-item kernel and with the persistent kernel (whose work counters must be
back at zero after every replay); one-node trees (the decode kernel); and
the typical-acceptance and candidate calls.
"""
import numpy as np
import pytest
import torch

from synth import make_choices, make_head_logits, make_logits, make_workload
from tests._helpers import dev, verifier

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


@pytest.mark.parametrize("name,kw,flags", [
    ("vicuna7b_b16", dict(batch=4, heads=4, ctx_range=(100, 900)), 0),
    ("vicuna7b_b16", dict(batch=4, heads=4, ctx_range=(100, 900)), 4),
    ("decode_b64", dict(batch=6, heads=4, ctx_range=(50, 2000)), 0),
])
def test_step_graph_replays_match_eager(name, kw, flags):
    wl = make_workload(name, 21, **kw)
    d = dev(wl)
    tv = verifier(wl, flags=flags)
    logits = make_logits(wl, 21, vocab=4096).cuda()
    cand = torch.remainder(d["cand_tokens"], 4096)
    pool0 = d["kv_pages"].clone()
    args = (d["q"], d["k_new"], d["v_new"])
    rest = (d["block_table"], d["ctx_lens"], d["tree_parent"], d["tree_depth"])

    # eager reference
    pool_e = pool0.clone()
    out_e = tv.verify(*args, pool_e, *rest)
    A_e, L_e, P_e = tv.argmax_accept(logits, cand, d["tree_parent"])
    tv.commit(d["k_new"], d["v_new"], L_e, P_e, pool_e, d["block_table"], d["ctx_lens"])
    torch.cuda.synchronize()

    # static buffers, captured once
    pool = pool0.clone()
    out = torch.empty_like(out_e)
    A, L, P = torch.empty_like(A_e), torch.empty_like(L_e), torch.empty_like(P_e)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        tv.verify(*args, pool, *rest, out=out)
        tv.argmax_accept(logits, cand, d["tree_parent"], A, L, P)
        tv.commit(d["k_new"], d["v_new"], L, P, pool, d["block_table"], d["ctx_lens"])
    torch.cuda.synchronize()
    for rep in range(4):
        out.zero_()
        A.fill_(-1)
        L.fill_(-1)
        P.fill_(-7)
        pool.copy_(pool0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(out), _bits(out_e)), rep
        assert torch.equal(A, A_e) and torch.equal(L, L_e) and torch.equal(P, P_e), rep
        assert torch.equal(_bits(pool), _bits(pool_e)), rep
    # the persistent kernel's counters are zero again: an eager call after
    # the replays still gives the same result
    out2 = tv.verify(*args, pool0, *rest)
    torch.cuda.synchronize()
    assert torch.equal(_bits(out2), _bits(out_e))


def test_typical_and_candidates_graph_replays_match_eager():
    wl = make_workload("vicuna7b_b16", 22, batch=5, heads=1, ctx_range=(16, 16))
    d = dev(wl)
    tv = verifier(wl)
    logits = make_logits(wl, 22, vocab=8192, scale=3.0, planted_margin=1.0).cuda()
    cand = torch.remainder(d["cand_tokens"], 8192)
    choices = make_choices(22, n=40, max_depth=4, topk=8)
    table = tv.medusa_tree(choices, 8, 4)
    hl = make_head_logits(5, 4, 8192, seed=22, ties=1).cuda()
    root = torch.arange(5, dtype=torch.int32, device="cuda") * 3

    S_e, OK_e, L_e, P_e = tv.accept_typical(logits, cand, d["tree_parent"], 0.8, 0.05, 0.4)
    C_e, Pc_e, Dc_e = tv.candidates(table, hl, 8, root)
    torch.cuda.synchronize()

    bufs = [torch.empty_like(x) for x in (S_e, OK_e, L_e, P_e, C_e, Pc_e, Dc_e)]
    S, OK, L, P, C, Pc, Dc = bufs
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        tv.accept_typical(logits, cand, d["tree_parent"], 0.8, 0.05, 0.4, S, OK, L, P)
        tv.candidates(table, hl, 8, root, C, Pc, Dc)
    torch.cuda.synchronize()
    ref = (S_e, OK_e, L_e, P_e, C_e, Pc_e, Dc_e)
    for rep in range(4):
        for t in bufs:
            t.fill_(-3)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip(bufs, ref):
            assert torch.equal(got, want), rep
    assert np.all(OK_e.cpu().numpy()[:, 0] == 1)
