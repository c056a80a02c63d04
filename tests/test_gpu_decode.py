"""GPU parity of the one-node (T = 1) decode kernel against the CPU oracle.

A descriptor with t_max == 1 takes the decode kernel: one workgroup per
(sequence, head) streams the whole context, no splits, no workspace.  Bars as
for the tree kernels: max-abs 1e-2 against the fp64 oracle (plus the output's
own bf16 rounding where a row sees a handful of keys).

Cases: contexts of 0 tokens (the root alone), 1 token, inside one page,
ending mid-page, and long enough to need more than one LDS window of block
ids (> 32768 tokens); more than 64 sequences (launch order without ranking);
grouped-query heads; a padding root (zero row); the full decode_b64 shape
(64 sequences, contexts 128..8192) on sampled sequences; agreement with the
tree kernels forced on the same input; repeated calls bit-identical; and a
verify -> accept -> commit step.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from synth import make_workload
from tests._helpers import ATOL, check_attention_rows, dev, oracle_verify_rows, pool_bits, verifier

pytestmark = pytest.mark.gpu

DECODE = 8  # TA_FLAG_DECODE_KERNEL


def _run(wl, flags=DECODE):
    d = dev(wl)
    tv = verifier(wl, flags=flags)
    from medusa_tree_attention_attn_amd._lib import tree_attn_plan_info
    kernel = tree_attn_plan_info(tv.desc)[0]
    out = tv.verify(d["q"], d["k_new"], d["v_new"], d["kv_pages"], d["block_table"],
                    d["ctx_lens"], d["tree_parent"], d["tree_depth"])
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), kernel


_check = check_attention_rows


CASES = [
    ("decode_b64", 0, dict(batch=4, heads=2, ctx_range=(100, 600))),
    ("decode_b64", 1, dict(batch=6, heads=3, ctx_range=(0, 40))),        # sub-page, mid-page
    ("decode_b64", 2, dict(batch=2, heads=2, ctx_range=(33000, 34100))),  # two id windows
    ("decode_b64", 3, dict(batch=70, heads=1, ctx_range=(1, 300))),      # > 64 sequences
    ("decode_b64", 4, dict(batch=5, heads=4, ctx_range=(2000, 9000))),
]


@pytest.mark.parametrize("name,seed,kw", CASES, ids=[f"s{s}" for _, s, _ in CASES])
def test_decode_kernel_matches_oracle(name, seed, kw):
    wl = make_workload(name, seed, **kw)
    print(f"decode {kw} seed={seed}", flush=True)
    got, kernel = _run(wl)
    assert kernel == "verify_decode_kernel"
    seqs = list(range(wl.spec.batch))
    _check(got, oracle_verify_rows(wl, seqs), wl, seqs)


def test_decode_tiny_contexts():
    """Contexts of 0 (the root alone), 1, 15, 16, 17 and 33 tokens."""
    wl = make_workload("decode_b64", 14, batch=6, heads=2, ctx_range=(40, 60))
    ctx = np.array([0, 1, 15, 16, 17, 33], dtype=np.int32)
    wl = dataclasses.replace(wl, ctx_lens=ctx)
    got, _ = _run(wl)
    seqs = list(range(6))
    _check(got, oracle_verify_rows(wl, seqs), wl, seqs)


def test_decode_full_shape_sampled():
    wl = make_workload("decode_b64", 0)
    got, kernel = _run(wl)
    assert kernel == "verify_decode_kernel"
    order = np.argsort(wl.ctx_lens)
    seqs = sorted({int(order[0]), int(order[1]), int(order[-1]), int(order[-2]),
                   int(order[len(order) // 2])})
    heads = [0, 17, 31]
    print(f"decode full shape: sequences {seqs} (ctx {wl.ctx_lens[seqs].tolist()})", flush=True)
    _check(got[seqs][:, :, heads], oracle_verify_rows(wl, seqs, heads), wl, seqs)


def test_decode_grouped_query_heads():
    wl = make_workload("decode_b64", 9, batch=3, heads=8, ctx_range=(50, 700))
    kn = wl.k_new[:, :, ::4].contiguous()
    vn = wl.v_new[:, :, ::4].contiguous()
    pool = wl.kv_pages[:, :, ::4].contiguous()
    spec = dataclasses.replace(wl.spec, kv_heads=2)
    wl = dataclasses.replace(wl, spec=spec, k_new=kn, v_new=vn, kv_pages=pool)
    got, _ = _run(wl)
    _check(got, oracle_verify_rows(wl, [0, 1, 2]), wl, [0, 1, 2])


def test_decode_padding_root_gives_zero_row():
    wl = make_workload("decode_b64", 10, batch=3, heads=2, ctx_range=(20, 200))
    par = wl.tree_parent.copy()
    par[1, 0] = oracle.PAD_PARENT
    wl = dataclasses.replace(wl, tree_parent=par)
    got, _ = _run(wl)
    assert np.all(got[1] == 0.0)
    _check(got, oracle_verify_rows(wl, [0, 1, 2]), wl, [0, 1, 2])


@pytest.mark.parametrize("flags", [0, 2, 4, 1])
def test_decode_agrees_with_tree_kernels(flags):
    """The decode kernel against the grid kernel's small-tree path (the
    default for a 1500-token bound, and forced), the persistent and the
    plain kernel."""
    wl = make_workload("decode_b64", 11, batch=4, heads=3, ctx_range=(0, 1500))
    a, ka = _run(wl)
    b, kb = _run(wl, flags=flags)
    assert ka == "verify_decode_kernel" and kb != ka
    real = wl.tree_parent != oracle.PAD_PARENT
    assert float(np.abs(a - b)[real].max()) <= 2 * ATOL


def test_decode_is_deterministic():
    wl = make_workload("decode_b64", 12, batch=4, heads=4, ctx_range=(100, 3000))
    a, _ = _run(wl)
    b, _ = _run(wl)
    assert np.array_equal(a, b)


def test_decode_step_with_accept_and_commit():
    """verify -> accept -> commit with one-node trees: every sequence accepts
    its root (length 1) and the commit writes the root's rotated key at
    position ctx_len, bit-exact with the oracle."""
    wl = make_workload("decode_b64", 13, batch=5, heads=2, ctx_range=(10, 500))
    d = dev(wl)
    tv = verifier(wl)
    out = tv.verify(d["q"], d["k_new"], d["v_new"], d["kv_pages"], d["block_table"],
                    d["ctx_lens"], d["tree_parent"], d["tree_depth"])
    L, P = tv.accept(d["node_argmax"], d["cand_tokens"], d["tree_parent"])
    tv.commit(d["k_new"], d["v_new"], L, P, d["kv_pages"], d["block_table"], d["ctx_lens"])
    torch.cuda.synchronize()
    assert L.cpu().tolist() == [1] * 5 and P.cpu()[:, 0].tolist() == [0] * 5
    rope = oracle.rope_table(wl.spec.head_dim, wl.max_ctx_len + wl.spec.t_max)
    pool_ref = oracle.commit(wl.k_new, wl.v_new, np.ones(5, np.int32),
                             np.zeros((5, 1), np.int32), wl.kv_pages, wl.block_table,
                             wl.ctx_lens, rope)
    assert np.array_equal(pool_bits(d["kv_pages"].cpu()), pool_bits(pool_ref))
    seqs = list(range(5))
    _check(out.float().cpu().numpy(), oracle_verify_rows(wl, seqs), wl, seqs)
