"""Out-of-range device values never cause an out-of-bounds access.

The header leaves outputs unspecified when device-resident values are out
of range (context lengths, block ids, tree links and depths, accepted paths,
token ids), but every kernel bounds-checks them.  Here each call is given
such garbage: it must complete, and a valid call made afterwards must still
match the oracle (the device and the library are unharmed).

Kernels covered: the three tree kernels (one workgroup per work item, the
persistent one that takes work items from a counter, and the plain
one-wavefront-per-node kernel), the decode kernel, acceptance, the fused
acceptance + commit, the commit with a garbage path, the greedy-token
argmax + acceptance and typical acceptance.
"""
import numpy as np
import pytest
import torch

import oracle
from synth import make_logits, make_workload
from tests._helpers import dev, oracle_verify_rows, verifier

pytestmark = pytest.mark.gpu


def _garbage(wl, seed):
    rng = np.random.default_rng(seed)
    B, T = wl.tree_parent.shape
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    return dict(
        ctx_lens=i32(rng.integers(-50, 3 * wl.max_ctx_len, size=B)),
        block_table=i32(rng.integers(-5, wl.num_blocks + 40, size=wl.block_table.shape)),
        tree_parent=i32(rng.integers(-4, T + 8, size=(B, T))),
        tree_depth=i32(rng.integers(-9, 200, size=(B, T))),
        tokens=i32(rng.integers(-100, 50000, size=(B, T))),
        accept_len=i32(rng.integers(-3, T + 9, size=B)),
        accept_path=i32(rng.integers(-5, T + 20, size=(B, T))),
    )


@pytest.mark.parametrize("name,kw,flags", [
    ("vicuna7b_b16", dict(batch=5, heads=3, ctx_range=(10, 900)), 2),   # grid kernel
    ("vicuna7b_b16", dict(batch=5, heads=3, ctx_range=(10, 900)), 4),   # persistent kernel
    ("vicuna7b_b16", dict(batch=5, heads=3, ctx_range=(10, 900)), 1),   # plain kernel
    ("decode_b64", dict(batch=5, heads=3, ctx_range=(10, 900)), 0),     # decode kernel
    ("decode_b64", dict(batch=5, heads=3, ctx_range=(10, 900)), 2),     # small-tree path
], ids=["grid", "persistent", "simple", "decode", "grid-small-trees"])
def test_garbage_device_values_are_contained(name, kw, flags):
    wl = make_workload(name, 31, **kw)
    d = dev(wl)
    tv = verifier(wl, flags=flags)
    g = _garbage(wl, 31)
    pool = d["kv_pages"].clone()
    print(f"garbage inputs: {name} {kw} flags={flags}", flush=True)
    for rep in range(2):
        tv.verify(d["q"], d["k_new"], d["v_new"], pool, g["block_table"], g["ctx_lens"],
                  g["tree_parent"], g["tree_depth"])
        L, P = tv.accept(g["tokens"], g["tokens"].flip(1), g["tree_parent"])
        tv.commit(d["k_new"], d["v_new"], g["accept_len"], g["accept_path"], pool,
                  g["block_table"], g["ctx_lens"])
        tv.accept_commit(g["tokens"], g["tokens"].flip(1), g["tree_parent"], d["k_new"],
                         d["v_new"], pool, g["block_table"], g["ctx_lens"])
        logits = make_logits(wl, 31, vocab=1000).cuda()
        tv.argmax_accept(logits, g["tokens"], g["tree_parent"])
        tv.accept_typical(logits, g["tokens"], g["tree_parent"])
        torch.cuda.synchronize()
    # the library and the device still work: a valid call is exact
    out = tv.verify(d["q"], d["k_new"], d["v_new"], d["kv_pages"], d["block_table"],
                    d["ctx_lens"], d["tree_parent"], d["tree_depth"])
    torch.cuda.synchronize()
    seqs = list(range(wl.spec.batch))
    ref = oracle_verify_rows(wl, seqs)
    real = wl.tree_parent != oracle.PAD_PARENT
    assert float(np.abs(out.float().cpu().numpy() - ref)[real].max()) <= 1e-2
