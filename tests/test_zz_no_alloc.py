"""The allocation-free verify entry point (tree_attn_verify_noalloc) against
tree_attn_verify: the same kernels run with the library's static device
workspace instead of the caller's, so the outputs must be bit-identical, and
within the attention bar of the oracle.  Each case makes two calls in a row,
the second with a smaller input, so the second runs over whatever the first
left in the shared array; the cases cover the split partials of the grid
kernel, the persistent kernel's work counters and partials, and a plan with
no partials."""
import numpy as np
import pytest
import torch

from synth import make_workload
from tests._helpers import check_attention_rows, dev, oracle_verify_rows, verifier

pytestmark = pytest.mark.gpu

CASES = [
    # grid kernel, 8 splits per (sequence, head) then fewer
    ("grid-splits", 0,
     ("vicuna7b_bs1", 0, {}),
     ("vicuna7b_bs1", 1, dict(heads=8, ctx_range=(200, 400), tree_sizes=(26,)))),
    # persistent kernel (work counters) with 256-token splits
    ("persistent-splits", 4,
     ("vicuna7b_b16", 40, dict(batch=4, heads=8, ctx_range=(500, 1500))),
     ("vicuna7b_b16", 41, dict(batch=2, heads=4, ctx_range=(100, 600)))),
    # one split: the counters only
    ("unsplit", 0,
     ("vicuna7b_b16", 42, dict(batch=16, heads=32, ctx_range=(256, 2048))),
     ("vicuna7b_b16", 43, dict(batch=9, heads=32, ctx_range=(256, 1024)))),
]


@pytest.mark.parametrize("name,flags,first,second", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_verify(name, flags, first, second):
    split = 256 if name == "persistent-splits" else 0
    wls = [make_workload(n, s, **kw) for n, s, kw in (first, second)]
    runs = []
    for wl in wls:
        d = dev(wl)
        tv = verifier(wl, flags=flags, split_tokens=split)
        args = (d["q"], d["k_new"], d["v_new"], d["kv_pages"], d["block_table"], d["ctx_lens"],
                d["tree_parent"], d["tree_depth"])
        ref = tv.verify(*args)
        runs.append((wl, tv, args, ref))
    torch.cuda.synchronize()
    outs = []
    for wl, tv, args, _ in runs:   # two calls in a row, the second smaller
        print(f"noalloc {name}: batch {wl.spec.batch} heads {wl.spec.heads} "
              f"ctx {int(wl.ctx_lens.min())}..{int(wl.ctx_lens.max())}", flush=True)
        outs.append(tv.verify_noalloc(*args, out=torch.full_like(args[0], 7.0)))
    torch.cuda.synchronize()
    for (wl, tv, args, ref), out in zip(runs, outs):
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
        seqs = list(range(wl.spec.batch))
        check_attention_rows(out.float().cpu().numpy(), oracle_verify_rows(wl, seqs), wl, seqs)
