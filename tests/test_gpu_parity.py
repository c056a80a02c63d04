"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars: accept_len, accept_path and the KV pool after commit are bit-exact;
attention outputs are within max-abs 1e-2 of the fp64 oracle (bf16 or fp32
inputs, fp32 accumulation, output rounded to the input dtype).  The RoPE
table the library builds is bit-identical to the oracle's own.

Sizes: the small presets run whole; the 16-sequence 7B preset runs whole for
seed 0; the 13B and stress presets run at full size on the GPU and are checked
on sampled sequences (sub-problems holding only the pages those sequences
reference), chosen to include the longest and shortest contexts and every tree
size of the stress mix.  Edge cases: empty context, single-node trees,
contexts that end mid-page, padded (ragged) trees, chains reaching depth 63,
grouped-query heads.  The MFMA path has two kernels (one workgroup per work
item, and a persistent one that takes work items from a counter); both are
run on the edge cases, the persistent one also on consecutive calls that
share its counters.
"""
import numpy as np
import pytest
import torch

import oracle
from synth import make_workload
from tests._helpers import (ATOL, check_attention_rows, dev, oracle_verify_rows, pool_bits,
                            verifier)

pytestmark = pytest.mark.gpu

def _verify_gpu(wl, flags=0, max_ctx_len=None, split_tokens=0):
    d = dev(wl)
    tv = verifier(wl, flags=flags, max_ctx_len=max_ctx_len, split_tokens=split_tokens)
    out = tv.verify(d["q"], d["k_new"], d["v_new"], d["kv_pages"], d["block_table"],
                    d["ctx_lens"], d["tree_parent"], d["tree_depth"])
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


_check_rows = check_attention_rows


FULL_CASES = [
    ("tiny", s, {}) for s in range(5)
] + [
    ("vicuna7b_bs1", 0, {}),
    ("vicuna7b_bs1", 1, {}),
    ("vicuna7b_b16", 0, {}),
    # several tiles and a ragged tail per sequence, small enough to check whole
    ("vicuna7b_b16", 3, dict(batch=3, heads=4, ctx_range=(1, 1100))),
    # empty contexts: the root attends only to itself
    ("vicuna7b_b16", 4, dict(batch=2, heads=2, ctx_range=(0, 0))),
    # contexts ending mid-page, trees of every stress size (ragged padding)
    ("stress_b64", 5, dict(batch=8, heads=2, ctx_range=(1, 77))),
    # single-node trees = plain paged decode
    ("stress_b64", 6, dict(batch=4, heads=2, ctx_range=(100, 600), tree_sizes=(1,))),
    # deep random trees (depth cap 63)
    ("vicuna7b_bs1", 7, dict(batch=2, heads=2, ctx_range=(30, 300), tree_sizes=(64,),
                             max_depth=63)),
    # head_dim 64 in bf16
    ("vicuna7b_b16", 14, dict(batch=3, heads=3, head_dim=64, ctx_range=(0, 500))),
]


KERNEL_FLAGS = {"default": 0, "simple": 1, "grid": 2, "persistent": 4}


@pytest.mark.parametrize("name,seed,kw", FULL_CASES,
                         ids=[f"{n}-s{s}-{i}" for i, (n, s, _) in enumerate(FULL_CASES)])
@pytest.mark.parametrize("kernel", ["default", "persistent", "simple"])
def test_verify_full(name, seed, kw, kernel):
    wl = make_workload(name, seed, **kw)
    flags = KERNEL_FLAGS[kernel]
    print(f"verify {name} seed={seed} {kw} kernel={kernel}", flush=True)
    got = _verify_gpu(wl, flags)
    ref = oracle_verify_rows(wl, range(wl.spec.batch))
    _check_rows(got, ref, wl, list(range(wl.spec.batch)))


@pytest.mark.parametrize("kernel", ["grid", "persistent"])
@pytest.mark.parametrize("split_tokens", [64, 192, 512, 4096])
def test_verify_split_sizes(split_tokens, kernel):
    """One, a few and many split-KV work items per (sequence, head): the
    partials and their merge must agree with the oracle."""
    wl = make_workload("vicuna7b_b16", 15, batch=4, heads=4, ctx_range=(1, 2000))
    print(f"verify split_tokens={split_tokens} kernel={kernel}", flush=True)
    got = _verify_gpu(wl, flags=KERNEL_FLAGS[kernel], split_tokens=split_tokens)
    ref = oracle_verify_rows(wl, range(4))
    _check_rows(got, ref, wl, list(range(4)))


def test_verify_split_ranked_long_short_pairs():
    """Split items ranked by length and paired long with short: 8 sequences x
    24 heads with 512-token splits give 17 (sequence, split) groups, 408 work
    items, between one and two per CU on a 256-CU device, so the launch slots
    past the CU count take the shortest items in reverse order."""
    wl = make_workload("vicuna7b_b16", 21, batch=8, heads=24, ctx_range=(0, 1500))
    print("verify ranked split items, 8x24, split_tokens=512, grid kernel", flush=True)
    got = _verify_gpu(wl, flags=KERNEL_FLAGS["grid"], split_tokens=512)
    ref = oracle_verify_rows(wl, range(8))
    _check_rows(got, ref, wl, list(range(8)))


def test_verify_repeated_calls_reuse_workspace():
    """The arrival counters reset themselves: repeated calls on one workspace
    give identical results."""
    wl = make_workload("vicuna7b_b16", 16, batch=3, heads=4, ctx_range=(700, 1900))
    d = dev(wl)
    tv = verifier(wl, split_tokens=256)
    outs = []
    for _ in range(3):
        o = tv.verify(d["q"], d["k_new"], d["v_new"], d["kv_pages"], d["block_table"],
                      d["ctx_lens"], d["tree_parent"], d["tree_depth"])
        outs.append(o.clone())
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
    ref = oracle_verify_rows(wl, range(3))
    _check_rows(outs[0].float().cpu().numpy(), ref, wl, [0, 1, 2])


@pytest.mark.parametrize("kernel", ["grid", "persistent"])
def test_verify_chain_depth_63(kernel):
    wl = make_workload("vicuna7b_bs1", 8, batch=2, heads=2, ctx_range=(17, 40),
                       tree_sizes=(64,), chain=True)
    got = _verify_gpu(wl, flags=KERNEL_FLAGS[kernel])
    ref = oracle_verify_rows(wl, [0, 1])
    _check_rows(got, ref, wl, [0, 1])


def test_persistent_kernel_counters_reset_between_calls():
    """The persistent kernel takes work items from counters in the workspace
    and its last workgroup zeroes them: consecutive calls on one workspace,
    with different numbers of work items (so different grids), each match
    the oracle, and a repeat of the first call is bit-identical to it."""
    from medusa_tree_attention_attn_amd import TreeVerifier
    big = make_workload("stress_b64", 21, batch=40, heads=32, ctx_range=(1, 900))
    small = make_workload("stress_b64", 22, batch=3, heads=5, ctx_range=(0, 300))
    s = big.spec
    tv = TreeVerifier(batch=s.batch, t_max=s.t_max, num_heads=32, num_kv_heads=32,
                      head_dim=128, max_blocks_per_seq=big.max_blocks,
                      num_blocks=big.num_blocks, max_ctx_len=big.max_ctx_len,
                      dtype=torch.bfloat16, flags=KERNEL_FLAGS["persistent"],
                      split_tokens=4096)
    tv_small = TreeVerifier(batch=3, t_max=s.t_max, num_heads=5, num_kv_heads=5,
                            head_dim=128, max_blocks_per_seq=small.max_blocks,
                            num_blocks=small.num_blocks, max_ctx_len=small.max_ctx_len,
                            dtype=torch.bfloat16, flags=KERNEL_FLAGS["persistent"],
                            split_tokens=4096)
    # share one workspace between the two descriptors
    assert tv_small.workspace_bytes_needed <= tv.workspace.numel()
    tv_small.desc.workspace = tv.workspace.data_ptr()
    tv_small.desc.workspace_bytes = tv.workspace.numel()
    db, ds = dev(big), dev(small)
    args = lambda d: (d["q"], d["k_new"], d["v_new"], d["kv_pages"], d["block_table"],
                      d["ctx_lens"], d["tree_parent"], d["tree_depth"])
    o1 = tv.verify(*args(db)).clone()
    o2 = tv_small.verify(*args(ds)).clone()
    o3 = tv.verify(*args(db)).clone()
    torch.cuda.synchronize()
    assert torch.equal(o1, o3)
    _check_rows(o2.float().cpu().numpy(), oracle_verify_rows(small, range(3)), small, [0, 1, 2])
    seqs = [0, 17, 39]
    ref = oracle_verify_rows(big, seqs)
    _check_rows(o1.float().cpu().numpy()[seqs], ref, big, seqs)


def _sample_seqs(wl, k):
    order = np.argsort(wl.ctx_lens)
    picks = {int(order[0]), int(order[-1])}
    for t in sorted(set(wl.tree_sizes.tolist())):
        picks.add(int(np.flatnonzero(wl.tree_sizes == t)[0]))
    rng = np.random.default_rng(wl.seed)
    while len(picks) < k:
        picks.add(int(rng.integers(wl.spec.batch)))
    return sorted(picks)


@pytest.mark.parametrize("name,seed,nseq", [
    ("vicuna7b_b16", 1, 16),   # every sequence
    ("vicuna13b_b8", 0, 8),    # every sequence
    ("stress_b64", 0, 16),     # 16 of 64: longest, shortest, every tree size, random others
])
def test_verify_sampled_full_size(name, seed, nseq):
    """Full-size launches (the default kernel choice, as the benchmark runs
    them), checked on every head of the sampled sequences."""
    wl = make_workload(name, seed)
    print(f"verify full-size {name} seed={seed}", flush=True)
    got = _verify_gpu(wl)
    seqs = _sample_seqs(wl, nseq)
    print(f"  checking {len(seqs)} sequences x {wl.spec.heads} heads", flush=True)
    ref = oracle_verify_rows(wl, seqs)
    _check_rows(got[seqs], ref, wl, seqs)


@pytest.mark.parametrize("kernel", ["grid", "persistent"])
def test_verify_grouped_query_heads(kernel):
    wl = make_workload("vicuna7b_b16", 9, batch=2, heads=8, ctx_range=(50, 400))
    # 8 query heads sharing 2 KV heads: keep every 4th KV head of the draw
    kn = wl.k_new[:, :, ::4].contiguous()
    vn = wl.v_new[:, :, ::4].contiguous()
    pool = wl.kv_pages[:, :, ::4].contiguous()
    import dataclasses
    spec = dataclasses.replace(wl.spec, kv_heads=2)
    wl = dataclasses.replace(wl, spec=spec, k_new=kn, v_new=vn, kv_pages=pool)
    got = _verify_gpu(wl, flags=KERNEL_FLAGS[kernel])
    ref = oracle_verify_rows(wl, [0, 1])
    _check_rows(got, ref, wl, [0, 1])



@pytest.mark.parametrize("batch,kv_heads,split_tokens,ctx_range", [
    (3, 8, 0, (100, 700)),     # fewer items than CUs
    (9, 8, 0, (100, 700)),     # 288 items: long and short halves on shared CUs
    (9, 4, 256, (100, 700)),   # split items (ranked groups of (sequence, split))
    (3, 2, 0, (100, 700)),     # 16 query heads per KV head
    (66, 8, 0, (1, 90)),       # more than 64 groups: (sequence, head) order
], ids=["b3-kv8", "b9-kv8", "b9-kv4-split", "b3-kv2", "b66-kv8"])
def test_verify_grouped_heads_launch_order(batch, kv_heads, split_tokens, ctx_range):
    """32 query heads on fewer KV heads: the launch order puts the query heads
    of one KV head on one XCD (a permutation of the heads of each (sequence,
    split) group).  Every head of every sequence (of the first nine at batch
    66) against the oracle."""
    wl = make_workload("vicuna7b_b16", 12, batch=batch, heads=32, kv_heads=kv_heads,
                       ctx_range=ctx_range)
    got = _verify_gpu(wl, split_tokens=split_tokens)
    seqs = list(range(min(batch, 9)))
    ref = oracle_verify_rows(wl, seqs)
    _check_rows(got[seqs], ref, wl, seqs)


MIXED_SIZES = (1, 2, 4, 8, 26, 64)


def _mixed_workload(seed0, batch, **kw):
    """A workload whose trees take every size of MIXED_SIZES (the first seed
    from seed0 on whose draw covers them all)."""
    for seed in range(seed0, seed0 + 100):
        wl = make_workload("stress_b64", seed, batch=batch, tree_sizes=MIXED_SIZES, **kw)
        if set(wl.tree_sizes.tolist()) == set(MIXED_SIZES):
            return wl
    raise AssertionError("no seed covers every tree size")


@pytest.mark.parametrize("kernel", ["default", "persistent", "simple"])
@pytest.mark.parametrize("split_tokens", [0, 128])
@pytest.mark.parametrize("ctx_range", [(0, 700), (0, 20)])
def test_verify_mixed_tree_sizes(kernel, split_tokens, ctx_range):
    """Trees of 1, 2, 4, 8, 26 and 64 nodes side by side in one batch.  The
    grid kernel routes each work item on the device: trees of at most 2 real
    nodes to its vector-ALU small-tree path, the others to the matrix cores;
    with 128-token splits the small-tree path leaves split partials for the
    merge kernel.  Contexts ending mid-page, and of 0..20 tokens (empty and
    sub-page contexts)."""
    wl = _mixed_workload(40, 18, heads=4, ctx_range=ctx_range)
    print(f"mixed trees {sorted(wl.tree_sizes.tolist())} kernel={kernel} split={split_tokens}",
          flush=True)
    got = _verify_gpu(wl, flags=KERNEL_FLAGS[kernel], split_tokens=split_tokens)
    seqs = list(range(wl.spec.batch))
    _check_rows(got, oracle_verify_rows(wl, seqs), wl, seqs)


def test_verify_mixed_tree_sizes_grouped_query_heads():
    """The small-tree path with 8 query heads over 2 KV heads."""
    import dataclasses
    wl = _mixed_workload(60, 12, heads=8, ctx_range=(20, 500))
    kn = wl.k_new[:, :, ::4].contiguous()
    vn = wl.v_new[:, :, ::4].contiguous()
    pool = wl.kv_pages[:, :, ::4].contiguous()
    spec = dataclasses.replace(wl.spec, kv_heads=2)
    wl = dataclasses.replace(wl, spec=spec, k_new=kn, v_new=vn, kv_pages=pool)
    got = _verify_gpu(wl)
    seqs = list(range(wl.spec.batch))
    _check_rows(got, oracle_verify_rows(wl, seqs), wl, seqs)


@pytest.mark.parametrize("kernel", ["grid", "persistent"])
def test_verify_invalid_page_reads_page_zero(kernel):
    """A block id outside the pool, inside a context, is never used as an
    address: the MFMA kernels read pool page 0 for it (its tokens are scored
    with page 0's K and V), so the result equals the oracle run on the same
    table with those ids replaced by 0."""
    import dataclasses
    wl = make_workload("vicuna7b_b16", 23, batch=3, heads=4, ctx_range=(300, 700))
    table = wl.block_table.copy()
    table[0, 3] = wl.num_blocks + 5                        # past the pool
    table[1, int(wl.ctx_lens[1]) // 16 - 1] = -3           # negative, the last full page
    table[2, 0] = np.iinfo(np.int32).max
    bad = dataclasses.replace(wl, block_table=table)
    fixed = dataclasses.replace(wl, block_table=np.where(
        (table < 0) | (table >= wl.num_blocks), 0, table).astype(np.int32))
    got = _verify_gpu(bad, flags=KERNEL_FLAGS[kernel])
    ref = oracle_verify_rows(fixed, range(3))
    _check_rows(got, ref, fixed, [0, 1, 2])


def test_verify_is_deterministic():
    wl = make_workload("vicuna7b_b16", 2, batch=4, heads=4, ctx_range=(200, 1500))
    a = _verify_gpu(wl)
    b = _verify_gpu(wl)
    assert np.array_equal(a, b)


def test_verify_larger_max_ctx_bound():
    """The grid is sized by the host bound; a loose bound changes nothing."""
    wl = make_workload("vicuna7b_b16", 10, batch=3, heads=2, ctx_range=(100, 900))
    a = _verify_gpu(wl)
    b = _verify_gpu(wl, max_ctx_len=wl.max_blocks * 16 - wl.spec.t_max)
    assert np.max(np.abs(a - b)) <= 1e-6 or np.array_equal(a, b)


# ----------------------------------------------------------------- accept --

def _accept_gpu(wl):
    d = dev(wl)
    tv = verifier(wl)
    L, P = tv.accept(d["node_argmax"], d["cand_tokens"], d["tree_parent"])
    torch.cuda.synchronize()
    return L.cpu().numpy(), P.cpu().numpy()


@pytest.mark.parametrize("name", ["tiny", "vicuna7b_bs1", "vicuna7b_b16", "vicuna13b_b8",
                                  "stress_b64"])
def test_accept_bit_exact(name):
    for seed in range(5):
        wl = make_workload(name, seed, heads=1, ctx_range=(16, 16))
        L, P = _accept_gpu(wl)
        Lr, Pr = oracle.accept_greedy(wl.node_argmax, wl.cand_tokens, wl.tree_parent)
        assert np.array_equal(L, Lr) and np.array_equal(P, Pr), (name, seed)


def test_accept_exhaustive_small_trees_on_gpu():
    """Every tree with T <= 7 nodes x every edge-match pattern, as one batch
    per T (duplicate sibling tokens included)."""
    import itertools
    from medusa_tree_attention_attn_amd import TreeVerifier
    rng = np.random.default_rng(0)
    for T in range(1, 8):
        rows_p, rows_c, rows_a = [], [], []
        for ps in itertools.product(*[range(i) for i in range(1, T)]):
            par = [-1] + list(ps)
            for pat in itertools.product([False, True], repeat=T - 1):
                amax = rng.integers(100, 200, size=T)
                cand = [0] + [int(amax[par[i]]) if pat[i - 1] else int(amax[par[i]]) + 1000
                              for i in range(1, T)]
                rows_p.append(par)
                rows_c.append(cand)
                rows_a.append(amax)
        P = np.array(rows_p, dtype=np.int32)
        C = np.array(rows_c, dtype=np.int32)
        A = np.array(rows_a, dtype=np.int32)
        B = P.shape[0]
        tv = TreeVerifier(batch=B, t_max=T, num_heads=1, num_kv_heads=1, head_dim=64,
                          max_blocks_per_seq=1, num_blocks=1, max_ctx_len=0,
                          dtype=torch.float32)
        g = lambda a: torch.from_numpy(a).cuda()
        L, path = tv.accept(g(A), g(C), g(P))
        torch.cuda.synchronize()
        Lr, Pr = oracle.accept_greedy(A, C, P)
        assert np.array_equal(L.cpu().numpy(), Lr), T
        assert np.array_equal(path.cpu().numpy(), Pr), T


def test_accept_all_and_none_match():
    wl = make_workload("vicuna7b_b16", 11, heads=1, ctx_range=(16, 16))
    for val in (0, 1):
        amax = np.full_like(wl.node_argmax, 5)
        cand = np.full_like(wl.cand_tokens, 5 + val)
        import dataclasses
        w2 = dataclasses.replace(wl, node_argmax=amax, cand_tokens=cand)
        L, P = _accept_gpu(w2)
        Lr, Pr = oracle.accept_greedy(amax, cand, wl.tree_parent)
        assert np.array_equal(L, Lr) and np.array_equal(P, Pr)



@pytest.mark.parametrize("mismatch_depth", [None, 1, 17, 40, 63])
def test_accept_deep_chains(mismatch_depth):
    """Chains of 64 nodes (depth 63), where the acceptance takes one step per
    tree level and reads the path back through every level: every edge
    matches, or the first mismatch sits at a given depth (at another depth
    in the second sequence; the third matches throughout).  The separate
    acceptance and the fused acceptance + commit against the oracle, the
    whole pool bit for bit."""
    import dataclasses
    wl = make_workload("vicuna7b_bs1", 5, batch=3, heads=2, ctx_range=(1, 200),
                       tree_sizes=(64,), chain=True)
    dep = np.asarray(wl.tree_depth)
    assert dep.max() == 63
    amax = np.full_like(wl.node_argmax, 7)
    cand = np.full_like(wl.cand_tokens, 7)
    if mismatch_depth is not None:
        cand[0][dep[0] == mismatch_depth] = 8
        cand[1][dep[1] == (mismatch_depth + 1) // 2] = 8
    wl = dataclasses.replace(wl, node_argmax=amax, cand_tokens=cand)
    Lr, Pr = oracle.accept_greedy(amax, cand, wl.tree_parent)
    expect = [mismatch_depth or 64, (mismatch_depth + 1) // 2 if mismatch_depth else 64, 64]
    assert list(Lr) == expect
    L, P = _accept_gpu(wl)
    assert np.array_equal(L, Lr) and np.array_equal(P, Pr)
    d = dev(wl)
    tv = verifier(wl)
    L2, P2 = tv.accept_commit(d["node_argmax"], d["cand_tokens"], d["tree_parent"], d["k_new"],
                              d["v_new"], d["kv_pages"], d["block_table"], d["ctx_lens"])
    torch.cuda.synchronize()
    assert np.array_equal(L2.cpu().numpy(), Lr) and np.array_equal(P2.cpu().numpy(), Pr)
    rope = oracle.rope_table(wl.spec.head_dim, wl.max_ctx_len + wl.spec.t_max)
    ref = oracle.commit(wl.k_new, wl.v_new, Lr, Pr, wl.kv_pages, wl.block_table, wl.ctx_lens,
                        rope)
    assert torch.equal(pool_bits(d["kv_pages"].cpu()), pool_bits(ref))


# ----------------------------------------------------------------- commit --

def _commit_gpu(wl, L=None, P=None):
    d = dev(wl)
    tv = verifier(wl)
    if L is None:
        Lg, Pg = tv.accept(d["node_argmax"], d["cand_tokens"], d["tree_parent"])
    else:
        Lg = torch.from_numpy(L).cuda()
        Pg = torch.from_numpy(P).cuda()
    tv.commit(d["k_new"], d["v_new"], Lg, Pg, d["kv_pages"], d["block_table"], d["ctx_lens"])
    torch.cuda.synchronize()
    return d["kv_pages"], Lg.cpu().numpy(), Pg.cpu().numpy(), tv


@pytest.mark.parametrize("name,seed,kw", [
    ("tiny", 0, {}), ("tiny", 1, dict(ctx_range=(0, 31))),
    ("vicuna7b_bs1", 0, {}), ("vicuna7b_b16", 0, {}), ("vicuna13b_b8", 0, {}),
    ("stress_b64", 3, dict(batch=12, heads=4, ctx_range=(0, 200))),
])
def test_commit_bit_exact_whole_pool(name, seed, kw):
    wl = make_workload(name, seed, **kw)
    # force long accepted paths so every depth is exercised
    amax = np.full_like(wl.node_argmax, 9)
    cand = np.full_like(wl.cand_tokens, 9)
    L, P = oracle.accept_greedy(amax, cand, wl.tree_parent)
    pool_gpu, _, _, tv = _commit_gpu(wl, L, P)
    rope = oracle.rope_table(wl.spec.head_dim, wl.max_ctx_len + wl.spec.t_max)
    ref = oracle.commit(wl.k_new, wl.v_new, L, P, wl.kv_pages, wl.block_table, wl.ctx_lens, rope)
    got = pool_bits(pool_gpu.cpu())
    exp = pool_bits(ref)
    diff = (got != exp).nonzero()
    assert diff.numel() == 0, f"{diff.shape[0]} differing elements, first {diff[:4].tolist()}"


def test_commit_stress_full_size():
    wl = make_workload("stress_b64", 0)
    before = wl.kv_pages.to("cuda")
    pool_gpu, L, P, _ = _commit_gpu(wl)
    Lr, Pr = oracle.accept_greedy(wl.node_argmax, wl.cand_tokens, wl.tree_parent)
    assert np.array_equal(L, Lr) and np.array_equal(P, Pr)
    # touched pages: every page of the committed slots
    touched = set()
    for b in range(wl.spec.batch):
        for i in range(int(L[b])):
            touched.add(int(wl.block_table[b, (int(wl.ctx_lens[b]) + i) // 16]))
    touched = sorted(touched)
    idx = torch.tensor(touched, device="cuda")
    mask = torch.ones(wl.num_blocks, dtype=torch.bool, device="cuda")
    mask[idx] = False
    assert torch.equal(pool_bits(pool_gpu[mask]), pool_bits(before[mask]))
    # the touched pages against the oracle on the sub-problem
    rope = oracle.rope_table(128, wl.max_ctx_len + wl.spec.t_max)
    sub_pool = wl.kv_pages.index_select(0, torch.tensor(touched))
    remap = {blk: k for k, blk in enumerate(touched)}
    table = np.array([[remap.get(int(x), -1) for x in row] for row in wl.block_table],
                     dtype=np.int32)
    ref = oracle.commit(wl.k_new, wl.v_new, L, P, sub_pool, table, wl.ctx_lens, rope)
    got = pool_gpu.index_select(0, idx).cpu()
    assert torch.equal(pool_bits(got), pool_bits(ref))


@pytest.mark.parametrize("name,seed,kw", [
    ("tiny", 0, {}), ("tiny", 2, dict(ctx_range=(0, 31))),
    ("vicuna7b_bs1", 1, {}), ("vicuna7b_b16", 0, {}), ("vicuna13b_b8", 1, {}),
    ("stress_b64", 4, dict(batch=12, heads=4, ctx_range=(0, 200))),
])
def test_accept_commit_fused_bit_exact(name, seed, kw):
    """The one-launch acceptance + commit against the oracle's accept_greedy
    then commit: accept_len, accept_path and every byte of the pool."""
    wl = make_workload(name, seed, **kw)
    d = dev(wl)
    tv = verifier(wl)
    L, P = tv.accept_commit(d["node_argmax"], d["cand_tokens"], d["tree_parent"], d["k_new"],
                            d["v_new"], d["kv_pages"], d["block_table"], d["ctx_lens"])
    torch.cuda.synchronize()
    Lr, Pr = oracle.accept_greedy(wl.node_argmax, wl.cand_tokens, wl.tree_parent)
    assert np.array_equal(L.cpu().numpy(), Lr) and np.array_equal(P.cpu().numpy(), Pr)
    rope = oracle.rope_table(wl.spec.head_dim, wl.max_ctx_len + wl.spec.t_max)
    ref = oracle.commit(wl.k_new, wl.v_new, Lr, Pr, wl.kv_pages, wl.block_table, wl.ctx_lens,
                        rope)
    diff = (pool_bits(d["kv_pages"].cpu()) != pool_bits(ref)).nonzero()
    assert diff.numel() == 0, f"{diff.shape[0]} differing elements"


def test_accept_commit_fused_long_paths():
    """Every candidate matches: the accepted path reaches the deepest node."""
    wl = make_workload("vicuna13b_b8", 2, heads=4, ctx_range=(1, 300))
    import dataclasses
    wl = dataclasses.replace(wl, node_argmax=np.full_like(wl.node_argmax, 9),
                             cand_tokens=np.full_like(wl.cand_tokens, 9))
    d = dev(wl)
    tv = verifier(wl)
    L, P = tv.accept_commit(d["node_argmax"], d["cand_tokens"], d["tree_parent"], d["k_new"],
                            d["v_new"], d["kv_pages"], d["block_table"], d["ctx_lens"])
    torch.cuda.synchronize()
    Lr, Pr = oracle.accept_greedy(wl.node_argmax, wl.cand_tokens, wl.tree_parent)
    assert np.array_equal(L.cpu().numpy(), Lr) and np.array_equal(P.cpu().numpy(), Pr)
    assert Lr.min() == wl.tree_depth.max(axis=1).min() + 1
    rope = oracle.rope_table(wl.spec.head_dim, wl.max_ctx_len + wl.spec.t_max)
    ref = oracle.commit(wl.k_new, wl.v_new, Lr, Pr, wl.kv_pages, wl.block_table, wl.ctx_lens,
                        rope)
    assert torch.equal(pool_bits(d["kv_pages"].cpu()), pool_bits(ref))


# ------------------------------------------------------------------- rope --

@pytest.mark.parametrize("d", [64, 128])
def test_rope_table_bit_exact(d):
    from medusa_tree_attention_attn_amd import tree_attn_rope_table
    n = 8192 + 64 + 64
    t = torch.empty((n, d // 2, 2), dtype=torch.float32, device="cuda")
    tree_attn_rope_table(d, 10000.0, n, t, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    got = t.cpu().numpy()
    ref = oracle.rope_table(d, n)
    bad = np.flatnonzero(got.view(np.uint32).ravel() != ref.view(np.uint32).ravel())
    assert bad.size == 0, f"{bad.size} of {ref.size} table entries differ"


# ------------------------------------------------------------- full step --

def test_two_chained_steps_match_oracle():
    """verify -> accept -> commit, then verify again at ctx + accept_len:
    both verifies and the commit agree with the oracle run the same way."""
    wl = make_workload("vicuna7b_b16", 12, batch=4, heads=4, ctx_range=(40, 700),
                       tree_sizes=(30,))
    d = dev(wl)
    tv = verifier(wl, max_ctx_len=wl.max_ctx_len + wl.max_depth + 1)
    out1 = tv.verify(d["q"], d["k_new"], d["v_new"], d["kv_pages"], d["block_table"],
                     d["ctx_lens"], d["tree_parent"], d["tree_depth"])
    L, P = tv.accept(d["node_argmax"], d["cand_tokens"], d["tree_parent"])
    tv.commit(d["k_new"], d["v_new"], L, P, d["kv_pages"], d["block_table"], d["ctx_lens"])
    ctx2 = d["ctx_lens"] + L
    # second step reuses the tree but with fresh q/k/v draws
    w2 = make_workload("vicuna7b_b16", 13, batch=4, heads=4, ctx_range=(40, 700),
                       tree_sizes=(30,))
    out2 = tv.verify(w2.q.cuda(), w2.k_new.cuda(), w2.v_new.cuda(), d["kv_pages"],
                     d["block_table"], ctx2, d["tree_parent"], d["tree_depth"])
    torch.cuda.synchronize()
    Lr, Pr = oracle.accept_greedy(wl.node_argmax, wl.cand_tokens, wl.tree_parent)
    assert np.array_equal(L.cpu().numpy(), Lr) and np.array_equal(P.cpu().numpy(), Pr)
    rope = oracle.rope_table(128, wl.max_ctx_len + wl.max_depth + 1 + wl.spec.t_max)
    pool1 = oracle.commit(wl.k_new, wl.v_new, Lr, Pr, wl.kv_pages, wl.block_table,
                          wl.ctx_lens, rope)
    assert torch.equal(pool_bits(d["kv_pages"].cpu()), pool_bits(pool1))
    r1 = oracle.verify(wl.q, wl.k_new, wl.v_new, wl.kv_pages, wl.block_table, wl.ctx_lens,
                       wl.tree_parent, wl.tree_depth)
    r2 = oracle.verify(w2.q, w2.k_new, w2.v_new, pool1, wl.block_table, wl.ctx_lens + Lr,
                       wl.tree_parent, wl.tree_depth)
    real = wl.tree_parent != oracle.PAD_PARENT
    assert np.abs(out1.float().cpu().numpy() - r1)[real].max() <= ATOL
    assert np.abs(out2.float().cpu().numpy() - r2)[real].max() <= ATOL


def _poison_unused_slots(wl):
    """NaN in every cache slot the context does not cover: the tail of each
    sequence's last page and all its pages past the context (the ones
    reserved for the commit)."""
    pool = wl.kv_pages.clone()
    nan = float("nan")
    for b in range(wl.spec.batch):
        ctx = int(wl.ctx_lens[b])
        for lb in range(wl.max_blocks):
            blk = int(wl.block_table[b, lb])
            if blk < 0:
                continue
            first = max(0, ctx - 16 * lb)       # slots of this page past the context
            if first < 16:
                pool[blk, :, :, first:] = nan
    import dataclasses
    return dataclasses.replace(wl, kv_pages=pool)


@pytest.mark.parametrize("name,kw,kernel", [
    ("vicuna7b_b16", dict(batch=4, heads=3, ctx_range=(1, 700)), "default"),
    ("vicuna7b_b16", dict(batch=4, heads=3, ctx_range=(1, 700)), "persistent"),
    ("vicuna7b_b16", dict(batch=4, heads=3, ctx_range=(1, 700)), "simple"),
    ("stress_b64", dict(batch=6, heads=2, ctx_range=(1, 300)), "default"),
    ("decode_b64", dict(batch=5, heads=2, ctx_range=(1, 500)), "default"),
])
def test_verify_ignores_nan_in_unused_cache_slots(name, kw, kernel):
    """Slots past ctx_len are never part of the softmax; whatever they hold
    (here NaN) must not reach the output."""
    wl = _poison_unused_slots(make_workload(name, 15, **kw))
    print(f"verify with NaN past the context: {name} {kw} kernel={kernel}", flush=True)
    got = _verify_gpu(wl, KERNEL_FLAGS[kernel])
    assert not np.isnan(got).any()
    ref = oracle_verify_rows(wl, range(wl.spec.batch))
    _check_rows(got, ref, wl, list(range(wl.spec.batch)))
