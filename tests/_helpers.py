"""Plumbing shared by the GPU parity tests: device copies of a workload,
compact sub-problems for sampled oracle checks, and the oracle calls."""
from __future__ import annotations

import os

import numpy as np
import torch

import oracle


def dev(wl, device="cuda"):
    """Device tensors of a workload (inputs only; nothing computed)."""
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)
    return dict(
        q=wl.q.to(device), k_new=wl.k_new.to(device), v_new=wl.v_new.to(device),
        kv_pages=wl.kv_pages.to(device), block_table=i32(wl.block_table),
        ctx_lens=i32(wl.ctx_lens), tree_parent=i32(wl.tree_parent),
        tree_depth=i32(wl.tree_depth), node_argmax=i32(wl.node_argmax),
        cand_tokens=i32(wl.cand_tokens))


def verifier(wl, flags=0, device="cuda", max_ctx_len=None, split_tokens=0):
    from medusa_tree_attention_attn_amd import TreeVerifier
    s = wl.spec
    return TreeVerifier(batch=s.batch, t_max=s.t_max, num_heads=s.heads,
                        num_kv_heads=s.kv_heads, head_dim=s.head_dim,
                        max_blocks_per_seq=wl.max_blocks, num_blocks=wl.num_blocks,
                        max_ctx_len=wl.max_ctx_len if max_ctx_len is None else max_ctx_len,
                        dtype=wl.torch_dtype, device=device, flags=flags,
                        split_tokens=split_tokens)


def sub_problem(wl, seqs):
    """Sequences `seqs` with only the pages they reference, renumbered: the
    oracle then needs no copy of the whole pool."""
    seqs = list(seqs)
    table = wl.block_table[seqs]
    used = np.unique(table[table >= 0])
    remap = -np.ones(wl.num_blocks, dtype=np.int64)
    remap[used] = np.arange(len(used))
    new_table = np.where(table >= 0, remap[np.maximum(table, 0)], -1).astype(np.int32)
    pool = wl.kv_pages.index_select(0, torch.from_numpy(used))
    return dict(q=wl.q[seqs], k_new=wl.k_new[seqs], v_new=wl.v_new[seqs], kv_pages=pool,
                block_table=new_table, ctx_lens=wl.ctx_lens[seqs],
                tree_parent=wl.tree_parent[seqs], tree_depth=wl.tree_depth[seqs])


def _host_threads() -> int:
    """Threads for the oracle checks: the CPUs this process may run on,
    capped at 8 (the per-node loops of the oracle hold the interpreter
    lock between NumPy calls, so more threads only contend for it)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(8, n))


def oracle_verify_rows(wl, seqs, heads=None):
    """Oracle output [len(seqs)][T][len(heads)][d] for the sampled rows.  The
    (sequence, head) pairs are independent calls of the oracle, spread over a
    thread pool (NumPy releases the interpreter lock in its array work), each
    with a one-thread BLAS."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits
    sp = sub_problem(wl, seqs)
    f = lambda t: t.to(torch.float32).numpy()
    q, kn, vn, pool = f(sp["q"]), f(sp["k_new"]), f(sp["v_new"]), f(sp["kv_pages"])
    heads = list(range(wl.spec.heads)) if heads is None else list(heads)
    T, d = wl.spec.t_max, wl.spec.head_dim
    out = np.zeros((len(seqs), T, len(heads), d))

    def one(job):
        bi, hi = job
        out[bi, :, hi] = oracle.verify_head(q, kn, vn, pool, sp["block_table"],
                                            sp["ctx_lens"], sp["tree_parent"],
                                            sp["tree_depth"], bi, heads[hi])

    jobs = [(bi, hi) for bi in range(len(seqs)) for hi in range(len(heads))]
    with threadpool_limits(1):
        if len(jobs) < 4:
            for j in jobs:
                one(j)
        else:
            with ThreadPoolExecutor(max_workers=_host_threads()) as ex:
                list(ex.map(one, jobs))
    return out


def pool_bits(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


# Attention bar.  `out` has q's dtype, so the result is rounded to bf16 after
# the fp32 accumulation: that rounding alone is up to 2^-8 * |out|, which
# exceeds 1e-2 once |out| > 2.56.  That only happens for nodes that attend to
# a handful of keys.  The bound is therefore set row by row (one row = one
# (sequence, node, head) output vector): every row of a sequence whose
# context holds at least 128 tokens is held to the plain max-abs 1e-2; only
# the rows of sequences with shorter contexts get the output-rounding term on
# top.
ATOL = 1e-2
RTOL_OUT_ROUNDING = 2.0 ** -8
SHORT_CTX = 128


def check_attention_rows(got, ref, wl, seqs):
    """got, ref: [len(seqs)][T][heads][d].  Padding rows must be exact zeros;
    each real row is held to its own bound (see ATOL above).  Returns the
    worst error over the rows held to the plain bound."""
    seqs = list(seqs)
    real = wl.tree_parent[seqs] != oracle.PAD_PARENT        # [len(seqs)][T]
    err = np.abs(got - ref)
    assert np.all(got[~real] == 0.0), "padding rows must be zero"
    short = np.asarray(wl.ctx_lens)[seqs] < SHORT_CTX       # [len(seqs)]
    bound = np.where(short[:, None, None, None], ATOL + RTOL_OUT_ROUNDING * np.abs(ref), ATOL)
    long_rows = real & ~short[:, None]
    short_rows = real & short[:, None]
    worst_long = float(err[long_rows].max()) if long_rows.any() else 0.0
    worst_short = float(err[short_rows].max()) if short_rows.any() else 0.0
    print(f"  max |gpu - oracle|: {worst_long:.3e} on {int(long_rows.sum())} node rows with "
          f"ctx >= {SHORT_CTX}, {worst_short:.3e} on {int(short_rows.sum())} with shorter "
          f"contexts", flush=True)
    assert worst_long <= ATOL, worst_long
    assert np.all(err[real] <= bound[real]), float((err / bound)[real].max())
    return worst_long
