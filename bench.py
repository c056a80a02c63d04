"""Benchmark of the Medusa tree-verify step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = tree_attn_verify -> tree_accept_commit (greedy acceptance and the
KV commit of the accepted path in one launch; --separate-accept-commit runs
tree_accept_greedy -> kv_commit_path instead) over one
batch of the synthetic workload (default: batch 16, 32 heads, head_dim 128,
bf16, contexts uniform in [256, 2048], trees of 64 nodes of depth <= 4,
acceptance probability 0.3).  Untimed steps for --prewarm-ms (the GPU's
clocks ramp up under sustained load; every timed measurement below is
preceded by such a pre-warm of the same calls), W untimed steps, then
exactly K timed steps
launched from Python between two device synchronisations; the same K steps
replayed as one captured HIP graph are reported beside them
(ms_per_step_graph).  Inputs are resident in HBM before the
timed region; the steps rotate over enough copies of the inputs and of the KV
pool (>= 1 GB in total) that the 256 MB Infinity Cache cannot serve a repeat.

Prints one JSON line: verified tree-tokens/s, the verify kernel's HBM
roofline fraction from its HIP-event launch time and its algorithmic bytes,
the greedy-token argmax (and argmax fused with acceptance) on synthetic
logits, and the oracle timed on this host's CPU.  The oracle leg
(cpu_baseline) also checks the outputs of the timed run against the oracle
before anything is printed; with --no-cpu-baseline that check is skipped and
the line says so.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "verify_mfma_vicuna7b_b16_traffic.json")


def counted_traffic(workload: str, kernel: str):
    """HBM bytes per verify launch from the committed rocprofv3 counter runs
    (FETCH_SIZE / WRITE_SIZE scaled by a plain copy of known size), or None
    when the kernel sources changed since the counters were taken or the
    workload differs."""
    import hashlib
    try:
        rec = json.load(open(TRAFFIC_RECORD))
    except (OSError, ValueError):
        return None
    if not rec.get("workload", "").startswith(workload + " ") or rec.get("kernel") != kernel:
        return None
    h = hashlib.sha256()
    for f in rec["sources"]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return rec["traffic_bytes_per_launch"] if h.hexdigest() == rec["sources_sha256"] else None
# The grid verify kernel's code: its device code and the headers it takes
# device code from (the host-side plan and launch declarations do not change
# what one launch moves for a given plan).
VERIFY_SOURCES = [
    "medusa_tree_attention_attn_amd/csrc/verify_mfma.hip",
    "medusa_tree_attention_attn_amd/csrc/mfma_tile.h",
    "medusa_tree_attention_attn_amd/csrc/page_stream.h",
    "medusa_tree_attention_attn_amd/csrc/common.h",
]


def write_traffic_record(fetch_csv: str, write_csv: str, workload: str, seed: int):
    """Turn two rocprofv3 counter runs of this script (`--pmc FETCH_SIZE`,
    then `--pmc WRITE_SIZE`, both with --calibrate-copy, csv output) into the
    traffic record: per-dispatch means of the verify kernel, each scaled by
    what the same counter reads for the 512 MiB device copies."""
    import csv
    import hashlib

    def per_kernel(path, counter):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        verify = [float(r["Counter_Value"]) for r in rows
                  if "verify_mfma_kernel(" in r["Kernel_Name"]]
        copies = sorted(float(r["Counter_Value"]) for r in rows
                        if "copyBuffer" in r["Kernel_Name"])
        if not verify or len(copies) < 5:
            raise SystemExit(f"{path}: no verify dispatches or no calibration copies")
        return sum(verify) / len(verify), len(verify), sum(copies[-5:]) / 5

    copy_kb = (512 << 20) / 1024
    f_kb, nf, f_copy = per_kernel(fetch_csv, "FETCH_SIZE")
    w_kb, nw, w_copy = per_kernel(write_csv, "WRITE_SIZE")
    f_scale, w_scale = copy_kb / f_copy, copy_kb / w_copy
    h = hashlib.sha256()
    for f in VERIFY_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    rec = {
        "kernel": "verify_mfma_kernel",
        "workload": f"{workload} seed {seed}",
        "sources": VERIFY_SOURCES,
        "sources_sha256": h.hexdigest(),
        "dispatches": [nf, nw],
        "fetch_size_kb_per_dispatch": round(f_kb, 1),
        "write_size_kb_per_dispatch": round(w_kb, 1),
        "copy_calibration": {"bytes": float(512 << 20), "fetch_size_kb": round(f_copy, 1),
                             "write_size_kb": round(w_copy, 1), "fetch_scale": round(f_scale, 4),
                             "write_scale": round(w_scale, 4)},
        "traffic_bytes_per_launch": int(round((f_kb * f_scale + w_kb * w_scale) * 1024)),
    }
    with open(TRAFFIC_RECORD, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec))


POOL_BYTES_TARGET = 1 << 30
# Typical acceptance settings measured and checked: temperature, epsilon
# (posterior threshold) and delta (its entropy factor), as commonly set for Medusa.
TYPICAL = (1.0, 0.09, 0.3)


def algorithmic_bytes(wl, accept_len=None):
    """Bytes the step must move (per launch), from the workload's shapes:
    verify: cached K/V of every context token, q + out + k_new + v_new of every
    real node, block-table entries, tree metadata, RoPE rows of the distinct
    positions; accept: argmax/candidates/parents + outputs; commit: the
    accepted rows read from k_new/v_new and written to the pool."""
    s = wl.spec
    es = 2 if s.dtype == "bf16" else 4
    ctx = wl.ctx_lens.astype(np.int64)
    tb = wl.tree_sizes.astype(np.int64)
    d, H, Hkv = s.head_dim, s.heads, s.kv_heads
    kv = int((ctx * 2 * Hkv * d * es).sum())
    qo = int((tb * 2 * H * d * es).sum())
    kvn = int((tb * 2 * Hkv * d * es).sum())
    table = int(((ctx + 15) // 16 * 4).sum())
    meta = int((tb * 8).sum())
    depth_rows = np.array([wl.tree_depth[b, : wl.tree_sizes[b]].max() + 1
                           for b in range(s.batch)], dtype=np.int64)
    rope = int((depth_rows * (d // 2) * 8).sum())
    verify = kv + qo + kvn + table + meta + rope
    accept = int((tb * 12).sum()) + s.batch * (4 + 4 * s.t_max)
    commit = 0
    if accept_len is not None:
        commit = int((np.asarray(accept_len, dtype=np.int64) * 2 * Hkv * d * es * 2).sum())
    return dict(verify=verify, accept=accept, commit=commit, kv=kv,
                step=verify + accept + commit)


def _i32(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)


def _host_threads() -> int:
    """CPUs this process may run on (its affinity mask)."""
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _cpu_model() -> str:
    """The host CPU's model name (lscpu, else /proc/cpuinfo)."""
    import subprocess
    try:
        r = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10)
        for line in r.stdout.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_heads(wl, seqs, threads):
    """Oracle attention [len(seqs)][T][H][d] of the given sequences, every
    head: the independent (sequence, head) calls of oracle.verify_head spread
    over `threads` threads, each with a one-thread BLAS.  Each sequence is
    handed over as a sub-problem holding only the pages it references."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    from threadpoolctl import threadpool_limits
    f = lambda t: t.to(torch.float32).numpy()
    subs = []
    for b in seqs:
        table = wl.block_table[[b]]
        used = np.unique(table[table >= 0])
        remap = -np.ones(wl.num_blocks, dtype=np.int64)
        remap[used] = np.arange(len(used))
        t2 = np.where(table >= 0, remap[np.maximum(table, 0)], -1).astype(np.int32)
        subs.append((f(wl.q[[b]]), f(wl.k_new[[b]]), f(wl.v_new[[b]]),
                     f(wl.kv_pages.index_select(0, torch.from_numpy(used))), t2,
                     wl.ctx_lens[[b]], wl.tree_parent[[b]], wl.tree_depth[[b]]))
    H, T, d = wl.spec.heads, wl.spec.t_max, wl.spec.head_dim
    out = np.zeros((len(seqs), T, H, d))

    def one(job):
        i, h = job
        out[i, :, h] = oracle.verify_head(*subs[i], 0, h)

    with threadpool_limits(1), ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(one, [(i, h) for i in range(len(seqs)) for h in range(H)]))
    return out


def _oracle_parity(wl, out, L, P, pool_after):
    """(cpu_baseline leg) Outputs of the timed run against the CPU oracle,
    for every sequence of the batch: acceptance bit-exact; attention within
    max-abs 1e-2 on every head of every node; the pages holding the
    committed rows bit-exact."""
    import oracle
    Lr, Pr = oracle.accept_greedy(wl.node_argmax, wl.cand_tokens, wl.tree_parent)
    ok_accept = np.array_equal(L, Lr) and np.array_equal(P, Pr)
    seqs = list(range(wl.spec.batch))
    ref = _oracle_heads(wl, seqs, min(8, _host_threads()))
    real = wl.tree_parent != oracle.PAD_PARENT
    worst = float(np.abs(out.float().numpy() - ref)[real].max())
    # commit: the pages holding the accepted rows
    rope = oracle.rope_table(wl.spec.head_dim, wl.max_ctx_len + wl.spec.t_max)
    ok_commit = True
    for b in seqs:
        pages = sorted({int(wl.block_table[b, (int(wl.ctx_lens[b]) + i) // 16])
                        for i in range(int(Lr[b]))})
        sub = wl.kv_pages.index_select(0, torch.tensor(pages))
        remap = {p: k for k, p in enumerate(pages)}
        t2 = np.array([[remap.get(int(x), -1) for x in wl.block_table[b]]], dtype=np.int32)
        ref_pool = oracle.commit(wl.k_new[[b]], wl.v_new[[b]], Lr[[b]], Pr[[b]], sub, t2,
                                 wl.ctx_lens[[b]], rope)
        got = pool_after.index_select(0, torch.tensor(pages))
        ok_commit &= torch.equal(got.view(torch.int16), ref_pool.view(torch.int16))
    return dict(accept_bit_exact=bool(ok_accept), commit_bit_exact=bool(ok_commit),
                attn_max_abs_err=worst, checked_sequences=len(seqs),
                ok=bool(ok_accept and ok_commit and worst <= 1e-2))


def cpu_baseline_leg(wl, timed, posterior_out):
    """The CPU oracle's leg of the benchmark, first half: its results check
    the outputs of the timed GPU run (and of the greedy-token measurement).
    The oracle's own timing runs in cpu_baseline_worker.  Returns the parity
    record."""
    import oracle
    parity = _oracle_parity(wl, *timed)
    if posterior_out is not None:
        from oracle.candidates import assemble_candidates
        from oracle.posterior import vocab_argmax
        logits = posterior_out["logits"]
        A, L, P = posterior_out["greedy"]
        ref = vocab_argmax(logits)
        Lr, Pr = oracle.accept_greedy(ref, wl.cand_tokens, wl.tree_parent)
        parity["posterior_bit_exact"] = bool(np.array_equal(A, ref) and np.array_equal(L, Lr)
                                             and np.array_equal(P, Pr))
        parity["typical"] = _typical_parity(wl, logits, *posterior_out["typical"])
        hl, choices, root, topk, C, Pc, Dc = posterior_out["candidates"]
        Cr, Pcr, Dcr = assemble_candidates(hl, choices, root, wl.spec.t_max, topk)
        parity["candidates_bit_exact"] = bool(np.array_equal(C, Cr) and np.array_equal(Pc, Pcr)
                                              and np.array_equal(Dc, Dcr))
        parity["ok"] = (parity["ok"] and parity["posterior_bit_exact"]
                        and parity["typical"]["ok"] and parity["candidates_bit_exact"])
    return parity


def _typical_parity(wl, logits, S, OK, L, P):
    """Typical acceptance against the oracle: per-node (lse, entropy) within
    1e-4, per-child results exact outside a relative 1e-4 band around the
    threshold, and the path exactly the oracle's rule over the GPU's own
    per-child results."""
    from oracle.posterior import _longest_path, softmax_stats, typical_accept
    temp, eps, delta = TYPICAL
    par = np.asarray(wl.tree_parent)
    cand = np.asarray(wl.cand_tokens)
    p, H = softmax_stats(logits, temp)
    x = logits.to(torch.float64).numpy() / temp
    m = x.max(axis=-1)
    lse = m + np.log(np.exp(x - m[..., None]).sum(axis=-1))
    del x
    Lr, Pr, okr = typical_accept(logits, cand, par, temp, eps, delta)
    thr = np.minimum(eps, delta * np.exp(-H))
    B, T = par.shape
    near = np.zeros((B, T), dtype=bool)
    for b in range(B):
        for i in range(1, T):
            n = par[b, i]
            if n >= 0:
                near[b, i] = abs(p[b, n, cand[b, i]] - thr[b, n]) <= 1e-4 * thr[b, n]
    del p
    err_lse = float(np.abs(S[..., 0] - lse).max())
    err_h = float(np.abs(S[..., 1] - H).max())
    ok_nodes = bool(np.array_equal(OK[~near], okr[~near].astype(np.int32)))
    Lg, Pg = _longest_path(OK.astype(bool), par)
    ok_path = bool(np.array_equal(L, Lg) and np.array_equal(P, Pg))
    clean = ~near.any(axis=1)
    ok_oracle_path = bool(np.array_equal(L[clean], Lr[clean]) and
                          np.array_equal(P[clean], Pr[clean]))
    return dict(lse_max_abs_err=err_lse, entropy_max_abs_err=err_h,
                nodes_near_threshold=int(near.sum()), node_ok_exact=ok_nodes,
                path_exact=ok_path and ok_oracle_path,
                ok=bool(err_lse <= 1e-4 + 1e-5 * np.abs(lse).max() and err_h <= 1e-4 + 1e-5 *
                        np.abs(H).max() and ok_nodes and ok_path and ok_oracle_path))


_ORACLE_ARGS = None  # the workload's arrays, inherited by the oracle's worker processes


def _oracle_pair(job):
    """One (sequence, head) of the oracle's attention, in a worker process."""
    import oracle
    b, h = job
    return oracle.verify_head(*_ORACLE_ARGS, b, h)


def _oracle_timing(wl):
    """The oracle as it stands, timed on one full step of the workload on
    every CPU of this process's affinity mask: oracle.verify_head of every
    (sequence, head) pair over a pool of that many forked processes (each
    with a one-thread BLAS), then the acceptance walk and the commit.  One
    untimed step, then the median of three timed steps.  `cpu_util` is the
    CPU time of this process and its workers over the wall time of the timed
    steps: the cores actually kept busy.  Runs in a process that never
    touches the GPU (see cpu_baseline_worker)."""
    import multiprocessing as mp

    import oracle
    import psutil
    from threadpoolctl import threadpool_limits
    global _ORACLE_ARGS
    threads = _host_threads()
    f = lambda t: t.to(torch.float32).numpy()
    _ORACLE_ARGS = (f(wl.q), f(wl.k_new), f(wl.v_new), f(wl.kv_pages), wl.block_table,
                    wl.ctx_lens, wl.tree_parent, wl.tree_depth)
    rope = oracle.rope_table(wl.spec.head_dim, wl.max_ctx_len + wl.spec.t_max)
    jobs = [(b, h) for b in range(wl.spec.batch) for h in range(wl.spec.heads)]
    me = psutil.Process()

    def cpu_seconds():
        procs = [me] + me.children(recursive=True)
        t = 0.0
        for p in procs:
            try:
                c = p.cpu_times()
                t += c.user + c.system
            except psutil.Error:
                pass
        return t

    with threadpool_limits(1), mp.get_context("fork").Pool(threads) as pool:
        def step():
            pool.map(_oracle_pair, jobs, chunksize=max(1, len(jobs) // (4 * threads)))
            L, P = oracle.accept_greedy(wl.node_argmax, wl.cand_tokens, wl.tree_parent)
            oracle.commit(wl.k_new, wl.v_new, L, P, wl.kv_pages, wl.block_table, wl.ctx_lens,
                          rope)

        step()  # untimed
        times, cpu = [], 0.0
        for _ in range(3):
            c0, t0 = cpu_seconds(), time.perf_counter()
            step()
            times.append(time.perf_counter() - t0)
            cpu += cpu_seconds() - c0
    dt = float(np.median(times))
    return dict(value=round(wl.tree_tokens / dt, 2), unit="tree-tokens/s", cores=threads,
                kind="oracle", cpu_model=_cpu_model(),
                cpu_util=round(cpu / sum(times), 2),
                sample=f"full steps of the workload (oracle.verify_head of all {wl.spec.batch}x"
                       f"{wl.spec.heads} (sequence, head) pairs over {threads} processes, "
                       f"acceptance, commit), seed {wl.seed}: 1 untimed + median of 3 timed "
                       f"steps ({', '.join(f'{t:.2f}' for t in times)} s)",
                seconds=dt)


def cpu_baseline_worker(workload: str, seed: int):
    """The oracle timing in a process of its own, started before the
    benchmark touches the GPU (so its worker processes are forked from a
    process without GPU state).  It waits for a line on stdin, sent once the
    GPU measurements are done, so the two never compete for the host; then
    it prints the timing as one JSON line."""
    from synth import make_workload
    if not sys.stdin.readline():
        return
    res = _oracle_timing(make_workload(workload, seed))
    print(json.dumps(res), flush=True)


def start_cpu_baseline_worker(workload: str, seed: int):
    import subprocess
    return subprocess.Popen([sys.executable, os.path.abspath(__file__), "--cpu-baseline-worker",
                             "--workload", workload, "--seed", str(seed)],
                            stdin=subprocess.PIPE, stdout=subprocess.PIPE, text=True)


def finish_cpu_baseline_worker(proc, log):
    out, _ = proc.communicate("go\n", timeout=900)
    if proc.returncode != 0:
        raise SystemExit(f"oracle timing process failed (exit {proc.returncode})")
    res = json.loads(out.strip().splitlines()[-1])
    log(f"cpu baseline: {res}")
    res.pop("seconds", None)
    return res


def _prewarm(fn, ms):
    """Untimed calls fn(k), k = 0, 1, ..., for `ms` of wall time; the host
    waits every 8 calls so it cannot run far ahead of the GPU.  The GPU's
    clocks ramp up over the first tens of milliseconds of sustained load
    and drop again while it idles."""
    t_end = time.perf_counter() + ms / 1e3
    k = 0
    while time.perf_counter() < t_end:
        fn(k)
        k += 1
        if k % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def time_calls(fn, n_inputs, reps, outputs, prewarm_ms=100.0):
    """Average microseconds per call of fn(k) (k picks input k % n_inputs):
      eager  back-to-back calls from Python between two events: what a
             caller sees, host overhead included when it exceeds the GPU's
             share;
      gpu    the same calls captured once into a HIP graph and replayed:
             the kernels' own time (launch gaps of a replayed graph only).
    Each timing follows prewarm_ms of untimed calls of the same kind.  The
    graph's outputs after the replay must equal the eager ones (both end on
    the same input); otherwise gpu is None."""
    _prewarm(lambda k: fn(k % n_inputs), prewarm_ms)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for k in range(reps):
        fn(k % n_inputs)
    b.record()
    torch.cuda.synchronize()
    eager = a.elapsed_time(b) * 1e3 / reps
    ref = [t.clone() for t in outputs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for k in range(reps):
            fn(k % n_inputs)
    torch.cuda.synchronize()
    _prewarm(lambda k: g.replay(), prewarm_ms)
    gpu = []
    for _ in range(3):
        for t in outputs:
            t.fill_(-7)          # replays must rewrite every output
        torch.cuda.synchronize()
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        if not all(torch.equal(t, r) for t, r in zip(outputs, ref)):
            return round(eager, 2), None
        gpu.append(a.elapsed_time(b) * 1e3 / reps)
    del g
    return round(eager, 2), round(min(gpu), 2)


def read_ceiling(dev, prewarm_ms, reps=20):
    """The device's read-stream rate: tree_attn_stream_read (16-byte
    non-temporal loads, the KV stream's width and policy) over alternating
    halves of a 2 GiB buffer, so each call reads 1 GiB that the 256 MB
    Infinity Cache cannot hold; HIP events around `reps` back-to-back calls
    after a pre-warm."""
    from medusa_tree_attention_attn_amd import tree_attn_stream_read
    half = 1 << 30
    buf = torch.ones(2 * half, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    parts = (buf[:half], buf[half:])
    fn = lambda k: tree_attn_stream_read(parts[k % 2], sink)
    _prewarm(fn, prewarm_ms)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for k in range(reps):
        fn(k)
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / reps
    del buf, parts
    gbs = half / (us * 1e-6) / 1e9
    return {"GB/s": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
            "probe": f"tree_attn_stream_read: 1 GiB contiguous per call, one workgroup per CU, 16-byte non-temporal "
                     f"loads, {reps} calls, {us:.1f} us each"}


def posterior_bench(wl, tv, dev, seed, log, reps=50):
    """The greedy token of every node from synthetic bf16 logits [B][T][vocab]
    (tree_vocab_argmax), the same fused with acceptance
    (tree_argmax_accept), typical acceptance (tree_accept_typical) and the
    next step's candidate tree (tree_medusa_candidates), each over rotating
    input copies (>= 1 GB, beyond the Infinity Cache), timed eager and as a
    replayed graph (time_calls), with the HBM fraction of the input stream
    at the graph's time.  Returns the figures and the outputs of the last
    calls for the oracle leg to check."""
    from synth import make_logits
    logits = make_logits(wl, seed)
    nb = logits.numel() * logits.element_size()
    copies = max(2, math.ceil(POOL_BYTES_TARGET / nb))
    xs = [logits.to(dev) for _ in range(copies)]
    cand, par = _i32(wl.cand_tokens, dev), _i32(wl.tree_parent, dev)
    B, T = wl.node_argmax.shape
    A = torch.empty((B, T), dtype=torch.int32, device=dev)
    L = torch.empty((B,), dtype=torch.int32, device=dev)
    P = torch.empty((B, T), dtype=torch.int32, device=dev)
    S = torch.empty((B, T, 2), dtype=torch.float32, device=dev)
    OK = torch.empty((B, T), dtype=torch.int32, device=dev)
    Lt, Pt = torch.empty_like(L), torch.empty_like(P)
    out = {"logits": f"bf16 [{B}][{T}][{logits.shape[-1]}], {copies} rotating copies",
           "bytes_per_launch": nb + B * T * 4}

    def record(name, eager, gpu, nbytes):
        us = gpu if gpu is not None else eager
        gbs = nbytes / (us * 1e-6) / 1e9
        out[name] = {"us": us, "eager_us": eager, "graph": gpu is not None,
                     "GB/s": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4)}

    temp, eps, delta = TYPICAL
    for name, fn, outs in (
            ("vocab_argmax", lambda k: tv.vocab_argmax(xs[k], A), [A]),
            ("argmax_accept", lambda k: tv.argmax_accept(xs[k], cand, par, A, L, P), [A, L, P]),
            ("typical_accept", lambda k: tv.accept_typical(xs[k], cand, par, temp, eps, delta,
                                                           S, OK, Lt, Pt), [S, OK, Lt, Pt])):
        record(name, *time_calls(fn, copies, reps, outs), out["bytes_per_launch"])
    del xs
    # Candidate tree for the next step: 4 Medusa heads' logits, a 63-path
    # choices list (top-10 ranks, depth <= 4) numbered once.
    from synth import make_choices, make_head_logits
    n_heads, topk = 4, 10
    choices = make_choices(seed, n=63, max_depth=4, topk=topk)
    table = tv.medusa_tree(choices, topk, n_heads)
    hl = make_head_logits(B, n_heads, logits.shape[-1], seed=seed)
    root = torch.from_numpy(np.asarray(wl.node_argmax[:, 0], dtype=np.int32))
    hb = hl.numel() * hl.element_size()
    hcopies = max(2, math.ceil(POOL_BYTES_TARGET / hb))
    hs = [hl.to(dev) for _ in range(hcopies)]
    root_d = root.to(dev)
    C = torch.empty((B, T), dtype=torch.int32, device=dev)
    Pc = torch.empty_like(C)
    Dc = torch.empty_like(C)
    record("medusa_candidates",
           *time_calls(lambda k: tv.candidates(table, hs[k], topk, root_d, C, Pc, Dc), hcopies,
                       reps, [C, Pc, Dc]), hb + 3 * B * T * 4)
    out["medusa_candidates"].update(
        head_logits=f"bf16 [{B}][{n_heads}][{hl.shape[-1]}], {hcopies} rotating copies",
        choices=f"{len(choices)} paths, top-{topk}")
    del hs
    log(f"posterior: {out}")
    host = lambda t: t.cpu().numpy()
    return out, dict(logits=logits, greedy=(host(A), host(L), host(P)),
                     typical=(host(S), host(OK), host(Lt), host(Pt)),
                     candidates=(hl, choices, root.numpy(), topk, host(C), host(Pc), host(Dc)))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="vicuna7b_b16")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--split-tokens", type=int, default=0)
    ap.add_argument("--kernel", choices=("auto", "grid", "persistent", "simple", "decode"),
                    default="auto", help="verify kernel (auto: the library's choice)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-posterior", action="store_true",
                    help="skip the greedy-token argmax measurement")
    ap.add_argument("--separate-accept-commit", action="store_true",
                    help="acceptance and commit as two launches instead of the fused one")
    ap.add_argument("--prewarm-ms", type=float, default=100.0,
                    help="untimed steps for this long before the W warmup steps: the GPU's "
                         "clocks ramp up over the first tens of milliseconds of load")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run plain 512 MiB device copies (for counter scaling)")
    ap.add_argument("--cpu-baseline-worker", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--traffic-record", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the verify kernel's traffic record from two rocprofv3 "
                         "counter-collection CSVs of this script, then exit (no GPU used)")
    args = ap.parse_args()
    if args.traffic_record:
        write_traffic_record(*args.traffic_record, args.workload, args.seed)
        return
    if args.cpu_baseline_worker:
        cpu_baseline_worker(args.workload, args.seed)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported "
              "(the tree-verify step shards by sequence or head with no exchange; "
              "multi-GPU runs are not part of it)", file=sys.stderr)
        sys.exit(2)
    # The oracle's timing process starts before anything touches the GPU.
    cpu_worker = None if args.no_cpu_baseline else start_cpu_baseline_worker(args.workload,
                                                                             args.seed)
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    from medusa_tree_attention_attn_amd import TreeVerifier
    from synth import make_workload

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t_gen = time.perf_counter()
    wl = make_workload(args.workload, args.seed)
    s = wl.spec
    log = lambda *a: print(*a, file=sys.stderr, flush=True)
    log(f"workload {s.name} seed {args.seed}: generated in {time.perf_counter() - t_gen:.1f}s, "
        f"{wl.tree_tokens} tree tokens, pool {wl.kv_pages.numel() * 2 / 1e6:.0f} MB")

    pool_bytes = wl.kv_pages.numel() * wl.kv_pages.element_size()
    copies = max(1, min(8, math.ceil(POOL_BYTES_TARGET / max(pool_bytes, 1))))
    sets = []
    for _ in range(copies):
        sets.append(dict(q=wl.q.to(dev), k=wl.k_new.to(dev), v=wl.v_new.to(dev),
                         pool=wl.kv_pages.to(dev), out=torch.empty_like(wl.q, device=dev)))
    table, ctx = _i32(wl.block_table, dev), _i32(wl.ctx_lens, dev)
    par, dep = _i32(wl.tree_parent, dev), _i32(wl.tree_depth, dev)
    amax, cand = _i32(wl.node_argmax, dev), _i32(wl.cand_tokens, dev)
    L = torch.empty((s.batch,), dtype=torch.int32, device=dev)
    P = torch.empty((s.batch, s.t_max), dtype=torch.int32, device=dev)
    tv = TreeVerifier(batch=s.batch, t_max=s.t_max, num_heads=s.heads, num_kv_heads=s.kv_heads,
                      head_dim=s.head_dim, max_blocks_per_seq=wl.max_blocks,
                      num_blocks=wl.num_blocks, max_ctx_len=wl.max_ctx_len,
                      dtype=wl.torch_dtype, split_tokens=args.split_tokens,
                      flags={"auto": 0, "simple": 1, "grid": 2, "persistent": 4,
                             "decode": 8}[args.kernel])
    from medusa_tree_attention_attn_amd._lib import tree_attn_plan_info
    kernel_name, n_splits, split_tokens = tree_attn_plan_info(tv.desc)
    log(f"{copies} rotating input copies ({copies * pool_bytes / 1e9:.2f} GB of KV pool), "
        f"workspace {tv.workspace.numel() / 1e6:.1f} MB; {kernel_name}, {n_splits} split(s) "
        f"of {split_tokens} tokens")

    def verify(k):
        st = sets[k % copies]
        tv.verify(st["q"], st["k"], st["v"], st["pool"], table, ctx, par, dep, out=st["out"])

    def accept_commit(k):
        st = sets[k % copies]
        if args.separate_accept_commit:
            tv.accept(amax, cand, par, L, P)
            tv.commit(st["k"], st["v"], L, P, st["pool"], table, ctx)
        else:
            tv.accept_commit(amax, cand, par, st["k"], st["v"], st["pool"], table, ctx, L, P)

    def step(k):
        verify(k)
        accept_commit(k)

    if args.calibrate_copy:
        src = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("calibration copies: 5 x 512 MiB device-to-device")

    # The timed steps: W warmup steps, then K steps launched from Python
    # between two events.  The same K steps are also captured as one HIP
    # graph and replayed (what a serving loop that replays its launches
    # would see); that figure is reported beside the eager one, and only if
    # the replay leaves the same bits as the eager steps.
    def time_steps(run):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t = time.perf_counter()
        a.record()
        run()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / args.steps, time.perf_counter() - t

    def eager_steps(first, n):
        for k in range(first, first + n):
            step(k)

    # The GPU's clocks ramp up over the first tens of milliseconds of
    # sustained load, and drop again while it idles (the 13B-shaped verify:
    # 152, 133, 129, then 127.5 us per launch over successive groups of 50).
    # Before each timed measurement, untimed calls of the measured function
    # fill prewarm_ms, so it sees the steady state a serving loop runs at;
    # the host waits every 8 calls so it cannot run far ahead of the GPU.
    def prewarm(fn):
        _prewarm(fn, args.prewarm_ms)

    prewarm(step)
    eager_steps(0, args.warmup)
    torch.cuda.synchronize()
    ms_per_step, wall = time_steps(lambda: eager_steps(args.warmup, args.steps))
    ms_per_step_graph = None
    if args.steps > 0:
        last = (args.warmup + args.steps - 1) % copies
        st = sets[last]
        bits = lambda t: t.view(torch.int16) if t.dtype == torch.bfloat16 else t
        ref = [t.clone() for t in (st["out"], L, P, st["pool"])]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            eager_steps(args.warmup, args.steps)
        torch.cuda.synchronize()
        prewarm(lambda k: g.replay())  # the first replay also uploads the graph
        t_graph = time_steps(g.replay)[0]
        if all(torch.equal(bits(x), bits(y))
               for x, y in zip(ref, (st["out"], L, P, st["pool"]))):
            ms_per_step_graph = t_graph
        else:
            log("graph replay differs from the eager steps: no graph figure")
        del g, ref

    # Verify-kernel launch time for the roofline: the same launches back to
    # back on the library's stream (torch's current stream) between two
    # events, so event and launch overheads are amortised; rocprofv3's
    # per-dispatch duration of the same command agrees with it.
    nv = max(args.steps, 20)
    prewarm(verify)
    va = torch.cuda.Event(enable_timing=True)
    vb = torch.cuda.Event(enable_timing=True)
    va.record()
    for k in range(nv):
        verify(k)
    vb.record()
    torch.cuda.synchronize()
    v_avg = va.elapsed_time(vb) / nv
    va.record()
    for k in range(nv):
        accept_commit(k)
    vb.record()
    torch.cuda.synchronize()
    ac_avg = va.elapsed_time(vb) / nv
    # The same acceptance + commit launches as a replayed graph: the GPU's
    # own time per call (the eager figure above is host-bound when the
    # kernel is shorter than the Python call).
    ac_gpu = None if args.separate_accept_commit else \
        time_calls(accept_commit, copies, nv, [L, P])[1]
    ceiling = read_ceiling(dev, args.prewarm_ms)
    log(f"read ceiling: {ceiling}")
    # restore the outputs of the step loop's last step for the parity check
    step(args.warmup + args.steps - 1)
    torch.cuda.synchronize()

    posterior, posterior_out = (None, None) if args.no_posterior else \
        posterior_bench(wl, tv, dev, args.seed, log)

    # The oracle leg: parity of the timed run's outputs (last copy used by the
    # last step), then the oracle's own timing.
    cpu = None
    chk = {"checked": False, "why": "--no-cpu-baseline: the oracle leg did not run"}
    if not args.no_cpu_baseline:
        last = sets[(args.warmup + args.steps - 1) % copies]
        chk = cpu_baseline_leg(
            wl, (last["out"].cpu(), L.cpu().numpy(), P.cpu().numpy(), last["pool"].cpu()),
            posterior_out)
        log(f"parity of timed outputs: {chk}")
        cpu = finish_cpu_baseline_worker(cpu_worker, log)
        if not chk["ok"]:
            print(json.dumps({"metric": "verified tree-tokens/s", "error": "parity failed",
                              "parity": chk}))
            sys.exit(1)

    nbytes = algorithmic_bytes(wl, L.cpu().numpy())
    achieved = nbytes["verify"] / (v_avg * 1e-3) / 1e9
    tokens_per_s = wl.tree_tokens / (ms_per_step * 1e-3)
    result = {
        "metric": "verified tree-tokens/s (verify+accept+commit step)",
        "value": round(tokens_per_s, 1),
        "unit": "tree-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if s.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{s.name}: batch {s.batch}, {s.heads} heads, head_dim {s.head_dim}, "
                        f"{s.dtype}, contexts U[{s.ctx_range[0]},{s.ctx_range[1]}], trees of "
                        f"{'/'.join(map(str, s.tree_sizes))} nodes, depth <= {s.max_depth}, "
                        f"match p={s.p_match}, seed {args.seed}",
            "global_batch": s.batch,
            "tree_tokens_per_step": wl.tree_tokens,
            "mean_ctx": float(wl.ctx_lens.mean()),
            "split_tokens": split_tokens,
            "splits": n_splits,
            "rotating_copies": copies,
            "parallelism": "single GPU",
            "prewarm_ms": args.prewarm_ms,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": kernel_name + (" + combine_kernel" if n_splits > 1 else ""),
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": (counted_traffic(args.workload, kernel_name)
                        if args.seed == 0 and args.split_tokens == 0 else None),
            "bytes_per_launch": nbytes["verify"],
            "avg_launch_us": round(v_avg * 1e3, 2),
            "ceiling": ceiling,
            "frac_of_ceiling": round(achieved / ceiling["GB/s"], 4),
        },
        "ms_per_step_graph": (round(ms_per_step_graph, 5) if ms_per_step_graph else None),
        "step_hbm_gbs": round(nbytes["step"] / (ms_per_step * 1e-3) / 1e9, 1),
        "per_call_us": {"verify": round(v_avg * 1e3, 2),
                        ("accept, commit" if args.separate_accept_commit else "accept_commit"):
                            round(ac_avg * 1e3, 2),
                        "accept_commit_graph": ac_gpu},
        "parity": {k: v for k, v in chk.items() if k != "ok"},
        "posterior": posterior,
        "cpu_baseline": cpu,
        "wall_s": round(wall, 3),
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
