"""Benchmark of the decode-attention step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-extra]

A step is one pass of the whole hot path over one batch through the C ABI:
kvd_decode_step, which does RoPE at each token's position, the paged append
and split-K decode attention (one fused kernel on matrix-core plans, plus the
split combine).  The same work as two calls (kvd_rope_append_kv, then
kvd_decode_attention) and the attention call alone are timed beside it.

The headline workload is the long-context layer (batch 4, 64 q / 8 kv heads,
head_dim 128, context 131072, paged bf16 cache with block 64), the largest
configuration of the five; the others are reported under their own names.
Inputs are seeded synthetic tensors already resident in HBM.  Successive
steps rotate over several layers' caches (distinct buffers, at least 1 GiB in
all) so that no step finds its cache in the 256 MB Infinity Cache left behind
by the previous one.

Rank 0 prints ONE JSON line.  `value` is tokens/s of the whole step (B*T new
tokens per step) over exactly K timed steps; `roofline` is for the step call
(the fused kernel and the combine): algorithmic bytes per call / its average
duration over those K steps, measured with HIP events on the launch stream.
Every workload (the headline included) is also timed as the median of 20
repetitions of 20 back-to-back calls, and as the median of 20 replays of a
HIP graph holding 20 calls; each is reported as a fraction of the 8 TB/s peak
and of a plain streaming-read kernel's rate on the same device.
`cpu_baseline` times the fp64 oracle on the host cores on a bounded sample of
the headline workload; every other workload carries its own oracle rate.
"""
import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

from kv_cached_decode_amd import binding as kb  # noqa: E402
from kv_cached_decode_amd import workloads  # noqa: E402

PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
HEADLINE = "long_ctx"
REPS, CALLS = 20, 20
KERNEL_SOURCES = ["kvd.cpp", "attn_valu.hip", "attn_mfma.hip", "attn_prefill.hip", "attn_combine.hip",
                  "rope_append.hip", "kvd_internal.h", "bf16_round.h", "rope_math.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_sources_sha():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "kv_cached_decode_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def to_dev_pool(pool, dev):
    if pool.dtype == np.uint16:
        return torch.from_numpy(pool.view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(pool).to(dev)


def describe_data(spec):
    """The input recipe of a workload, in words."""
    dist = {"uniform0.1": "U[-0.1, 0.1]", "normal": "N(0,1)", "normal_scaled": "N(0,1)/sqrt(128)"}[spec.dist]
    parts = [f"seeded {dist} values", f"{spec.kv_dtype} cache"]
    if isinstance(spec.ctx, tuple):
        parts.append(f"ragged contexts U{{{spec.ctx[0]}..{spec.ctx[1]}}}")
    if spec.chunk:
        parts.append(f"ragged chunks U{{{spec.chunk[0]}..{spec.chunk[1]}}} new tokens")
    if spec.big_keys:
        parts.append(f"{spec.big_keys} keys per sequence scaled by {spec.big_key_factor:g}")
    table = {"inorder": "in-order paged table", "shuffled": "shuffled paged table",
             "single": "contiguous cache (one block per sequence)"}[spec.table]
    parts.append(f"{table}, block {spec.block_size}")
    if spec.spare_frac:
        parts.append(f"{spec.spare_frac:.0%} spare blocks and every tail slot NaN/Inf-poisoned")
    if spec.prefix:
        parts.append("cache built by appends of raw prefix tokens")
    return "synthetic (" + "; ".join(parts) + ")"


def workload_text(w):
    s = w.spec
    ctx = f"context {s.ctx[0]}..{s.ctx[1]}" if isinstance(s.ctx, tuple) else f"context {s.ctx}"
    t = f"T={s.q_tokens}" + (f" (chunks {s.chunk[0]}..{s.chunk[1]})" if s.chunk else "")
    return (f"{s.name}: decode step of one attention layer, B={s.num_seqs} {t} Hq={s.n_q_heads} "
            f"Hkv={s.n_kv_heads} D={s.head_dim} {ctx} bs={s.block_size} {s.kv_dtype}")


class Layers:
    """`n` layers' caches of one workload, resident on the GPU."""

    def __init__(self, w, n, dev, kernel, num_splits):
        s = w.spec
        self.w = w
        self.kernel, self.num_splits = kernel, num_splits
        table = torch.from_numpy(w.block_table).to(dev)
        seq_lens = torch.from_numpy(w.seq_lens).to(dev)
        q_lens = torch.from_numpy(w.q_lens).to(dev) if w.q_lens is not None else None
        kd, vd = to_dev_pool(w.k_pool, dev), to_dev_pool(w.v_pool, dev)
        self.kv = []
        for i in range(n):
            k = kd if i == 0 else kd.clone()
            v = vd if i == 0 else vd.clone()
            self.kv.append(kb.PagedKV(k, v, table, seq_lens, s.n_q_heads, s.q_tokens, w.max_seq_len,
                                      q_lens=q_lens))
        self.q = torch.from_numpy(w.q).to(dev)
        self.k = torch.from_numpy(w.k).to(dev)
        self.v = torch.from_numpy(w.v).to(dev)
        self.q_rot = torch.empty_like(self.q)
        self.out = torch.empty_like(self.q)
        self.ws = kb.workspace(self.kv[0], num_splits, kernel)
        if self.ws is not None:
            self.ws = self.ws.clone()
        self.plan = kb.decode_attention_plan(self.kv[0], num_splits, kernel)
        # The step's output is the attention output; the rotated queries are
        # an intermediate.  The matrix-core plans rotate them inside the
        # attention kernel (the decode kernel also appends; the prefill kernel
        # runs after the RoPE/append kernel has appended) and need no buffer
        # for them; the vector-ALU plans run the two kernels in a row and get
        # one, as a caller would pass it, rather than reusing `out`.
        fused = self.plan[2] == kb.KVD_KERNEL_MFMA
        self.step_q_rot = None if fused else self.q_rot

    def step(self, i):
        kv = self.kv[i % len(self.kv)]
        s = self.w.spec
        kb.decode_step(kv, self.q, self.k, self.v, self.out, self.step_q_rot, False, s.rope_base, s.layout,
                       0.0, self.ws, self.num_splits, self.kernel)

    def two_calls(self, i):
        kv = self.kv[i % len(self.kv)]
        s = self.w.spec
        kb.rope_append_kv(kv, self.q, self.k, self.v, self.q_rot, s.rope_base, s.layout)
        kb.decode_attention(kv, self.q_rot, self.out, 0.0, self.ws, self.num_splits, self.kernel)

    def attention(self, i):
        kv = self.kv[i % len(self.kv)]
        kb.decode_attention(kv, self.q_rot, self.out, 0.0, self.ws, self.num_splits, self.kernel)


def timed(fn, steps, warmup):
    """The contract's timing: `warmup` untimed calls, then exactly `steps`
    calls bracketed by synchronisation and timed with HIP events on the
    launch stream.  Returns ms per call."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        fn(i)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def reps_timed(fn, reps=REPS, calls=CALLS):
    """`reps` repetitions of `calls` back-to-back calls, each repetition
    between its own pair of HIP events.  Returns the median ms per call and
    the spread (min, max) over the repetitions."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    torch.cuda.synchronize()
    i = 0
    ev[0].record()
    for r in range(reps):
        for _ in range(calls):
            fn(i)
            i += 1
        ev[r + 1].record()
    torch.cuda.synchronize()
    per = [ev[r].elapsed_time(ev[r + 1]) / calls for r in range(reps)]
    return statistics.median(per), (min(per), max(per))


def graph_timed(fn, results, calls=CALLS, replays=REPS):
    """Device time per call without the host's launch cost: calls 0..calls-1
    of `fn` captured in one HIP graph, replayed `replays` times, each replay
    between its own HIP events; the median ms per call.  The graph's results
    must equal those of the same calls made eagerly (None otherwise)."""
    # the same start for the eager calls and the replay (rows a call leaves
    # as they are, such as padding rows, must match too)
    for r in results:
        r.zero_()
    for i in range(calls):
        fn(i)
    torch.cuda.synchronize()
    eager = [r.clone() for r in results]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for i in range(calls):
            fn(i)
    torch.cuda.synchronize()
    for r in results:
        r.zero_()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    if not all(torch.equal(r, e) for r, e in zip(results, eager)):
        return None
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(replays + 1)]
    ev[0].record()
    for r in range(replays):
        g.replay()
        ev[r + 1].record()
    torch.cuda.synchronize()
    per = [ev[r].elapsed_time(ev[r + 1]) / calls for r in range(replays)]
    del g
    return statistics.median(per)


def graph_timed_us(fn, results, calls=32, replays=20):
    """graph_timed for a call that takes no index, in microseconds."""
    ms = graph_timed(lambda i: fn(), results, calls, replays)
    return None if ms is None else ms * 1e3


def prewarm(L, seconds=0.3):
    """Untimed: run the three call kinds in turn until the GPU's clocks have
    settled, so that the first kind timed is not the one that pays for it."""
    t0 = time.time()
    i = 0
    while time.time() - t0 < seconds:
        for fn in (L.step, L.two_calls, L.attention):
            for _ in range(4):
                fn(i)
                i += 1
        torch.cuda.synchronize()


def layers_for(w):
    # rotate over enough distinct caches to cover >= 1 GiB (4x the MALL)
    kv_bytes = w.k_pool.nbytes + w.v_pool.nbytes
    return int(min(8, max(1, -(-(1 << 30) // kv_bytes))))


def stream_probe(dev, nbytes=2 << 30):
    """The plain streaming-read kernel (kvd_probe_stream_read) over a 2 GiB
    buffer at several grid shapes: the median GB/s of 20 timed reads each.
    Returns the best shape's figure and the whole sweep."""
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    sweep = []
    for wgs in (256, 512, 1024, 2048):
        for threads in (256, 512, 1024):
            for unroll in (4, 16):
                fn = lambda i: kb.probe_stream_read(buf, wgs, threads, unroll, sink)  # noqa: E731
                for i in range(3):
                    fn(i)
                ms, _ = reps_timed(fn, reps=20, calls=1)
                sweep.append({"workgroups": wgs, "threads": threads, "unroll": unroll,
                              "GBs": round(nbytes / (ms * 1e-3) / 1e9, 1)})
    del buf
    torch.cuda.empty_cache()
    best = max(sweep, key=lambda r: r["GBs"])
    one_per_cu = max((r for r in sweep if r["workgroups"] == 256), key=lambda r: r["GBs"])
    return {"GBs": best["GBs"], "frac_of_peak": round(best["GBs"] / PEAK_HBM_GBS, 4),
            "best_shape": {k: best[k] for k in ("workgroups", "threads", "unroll")},
            "GBs_256_workgroups": one_per_cu["GBs"], "bytes_read": nbytes, "sweep": sweep}


def oracle_rate(w, budget_s=3.0):
    """The fp64 oracle (as it stands) on the host cores for this workload:
    RoPE + append of every new token, then attention over a seeded sample of
    query rows that grows until it takes about budget_s (every row if that
    is sooner).  Returns query tokens/s, counting a row's share of its token."""
    import oracle
    s = w.spec
    dt = oracle.ORACLE_BF16 if s.kv_dtype == "bf16" else oracle.ORACLE_F32
    oc = oracle.OracleCache(num_seqs=s.num_seqs, q_tokens=s.q_tokens, n_q_heads=s.n_q_heads,
                            n_kv_heads=s.n_kv_heads, head_dim=s.head_dim, block_size=s.block_size,
                            k_pool=w.k_pool.copy(), v_pool=w.v_pool.copy(), block_table=w.block_table,
                            seq_lens=w.seq_lens, cache_dtype=dt, q_lens=w.q_lens)
    t0 = time.perf_counter()
    q_rot = oc.rope_append_kv(w.q, w.k, w.v, s.rope_base, s.layout)
    t_rope = time.perf_counter() - t0
    total = s.num_seqs * s.q_tokens * s.n_q_heads
    rng = np.random.default_rng(0)
    n = max(1, total // 64)
    while True:
        rows = np.sort(rng.choice(total, size=min(n, total), replace=False)).astype(np.int64)
        t1 = time.perf_counter()
        oc.decode_attention_rows(q_rot, rows)
        t_attn = time.perf_counter() - t1
        if t_attn >= budget_s / 2 or rows.size == total:
            break
        n *= 4
    real_tokens = int(w.q_lens.sum()) if w.q_lens is not None else s.num_seqs * s.q_tokens
    # time of a whole step at this rate: RoPE/append as measured, attention
    # scaled from the sample to every row
    t_step = t_rope + t_attn * total / rows.size
    return {"tokens_per_s": round(real_tokens / t_step, 2), "cores": oracle.threads(),
            "sample": f"RoPE+append of all {real_tokens} new tokens ({t_rope:.2f} s), attention of "
                      f"{rows.size} of {total} query rows ({t_attn:.2f} s), scaled to the whole step"}


def measure(name, steps, warmup, dev, kernel=0, num_splits=0, reps=REPS, graph=True, contract=False,
            oracle_budget=3.0):
    """Time one workload.  With `contract`, the step is first timed over
    exactly `steps` calls after `warmup` (the headline's figures)."""
    w = workloads.make_workload(workloads.CONFIGS[name])
    n_layers = layers_for(w)
    L = Layers(w, n_layers, dev, kernel, num_splits)
    s = w.spec
    prewarm(L)
    res = {"workload": workload_text(w), "data": describe_data(s), "layers_rotated": n_layers,
           "plan": {"splits": L.plan[0], "keys_per_split": L.plan[1],
                    "kernel": ["auto", "valu", "mfma"][L.plan[2]]}}
    if contract:
        res["contract_step_ms"] = timed(L.step, steps, warmup)
    step_ms, step_spread = reps_timed(L.step, reps)
    two_ms, _ = reps_timed(L.two_calls, reps)
    attn_ms, _ = reps_timed(L.attention, reps)
    graph_ms = graph_timed(L.step, [L.out]) if graph else None
    nb = w.algorithmic_bytes()
    tokens = int(w.q_lens.sum()) if w.q_lens is not None else s.num_seqs * s.q_tokens
    res.update({
        "step_ms": step_ms, "step_ms_spread": list(step_spread), "graph_step_ms": graph_ms,
        "two_call_step_ms": two_ms, "attn_ms": attn_ms,
        "tokens_per_s": tokens / (step_ms * 1e-3),
        "attn_tokens_per_s": tokens / (attn_ms * 1e-3),
        "attn_bytes": nb["attention"], "step_bytes": nb["step"],
        "attn_GBs": nb["attention"] / (attn_ms * 1e-3) / 1e9,
        "step_GBs": nb["step"] / (step_ms * 1e-3) / 1e9,
    })
    res["attn_frac_of_peak"] = res["attn_GBs"] / PEAK_HBM_GBS
    res["step_frac_of_peak"] = res["step_GBs"] / PEAK_HBM_GBS
    if graph_ms is not None:
        res["graph_step_GBs"] = nb["step"] / (graph_ms * 1e-3) / 1e9
        res["graph_step_frac_of_peak"] = res["graph_step_GBs"] / PEAK_HBM_GBS
    if w.q_lens is not None:
        # a prefill chunk leans on the matrix cores: algorithmic flops of the
        # attention call against the dense bf16 peak
        res["attn_TFLOPs"] = w.algorithmic_flops() / (attn_ms * 1e-3) / 1e12
        res["attn_frac_of_bf16_peak"] = res["attn_TFLOPs"] / PEAK_BF16_TFLOPS
    del L
    torch.cuda.empty_cache()
    if oracle_budget:
        res["oracle"] = oracle_rate(w, oracle_budget)
    return w, res


def measure_cp_shard(steps, warmup, dev, parts=8):
    """One GPU's share of the long-context layer under context parallelism
    over `parts` GPUs: a shard holding 131072/parts keys of each sequence
    exports (out, lse) for every query row, then the `parts` partials are
    merged.  The shards are the first parts-1 key ranges of the cache (each a
    distinct 268 MB region, rotated like layers); the new token lies past
    all of them, so every held key is visible."""
    w = workloads.make_workload(workloads.CONFIGS["long_ctx"])
    s = w.spec
    ctx = int(w.seq_lens.min()) - s.q_tokens
    n = ctx // parts
    bs = s.block_size
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)  # noqa: E731
    kd, vd = to_dev_pool(w.k_pool, dev), to_dev_pool(w.v_pool, dev)
    kvs = []
    for k in range(parts - 1):
        table = w.block_table[:, (k * n) // bs:]
        table = np.concatenate([table, np.full((s.num_seqs, (k * n) // bs), -1, np.int32)], 1)
        kvs.append(kb.PagedKV(kd, vd, t(table), t(np.full(s.num_seqs, n)), s.n_q_heads, s.q_tokens, n,
                              key_pos0=t(np.full(s.num_seqs, k * n)),
                              q_pos=t(w.seq_lens.astype(np.int64) - s.q_tokens)))
    q = torch.from_numpy(w.q).to(dev)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    ws = kb.workspace(kvs[0])
    ws = ws.clone() if ws is not None else None
    plan = kb.decode_attention_plan(kvs[0])
    shard_ms = timed(lambda i: kb.decode_attention_lse(kvs[i % len(kvs)], q, out, lse, 0.0, ws), steps, warmup)
    outs = torch.randn((parts,) + tuple(q.shape), dtype=torch.float32, device=dev)
    lses = torch.randn((parts,) + tuple(q.shape[:3]), dtype=torch.float32, device=dev)
    mo, ml = torch.empty_like(q), torch.empty_like(lse)
    merge_ms = timed(lambda i: kb.merge_partials(outs, lses, mo, ml), steps, warmup)
    merge_graph_us = graph_timed_us(lambda: kb.merge_partials(outs, lses, mo, ml), (mo, ml))
    rows = s.num_seqs * s.q_tokens * s.n_q_heads
    shard_bytes = s.num_seqs * n * s.n_kv_heads * s.head_dim * 2 * 2 + rows * s.head_dim * 4 * 2 + rows * 4 \
        + s.num_seqs * (n // bs) * 4
    del kvs, kd, vd
    torch.cuda.empty_cache()
    return {"workload": f"long_ctx shard of {parts}: B={s.num_seqs} Hq={s.n_q_heads} Hkv={s.n_kv_heads} "
                        f"D={s.head_dim}, {n} keys per sequence, exports (out, lse)",
            "plan": {"splits": plan[0], "keys_per_split": plan[1], "kernel": ["auto", "valu", "mfma"][plan[2]]},
            "shard_ms": round(shard_ms, 4), "shard_GBs": round(shard_bytes / (shard_ms * 1e-3) / 1e9, 1),
            "shard_frac_of_peak": round(shard_bytes / (shard_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "merge_ms": round(merge_ms, 4),
            "merge_graph_us": None if merge_graph_us is None else round(merge_graph_us, 2),
            "exchange_bytes_per_gpu": rows * (s.head_dim + 1) * 4}


def cpu_baseline(w, budget_s=12.0):
    """The fp64 oracle (as it stands) on the host cores: RoPE + append +
    attention of the same workload, repeated until about `budget_s` seconds."""
    import oracle
    s = w.spec
    dt = oracle.ORACLE_BF16 if s.kv_dtype == "bf16" else oracle.ORACLE_F32
    reps, t0 = 0, time.perf_counter()
    while True:
        oc = oracle.OracleCache(num_seqs=s.num_seqs, q_tokens=s.q_tokens, n_q_heads=s.n_q_heads,
                                n_kv_heads=s.n_kv_heads, head_dim=s.head_dim, block_size=s.block_size,
                                k_pool=w.k_pool, v_pool=w.v_pool, block_table=w.block_table,
                                seq_lens=w.seq_lens, cache_dtype=dt, q_lens=w.q_lens)
        t1 = time.perf_counter()
        oc.decode_attention(oc.rope_append_kv(w.q, w.k, w.v, s.rope_base, s.layout))
        reps += 1
        t_work = time.perf_counter() - t1
        if time.perf_counter() - t0 >= budget_s or reps >= 50:
            break
    elapsed = time.perf_counter() - t0
    tokens = (int(w.q_lens.sum()) if w.q_lens is not None else s.num_seqs * s.q_tokens) * reps
    return {"value": tokens / elapsed, "unit": "tokens/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": f"{reps} full {s.name} step(s) (RoPE+append+attention, all {s.num_seqs * s.q_tokens} "
                      f"query tokens), fp64, OpenMP over query rows; last rep {t_work:.2f} s"}


CALIB_BYTES = 512 << 20


def copy_calibration(dev, nbytes=CALIB_BYTES):
    """A plain streaming kernel of known traffic (reads nbytes, writes nbytes:
    torch.neg on fp32), outside every timed region, whose FETCH_SIZE /
    WRITE_SIZE scale the counters of a profiled run."""
    a = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.neg(a, out=b)
    torch.cuda.synchronize()


def stored_traffic(workload):
    """HBM bytes per decode-step call from the committed counter runs, or None
    if the kernels changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    entry = t.get(workload)
    if not entry or entry.get("kernel_sources_sha") != kernel_sources_sha():
        return None
    return entry.get("step_bytes_per_launch")


# ---------------------------------------------------------------- profile summary
def _csv_rows(d, suffix):
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)
    rows = []
    for f in files:
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    return rows


def _median(v):
    v = sorted(v)
    return v[len(v) // 2] if v else float("nan")


def summarize(prof_dir, workload, commands, record=True):
    """Turn rocprofv3 CSV output (kt/ kernel trace, fetch/ FETCH_SIZE,
    write/ WRITE_SIZE, util/ utilisation counters, tcc/ L2 hits and misses,
    mix/ request sizes, issue/ and insts/ issue, stall and instruction counts,
    mops/ matrix-core operations)
    into a markdown summary on stdout and, with `record` (runs of the
    automatic plan), record the calibrated traffic per call."""
    import collections
    w = workloads.make_workload(workloads.CONFIGS[workload])
    alg = w.algorithmic_bytes()
    out = [f"# {workload}: decode-step kernels on MI355X (rocprofv3)", "",
           workload_text(w), "", describe_data(w.spec), ""]
    out += ["Commands (repository root):", "", "```"] + commands + ["```", ""]

    trace = _csv_rows(os.path.join(prof_dir, "kt"), "kernel_trace.csv")
    dur = collections.defaultdict(list)
    for r in trace:
        dur[r["Kernel_Name"]].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0)
    ours = {k: v for k, v in dur.items() if k.startswith(("attn_", "rope_append", "decode_step"))}
    out += ["## Kernel durations (--kernel-trace --stats)", "",
            "| kernel | calls | mean us | median us | min us |", "|---|---|---|---|---|"]
    for k, v in sorted(ours.items()):
        out.append(f"| {k} | {len(v)} | {sum(v) / len(v):.2f} | {_median(v):.2f} | {min(v):.2f} |")
    # the step call: the fused kernel (or RoPE/append + attention) and the
    # combine; the attention call alone: the attention kernel and the combine
    combine = [k for k in ours if k.startswith("attn_combine")]
    attn_names = [k for k in ours if k.startswith("attn_")]
    fused = [k for k in ours if k.startswith("decode_step")]
    step_names = (fused + combine) if fused else list(ours)
    step_us = sum(_median(ours[k]) for k in step_names)
    attn_us = sum(_median(ours[k]) for k in attn_names)
    out += ["", f"Decode-step call (sum of medians of {', '.join(sorted(step_names))}): "
                f"{step_us:.2f} us -> {alg['step'] / step_us / 1e3:.0f} GB/s algorithmic "
                f"({alg['step'] / step_us / 1e3 / PEAK_HBM_GBS:.1%} of 8 TB/s).",
            f"Decode-attention call alone (sum of medians of {', '.join(sorted(attn_names))}): "
            f"{attn_us:.2f} us -> {alg['attention'] / attn_us / 1e3:.0f} GB/s algorithmic "
            f"({alg['attention'] / attn_us / 1e3 / PEAK_HBM_GBS:.1%} of 8 TB/s).", ""]

    def per_kernel(sub, counter):
        vals = collections.defaultdict(list)
        for r in _csv_rows(os.path.join(prof_dir, sub), "counter_collection.csv"):
            if r["Counter_Name"] == counter:
                vals[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        return vals

    fetch, write = per_kernel("fetch", "FETCH_SIZE"), per_kernel("write", "WRITE_SIZE")
    calib_kib = CALIB_BYTES / 1024.0
    f_cal = [x for x in fetch.get("vectorized_elementwise_kernel", []) if x > 0.25 * calib_kib]
    w_cal = [x for x in write.get("vectorized_elementwise_kernel", []) if x > 0.25 * calib_kib]
    f_fac = _median(f_cal) / calib_kib if f_cal else float("nan")
    w_fac = _median(w_cal) / calib_kib if w_cal else float("nan")
    out += ["## HBM traffic (--pmc FETCH_SIZE, then --pmc WRITE_SIZE; KiB per dispatch)", "",
            f"Calibration: a plain fp32 negate of {CALIB_BYTES >> 20} MiB (reads and writes "
            f"{CALIB_BYTES >> 20} MiB) reads FETCH_SIZE = {_median(f_cal):.0f} KiB "
            f"(factor {f_fac:.4f}) and WRITE_SIZE = {_median(w_cal):.0f} KiB (factor {w_fac:.4f}); "
            "counter values below are divided by these factors.", "",
            "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | read MB (scaled) | written MB (scaled) |",
            "|---|---|---|---|---|"]
    per_k = {}
    for k in sorted(set(fetch) & set(ours)):
        fk, wk = _median(fetch[k]), _median(write.get(k, [0.0]))
        rd, wr = fk / f_fac * 1024, wk / w_fac * 1024
        per_k[k] = rd + wr
        out.append(f"| {k} | {fk:.0f} | {wk:.0f} | {rd / 1e6:.2f} | {wr / 1e6:.2f} |")
    step_traffic = sum(per_k.get(k, 0.0) for k in step_names)
    traffic = sum(per_k.get(k, 0.0) for k in attn_names)
    out += ["", f"Decode-step call: {step_traffic / 1e6:.2f} MB of HBM traffic vs "
                f"{alg['step'] / 1e6:.2f} MB algorithmic ({step_traffic / alg['step']:.3f}x).",
            f"Decode-attention call alone: {traffic / 1e6:.2f} MB of HBM traffic vs "
            f"{alg['attention'] / 1e6:.2f} MB algorithmic ({traffic / alg['attention']:.3f}x).", ""]

    tcc = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in _csv_rows(os.path.join(prof_dir, "tcc"), "counter_collection.csv"):
        tcc[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    if tcc:
        out += ["## L2 reuse (--pmc TCC_HIT_sum TCC_MISS_sum; requests per dispatch)", "",
                "| kernel | TCC_HIT | TCC_MISS | hit rate |", "|---|---|---|---|"]
        for k in sorted(tcc):
            if not k.startswith(("attn_", "decode_step", "rope_append")):
                continue
            h = _median(tcc[k].get("TCC_HIT_sum", [0.0]))
            m = _median(tcc[k].get("TCC_MISS_sum", [0.0]))
            out.append(f"| {k} | {h:.0f} | {m:.0f} | {h / max(h + m, 1.0):.1%} |")
        out.append("")

    mix = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in _csv_rows(os.path.join(prof_dir, "mix"), "counter_collection.csv"):
        mix[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    if mix:
        out += ["## L2-to-memory read requests (--pmc TCC_EA0_RDREQ_sum TCC_EA0_RDREQ_32B_sum "
                "TCC_BUBBLE_sum TCC_EA0_RDREQ_DRAM_sum; per dispatch)", "",
                "FETCH_SIZE counts TCC_BUBBLE requests as 128 bytes, TCC_EA0_RDREQ_32B as 32 and the rest "
                "as 64; the calibration copy shows how a plain stream's requests fall.", "",
                "| kernel | RDREQ | RDREQ_32B | BUBBLE | RDREQ_DRAM | MB if all RDREQ are 128 B |",
                "|---|---|---|---|---|---|"]
        for k in sorted(mix):
            if not k.startswith(("attn_", "decode_step", "rope_append", "vectorized_elementwise")):
                continue
            m = {c: _median(v) for c, v in mix[k].items()}
            rq = m.get("TCC_EA0_RDREQ_sum", 0.0)
            out.append(f"| {k} | {rq:.0f} | {m.get('TCC_EA0_RDREQ_32B_sum', 0):.0f} | "
                       f"{m.get('TCC_BUBBLE_sum', 0):.0f} | {m.get('TCC_EA0_RDREQ_DRAM_sum', 0):.0f} | "
                       f"{rq * 128 / 1e6:.2f} |")
        out.append("")

    util = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in _csv_rows(os.path.join(prof_dir, "util"), "counter_collection.csv"):
        util[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    if util:
        out += ["## Utilisation (one --pmc run)", "",
                "GRBM_GUI_ACTIVE is summed over the 8 XCDs by the collector; per-XCD cycles = sum / 8. "
                "VALU busy = SQ_ACTIVE_INST_VALU / (256 CUs x cycles); MFMA busy = "
                "SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x cycles).", "",
                "| kernel | cycles | VALU busy | MFMA busy | VALU instr / wave | LDS bank conflicts |",
                "|---|---|---|---|---|---|"]
        for k in sorted(util):
            if not k.startswith(("attn_", "decode_step")):
                continue
            m = {c: _median(v) for c, v in util[k].items()}
            cyc = m.get("GRBM_GUI_ACTIVE", float("nan")) / 8
            out.append(f"| {k} | {cyc:.0f} | {m.get('SQ_ACTIVE_INST_VALU', 0) / 256 / cyc:.1%} | "
                       f"{m.get('SQ_VALU_MFMA_BUSY_CYCLES', 0) / 1024 / cyc:.2%} | "
                       f"{m.get('SQ_INSTS_VALU', 0) / max(m.get('SQ_WAVES', 1), 1):.0f} | "
                       f"{m.get('SQ_LDS_BANK_CONFLICT', 0):.0f} |")
        out.append("")

    # matrix-core work: SQ_INSTS_VALU_MFMA_MOPS_* count in units of 512 flops
    # (32 for one 16x16x32 instruction)
    mops = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in _csv_rows(os.path.join(prof_dir, "mops"), "counter_collection.csv"):
        mops[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    if mops:
        aflops = w.algorithmic_flops()
        out += ["## Matrix-core work (--pmc SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_F16 "
                "SQ_INSTS_VALU_MFMA_MOPS_F32 GRBM_GUI_ACTIVE)", "",
                "The MOPS counters count matrix-core work in units of 512 flops (32 per 16x16x32 "
                "instruction). The rate divides by the kernel's median duration above; the last column "
                f"compares with the attention's algorithmic {aflops / 1e9:.2f} GFLOP (q.K and the "
                "weighted V sum of every real query row over the keys it sees).", "",
                "| kernel | bf16 GFLOP | fp16 GFLOP | fp32 GFLOP | TFLOP/s at the median duration | "
                "matrix-core / algorithmic flops |", "|---|---|---|---|---|---|"]
        for k in sorted(mops):
            if not k.startswith(("attn_", "decode_step")) or k not in ours:
                continue
            m = {c: _median(v) * 512 for c, v in mops[k].items()}
            tot = sum(m.get(f"SQ_INSTS_VALU_MFMA_MOPS_{t}", 0.0) for t in ("BF16", "F16", "F32"))
            if tot == 0:
                continue
            out.append(f"| {k} | {m.get('SQ_INSTS_VALU_MFMA_MOPS_BF16', 0) / 1e9:.2f} | "
                       f"{m.get('SQ_INSTS_VALU_MFMA_MOPS_F16', 0) / 1e9:.2f} | "
                       f"{m.get('SQ_INSTS_VALU_MFMA_MOPS_F32', 0) / 1e9:.2f} | "
                       f"{tot / (_median(ours[k]) * 1e-6) / 1e12:.1f} | {tot / aflops:.2f}x |")
        out.append("")

    # where the waves' time goes: issuing, waiting on a counter (s_waitcnt,
    # barriers), or holding an instruction that cannot issue yet; and the
    # instruction mix per wave
    issue = collections.defaultdict(lambda: collections.defaultdict(list))
    for sub in ("issue", "insts"):
        for r in _csv_rows(os.path.join(prof_dir, sub), "counter_collection.csv"):
            issue[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    if issue:
        out += ["## Issue and stalls (--pmc SQ_WAVE_CYCLES SQ_ACTIVE_INST_ANY SQ_WAIT_ANY SQ_WAIT_INST_ANY "
                "SQ_ACTIVE_INST_LDS SQ_WAIT_INST_LDS SQ_VALU_MFMA_COEXEC_CYCLES SQ_INSTS_MFMA, then "
                "--pmc SQ_INSTS_VALU SQ_INSTS_SALU SQ_INSTS_LDS SQ_INSTS_VALU_TRANS_F32 SQ_WAVES "
                "SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE)", "",
                "Shares of the waves' lifetime (SQ_WAVE_CYCLES): issuing instructions (SQ_ACTIVE_INST_ANY), "
                "waiting (SQ_WAIT_ANY: on s_waitcnt counters, barriers, dependencies) and waiting for an "
                "instruction to issue (SQ_WAIT_INST_ANY). Co-execution: cycles with the matrix cores and "
                "the vector ALU busy at once (SQ_VALU_MFMA_COEXEC_CYCLES), as a share of the matrix cores' "
                "busy cycles. Instructions per wave count every wave of the grid, those of empty units "
                "included (SQ_INSTS_VALU includes the MFMAs).", "",
                "| kernel | issuing | waiting | waiting for issue | co-execution | MFMA / wave | "
                "VALU / wave | SALU / wave | LDS / wave | exp / wave |",
                "|---|---|---|---|---|---|---|---|---|---|"]
        for k in sorted(issue):
            if not k.startswith(("attn_", "decode_step")):
                continue
            m = {c: _median(v) for c, v in issue[k].items()}
            wc = max(m.get("SQ_WAVE_CYCLES", 0.0), 1.0)
            nw = max(m.get("SQ_WAVES", 1.0), 1.0)
            busy = max(m.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0), 1.0)
            out.append(f"| {k} | {m.get('SQ_ACTIVE_INST_ANY', 0) / wc:.1%} | {m.get('SQ_WAIT_ANY', 0) / wc:.1%} | "
                       f"{m.get('SQ_WAIT_INST_ANY', 0) / wc:.1%} | "
                       f"{m.get('SQ_VALU_MFMA_COEXEC_CYCLES', 0) / busy:.1%} | "
                       f"{m.get('SQ_INSTS_MFMA', 0) / nw:.0f} | {m.get('SQ_INSTS_VALU', 0) / nw:.0f} | "
                       f"{m.get('SQ_INSTS_SALU', 0) / nw:.0f} | {m.get('SQ_INSTS_LDS', 0) / nw:.0f} | "
                       f"{m.get('SQ_INSTS_VALU_TRANS_F32', 0) / nw:.0f} |")
        out.append("")
    print("\n".join(out))

    if not record:
        return
    entry = {"kernel_sources_sha": kernel_sources_sha(), "step_bytes_per_launch": round(step_traffic),
             "attn_bytes_per_launch": round(traffic), "fetch_factor": f_fac, "write_factor": w_fac,
             "step_us_trace": step_us, "attn_us_trace": attn_us}
    try:
        with open(TRAFFIC_FILE) as f:
            allt = json.load(f)
    except (OSError, ValueError):
        allt = {}
    allt[workload] = entry
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(allt, f, indent=1, sort_keys=True)


def rounded(d):
    return {k: (round(v, 4) if isinstance(v, float) else v) for k, v in d.items()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=HEADLINE, choices=workloads.CONFIG_ORDER)
    ap.add_argument("--kernel", type=int, default=0, help="0 auto, 1 VALU, 2 MFMA")
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--reps", type=int, default=REPS, help="repetitions of 20 calls per median")
    ap.add_argument("--no-extra", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu", action="store_true", help="skip every CPU oracle timing")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replays")
    ap.add_argument("--no-probe", action="store_true", help="skip the streaming-read probe")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--summarize", metavar="PROFILE_DIR",
                    help="write the profile summary of rocprofv3 output in PROFILE_DIR and exit")
    ap.add_argument("--command", action="append", default=[],
                    help="(with --summarize) a profiling command to quote in the summary")
    args = ap.parse_args()
    if args.summarize:
        summarize(args.summarize, args.workload, args.command, record=args.kernel == 0)
        return
    if args.gpus != 1:
        print(f"bench.py: measures one GPU; --gpus {args.gpus} is not supported "
              "(the path shards by sequence, kv head or key range with no exchange inside the "
              "attention step; see the design notes)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py: no GPU", file=sys.stderr)
        sys.exit(1)
    dev = "cuda:0"
    kb.lib()
    if args.calibrate_copy:
        copy_calibration(dev)
    probe = None if args.no_probe else stream_probe(dev)
    print(f"[bench] probe {probe and probe['GBs']} GB/s", file=sys.stderr, flush=True)

    w, head = measure(args.workload, args.steps, args.warmup, dev, args.kernel, args.splits, args.reps,
                      graph=not args.no_graph, contract=True, oracle_budget=0)
    print(f"[bench] {args.workload}: {head['contract_step_ms']:.4f} ms per step", file=sys.stderr, flush=True)
    extra = {}
    if not args.no_extra:
        for name in workloads.CONFIG_ORDER:
            if name == args.workload:
                continue
            _, r = measure(name, 0, 0, dev, args.kernel, args.splits, args.reps, graph=not args.no_graph,
                           oracle_budget=0 if args.no_cpu else 3.0)
            extra[name] = rounded(r)
            print(f"[bench] {name}: {r['step_ms']:.4f} ms per step", file=sys.stderr, flush=True)
        extra["long_ctx_cp8_shard"] = measure_cp_shard(max(10, args.steps // 4), max(2, args.warmup // 4), dev)
    cpu = None if args.no_cpu else cpu_baseline(w)
    if probe:
        for r in [head] + [r for r in extra.values() if "step_GBs" in r]:
            r["step_frac_of_probe"] = round(r["step_GBs"] / probe["GBs"], 4)
            r["attn_frac_of_probe"] = round(r["attn_GBs"] / probe["GBs"], 4)

    s = w.spec
    tokens = int(w.q_lens.sum()) if w.q_lens is not None else s.num_seqs * s.q_tokens
    step_ms = head["contract_step_ms"]
    achieved = head["step_bytes"] / (step_ms * 1e-3) / 1e9
    traffic = stored_traffic(args.workload)
    line = {
        "metric": "decode-attention tokens/s and achieved HBM GB/s (% of peak), 1xMI355X",
        "value": tokens / (step_ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if s.kv_dtype == "bf16" else "fp32",
        "accumulate_dtype": "fp32",
        "data": head["data"],
        "config": {"workload": head["workload"], "batch": s.num_seqs, "q_tokens_per_seq": s.q_tokens,
                   "context": int(w.max_seq_len - s.q_tokens), "layers_rotated": head["layers_rotated"],
                   "plan": head["plan"]},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                     "kernel": "kvd_decode_step (fused RoPE + append + split-K attention kernel, "
                               "then the split combine)",
                     "algorithmic_bytes_per_launch": head["step_bytes"], "avg_launch_ms": step_ms,
                     "frac_of_probe": round(achieved / probe["GBs"], 4) if probe else None},
        "median_of_reps": {"step_ms": head["step_ms"], "step_ms_spread": head["step_ms_spread"],
                           "step_frac_of_peak": head["step_frac_of_peak"],
                           "step_frac_of_probe": head.get("step_frac_of_probe"),
                           "graph_step_ms": head["graph_step_ms"],
                           "graph_step_frac_of_peak": head.get("graph_step_frac_of_peak"),
                           "reps": args.reps, "calls_per_rep": CALLS},
        "two_call_step_ms": head["two_call_step_ms"],
        "attention_call": {"ms": head["attn_ms"], "GBs": head["attn_GBs"],
                           "frac": head["attn_frac_of_peak"], "algorithmic_bytes": head["attn_bytes"],
                           "tokens_per_s": head["attn_tokens_per_s"]},
        "stream_probe": probe and {k: v for k, v in probe.items() if k != "sweep"},
        "cpu_baseline": cpu,
        "other_workloads": extra,
    }
    print(json.dumps(line), flush=True)
    if probe and os.environ.get("KVD_BENCH_PROBE_SWEEP"):
        with open(os.environ["KVD_BENCH_PROBE_SWEEP"], "w") as f:
            json.dump(probe, f, indent=1)


if __name__ == "__main__":
    main()
