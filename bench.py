"""Benchmark of the decode-attention step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-extra]

A step is one pass of the whole hot path over one batch through the C ABI:
kvd_decode_step, which does RoPE at each token's position, the paged append
and split-K decode attention (one fused kernel on matrix-core plans, plus the
split combine).  The same work as two calls (kvd_rope_append_kv, then
kvd_decode_attention) and the attention call alone are timed beside it.
The headline workload is the Llama-3-8B-shaped layer (batch 16, 32 q / 8 kv
heads, head_dim 128, context 4096, bf16 cache).  Inputs are seeded synthetic
tensors already resident in HBM.  Successive steps rotate over several
layers' caches (distinct buffers) so that no step finds its cache in the
256 MB Infinity Cache left behind by the previous one.

Rank 0 prints ONE JSON line.  `value` is tokens/s of the whole step (B*T new
tokens per step).  `roofline` is for the step call (the fused kernel and the
combine): algorithmic bytes per call / its average duration measured with HIP
events on the launch stream.  `cpu_baseline` times the fp64 oracle on the
host cores on a bounded sample of the same workload.
"""
import argparse
import hashlib
import json
import os
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
HEADLINE = "llama3_8b"
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
        # an intermediate.  A matrix-core decode plan runs as one kernel and
        # needs no buffer for them; the other plans (prefill tiles, the
        # vector-ALU kernel) run the two kernels in a row and get one, as a
        # caller would pass it, rather than reusing `out`.
        rows = s.n_q_heads // s.n_kv_heads * s.q_tokens
        fused = self.plan[2] == kb.KVD_KERNEL_MFMA and rows <= 16
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
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        fn(i)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps   # ms per call


def graph_timed_us(fn, results, calls=32, replays=20):
    """Device time of one call of `fn` without the host's launch cost: `calls`
    launches captured in one HIP graph, replayed `replays` times.  The graph's
    results must equal those of an eager call (None is returned otherwise)."""
    fn()
    torch.cuda.synchronize()
    eager = [r.clone() for r in results]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            fn()
    for r in results:
        r.fill_(float("nan"))
    g.replay()
    torch.cuda.synchronize()
    if not all(torch.equal(r, e) for r, e in zip(results, eager)):
        return None
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(replays):
        g.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) * 1e3 / (replays * calls)


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


def measure(name, steps, warmup, dev, kernel=0, num_splits=0):
    w = workloads.make_workload(workloads.CONFIGS[name])
    n_layers = layers_for(w)
    L = Layers(w, n_layers, dev, kernel, num_splits)
    s = w.spec
    prewarm(L)
    step_ms = timed(L.step, steps, warmup)
    two_ms = timed(L.two_calls, steps, warmup)
    attn_ms = timed(L.attention, steps, warmup)
    nb = w.algorithmic_bytes()
    tokens = int(w.q_lens.sum()) if w.q_lens is not None else s.num_seqs * s.q_tokens
    res = {
        "workload": name, "layers_rotated": n_layers, "plan": {"splits": L.plan[0], "keys_per_split": L.plan[1],
                                                               "kernel": ["auto", "valu", "mfma"][L.plan[2]]},
        "step_ms": step_ms, "two_call_step_ms": two_ms, "attn_ms": attn_ms,
        "tokens_per_s": tokens / (step_ms * 1e-3),
        "attn_tokens_per_s": tokens / (attn_ms * 1e-3),
        "attn_bytes": nb["attention"], "step_bytes": nb["step"],
        "attn_GBs": nb["attention"] / (attn_ms * 1e-3) / 1e9,
        "step_GBs": nb["step"] / (step_ms * 1e-3) / 1e9,
    }
    res["attn_frac_of_peak"] = res["attn_GBs"] / PEAK_HBM_GBS
    res["step_frac_of_peak"] = res["step_GBs"] / PEAK_HBM_GBS
    if w.q_lens is not None:
        # a prefill chunk leans on the matrix cores: algorithmic flops of the
        # attention call against the dense bf16 peak
        res["attn_TFLOPs"] = w.algorithmic_flops() / (attn_ms * 1e-3) / 1e12
        res["attn_frac_of_bf16_peak"] = res["attn_TFLOPs"] / PEAK_BF16_TFLOPS
    del L
    torch.cuda.empty_cache()
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
                                seq_lens=w.seq_lens, cache_dtype=dt)
        t1 = time.perf_counter()
        oc.decode_attention(oc.rope_append_kv(w.q, w.k, w.v, s.rope_base, s.layout))
        reps += 1
        t_work = time.perf_counter() - t1
        if time.perf_counter() - t0 >= budget_s or reps >= 50:
            break
    elapsed = time.perf_counter() - t0
    tokens = s.num_seqs * s.q_tokens * reps
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


def summarize(prof_dir, workload, commands):
    """Turn rocprofv3 CSV output (kt/ kernel trace, fetch/ FETCH_SIZE,
    write/ WRITE_SIZE, util/ utilisation counters) into a markdown summary on
    stdout and record the calibrated traffic per decode-attention call."""
    import collections
    w = workloads.make_workload(workloads.CONFIGS[workload])
    alg = w.algorithmic_bytes()
    out = [f"# {workload}: decode-step kernels on MI355X (rocprofv3)", ""]
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
    print("\n".join(out))

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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=HEADLINE, choices=workloads.CONFIG_ORDER)
    ap.add_argument("--kernel", type=int, default=0, help="0 auto, 1 VALU, 2 MFMA")
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--no-extra", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--summarize", metavar="PROFILE_DIR",
                    help="write the profile summary of rocprofv3 output in PROFILE_DIR and exit")
    ap.add_argument("--command", action="append", default=[],
                    help="(with --summarize) a profiling command to quote in the summary")
    args = ap.parse_args()
    if args.summarize:
        summarize(args.summarize, args.workload, args.command)
        return
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU; --gpus {args.gpus} is not supported "
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

    w, head = measure(args.workload, args.steps, args.warmup, dev, args.kernel, args.splits)
    extra = {}
    if not args.no_extra:
        for name in workloads.CONFIG_ORDER:
            if name == args.workload:
                continue
            steps = max(10, args.steps // 4)
            _, r = measure(name, steps, max(2, args.warmup // 4), dev, args.kernel, args.splits)
            extra[name] = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()}
        extra["long_ctx_cp8_shard"] = measure_cp_shard(max(10, args.steps // 4), max(2, args.warmup // 4), dev)
    cpu = None if args.no_cpu else cpu_baseline(w)

    s = w.spec
    traffic = stored_traffic(args.workload)
    line = {
        "metric": "decode-attention tokens/s and achieved HBM GB/s (% of peak), 1xMI355X",
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["step_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 cache, fp32 accumulate" if s.kv_dtype == "bf16" else "fp32",
        "data": "synthetic (seeded; N(0,1)/sqrt(128) values, in-order paged table)",
        "config": {"workload": f"{s.name}: decode step of one attention layer, B={s.num_seqs} T={s.q_tokens} "
                               f"Hq={s.n_q_heads} Hkv={s.n_kv_heads} D={s.head_dim} context={w.max_seq_len - s.q_tokens} "
                               f"bs={s.block_size} {s.kv_dtype}",
                   "batch": s.num_seqs, "q_tokens_per_seq": s.q_tokens, "context": int(w.max_seq_len - s.q_tokens),
                   "layers_rotated": head["layers_rotated"], "plan": head["plan"]},
        "roofline": {"bound": "hbm", "achieved": head["step_GBs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": head["step_GBs"] / PEAK_HBM_GBS, "traffic": traffic,
                     "kernel": "kvd_decode_step (fused RoPE + append + split-K attention kernel, "
                               "then the split combine)",
                     "algorithmic_bytes_per_launch": head["step_bytes"], "avg_launch_ms": head["step_ms"]},
        "two_call_step_ms": head["two_call_step_ms"],
        "attention_call": {"ms": head["attn_ms"], "GBs": head["attn_GBs"],
                           "frac": head["attn_frac_of_peak"], "algorithmic_bytes": head["attn_bytes"],
                           "tokens_per_s": head["attn_tokens_per_s"]},
        "cpu_baseline": cpu,
        "other_workloads": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
