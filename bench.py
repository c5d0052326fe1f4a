"""Benchmark of the decode-attention step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-extra]

A step is one pass of the whole hot path over one batch: kvd_rope_append_kv
(RoPE at each token's position + paged append) followed by
kvd_decode_attention (split-K attention + combine), both through the C ABI.
The headline workload is the Llama-3-8B-shaped layer (batch 16, 32 q / 8 kv
heads, head_dim 128, context 4096, bf16 cache).  Inputs are seeded synthetic
tensors already resident in HBM.  Successive steps rotate over several
layers' caches (distinct buffers) so that no step finds its cache in the
256 MB Infinity Cache left behind by the previous one.

Rank 0 prints ONE JSON line.  `value` is tokens/s of the whole step (B*T new
tokens per step).  `roofline` is for the decode-attention call (the dominant
kernel): algorithmic bytes per call / its average duration measured with HIP
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
HEADLINE = "llama3_8b"
KERNEL_SOURCES = ["kvd.cpp", "attn_valu.hip", "attn_mfma.hip", "attn_combine.hip", "rope_append.hip",
                  "kvd_internal.h", "bf16_round.h"]
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
        kd, vd = to_dev_pool(w.k_pool, dev), to_dev_pool(w.v_pool, dev)
        self.kv = []
        for i in range(n):
            k = kd if i == 0 else kd.clone()
            v = vd if i == 0 else vd.clone()
            self.kv.append(kb.PagedKV(k, v, table, seq_lens, s.n_q_heads, s.q_tokens, w.max_seq_len))
        self.q = torch.from_numpy(w.q).to(dev)
        self.k = torch.from_numpy(w.k).to(dev)
        self.v = torch.from_numpy(w.v).to(dev)
        self.q_rot = torch.empty_like(self.q)
        self.out = torch.empty_like(self.q)
        self.ws = kb.workspace(self.kv[0], num_splits, kernel)
        if self.ws is not None:
            self.ws = self.ws.clone()
        self.plan = kb.decode_attention_plan(self.kv[0], num_splits, kernel)

    def step(self, i):
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


def layers_for(w):
    # rotate over enough distinct caches to cover >= 1 GiB (4x the MALL)
    kv_bytes = w.k_pool.nbytes + w.v_pool.nbytes
    return int(min(8, max(1, -(-(1 << 30) // kv_bytes))))


def measure(name, steps, warmup, dev, kernel=0, num_splits=0):
    w = workloads.make_workload(workloads.CONFIGS[name])
    n_layers = layers_for(w)
    L = Layers(w, n_layers, dev, kernel, num_splits)
    s = w.spec
    step_ms = timed(L.step, steps, warmup)
    attn_ms = timed(L.attention, steps, warmup)
    nb = w.algorithmic_bytes()
    tokens = s.num_seqs * s.q_tokens
    res = {
        "workload": name, "layers_rotated": n_layers, "plan": {"splits": L.plan[0], "keys_per_split": L.plan[1],
                                                               "kernel": ["auto", "valu", "mfma"][L.plan[2]]},
        "step_ms": step_ms, "attn_ms": attn_ms,
        "tokens_per_s": tokens / (step_ms * 1e-3),
        "attn_tokens_per_s": tokens / (attn_ms * 1e-3),
        "attn_bytes": nb["attention"], "step_bytes": nb["step"],
        "attn_GBs": nb["attention"] / (attn_ms * 1e-3) / 1e9,
        "step_GBs": nb["step"] / (step_ms * 1e-3) / 1e9,
    }
    res["attn_frac_of_peak"] = res["attn_GBs"] / PEAK_HBM_GBS
    del L
    torch.cuda.empty_cache()
    return w, res


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


def stored_traffic():
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_sources_sha") != kernel_sources_sha():
        return None   # kernels changed since the counters were taken
    return t.get("attn_bytes_per_launch")


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
    args = ap.parse_args()
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
    cpu = None if args.no_cpu else cpu_baseline(w)

    s = w.spec
    traffic = stored_traffic()
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
        "roofline": {"bound": "hbm", "achieved": head["attn_GBs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": head["attn_GBs"] / PEAK_HBM_GBS, "traffic": traffic,
                     "kernel": "kvd_decode_attention (split-K attention + combine)",
                     "algorithmic_bytes_per_launch": head["attn_bytes"], "avg_launch_ms": head["attn_ms"]},
        "step_GBs": head["step_GBs"],
        "attn_tokens_per_s": head["attn_tokens_per_s"],
        "cpu_baseline": cpu,
        "other_workloads": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
