"""Helpers for the GPU tests: upload a workload, run the HIP path through the
C ABI (via the thin binding), run the oracle on the same inputs, compare."""
import functools
import json
import os
import sys

import numpy as np
import torch

from helpers import oracle_cache
from kv_cached_decode_amd import binding as kb
from kv_cached_decode_amd import workloads

DEV = "cuda:0"


def note(*a):
    """Name the case before a GPU step (flushed, so a crash still shows it)."""
    print("[gpu-case]", *a, file=sys.stderr, flush=True)


def to_dev_pool(pool):
    if pool.dtype == np.uint16:
        return torch.from_numpy(pool.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(pool).to(DEV)


def to_host_pool(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


@functools.lru_cache(maxsize=2)
def cached_workload(spec):
    return workloads.make_workload(spec)


def check_table(table, seq_lens, block_size, num_blocks):
    """Host check before any launch: every block a sequence's keys need is
    allocated (an id in the pool), so no kernel can address outside it."""
    table = np.asarray(table)
    for b, L in enumerate(np.asarray(seq_lens)):
        need = table[b, :-(-int(L) // block_size)]
        assert need.size == -(-int(L) // block_size), f"sequence {b}: table too narrow for {L} keys"
        assert np.all((need >= 0) & (need < num_blocks)), f"sequence {b}: unallocated block for {L} keys"


class GpuCase:
    """A workload resident on the GPU, ready for the step."""

    def __init__(self, w, seq_lens=None, q_tokens=None, window=0, block_table=None, q_lens=None):
        self.w = w
        s = w.spec
        self.k_cache = to_dev_pool(w.k_pool)
        self.v_cache = to_dev_pool(w.v_pool)
        self.table = torch.from_numpy(w.block_table if block_table is None else block_table).to(DEV)
        sl = w.seq_lens if seq_lens is None else seq_lens
        check_table(w.block_table if block_table is None else block_table, sl, s.block_size, w.num_blocks)
        self.seq_lens = torch.from_numpy(np.ascontiguousarray(sl, dtype=np.int32)).to(DEV)
        T = q_tokens or s.q_tokens
        ql = w.q_lens if q_lens is None else q_lens
        self.q_lens = None if ql is None else torch.from_numpy(np.ascontiguousarray(ql, np.int32)).to(DEV)
        self.kv = kb.PagedKV(self.k_cache, self.v_cache, self.table, self.seq_lens, s.n_q_heads, T,
                             max(int(np.max(sl)), T) if len(sl) else T, window, q_lens=self.q_lens)
        self.q = torch.from_numpy(w.q).to(DEV)
        self.k = torch.from_numpy(w.k).to(DEV)
        self.v = torch.from_numpy(w.v).to(DEV)

    def step(self, kernel=kb.KVD_KERNEL_AUTO, num_splits=0, scale=0.0):
        s = self.w.spec
        # zeroed: the rows of padding tokens (ragged chunks) are left as they are
        q_rot = kb.rope_append_kv(self.kv, self.q, self.k, self.v, torch.zeros_like(self.q),
                                  rope_base=s.rope_base, layout=s.layout)
        out = kb.decode_attention(self.kv, q_rot, softmax_scale=scale, num_splits=num_splits,
                                  kernel=kernel)
        torch.cuda.synchronize()
        return q_rot.cpu().numpy(), out.cpu().numpy()

    def attention(self, q_rot, kernel=kb.KVD_KERNEL_AUTO, num_splits=0, scale=0.0):
        out = kb.decode_attention(self.kv, q_rot, softmax_scale=scale, num_splits=num_splits,
                                  kernel=kernel)
        torch.cuda.synchronize()
        return out.cpu().numpy()

    def pools(self):
        return to_host_pool(self.k_cache), to_host_pool(self.v_cache)


def oracle_step(w, rows=None, scale=None, window=0, block_table=None):
    """Oracle RoPE + append + attention on host copies.  Returns (q_rot fp64,
    out fp64 for all rows or the given flat rows, k_pool, v_pool)."""
    s = w.spec
    oc = oracle_cache(w, window=window, block_table=block_table)
    q_rot = oc.rope_append_kv(w.q, w.k, w.v, s.rope_base, s.layout)
    if rows is None:
        out = oc.decode_attention(q_rot, scale=scale)
    else:
        out, _ = oc.decode_attention_rows(q_rot, rows, scale=scale)
    return q_rot, out, oc.k_pool, oc.v_pool


def rel_err(gpu, ref):
    """Normwise relative error max|gpu - ref| / max|ref| (the bf16 criterion)."""
    return float(np.max(np.abs(gpu - ref)) / max(np.max(np.abs(ref)), 1e-30))


def abs_err(gpu, ref):
    return float(np.max(np.abs(gpu - ref)))


def worst_row_err(gpu, ref, head_dim):
    """The largest per-row error: over query rows, max|gpu - ref| of the row
    divided by max|ref| of the row (the absolute error for a row whose
    reference is all zero, such as a padding row)."""
    g = np.asarray(gpu, np.float64).reshape(-1, head_dim)
    r = np.asarray(ref, np.float64).reshape(-1, head_dim)
    if g.size == 0:
        return 0.0
    num = np.max(np.abs(g - r), axis=1)
    den = np.max(np.abs(r), axis=1)
    return float(np.max(np.where(den > 0, num / np.where(den > 0, den, 1.0), num)))


def log_parity(label, **fields):
    """Print a parity result and, when KVD_PARITY_LOG names a file, append it
    there as one JSON line."""
    note("parity", label, " ".join(f"{k}={v:.3e}" if isinstance(v, float) else f"{k}={v}"
                                   for k, v in fields.items()))
    path = os.environ.get("KVD_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(dict(label=label, **fields)) + "\n")


def assert_parity(spec, gpu_out, ref_out, label=None):
    """fp32 caches: 1e-5 max-abs; bf16 caches with fp32 accumulation: 2e-3
    normwise relative.  The worst per-row error is reported beside it."""
    assert np.all(np.isfinite(gpu_out)), "non-finite output"
    row = worst_row_err(gpu_out, ref_out, spec.head_dim)
    if spec.kv_dtype == "f32":
        e = abs_err(gpu_out, ref_out)
        kind = "max_abs"
    else:
        e = rel_err(gpu_out, ref_out)
        kind = "normwise"
    if label is not None:
        log_parity(label, **{kind: e, "worst_row": row, "rows": int(np.size(gpu_out) // spec.head_dim)})
    if spec.kv_dtype == "f32":
        assert e <= 1e-5, f"{spec.name}: max-abs error {e:.3e} > 1e-5"
    else:
        assert e <= 2e-3, f"{spec.name}: normwise relative error {e:.3e} > 2e-3"
    return e


def assert_qrot(gpu_q, ref_q):
    """q_rot is the fp64 rotation rounded to fp32: within one fp32 rounding."""
    ref32 = ref_q.astype(np.float32)
    diff = np.abs(gpu_q.astype(np.float64) - ref_q)
    bound = np.abs(ref_q) * 2.0 ** -23 + 1e-30
    assert np.all(diff <= bound), f"q_rot off by more than an fp32 ulp ({np.max(diff / bound):.2f})"
    return int(np.sum(gpu_q != ref32))
