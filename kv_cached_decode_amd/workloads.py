"""Seeded synthetic inputs for the decode-attention step.

This module only draws random inputs and lays them out; it holds none of the
method's arithmetic (no RoPE, no rounding into the cache, no softmax).  Both
the GPU tests/benchmark and the CPU oracle take their inputs from here.

Workload shapes follow the five named configurations of the decode step:

* ``tiny_f32``       -- batch 1, 4 q heads = 4 kv heads, head_dim 16, a cache of
  32 tokens built by appends, decode at position 32, fp32 cache, values
  uniform in [-0.1, 0.1], RoPE base 10000.
* ``llama3_8b``      -- batch 16, 32 q / 8 kv heads, head_dim 128, context
  4096 for every sequence, bf16 cache, values N(0,1)/sqrt(128), base 500000.
* ``qwen3_0_6b_cb``  -- continuous batching: batch 64, 16 q / 8 kv heads,
  ragged contexts uniform in [128, 8192], paged bf16 (block 16, shuffled
  table), values N(0,1).
* ``long_ctx``       -- batch 4, 64 q / 8 kv heads, context 131072, paged bf16
  (block 64), values N(0,1) plus 16 seeded large-magnitude keys per sequence.
* ``mtp_verify``     -- batch 32, 4 query tokens per sequence (causal within
  the draft), 32 q / 8 kv heads, context 16384, paged bf16 (block 16).
* ``chunked_prefill`` -- batch 8 of Llama-3-8B-shaped layers taking a prefill
  chunk each: ragged chunks of 64..512 new tokens (uniform per sequence) on
  ragged contexts uniform in [0, 4096], paged bf16 (block 16, shuffled).
* ``llama2_7b_mha``  -- multi-head decode (one query row per kv head, where
  the two kernel families come closest): batch 16, 32 q = 32 kv heads,
  head_dim 128, context 4096, paged bf16 (block 16, shuffled), values N(0,1).

bf16 values are drawn as float32 and truncated to their top 16 bits (a
distribution choice, not a rounding the method performs).  Cache slots past
each sequence's context (the tail of its last block, the slots of the new
tokens) and unreferenced spare blocks are poisoned with NaN/Inf so that a
kernel that reads or weights them shows it.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional, Tuple, Union

import numpy as np

BF16_NAN = np.uint16(0x7FC0)
BF16_POS_INF = np.uint16(0x7F80)
BF16_NEG_INF = np.uint16(0xFF80)


@dataclass(frozen=True)
class Spec:
    name: str
    num_seqs: int
    q_tokens: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    block_size: int
    kv_dtype: str                      # "bf16" | "f32"
    ctx: Union[int, Tuple[int, int]]   # context before the step: fixed, or uniform [lo, hi]
    rope_base: float
    dist: str                          # "uniform0.1" | "normal" | "normal_scaled"
    table: str                         # "inorder" | "shuffled" | "single"
    spare_frac: float = 0.0
    big_keys: int = 0                  # large-magnitude key positions per sequence
    big_key_factor: float = 64.0
    prefix: bool = False               # cache built by appends from raw prefix tokens
    seed: int = 0
    layout: int = 0                    # RoPE pairing: 0 half, 1 interleaved
    chunk: Optional[Tuple[int, int]] = None   # ragged new tokens per sequence, uniform [lo, hi] <= T

    def with_(self, **kw) -> "Spec":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    "tiny_f32": Spec("tiny_f32", 1, 1, 4, 4, 16, 64, "f32", 32, 10000.0, "uniform0.1",
                     "single", prefix=True, seed=1),
    "llama3_8b": Spec("llama3_8b", 16, 1, 32, 8, 128, 64, "bf16", 4096, 500000.0,
                      "normal_scaled", "inorder", seed=2),
    "qwen3_0_6b_cb": Spec("qwen3_0_6b_cb", 64, 1, 16, 8, 128, 16, "bf16", (128, 8192),
                          10000.0, "normal", "shuffled", spare_frac=0.05, seed=3),
    "long_ctx": Spec("long_ctx", 4, 1, 64, 8, 128, 64, "bf16", 131072, 10000.0, "normal",
                     "shuffled", spare_frac=0.05, big_keys=16, seed=4),
    "mtp_verify": Spec("mtp_verify", 32, 4, 32, 8, 128, 16, "bf16", 16384, 10000.0, "normal",
                       "shuffled", spare_frac=0.05, seed=5),
    "chunked_prefill": Spec("chunked_prefill", 8, 512, 32, 8, 128, 16, "bf16", (0, 4096), 500000.0,
                            "normal_scaled", "shuffled", spare_frac=0.05, seed=7, chunk=(64, 512)),
    "llama2_7b_mha": Spec("llama2_7b_mha", 16, 1, 32, 32, 128, 16, "bf16", 4096, 10000.0, "normal",
                          "shuffled", spare_frac=0.05, seed=8),
}
CONFIG_ORDER = ["tiny_f32", "llama3_8b", "qwen3_0_6b_cb", "long_ctx", "mtp_verify", "chunked_prefill",
                "llama2_7b_mha"]


def small_variant(name: str) -> Spec:
    """The same structure at sizes the oracle finishes in seconds: several key
    tiles, ragged tails, more than one block per sequence."""
    s = CONFIGS[name]
    if name == "tiny_f32":
        return s
    if name == "llama3_8b":
        return s.with_(name=name + "_small", num_seqs=3, ctx=1000, seed=102)
    if name == "qwen3_0_6b_cb":
        return s.with_(name=name + "_small", num_seqs=9, ctx=(1, 700), seed=103)
    if name == "long_ctx":
        return s.with_(name=name + "_small", num_seqs=2, ctx=9000, seed=104)
    if name == "mtp_verify":
        return s.with_(name=name + "_small", num_seqs=5, ctx=(0, 600), seed=105)
    if name == "chunked_prefill":
        return s.with_(name=name + "_small", num_seqs=3, q_tokens=96, ctx=(0, 300), chunk=(1, 96),
                       seed=107)
    if name == "llama2_7b_mha":
        return s.with_(name=name + "_small", num_seqs=3, ctx=(1, 900), seed=108)
    raise KeyError(name)


@dataclass
class Workload:
    spec: Spec
    ctx_lens: np.ndarray          # int64 [B], context before the step
    seq_lens: np.ndarray          # int32 [B], keys after the new tokens are appended
    block_table: np.ndarray       # int32 [B][max_blocks_per_seq], -1 = unused
    k_pool: np.ndarray            # [num_blocks][Hkv][bs][D] uint16 (bf16 bits) or float32
    v_pool: np.ndarray
    q: np.ndarray                 # float32 [B][T][Hq][D] new queries (before RoPE)
    k: np.ndarray                 # float32 [B][T][Hkv][D] new keys (before RoPE)
    v: np.ndarray                 # float32 [B][T][Hkv][D] new values
    big_key_pos: Optional[np.ndarray] = None   # int64 [B][n] positions of large keys
    prefix_q: Optional[np.ndarray] = None      # float32 [B][P][Hq][D] raw prefix tokens
    prefix_k: Optional[np.ndarray] = None
    prefix_v: Optional[np.ndarray] = None
    q_lens: Optional[np.ndarray] = None        # int32 [B] new tokens per sequence (ragged chunks)
    extra: dict = field(default_factory=dict)

    @property
    def num_blocks(self) -> int:
        return int(self.k_pool.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.seq_lens.size else 0

    def algorithmic_bytes(self) -> dict:
        """Bytes the step must move, per call (see the roofline notes)."""
        s = self.spec
        B, T, Hq, Hkv, D = s.num_seqs, s.q_tokens, s.n_q_heads, s.n_kv_heads, s.head_dim
        esz = 2 if s.kv_dtype == "bf16" else 4
        keys = int(self.seq_lens.astype(np.int64).sum())
        kv_read = keys * Hkv * D * 2 * esz
        if self.q_lens is not None:
            T = float(np.mean(self.q_lens))        # real rows only
        qo = int(B * T * Hq * D * 4 * 2)
        table = int(sum((int(L) + s.block_size - 1) // s.block_size for L in self.seq_lens)) * 4
        attn = kv_read + qo + table + B * 4
        rope_append = B * T * (Hq * D * 4 * 2 + 2 * Hkv * D * (4 + esz)) + B * 4 + B * T * 4
        # the whole step: the cache read, q in, out, the new k/v in and their
        # append, the block table and seq_lens (no intermediate q_rot)
        step = attn + int(B * T * 2 * Hkv * D * (4 + esz))
        return {"kv_read": kv_read, "attention": attn, "rope_append": int(rope_append), "step": step}

    def algorithmic_flops(self) -> int:
        """Multiply-adds of the attention, 2 flops each: for every real query
        row, q.K over the keys it sees and the weighted sum of their V rows."""
        s = self.spec
        T = s.q_tokens
        n = self.q_lens if self.q_lens is not None else np.full(s.num_seqs, T)
        total = 0
        for b in range(s.num_seqs):
            L, nb = int(self.seq_lens[b]), int(n[b])
            vis = L - nb + 1 + np.arange(nb)                 # keys row t sees
            total += int(vis.sum())
        return total * s.n_q_heads * s.head_dim * 2 * 2


def _draw(rng, n, dist, dtype_out):
    if dist == "uniform0.1":
        x = rng.uniform(-0.1, 0.1, size=n).astype(np.float32)
    elif dist == "normal":
        x = rng.standard_normal(n, dtype=np.float32)
    elif dist == "normal_scaled":
        x = rng.standard_normal(n, dtype=np.float32) * np.float32(1.0 / np.sqrt(128.0))
    else:
        raise ValueError(dist)
    if dtype_out == "bf16":
        return (x.view(np.uint32) >> 16).astype(np.uint16)
    return x


def _fill_pool(seed_seq, pool, dist, kv_dtype, chunk=1 << 24):
    """Fill a pool chunk by chunk, each chunk from its own child generator of
    seed_seq, so the values do not depend on how many threads draw them."""
    flat = pool.reshape(-1)
    starts = list(range(0, flat.size, chunk))
    kids = seed_seq.spawn(len(starts))

    def job(i):
        n = min(chunk, flat.size - starts[i])
        flat[starts[i]:starts[i] + n] = _draw(np.random.default_rng(kids[i]), n, dist, kv_dtype)

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        list(ex.map(job, range(len(starts))))


def _poison_value(kv_dtype, which):
    if kv_dtype == "bf16":
        return [BF16_NAN, BF16_POS_INF, BF16_NEG_INF][which % 3]
    return np.float32([np.nan, np.inf, -np.inf][which % 3])


def make_workload(spec: Spec) -> Workload:
    rng = np.random.default_rng(spec.seed)
    B, T, Hq, Hkv, D, bs = (spec.num_seqs, spec.q_tokens, spec.n_q_heads, spec.n_kv_heads,
                            spec.head_dim, spec.block_size)
    if isinstance(spec.ctx, tuple):
        lo, hi = spec.ctx
        ctx = rng.integers(lo, hi + 1, size=B).astype(np.int64)
    else:
        ctx = np.full(B, int(spec.ctx), np.int64)
    q_lens = None
    if spec.chunk is not None:
        lo, hi = spec.chunk
        assert 0 <= lo <= hi <= T
        q_lens = rng.integers(lo, hi + 1, size=B).astype(np.int32)
    seq_lens = (ctx + (T if q_lens is None else q_lens)).astype(np.int32)
    nblk = [(int(L) + bs - 1) // bs for L in seq_lens]
    max_blocks = max(nblk) if B else 0
    total = int(sum(nblk))
    spare = int(np.ceil(spec.spare_frac * total))
    num_blocks = total + spare
    table = np.full((B, max_blocks), -1, np.int32)
    if spec.table == "shuffled":
        perm = rng.permutation(num_blocks).astype(np.int32)
    else:
        perm = np.arange(num_blocks, dtype=np.int32)
    off = 0
    for b in range(B):
        table[b, :nblk[b]] = perm[off:off + nblk[b]]
        off += nblk[b]
    spare_ids = perm[off:]

    np_dt = np.uint16 if spec.kv_dtype == "bf16" else np.float32
    shape = (num_blocks, Hkv, bs, D)
    k_pool = np.empty(shape, np_dt)
    v_pool = np.empty(shape, np_dt)
    if spec.prefix:
        k_pool[...] = _poison_value(spec.kv_dtype, 0)
        v_pool[...] = _poison_value(spec.kv_dtype, 0)
    else:
        k_seq, v_seq = np.random.SeedSequence([spec.seed, 1]), np.random.SeedSequence([spec.seed, 2])
        _fill_pool(k_seq, k_pool, spec.dist, spec.kv_dtype)
        _fill_pool(v_seq, v_pool, spec.dist, spec.kv_dtype)
    # poison every slot at or past the context: the new tokens' slots and the tail
    for b in range(B):
        for pos in range(int(ctx[b]), nblk[b] * bs):
            blk = table[b, pos // bs]
            k_pool[blk, :, pos % bs, :] = _poison_value(spec.kv_dtype, pos)
            v_pool[blk, :, pos % bs, :] = _poison_value(spec.kv_dtype, pos + 1)
    for i, blk in enumerate(spare_ids):
        k_pool[blk] = _poison_value(spec.kv_dtype, i)
        v_pool[blk] = _poison_value(spec.kv_dtype, i + 2)

    big = None
    if spec.big_keys and not spec.prefix:
        big = np.zeros((B, spec.big_keys), np.int64)
        for b in range(B):
            L = int(ctx[b])
            inner = rng.choice(np.arange(1, L - 1), size=spec.big_keys - 2, replace=False)
            pos = np.sort(np.concatenate([[0, L - 1], inner]))
            big[b] = pos
            for p in pos:
                blk = table[b, p // bs]
                row = k_pool[blk, :, p % bs, :]
                if spec.kv_dtype == "bf16":
                    f = (row.astype(np.uint32) << 16).view(np.float32) * np.float32(spec.big_key_factor)
                    k_pool[blk, :, p % bs, :] = (f.view(np.uint32) >> 16).astype(np.uint16)
                else:
                    k_pool[blk, :, p % bs, :] = row * np.float32(spec.big_key_factor)

    def raw(shape_):
        return _draw(rng, int(np.prod(shape_)), spec.dist, "f32").reshape(shape_)

    pq = pk = pv = None
    if spec.prefix:
        P = int(ctx.max()) + T
        pq, pk, pv = raw((B, P, Hq, D)), raw((B, P, Hkv, D)), raw((B, P, Hkv, D))
        idx = [np.arange(int(c), int(c) + T) for c in ctx]
        q = np.stack([pq[b, idx[b]] for b in range(B)]).astype(np.float32)
        k = np.stack([pk[b, idx[b]] for b in range(B)]).astype(np.float32)
        v = np.stack([pv[b, idx[b]] for b in range(B)]).astype(np.float32)
    else:
        q, k, v = raw((B, T, Hq, D)), raw((B, T, Hkv, D)), raw((B, T, Hkv, D))
    return Workload(spec, ctx, seq_lens, table, k_pool, v_pool,
                    np.ascontiguousarray(q), np.ascontiguousarray(k), np.ascontiguousarray(v),
                    big, pq, pk, pv, q_lens)


def sample_rows(spec: Spec, n: int, seed: int = 0) -> np.ndarray:
    """A seeded sample of flat query rows (b*T*Hq + t*Hq + h) that always
    includes the first and last row of every sequence."""
    rng = np.random.default_rng(10_000 + seed)
    per_seq = spec.q_tokens * spec.n_q_heads
    total = spec.num_seqs * per_seq
    ends = np.concatenate([np.arange(spec.num_seqs) * per_seq,
                           np.arange(spec.num_seqs) * per_seq + per_seq - 1])
    extra = rng.choice(total, size=min(n, total), replace=False)
    return np.unique(np.concatenate([ends, extra])).astype(np.int64)


# --------------------------------------------------------------------------
# The tiny decoder LM of ferric-core `examples/generate.rs` (its `Cfg` and
# `Layer`): 3 layers, 4 heads of 16, model width 64, MLP width 128, vocab 32,
# RoPE base 10000, RMSNorm eps 1e-5, prompt [3, 14, 1, 15] then 5 greedy
# steps.  Weights are seeded uniform draws standing in for the page's hash
# fill; the norm gains are 1 plus a draw, as on the page.
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class TinyLMConfig:
    n_layers: int = 3
    n_heads: int = 4
    head_dim: int = 16
    d_model: int = 64
    d_ff: int = 128
    vocab: int = 32
    rope_base: float = 10000.0
    eps: float = 1e-5
    weight_scale: float = 0.3
    seed: int = 9


TINY_LM = TinyLMConfig()
TINY_LM_PROMPT = (3, 14, 1, 15)
TINY_LM_GEN_STEPS = 5


def tiny_lm_weights(cfg: TinyLMConfig = TINY_LM) -> dict:
    """float32 weights, matrices stored [in][out] (a row vector times W):
    emb [vocab][d]; per layer wn1, wn2 [d]; wq, wk, wv, wo [d][d]; wg, wu
    [d][ff]; wd [ff][d]; then wln [d] and wlm [d][vocab]."""
    rng = np.random.default_rng(cfg.seed)
    a = cfg.weight_scale
    d, ff = cfg.d_model, cfg.d_ff

    def u(*shape):
        return rng.uniform(-a, a, size=shape).astype(np.float32)

    w = {"emb": u(cfg.vocab, d), "layers": []}
    for _ in range(cfg.n_layers):
        w["layers"].append({
            "wn1": (1.0 + u(d)).astype(np.float32), "wn2": (1.0 + u(d)).astype(np.float32),
            "wq": u(d, d), "wk": u(d, d), "wv": u(d, d), "wo": u(d, d),
            "wg": u(d, ff), "wu": u(d, ff), "wd": u(ff, d),
        })
    w["wln"] = (1.0 + u(d)).astype(np.float32)
    w["wlm"] = u(d, cfg.vocab)
    return w
