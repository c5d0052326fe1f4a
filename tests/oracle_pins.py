"""Pins for the CPU oracle: checks against what the pages and the mathematics
fix, independent of the oracle's own formulas.

Each ``check_*`` function raises AssertionError on a mismatch.  They are run
by test_oracle_pins.py against the real oracle and by test_oracle_mutants.py
against copies of the oracle with planted mistakes (each mistake must trip at
least one check).

What pins what:

* bf16 rounding -- torch's fp32->bf16 conversion (a library routine) and
  hand-derived tie / overflow / subnormal cases (tests/golden).
* RoPE -- closed forms at theta_0 = 1 and theta_1 = base^(-1/2); identity at
  position 0; the textbook complex-number form; the relative-position
  property; norm preservation.
* append -- the integer closed form of the slot address; a sentinel canary
  (exactly the target slots change); the stored bits against torch's bf16
  conversion and the complex-form RoPE.
* attention -- the pages' own criterion (ferric-core generate.rs: cached decode
  equals the last row of a full non-cached causal recompute); torch's
  scaled_dot_product_attention in fp64; weights sum to one; identical keys give
  the mean of V; a single key gives its V; constant V; a dominant key; linearity
  in V; block-permutation invariance; GQA = MHA on repeated heads; a verify row
  equals a shorter single-token decode; log-sum-exp against scipy.
"""
import json
import math
import os

import numpy as np
import torch

import oracle
from full_recompute import causal_attention, recompute_last_rows, rope_complex
from helpers import gather, oracle_cache, pool_as_f64
from kv_cached_decode_amd import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------- bf16 rounding
def check_bf16_matches_torch():
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-39).astype(np.float32),     # subnormal range
        np.clip(rng.standard_normal(2000) * 1e38, -3.3e38, 3.3e38).astype(np.float32),
        np.float32([0.0, -0.0, np.inf, -np.inf, 3.4e38, -3.4e38]),
        # exact ties: 8 significant bits + a half ulp
        ((rng.integers(128, 256, 2000) * 2 + 1).astype(np.float32) * np.float32(2.0 ** -9)),
    ])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.bf16_from_double(float(v)) for v in x], np.uint16)
    assert np.array_equal(ref, got), f"{int((ref != got).sum())} bf16 roundings differ from torch"


def check_bf16_golden():
    with open(os.path.join(GOLDEN, "bf16_rounding_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        x = float(c["x"]) if "inf" in c["x"] else float.fromhex(c["x"])
        got = oracle.bf16_from_double(x)
        assert got == int(c["bits"], 16), f"bf16({c['x']}) = {got:#06x}, expected {c['bits']} ({c['why']})"
    assert oracle.bf16_from_double(float("nan")) & 0x7FFF == 0x7FC0


def check_bf16_roundtrip():
    bits = np.arange(1 << 16, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    for b in range(0, 1 << 16, 97):
        if np.isnan(f[b]):
            continue
        v = oracle.bf16_to_double(b)
        assert v == float(f[b])
        assert oracle.bf16_from_double(v) == b


# ------------------------------------------------------------------------- RoPE
def check_rope_closed_form():
    c1, s1 = math.cos(1.0), math.sin(1.0)
    # D = 4: theta_0 = 1, theta_1 = base^(-1/2) = 0.01 for base 10000, so
    # position 1 turns pair 0 by 1 rad and position 100 turns pair 1 by 1 rad.
    cases = [
        (0, [1, 0, 0, 0], 1, [c1, 0, s1, 0]),
        (0, [0, 0, 1, 0], 1, [-s1, 0, c1, 0]),
        (0, [0, 1, 0, 0], 100, [0, c1, 0, s1]),
        (1, [1, 0, 0, 0], 1, [c1, s1, 0, 0]),
        (1, [0, 0, 0, 1], 100, [0, 0, -s1, c1]),
        (1, [0, 1, 0, 0], 1, [-s1, c1, 0, 0]),
    ]
    for layout, x, pos, want in cases:
        y = oracle.rope(np.array([[x]], np.float64), [pos], 10000.0, layout)[0, 0]
        assert np.allclose(y, want, rtol=0, atol=1e-15), (layout, x, pos, y, want)


def check_rope_position_zero_identity():
    x = np.random.default_rng(1).standard_normal((3, 5, 128))
    for layout in (0, 1):
        y = oracle.rope(x, [0, 0, 0], 500000.0, layout)
        assert np.array_equal(x, y)


def check_rope_complex_form():
    rng = np.random.default_rng(2)
    pos = np.concatenate([[0, 1, 2, 4095, 4096, 16387, 131072], rng.integers(0, 140000, 9)])
    for D, base in ((16, 10000.0), (128, 10000.0), (128, 500000.0), (64, 1e6)):
        x = rng.standard_normal((pos.size, 3, D))
        for layout in (0, 1):
            y = oracle.rope(x, pos, base, layout)
            ref = rope_complex(x, pos, base, layout)
            assert np.max(np.abs(y - ref)) < 1e-9, (D, base, layout, np.max(np.abs(y - ref)))


def check_rope_relative_position():
    rng = np.random.default_rng(3)
    D = 128
    for layout in (0, 1):
        for m, n in ((5, 3), (131072, 131000), (70000, 12), (16387, 16384)):
            q = rng.standard_normal((1, 1, D))
            k = rng.standard_normal((1, 1, D))
            lhs = np.sum(oracle.rope(q, [m], 10000.0, layout) * oracle.rope(k, [n], 10000.0, layout))
            rhs = np.sum(oracle.rope(q, [m - n], 10000.0, layout) * k)
            tol = 1e-9 * np.linalg.norm(q) * np.linalg.norm(k)
            assert abs(lhs - rhs) < tol, (layout, m, n, lhs, rhs)


def check_rope_norm():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((4, 2, 128))
    for layout in (0, 1):
        y = oracle.rope(x, [3, 999, 65536, 131073], 10000.0, layout)
        assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)


# ----------------------------------------------------------------------- append
def _sentinel_workload(kv_dtype, T=2, bs=4, seed=11):
    spec = workloads.Spec("append_probe", 3, T, 4, 2, 16, bs, kv_dtype, (0, 9), 10000.0,
                          "normal", "shuffled", spare_frac=0.5, seed=seed)
    return workloads.make_workload(spec)


def check_append_slots_and_bits():
    for kv_dtype in ("bf16", "f32"):
        w = _sentinel_workload(kv_dtype)
        s = w.spec
        sentinel = np.uint16(0x1234) if kv_dtype == "bf16" else np.float32(-777.0)
        kp = np.full_like(w.k_pool, sentinel)
        vp = np.full_like(w.v_pool, sentinel)
        oc = oracle_cache(w, k_pool=kp, v_pool=vp)
        q_rot = oc.rope_append_kv(w.q, w.k, w.v, s.rope_base, s.layout)
        changed_k = oc.k_pool != sentinel
        changed_v = oc.v_pool != sentinel
        expect = np.zeros_like(changed_k)
        for b in range(s.num_seqs):
            for t in range(s.q_tokens):
                pos = int(w.seq_lens[b]) - s.q_tokens + t
                blk = w.block_table[b, pos // s.block_size]
                expect[blk, :, pos % s.block_size, :] = True
        assert np.array_equal(changed_k, expect), "K append wrote outside its slots"
        assert np.array_equal(changed_v, expect), "V append wrote outside its slots"
        for b in range(s.num_seqs):
            pos = np.arange(int(w.seq_lens[b]) - s.q_tokens, int(w.seq_lens[b]))
            krot = rope_complex(w.k[b].astype(np.float64), pos, s.rope_base, s.layout)
            qrot = rope_complex(w.q[b].astype(np.float64), pos, s.rope_base, s.layout)
            assert np.max(np.abs(q_rot[b] - qrot)) < 1e-12
            for t, p in enumerate(pos):
                blk = w.block_table[b, p // s.block_size]
                ks = oc.k_pool[blk, :, p % s.block_size, :]
                vs = oc.v_pool[blk, :, p % s.block_size, :]
                if kv_dtype == "bf16":
                    vref = torch.from_numpy(w.v[b, t]).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
                    kref = np.vectorize(oracle.bf16_from_double, otypes=[np.uint16])(krot[t])
                    assert np.array_equal(vs, vref), "V not stored as bf16(v)"
                    assert np.array_equal(ks, kref), "K not stored as bf16(rope(k))"
                else:
                    assert np.array_equal(vs, w.v[b, t])
                    assert np.max(np.abs(ks.astype(np.float64) - krot[t])) <= 6e-8 * np.max(np.abs(krot[t]))


# -------------------------------------------------------------------- attention
def _build_by_appends(B, T, Hq, Hkv, D, bs, P, base, layout, dtype, seed):
    """A paged cache filled by appending each sequence's raw prefix T tokens at
    a time (the decode loop of generate.rs), returning the raw prefix too."""
    rng = np.random.default_rng(seed)
    assert P % T == 0
    nblk = (P + bs - 1) // bs
    num_blocks = B * nblk + 3
    perm = rng.permutation(num_blocks).astype(np.int32)
    table = perm[:B * nblk].reshape(B, nblk).copy()
    np_dt = {"f64": np.float64, "f32": np.float32, "bf16": np.uint16}[dtype]
    shape = (num_blocks, Hkv, bs, D)
    kp = np.full(shape, np.nan if dtype != "bf16" else 0x7FC0, np_dt)
    vp = np.full(shape, np.nan if dtype != "bf16" else 0x7FC0, np_dt)
    qr = rng.uniform(-1, 1, (B, P, Hq, D)).astype(np.float32)
    kr = rng.uniform(-1, 1, (B, P, Hkv, D)).astype(np.float32)
    vr = rng.uniform(-1, 1, (B, P, Hkv, D)).astype(np.float32)
    dt_code = {"f64": oracle.ORACLE_F64, "f32": oracle.ORACLE_F32, "bf16": oracle.ORACLE_BF16}[dtype]
    q_rot = None
    for start in range(0, P, T):
        seq_lens = np.full(B, start + T, np.int32)
        oc = oracle.OracleCache(num_seqs=B, q_tokens=T, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D,
                                block_size=bs, k_pool=kp, v_pool=vp, block_table=table,
                                seq_lens=seq_lens, cache_dtype=dt_code)
        q_rot = oc.rope_append_kv(np.ascontiguousarray(qr[:, start:start + T]),
                                  np.ascontiguousarray(kr[:, start:start + T]),
                                  np.ascontiguousarray(vr[:, start:start + T]), base, layout)
    return oc, q_rot, qr, kr, vr


CRITERION_SHAPES = [
    # B, T, Hq, Hkv, D, bs, P, base, layout
    (2, 1, 4, 4, 16, 4, 1, 10000.0, 0),
    (2, 1, 4, 4, 16, 4, 33, 10000.0, 0),
    (1, 1, 8, 2, 16, 1, 17, 500000.0, 1),
    (2, 3, 6, 3, 16, 16, 48, 10000.0, 0),
    (1, 4, 8, 2, 128, 16, 64, 10000.0, 1),
    (1, 1, 4, 1, 128, 64, 300, 500000.0, 0),
]


def check_cached_decode_equals_full_recompute():
    for (B, T, Hq, Hkv, D, bs, P, base, layout) in CRITERION_SHAPES:
        for dtype in ("f64", "f32"):
            oc, q_rot, qr, kr, vr = _build_by_appends(B, T, Hq, Hkv, D, bs, P, base, layout, dtype,
                                                      seed=P + D + Hq)
            out, lse = oc.decode_attention(q_rot, want_lse=True)
            store = None if dtype == "f64" else (lambda a: a.astype(np.float32).astype(np.float64))
            tol = 1e-12 if dtype == "f64" else 1e-6
            for b in range(B):
                ref, ref_lse = recompute_last_rows(qr[b], kr[b], vr[b], T, base, layout, store)
                err = np.max(np.abs(out[b] - ref))
                assert err < tol, (B, T, Hq, Hkv, D, bs, P, dtype, err)
                assert np.max(np.abs(lse[b] - ref_lse)) < max(tol, 1e-11)


def check_tiny_config_chain():
    """The tiny fp32 configuration: 32 appends at positions 0..31, then the
    decode step at position 32, against the full recompute of the 33 tokens."""
    w = workloads.make_workload(workloads.CONFIGS["tiny_f32"])
    s = w.spec
    for dtype, tol in (("f64", 1e-12), ("f32", 1e-7)):
        np_dt = np.float64 if dtype == "f64" else np.float32
        kp = np.full(w.k_pool.shape, np.nan, np_dt)
        vp = np.full(w.v_pool.shape, np.nan, np_dt)
        for p in range(33):
            oc = oracle_cache(w, seq_lens=np.array([p + 1], np.int32), k_pool=kp, v_pool=vp,
                              dtype=dtype)
            q_rot = oc.rope_append_kv(np.ascontiguousarray(w.prefix_q[:, p:p + 1]),
                                      np.ascontiguousarray(w.prefix_k[:, p:p + 1]),
                                      np.ascontiguousarray(w.prefix_v[:, p:p + 1]), s.rope_base)
            kp, vp = oc.k_pool, oc.v_pool
        out = oc.decode_attention(q_rot)
        store = None if dtype == "f64" else (lambda a: a.astype(np.float32).astype(np.float64))
        ref, _ = recompute_last_rows(w.prefix_q[0], w.prefix_k[0], w.prefix_v[0], 1, s.rope_base,
                                     s.layout, store)
        assert np.max(np.abs(out[0] - ref)) < tol, (dtype, np.max(np.abs(out[0] - ref)))


def _dense_sdpa(w, q64, b, t):
    """torch SDPA (fp64, CPU) for query token t of sequence b on gathered K/V."""
    s = w.spec
    g = s.n_q_heads // s.n_kv_heads
    n = int(w.seq_lens[b]) - s.q_tokens + t + 1
    K = np.stack([gather(pool_as_f64(w, w.k_pool), w.block_table[b], s.block_size, h, n)
                  for h in range(s.n_kv_heads)])
    V = np.stack([gather(pool_as_f64(w, w.v_pool), w.block_table[b], s.block_size, h, n)
                  for h in range(s.n_kv_heads)])
    Kt = torch.from_numpy(K).repeat_interleave(g, dim=0).contiguous()
    Vt = torch.from_numpy(V).repeat_interleave(g, dim=0).contiguous()
    Q = torch.from_numpy(q64[b, t]).unsqueeze(1)       # [Hq][1][D]
    return torch.nn.functional.scaled_dot_product_attention(Q, Kt, Vt).squeeze(1).numpy()


def _fill_new_slots(w):
    """Give the new tokens' slots valid values (attention-only checks)."""
    s = w.spec
    rng = np.random.default_rng(99)
    for b in range(s.num_seqs):
        for pos in range(int(w.ctx_lens[b]), int(w.seq_lens[b])):
            blk = w.block_table[b, pos // s.block_size]
            n = s.n_kv_heads * s.head_dim
            for pool in (w.k_pool, w.v_pool):
                if s.kv_dtype == "bf16":
                    pool[blk, :, pos % s.block_size, :] = (
                        rng.standard_normal(n, dtype=np.float32).view(np.uint32) >> 16
                    ).astype(np.uint16).reshape(s.n_kv_heads, s.head_dim)
                else:
                    pool[blk, :, pos % s.block_size, :] = rng.standard_normal(
                        (s.n_kv_heads, s.head_dim)).astype(np.float32)
    return w


def check_attention_matches_torch_sdpa():
    for name in ("qwen3_0_6b_cb", "mtp_verify"):
        spec = workloads.small_variant(name).with_(num_seqs=3)
        w = _fill_new_slots(workloads.make_workload(spec))
        q64 = w.q.astype(np.float64)
        out = oracle_cache(w).decode_attention(q64)
        for b in range(spec.num_seqs):
            for t in range(spec.q_tokens):
                ref = _dense_sdpa(w, q64, b, t)
                err = np.max(np.abs(out[b, t] - ref))
                assert err < 1e-12, (name, b, t, err)


def _tiny_cache(B=2, T=1, Hq=4, Hkv=2, D=16, bs=4, L=(7, 13), seed=5, dtype="f64"):
    spec = workloads.Spec("tiny_probe", B, T, Hq, Hkv, D, bs, "f32", L, 10000.0, "normal",
                          "shuffled", spare_frac=0.3, seed=seed)
    w = _fill_new_slots(workloads.make_workload(spec))
    return w, oracle_cache(w, dtype=dtype)


def check_weights_sum_to_one_and_lse():
    w, oc = _tiny_cache(B=3, T=2, L=(0, 40))
    q = w.q.astype(np.float64) * 3.0
    out, lse, wsum = oc.decode_attention(q, want_lse=True, want_wsum=True)
    assert np.max(np.abs(wsum - 1.0)) < 1e-13
    s = w.spec
    from scipy.special import logsumexp
    g = s.n_q_heads // s.n_kv_heads
    kf = pool_as_f64(w, w.k_pool)
    for b in range(s.num_seqs):
        for t in range(s.q_tokens):
            n = int(w.seq_lens[b]) - s.q_tokens + t + 1
            for h in range(s.n_q_heads):
                K = gather(kf, w.block_table[b], s.block_size, h // g, n)
                sc = K @ q[b, t, h] / math.sqrt(s.head_dim)
                assert abs(lse[b, t, h] - logsumexp(sc)) < 1e-12


def check_identical_keys_mean_v():
    w, oc = _tiny_cache(L=(20, 30))
    s = w.spec
    oc.k_pool[...] = 0.37                       # every key identical
    out = oc.decode_attention(w.q.astype(np.float64) * 5)
    vf = oc.v_pool
    for b in range(s.num_seqs):
        n = int(w.seq_lens[b])
        for h in range(s.n_q_heads):
            V = gather(vf, w.block_table[b], s.block_size, h // (s.n_q_heads // s.n_kv_heads), n)
            assert np.max(np.abs(out[b, 0, h] - V.mean(axis=0))) < 1e-14


def check_single_key_and_constant_v():
    w, oc = _tiny_cache(L=(0, 0))                # context 0: only the new token is visible
    s = w.spec
    out = oc.decode_attention(w.q.astype(np.float64))
    g = s.n_q_heads // s.n_kv_heads
    for b in range(s.num_seqs):
        blk = w.block_table[b, 0]
        for h in range(s.n_q_heads):
            assert np.array_equal(out[b, 0, h], oc.v_pool[blk, h // g, 0])
    w, oc = _tiny_cache(L=(5, 40))
    oc.v_pool[...] = -1.25
    out = oc.decode_attention(w.q.astype(np.float64))
    assert np.max(np.abs(out + 1.25)) < 1e-14


def check_dominant_key():
    """A key whose score exceeds every other by ~1e3 takes all the weight; the
    scores are large enough that a softmax without the running max overflows."""
    w, oc = _tiny_cache(L=(30, 30))
    s = w.spec
    q = np.zeros_like(w.q, dtype=np.float64)
    q[..., 0] = 1.0
    oc.k_pool[..., 0] = np.clip(oc.k_pool[..., 0], -1, 1)
    pos = 11
    g = s.n_q_heads // s.n_kv_heads
    for b in range(s.num_seqs):
        blk = w.block_table[b, pos // s.block_size]
        oc.k_pool[blk, :, pos % s.block_size, 0] = 8000.0
    out = oc.decode_attention(q)
    for b in range(s.num_seqs):
        blk = w.block_table[b, pos // s.block_size]
        for h in range(s.n_q_heads):
            assert np.max(np.abs(out[b, 0, h] - oc.v_pool[blk, h // g, pos % s.block_size])) < 1e-12


def check_linear_in_v():
    w, oc1 = _tiny_cache(L=(9, 25), seed=8)
    q = w.q.astype(np.float64)
    _, oc2 = _tiny_cache(L=(9, 25), seed=8)
    oc2.v_pool[...] = np.random.default_rng(3).standard_normal(oc2.v_pool.shape)
    _, oc3 = _tiny_cache(L=(9, 25), seed=8)
    oc3.v_pool[...] = 2.0 * oc1.v_pool - 3.0 * oc2.v_pool
    o1, o2, o3 = oc1.decode_attention(q), oc2.decode_attention(q), oc3.decode_attention(q)
    assert np.max(np.abs(o3 - (2.0 * o1 - 3.0 * o2))) < 1e-12


def check_block_permutation_invariance():
    w, oc = _tiny_cache(B=3, T=2, L=(3, 40), seed=9)
    q = w.q.astype(np.float64)
    out = oc.decode_attention(q)
    perm = np.random.default_rng(4).permutation(oc.k_pool.shape[0])   # new id of old block i
    kp = np.empty_like(oc.k_pool)
    vp = np.empty_like(oc.v_pool)
    kp[perm] = oc.k_pool
    vp[perm] = oc.v_pool
    table = np.where(w.block_table >= 0, perm[np.maximum(w.block_table, 0)], -1).astype(np.int32)
    oc2 = oracle_cache(w, k_pool=kp, v_pool=vp, block_table=table, dtype="f64")
    assert np.array_equal(out, oc2.decode_attention(q))


def check_gqa_equals_repeated_mha():
    w, oc = _tiny_cache(B=2, T=2, Hq=8, Hkv=2, L=(5, 30), seed=10)
    q = w.q.astype(np.float64)
    out = oc.decode_attention(q)
    g = 4
    kp = np.repeat(oc.k_pool, g, axis=1)
    vp = np.repeat(oc.v_pool, g, axis=1)
    s = w.spec
    mha = oracle.OracleCache(num_seqs=s.num_seqs, q_tokens=s.q_tokens, n_q_heads=8, n_kv_heads=8,
                             head_dim=s.head_dim, block_size=s.block_size,
                             k_pool=np.ascontiguousarray(kp), v_pool=np.ascontiguousarray(vp),
                             block_table=w.block_table, seq_lens=w.seq_lens,
                             cache_dtype=oracle.ORACLE_F64)
    assert np.array_equal(out, mha.decode_attention(q))


def check_verify_row_equals_shorter_decode():
    T = 3
    w, oc = _tiny_cache(B=2, T=T, L=(4, 30), seed=12)
    q = w.q.astype(np.float64)
    out = oc.decode_attention(q)
    for t in range(T):
        sl = (w.seq_lens - (T - 1 - t)).astype(np.int32)
        one = oracle_cache(w, seq_lens=sl, q_tokens=1, k_pool=oc.k_pool, v_pool=oc.v_pool,
                           dtype="f64")
        o1 = one.decode_attention(np.ascontiguousarray(q[:, t:t + 1]))
        assert np.array_equal(out[:, t], o1[:, 0]), t


def check_sliding_window_equals_truncated_cache():
    """Attention with a window of W keys equals full attention over a cache
    that holds only the last W keys of each sequence (the same stored rows,
    moved to positions 0..W-1), and a verify row with a window equals the
    shorter single-token decode with the same window."""
    for W in (1, 5, 33, 200):
        w, oc = _tiny_cache(B=3, T=1, L=(0, 120), seed=14)
        s = w.spec
        q = w.q.astype(np.float64)
        out_w = oracle_cache(w, k_pool=oc.k_pool, v_pool=oc.v_pool, dtype="f64", window=W).decode_attention(q)
        bs = s.block_size
        keep = [min(int(L), W) for L in w.seq_lens]
        nblk = max((k + bs - 1) // bs for k in keep)
        kp = np.full((s.num_seqs * nblk, s.n_kv_heads, bs, s.head_dim), np.nan)
        vp = np.full_like(kp, np.nan)
        table = np.arange(s.num_seqs * nblk, dtype=np.int32).reshape(s.num_seqs, nblk)
        for b in range(s.num_seqs):
            L = int(w.seq_lens[b])
            for new, old in enumerate(range(L - keep[b], L)):
                blk = w.block_table[b, old // bs]
                kp[table[b, new // bs], :, new % bs] = oc.k_pool[blk, :, old % bs]
                vp[table[b, new // bs], :, new % bs] = oc.v_pool[blk, :, old % bs]
        trunc = oracle.OracleCache(num_seqs=s.num_seqs, q_tokens=1, n_q_heads=s.n_q_heads,
                                   n_kv_heads=s.n_kv_heads, head_dim=s.head_dim, block_size=bs,
                                   k_pool=kp, v_pool=vp, block_table=table,
                                   seq_lens=np.array(keep, np.int32), cache_dtype=oracle.ORACLE_F64)
        assert np.array_equal(out_w, trunc.decode_attention(q)), W
    T = 3
    w, oc = _tiny_cache(B=2, T=T, L=(4, 60), seed=15)
    q = w.q.astype(np.float64)
    out = oracle_cache(w, k_pool=oc.k_pool, v_pool=oc.v_pool, dtype="f64", window=7).decode_attention(q)
    for t in range(T):
        sl = (w.seq_lens - (T - 1 - t)).astype(np.int32)
        one = oracle_cache(w, seq_lens=sl, q_tokens=1, k_pool=oc.k_pool, v_pool=oc.v_pool, dtype="f64",
                           window=7)
        assert np.array_equal(out[:, t], one.decode_attention(np.ascontiguousarray(q[:, t:t + 1]))[:, 0])


def _shard_cache(w, whole, cut0, cut1, window=0, q_tokens=None, dtype="f64"):
    """A cache that holds only global keys cut0[b] .. cut1[b]-1 of each
    sequence of `whole`, moved to local positions 0.., with the shard
    positions that say so."""
    s = w.spec
    bs = s.block_size
    n = (cut1 - cut0).astype(np.int64)
    nb = max(1, int(max((k + bs - 1) // bs for k in n)))
    fill = workloads.BF16_NAN if whole.k_pool.dtype == np.uint16 else np.nan
    kp = np.full((s.num_seqs * nb, s.n_kv_heads, bs, s.head_dim), fill, whole.k_pool.dtype)
    vp = np.full_like(kp, fill)
    table = np.arange(s.num_seqs * nb, dtype=np.int32).reshape(s.num_seqs, nb)
    for b in range(s.num_seqs):
        for i, gpos in enumerate(range(int(cut0[b]), int(cut1[b]))):
            blk = w.block_table[b, gpos // bs]
            kp[table[b, i // bs], :, i % bs] = whole.k_pool[blk, :, gpos % bs]
            vp[table[b, i // bs], :, i % bs] = whole.v_pool[blk, :, gpos % bs]
    T = q_tokens or s.q_tokens
    return oracle.OracleCache(num_seqs=s.num_seqs, q_tokens=T, n_q_heads=s.n_q_heads,
                              n_kv_heads=s.n_kv_heads, head_dim=s.head_dim, block_size=bs,
                              k_pool=kp, v_pool=vp, block_table=table, seq_lens=n.astype(np.int32),
                              cache_dtype=whole.cache_dtype, window=window,
                              key_pos0=cut0.astype(np.int32),
                              q_pos=(w.seq_lens - T).astype(np.int32))


def check_context_parallel_shards_merge_to_whole():
    """Context parallelism: each shard's (out, lse) over the keys it holds,
    merged by log-sum-exp weights, equals attention over the whole cache;
    a row that sees no key of a shard gets out = 0 and lse = -inf."""
    from scipy.special import logsumexp
    for window, seed in ((0, 21), (9, 22), (40, 23)):
        w, oc = _tiny_cache(B=4, T=2, L=(0, 60), seed=seed)
        s = w.spec
        q = w.q.astype(np.float64) * 2.0
        out_w, lse_w = oracle_cache(w, k_pool=oc.k_pool, v_pool=oc.v_pool, dtype="f64",
                                    window=window).decode_attention(q, want_lse=True)
        rng = np.random.default_rng(seed)
        L = w.seq_lens.astype(np.int64)
        # three shards per sequence at seeded cut points (empty shards included)
        cuts = np.sort(np.stack([rng.integers(0, L + 1) for _ in range(2)], 1), 1)
        cuts[0] = 0                      # sequence 0: two empty shards
        cuts[1] = L[1] - 1               # sequence 1: the last shard holds only key L-1,
                                         # which draft row 0 does not see
        edges = np.concatenate([np.zeros((s.num_seqs, 1), np.int64), cuts, L[:, None]], 1)
        outs, lses = [], []
        for k in range(3):
            sh = _shard_cache(w, oc, edges[:, k], edges[:, k + 1], window=window)
            o, l_ = sh.decode_attention(q, want_lse=True)
            empty = np.isneginf(l_)
            assert np.all(o[empty] == 0.0)
            outs.append(o)
            lses.append(l_)
        assert any(np.isneginf(l_).any() for l_ in lses), "want a shard some row cannot see"
        lse_m = logsumexp(np.stack(lses), axis=0)
        wts = np.exp(np.stack(lses) - lse_m)[..., None]
        out_m = np.sum(wts * np.stack(outs), axis=0)
        assert np.max(np.abs(out_m - out_w)) < 1e-12, window
        assert np.max(np.abs(lse_m - lse_w)) < 1e-12, window


def check_shard_append_rotates_at_global_position():
    """The shard holding a sequence's tail appends its new tokens at their
    global positions (the rotation) into its local slots: the stored rows and
    q_rot equal the whole-cache append's bit for bit.  A shard without the
    new tokens returns the same q_rot and leaves its pools untouched."""
    for dtype, kvd in (("f64", "f64"), ("bf16", "bf16")):
        spec = workloads.Spec("shard_append", 3, 2, 4, 2, 16, 4, kvd if kvd == "bf16" else "f32",
                              (5, 50), 10000.0, "normal", "shuffled", spare_frac=0.2, seed=24)
        w = workloads.make_workload(spec)
        whole = oracle_cache(w, dtype=dtype)
        q_whole = whole.rope_append_kv(w.q, w.k, w.v, spec.rope_base)
        L = w.seq_lens.astype(np.int64)
        cut = (L - spec.q_tokens) // 2
        tail = _shard_cache(w, oracle_cache(w, dtype=dtype), cut, L, dtype=dtype)
        q_tail = tail.rope_append_kv(w.q, w.k, w.v, spec.rope_base)
        assert np.array_equal(q_whole, q_tail)
        bs = spec.block_size
        for b in range(spec.num_seqs):
            for t in range(spec.q_tokens):
                gpos = int(L[b]) - spec.q_tokens + t
                loc = gpos - int(cut[b])
                a = whole.k_pool[w.block_table[b, gpos // bs], :, gpos % bs]
                c = tail.k_pool[tail.block_table[b, loc // bs], :, loc % bs]
                assert np.array_equal(a, c), (dtype, b, t)
                a = whole.v_pool[w.block_table[b, gpos // bs], :, gpos % bs]
                c = tail.v_pool[tail.block_table[b, loc // bs], :, loc % bs]
                assert np.array_equal(a, c), (dtype, b, t)
        # a shard that does not hold the new tokens (the head of every
        # sequence) rotates the queries alike and stores nothing
        head = _shard_cache(w, oracle_cache(w, dtype=dtype), np.zeros_like(cut), cut, dtype=dtype)
        k_before, v_before = head.k_pool.copy(), head.v_pool.copy()
        q_head = head.rope_append_kv(w.q, w.k, w.v, spec.rope_base)
        assert np.array_equal(q_whole, q_head)
        assert np.array_equal(head.k_pool.view(np.uint8), k_before.view(np.uint8))
        assert np.array_equal(head.v_pool.view(np.uint8), v_before.view(np.uint8))


def check_ragged_new_tokens():
    """Ragged chunks (q_lens[b] <= T new tokens per sequence): each real row
    equals the same sequence decoded alone with T = q_lens[b]; padding rows
    get out = 0 and lse = -inf; the append writes exactly the real tokens'
    slots (checked against a sentinel pool)."""
    T = 6
    spec = workloads.Spec("ragged", 4, T, 4, 2, 16, 4, "f32", (0, 30), 10000.0, "normal", "shuffled",
                          spare_frac=0.2, seed=25)
    w = workloads.make_workload(spec)
    q_lens = np.array([6, 1, 3, 0], np.int32)
    # the cache holds ctx + q_lens keys; the table covers ctx + T
    sl = (w.ctx_lens + q_lens).astype(np.int32)
    base = oracle_cache(w, seq_lens=sl, dtype="f64")
    sentinel = np.full_like(base.k_pool, 7.0)
    ragged = oracle.OracleCache(num_seqs=spec.num_seqs, q_tokens=T, n_q_heads=spec.n_q_heads,
                                n_kv_heads=spec.n_kv_heads, head_dim=spec.head_dim,
                                block_size=spec.block_size, k_pool=sentinel.copy(), v_pool=sentinel.copy(),
                                block_table=w.block_table, seq_lens=sl, cache_dtype=oracle.ORACLE_F64,
                                q_lens=q_lens)
    q_rot = ragged.rope_append_kv(w.q, w.k, w.v, spec.rope_base)
    changed = np.argwhere(np.any(ragged.k_pool != 7.0, axis=-1))
    assert len(changed) == int(q_lens.sum()) * spec.n_kv_heads
    bs = spec.block_size
    for b in range(spec.num_seqs):
        for t in range(int(q_lens[b])):
            pos = int(sl[b]) - int(q_lens[b]) + t
            assert np.all(ragged.k_pool[w.block_table[b, pos // bs], :, pos % bs] != 7.0)
    # the same append into the real cache, then attention
    full = oracle.OracleCache(num_seqs=spec.num_seqs, q_tokens=T, n_q_heads=spec.n_q_heads,
                              n_kv_heads=spec.n_kv_heads, head_dim=spec.head_dim, block_size=bs,
                              k_pool=base.k_pool, v_pool=base.v_pool, block_table=w.block_table,
                              seq_lens=sl, cache_dtype=oracle.ORACLE_F64, q_lens=q_lens)
    assert np.array_equal(full.rope_append_kv(w.q, w.k, w.v, spec.rope_base), q_rot)
    out, lse = full.decode_attention(q_rot, want_lse=True)
    assert np.all(np.isfinite(out))
    for b in range(spec.num_seqs):
        n = int(q_lens[b])
        assert np.all(out[b, n:] == 0.0) and np.all(np.isneginf(lse[b, n:]))
        if n == 0:
            continue
        one = oracle.OracleCache(num_seqs=1, q_tokens=n, n_q_heads=spec.n_q_heads,
                                 n_kv_heads=spec.n_kv_heads, head_dim=spec.head_dim, block_size=bs,
                                 k_pool=full.k_pool, v_pool=full.v_pool,
                                 block_table=np.ascontiguousarray(w.block_table[b:b + 1]),
                                 seq_lens=sl[b:b + 1], cache_dtype=oracle.ORACLE_F64)
        o1, l1 = one.decode_attention(np.ascontiguousarray(q_rot[b:b + 1, :n]), want_lse=True)
        assert np.array_equal(out[b, :n], o1[0]) and np.array_equal(lse[b, :n], l1[0])


def check_rows_api():
    w, oc = _tiny_cache(B=3, T=2, L=(3, 40), seed=13)
    q = w.q.astype(np.float64)
    out, lse = oc.decode_attention(q, want_lse=True)
    rows = np.array([0, 5, 7, 11], np.int64)
    o2, l2 = oc.decode_attention_rows(q, rows)
    assert np.array_equal(o2, out.reshape(-1, w.spec.head_dim)[rows])
    assert np.array_equal(l2, lse.reshape(-1)[rows])


ALL_CHECKS = [v for k, v in sorted(globals().items()) if k.startswith("check_")]
