"""GPU: context-parallel partial export and merge (CP/DCP, one of the
parallel modes of the ferrite page).  Each sequence's cache is cut into
contiguous key ranges (shards); the shard holding the tail appends the new
tokens, every shard exports (out, lse) over its keys, and the merge of the
partials must equal attention over the whole cache.  One GPU plays every
shard here: the shards share the physical pools and see them through their
own block tables and positions, as separate GPUs would see their own pools.

Tolerances: outputs as everywhere (bf16 caches 2e-3 normwise relative, fp32
caches 1e-5 max-abs).  lse follows the largest score, which carries the
relative error of the query as the matrix cores see it (a bf16 hi + lo pair,
about 16 significant bits, so 2^-16 ~ 1.5e-5 relative) plus fp32
accumulation: |lse - ref| <= 1e-4 + 3e-5 |ref|, and exactly -inf where a row
sees none of a shard's keys."""
import numpy as np
import pytest
import torch

from gpu_common import DEV, GpuCase, assert_parity, cached_workload, check_table, note
from helpers import oracle_cache
from kv_cached_decode_amd import binding as kb
from kv_cached_decode_amd import workloads

pytestmark = pytest.mark.gpu

def lse_ok(got, ref):
    return bool(np.all(np.abs(got - ref) <= 1e-4 + 3e-5 * np.abs(ref)))


def shard_cuts(w, P, seed):
    """[B][P+1] block-aligned cut points 0 = c_0 <= ... <= c_P = seq_len, with
    some empty shards; every cut lies at or before the first new token."""
    s = w.spec
    bs = s.block_size
    rng = np.random.default_rng(seed)
    L = w.seq_lens.astype(np.int64)
    cuts = np.zeros((s.num_seqs, P + 1), np.int64)
    for b in range(s.num_seqs):
        # the new tokens stay in the tail shard: no cut inside the last T keys
        top = (L[b] - s.q_tokens) // bs
        inner = np.sort(rng.integers(0, top + 1, size=P - 1)) * bs
        cuts[b, 1:P] = inner
        cuts[b, P] = L[b]
    cuts[0, 1:P] = 0                     # sequence 0: everything in the tail shard
    return cuts


def shard_kv(case, cuts, k, window=0):
    """The PagedKV of shard k: keys cuts[:, k] .. cuts[:, k+1] of each
    sequence, through a table that starts at the shard's first block."""
    w = case.w
    s = w.spec
    bs = s.block_size
    table = np.full_like(w.block_table, -1)
    for b in range(s.num_seqs):
        first = int(cuts[b, k]) // bs
        row = w.block_table[b, first:]
        table[b, :row.size] = row
    n = (cuts[:, k + 1] - cuts[:, k]).astype(np.int32)
    check_table(table, n, bs, w.num_blocks)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(DEV)  # noqa: E731
    return kb.PagedKV(case.k_cache, case.v_cache, t(table), t(n), s.n_q_heads, s.q_tokens,
                      max(1, int(n.max())), window, key_pos0=t(cuts[:, k]),
                      q_pos=t(w.seq_lens.astype(np.int64) - s.q_tokens)), table, n


def run_shards(case, cuts, kernel, window=0):
    """Tail-shard append, every shard's partial, then the merge.  Returns
    (q_rot, outs, lses, merged, merged_lse, shard tables and lengths)."""
    s = case.w.spec
    P = cuts.shape[1] - 1
    kvs = [shard_kv(case, cuts, k, window) for k in range(P)]
    q_rot = kb.rope_append_kv(kvs[-1][0], case.q, case.k, case.v, rope_base=s.rope_base, layout=s.layout)
    parts = [kb.decode_attention_lse(kv, q_rot, kernel=kernel) for kv, _, _ in kvs]
    outs = torch.stack([o for o, _ in parts])
    lses = torch.stack([l_ for _, l_ in parts])
    merged, mlse = kb.merge_partials(outs, lses)
    torch.cuda.synchronize()
    return (q_rot.cpu().numpy(), outs.cpu().numpy(), lses.cpu().numpy(), merged.cpu().numpy(),
            mlse.cpu().numpy(), [(t, n) for _, t, n in kvs])


CASES = [("llama3_8b", 3, 0, kb.KVD_KERNEL_MFMA), ("mtp_verify", 3, 0, kb.KVD_KERNEL_MFMA),
         ("qwen3_0_6b_cb", 4, 0, kb.KVD_KERNEL_AUTO), ("mtp_verify", 3, 64, kb.KVD_KERNEL_MFMA),
         ("llama3_8b", 2, 0, kb.KVD_KERNEL_VALU), ("long_ctx", 5, 1000, kb.KVD_KERNEL_AUTO)]


@pytest.mark.parametrize("name,P,window,kernel", CASES,
                         ids=[f"{n}-P{p}-w{w}-k{k}" for n, p, w, k in CASES])
def test_shards_merge_to_whole_cache(name, P, window, kernel):
    check_shards(workloads.small_variant(name), P, window, kernel)


@pytest.mark.parametrize("window", [0, 64])
def test_prefill_shards_merge_to_whole_cache(window):
    """A chunk of 40 new tokens per sequence (160 query rows per kv head: the
    prefill kernel) cut into 3 shards, the same checks."""
    check_shards(CP_PREFILL, 3, window, kb.KVD_KERNEL_AUTO)


def check_shards(spec, P, window, kernel):
    w = cached_workload(spec)
    note("context parallel", spec.name, P, window, kernel)
    case = GpuCase(w, window=window)
    cuts = shard_cuts(w, P, seed=P + window)
    q_rot, outs, lses, merged, mlse, shards = run_shards(case, cuts, kernel, window)

    # the tail shard's append lands in the same physical slots, bit for bit
    oc = oracle_cache(w, window=window)
    q_ref = oc.rope_append_kv(w.q, w.k, w.v, spec.rope_base, spec.layout)
    kp, vp = case.pools()
    assert np.array_equal(kp, oc.k_pool) and np.array_equal(vp, oc.v_pool)
    assert np.max(np.abs(q_rot - q_ref) / (np.abs(q_ref) + 1e-30)) <= 2.0 ** -23

    # the merge equals the whole cache
    out_ref, lse_ref = oc.decode_attention(q_ref, want_lse=True)
    assert_parity(spec, merged, out_ref)
    assert lse_ok(mlse, lse_ref), np.max(np.abs(mlse - lse_ref))

    # every shard's partial equals the oracle's shard
    for k, (table, n) in enumerate(shards):
        sh_oc = oracle_cache(w, seq_lens=n, block_table=table.clip(min=0), k_pool=oc.k_pool,
                             v_pool=oc.v_pool, window=window, key_pos0=cuts[:, k],
                             q_pos=w.seq_lens.astype(np.int64) - spec.q_tokens)
        o_ref, l_ref = sh_oc.decode_attention(q_ref, want_lse=True)
        empty = np.isneginf(l_ref)
        assert np.array_equal(np.isneginf(lses[k]), empty), f"shard {k}: empty rows differ"
        assert np.all(outs[k][empty] == 0.0)
        if (~empty).any():
            assert lse_ok(lses[k][~empty], l_ref[~empty])
            assert_parity(spec, outs[k][~empty], o_ref[~empty])


def test_merge_of_one_part_is_identity_and_all_empty_rows_are_zero():
    note("merge identity")
    g = torch.Generator(device="cpu").manual_seed(3)
    o = torch.randn(1, 40, 128, generator=g).to(DEV)
    l_ = torch.randn(1, 40, generator=g).to(DEV)
    l_[0, 5] = float("-inf")
    o[0, 5] = 0.0
    out, lse = kb.merge_partials(o, l_)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), o[0].cpu()) or torch.allclose(out.cpu(), o[0].cpu(), rtol=0, atol=0)
    assert torch.equal(lse.cpu(), l_[0].cpu())
    # two parts where both are empty for a row: out 0, lse -inf
    o2 = torch.stack([o[0], o[0]])
    l2 = torch.stack([l_[0], l_[0]])
    out2, lse2 = kb.merge_partials(o2, l2)
    torch.cuda.synchronize()
    assert torch.all(out2[5].cpu() == 0.0) and torch.isneginf(lse2[5].cpu())
    # equal parts: same output, lse + log 2
    assert torch.allclose(out2.cpu(), o[0].cpu(), rtol=1e-6, atol=1e-6)
    fin = torch.isfinite(l_[0]).cpu()
    assert torch.allclose(lse2.cpu()[fin], (l_[0].cpu() + np.log(2.0))[fin], rtol=0, atol=1e-5)


@pytest.mark.parametrize("P", [8, 12])
def test_merge_of_many_parts(P):
    """Eight parts (each thread loads every part at once) and twelve (weights
    formed in LDS first), with rows some parts did not see (lse -inf, output
    0) and one row no part saw: the merge formula in fp64."""
    note("merge parts", P)
    rng = np.random.default_rng(40 + P)
    rows, D = 57, 128
    o = rng.standard_normal((P, rows, D)).astype(np.float32)
    lse = (rng.standard_normal((P, rows)) * 3.0).astype(np.float32)
    empty = rng.random((P, rows)) < 0.25
    empty[:, 7] = True
    lse[empty] = -np.inf
    o[empty] = 0.0
    out, mlse = kb.merge_partials(torch.from_numpy(o).to(DEV), torch.from_numpy(lse).to(DEV))
    torch.cuda.synchronize()
    out, mlse = out.cpu().numpy(), mlse.cpu().numpy()
    l64 = lse.astype(np.float64)
    M = l64.max(axis=0)
    live = np.isfinite(M)
    w = np.where(live[None, :], np.exp(l64 - np.where(live, M, 0.0)[None, :]), 0.0)
    S = w.sum(axis=0)
    ref = np.einsum("pr,prd->rd", w, o.astype(np.float64)) / np.where(S > 0, S, 1.0)[:, None]
    assert np.all(out[~live] == 0.0) and np.all(np.isneginf(mlse[~live]))
    assert np.max(np.abs(out[live] - ref[live])) <= 1e-5 * np.max(np.abs(ref[live]))
    assert np.max(np.abs(mlse[live] - (M + np.log(np.where(S > 0, S, 1.0)))[live])) <= 1e-5


CP_PREFILL = workloads.Spec("cp_prefill", 3, 40, 32, 8, 128, 16, "bf16", (100, 500), 10000.0, "normal",
                            "shuffled", spare_frac=0.1, seed=83)


@pytest.mark.parametrize("sp,kernel", [(workloads.small_variant("mtp_verify"), kb.KVD_KERNEL_AUTO),
                                       (workloads.small_variant("llama3_8b"), kb.KVD_KERNEL_VALU),
                                       (CP_PREFILL, kb.KVD_KERNEL_AUTO)],
                         ids=["mtp_verify", "llama3_8b-valu", "prefill"])
def test_every_shard_runs_the_whole_step(sp, kernel):
    """Each shard calls kvd_decode_step with the same new tokens, as every GPU
    of a context-parallel group would: the shards that do not hold the new
    tokens rotate the queries and store nothing, the tail shard appends, so
    the pools end exactly as the oracle's whole-cache append leaves them, and
    each shard's output is its partial over the keys it holds."""
    spec = sp
    w = cached_workload(spec)
    note("every shard steps", spec.name, kernel)
    case = GpuCase(w)
    P = 3
    cuts = shard_cuts(w, P, seed=11)
    kvs = [shard_kv(case, cuts, k) for k in range(P)]
    oc = oracle_cache(w)
    q_ref = oc.rope_append_kv(w.q, w.k, w.v, spec.rope_base, spec.layout)
    for k, (kv, table, n) in enumerate(kvs):
        out, q_rot = kb.decode_step(kv, case.q, case.k, case.v, q_rot=torch.zeros_like(case.q),
                                    rope_base=spec.rope_base, layout=spec.layout, kernel=kernel)
        torch.cuda.synchronize()
        q_rot = q_rot.cpu().numpy()
        assert np.max(np.abs(q_rot - q_ref) / (np.abs(q_ref) + 1e-30)) <= 2.0 ** -23, k
        sh_oc = oracle_cache(w, seq_lens=n, block_table=table.clip(min=0), k_pool=oc.k_pool,
                             v_pool=oc.v_pool, key_pos0=cuts[:, k],
                             q_pos=w.seq_lens.astype(np.int64) - spec.q_tokens)
        o_ref, l_ref = sh_oc.decode_attention(q_ref, want_lse=True)
        out = out.cpu().numpy()
        empty = np.isneginf(l_ref)
        assert np.all(out[empty] == 0.0)
        if (~empty).any():
            assert_parity(spec, out[~empty], o_ref[~empty])
    kp, vp = case.pools()
    assert np.array_equal(kp, oc.k_pool) and np.array_equal(vp, oc.v_pool)
