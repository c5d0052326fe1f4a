"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

* The append is bit-exact: the whole K and V pools after the step equal the
  oracle's, bit for bit (the poisoned tail slots and spare blocks included).
* q_rot is the fp64 rotation rounded once to fp32.
* Attention: fp32 caches within 1e-5 max-abs, bf16 caches (fp32 accumulate)
  within 2e-3 normwise relative (max|gpu - ref| / max|ref|).
Small variants of the five configurations and the full configurations (in
the launch configuration the benchmark times) are checked on every row.
"""
import zlib

import numpy as np
import pytest
import torch

from full_recompute import recompute_last_rows
from gpu_common import (GpuCase, assert_parity, assert_qrot, cached_workload, note, oracle_step,
                        rel_err)
from helpers import oracle_cache
from kv_cached_decode_amd import binding as kb
from kv_cached_decode_amd import workloads

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="no GPU")

SMALL = [workloads.small_variant(n) for n in workloads.CONFIG_ORDER[1:]]
FULL = [workloads.CONFIGS[n] for n in workloads.CONFIG_ORDER[1:]]


@needs_gpu
@pytest.mark.parametrize("spec", SMALL, ids=lambda s: s.name)
def test_small_configs_all_rows(spec):
    w = cached_workload(spec)
    note("small", spec.name)
    case = GpuCase(w)
    q_gpu, out_gpu = case.step()
    kp, vp = case.pools()
    q_ref, out_ref, kp_ref, vp_ref = oracle_step(w)
    assert np.array_equal(kp, kp_ref), "K pool differs from the oracle's after the append"
    assert np.array_equal(vp, vp_ref), "V pool differs from the oracle's after the append"
    assert_qrot(q_gpu, q_ref)
    e = assert_parity(spec, out_gpu, out_ref, label=f"two_calls/{spec.name}")
    print(f"{spec.name}: error {e:.3e}")


@needs_gpu
@pytest.mark.parametrize("spec", FULL, ids=lambda s: s.name)
def test_full_configs_all_rows(spec):
    """The full configurations in the launch configuration the benchmark
    times (the automatic plan), every output row against the oracle."""
    w = cached_workload(spec)
    case = GpuCase(w)
    note("full", spec.name, "plan", kb.decode_attention_plan(case.kv))
    q_gpu, out_gpu = case.step()
    kp, vp = case.pools()
    q_ref, out_ref, kp_ref, vp_ref = oracle_step(w)
    assert np.array_equal(kp, kp_ref), "K pool differs from the oracle's after the append"
    assert np.array_equal(vp, vp_ref), "V pool differs from the oracle's after the append"
    assert_qrot(q_gpu, q_ref)
    e = assert_parity(spec, out_gpu, out_ref, label=f"two_calls/{spec.name}")
    print(f"{spec.name}: error {e:.3e} on every row")


@needs_gpu
@pytest.mark.parametrize("name", ["llama3_8b", "qwen3_0_6b_cb", "long_ctx", "llama2_7b_mha"])
def test_valu_kernel_full_configs(name):
    """The vector-ALU kernel (the family of fp32 caches and head dims other
    than 128) forced onto the full bf16 configurations, as its profiles time
    it, with its own automatic split plan: every output row against the
    oracle."""
    spec = workloads.CONFIGS[name]
    w = cached_workload(spec)
    case = GpuCase(w)
    note("valu full", name, "plan", kb.decode_attention_plan(case.kv, kernel=kb.KVD_KERNEL_VALU))
    _, out = case.step(kernel=kb.KVD_KERNEL_VALU)
    _, ref, _, _ = oracle_step(w)
    e = assert_parity(spec, out, ref, label=f"valu_full/{name}")
    print(f"{name} (vector ALU): error {e:.3e} on every row")


@needs_gpu
def test_tiny_config_append_chain():
    """Tiny fp32 configuration: 32 GPU appends at positions 0..31, then the
    decode step at position 32; pools and output against the oracle's chain and
    the output against the full non-cached recompute."""
    w = workloads.make_workload(workloads.CONFIGS["tiny_f32"])
    s = w.spec
    note("tiny chain")
    case = GpuCase(w)
    oc_k, oc_v = w.k_pool.copy(), w.v_pool.copy()
    for p in range(33):
        sl = np.array([p + 1], np.int32)
        case.seq_lens.copy_(torch.from_numpy(sl))
        case.kv.max_seq_len = p + 1
        case.q.copy_(torch.from_numpy(np.ascontiguousarray(w.prefix_q[:, p:p + 1])))
        case.k.copy_(torch.from_numpy(np.ascontiguousarray(w.prefix_k[:, p:p + 1])))
        case.v.copy_(torch.from_numpy(np.ascontiguousarray(w.prefix_v[:, p:p + 1])))
        q_gpu, out_gpu = case.step()
        oc = oracle_cache(w, seq_lens=sl, k_pool=oc_k, v_pool=oc_v)
        q_ref = oc.rope_append_kv(np.ascontiguousarray(w.prefix_q[:, p:p + 1]),
                                  np.ascontiguousarray(w.prefix_k[:, p:p + 1]),
                                  np.ascontiguousarray(w.prefix_v[:, p:p + 1]), s.rope_base)
        out_ref = oc.decode_attention(q_ref)
        oc_k, oc_v = oc.k_pool, oc.v_pool
        kp, vp = case.pools()
        assert np.array_equal(kp.view(np.uint32), oc_k.view(np.uint32)), p
        assert np.array_equal(vp.view(np.uint32), oc_v.view(np.uint32)), p
        assert_parity(s, out_gpu, out_ref)
    store = lambda a: a.astype(np.float32).astype(np.float64)  # noqa: E731
    ref, _ = recompute_last_rows(w.prefix_q[0], w.prefix_k[0], w.prefix_v[0], 1, s.rope_base,
                                 s.layout, store)
    assert np.max(np.abs(out_gpu[0] - ref)) <= 1e-5


@needs_gpu
@pytest.mark.parametrize("splits", [1, 2, 3, 5, 8, 1000])
def test_split_count_does_not_change_the_result(splits):
    spec = workloads.small_variant("llama3_8b")
    w = cached_workload(spec)
    note("splits", splits)
    case = GpuCase(w)
    _, out_auto = case.step()
    q_rot = kb.rope_append_kv(case.kv, case.q, case.k, case.v, rope_base=spec.rope_base)
    out = case.attention(q_rot, num_splits=splits)
    again = case.attention(q_rot, num_splits=splits)
    assert np.array_equal(out, again), "not deterministic for a fixed plan"
    q_ref, out_ref, _, _ = oracle_step(w)
    assert_parity(spec, out, out_ref)
    assert rel_err(out, out_auto) < 1e-5


@needs_gpu
@pytest.mark.parametrize("D,dtype", [(16, "f32"), (32, "bf16"), (64, "f32"), (256, "bf16")])
def test_split_merge_every_head_dim(D, dtype):
    """Three splits merged at every head dim (the merge lays D/4 threads on a
    row, 256/(D/4) rows a workgroup, the last one partly filled)."""
    spec = workloads.Spec(f"splits_d{D}", 3, 2, 8, 2, D, 16, dtype, (100, 900), 10000.0, "normal",
                          "shuffled", spare_frac=0.1, seed=D)
    w = cached_workload(spec)
    note("split merge", D, dtype)
    case = GpuCase(w)
    q_rot = kb.rope_append_kv(case.kv, case.q, case.k, case.v, rope_base=spec.rope_base)
    out = case.attention(q_rot, num_splits=3)
    _, out_ref, _, _ = oracle_step(w)
    assert_parity(spec, out, out_ref)


@needs_gpu
@pytest.mark.parametrize("D,dtype,layout,Hq,Hkv", [(128, "bf16", 1, 32, 8), (64, "f32", 1, 64, 8),
                                                  (16, "bf16", 0, 8, 2), (256, "f32", 0, 16, 4)])
def test_rope_append_many_tokens(D, dtype, layout, Hq, Hkv):
    """RoPE + append of 600 tokens (several head rounds a workgroup) in both
    pairings and every head dim: the pools bit for bit and q_rot within one
    fp32 rounding of the oracle."""
    spec = workloads.Spec(f"rope_many_d{D}", 3, 200, Hq, Hkv, D, 16, dtype, (0, 300), 500000.0, "normal",
                          "shuffled", spare_frac=0.1, seed=D + layout, layout=layout)
    w = cached_workload(spec)
    note("rope many tokens", D, dtype, layout)
    case = GpuCase(w)
    q_rot = kb.rope_append_kv(case.kv, case.q, case.k, case.v, rope_base=spec.rope_base, layout=layout)
    torch.cuda.synchronize()
    kp, vp = case.pools()
    oc = oracle_cache(w)
    q_ref = oc.rope_append_kv(w.q, w.k, w.v, spec.rope_base, layout)
    assert np.array_equal(kp.view(np.uint8), oc.k_pool.view(np.uint8)), "K pool differs"
    assert np.array_equal(vp.view(np.uint8), oc.v_pool.view(np.uint8)), "V pool differs"
    assert_qrot(q_rot.cpu().numpy(), q_ref)


EDGE = [
    # name, B, T, Hq, Hkv, D, bs, dtype, ctx, layout
    ("single_key", 3, 1, 8, 2, 128, 16, "bf16", 0, 0),
    ("draft_only", 2, 4, 8, 2, 128, 16, "bf16", 0, 0),
    ("block_size_1", 2, 1, 4, 2, 64, 1, "bf16", (1, 300), 0),
    ("block_size_1024", 2, 2, 4, 1, 128, 1024, "bf16", (1000, 3000), 0),
    ("d16_bf16", 2, 1, 4, 4, 16, 16, "bf16", (5, 900), 1),
    ("d32_f32", 2, 1, 4, 2, 32, 8, "f32", (5, 900), 0),
    ("d64_f32", 3, 2, 6, 3, 64, 32, "f32", (5, 700), 1),
    ("d128_f32", 2, 1, 8, 2, 128, 16, "f32", (100, 1500), 0),
    ("d256_bf16", 2, 1, 4, 2, 256, 16, "bf16", (100, 1500), 0),
    ("d256_f32", 2, 3, 4, 2, 256, 16, "f32", (10, 600), 0),
    ("many_rows_g16", 2, 1, 32, 2, 128, 16, "bf16", (10, 2000), 0),
    ("verify_t8", 2, 8, 8, 4, 128, 16, "bf16", (0, 900), 0),
    ("verify_t16_f32", 1, 16, 4, 4, 64, 16, "f32", 333, 1),
    ("interleaved", 3, 1, 8, 8, 128, 64, "bf16", (1, 2000), 1),
    # the largest chunk a step takes (T = 1024): 4096 and 1024 query rows per kv head
    ("chunk_t1024_g4", 1, 1024, 32, 8, 128, 16, "bf16", (0, 200), 0),
    ("chunk_t1024_mha", 2, 1024, 4, 4, 128, 64, "bf16", (10, 300), 1),
    # large blocks through each kernel: matrix-core decode with splits, the
    # prefill kernel (block ids staged per split), the vector-ALU kernel
    ("decode_bs_128", 4, 1, 32, 8, 128, 128, "bf16", (1000, 9000), 0),
    ("prefill_bs_256", 2, 40, 8, 2, 128, 256, "bf16", (100, 2500), 0),
    ("prefill_bs_1024", 1, 24, 16, 4, 128, 1024, "bf16", (2000, 5000), 1),
    ("valu_bs_512_f32", 2, 1, 8, 2, 128, 512, "f32", (100, 3000), 1),
]


@needs_gpu
@pytest.mark.parametrize("case_", EDGE, ids=lambda c: c[0])
def test_edge_cases(case_):
    name, B, T, Hq, Hkv, D, bs, dtype, ctx, layout = case_
    spec = workloads.Spec(name, B, T, Hq, Hkv, D, bs, dtype, ctx, 10000.0, "normal", "shuffled",
                          spare_frac=0.2, seed=zlib.crc32(name.encode()) % 1000, layout=layout)
    w = workloads.make_workload(spec)
    note("edge", name)
    case = GpuCase(w)
    q_gpu, out_gpu = case.step()
    kp, vp = case.pools()
    q_ref, out_ref, kp_ref, vp_ref = oracle_step(w)
    assert np.array_equal(kp.view(np.uint16), kp_ref.view(np.uint16))
    assert np.array_equal(vp.view(np.uint16), vp_ref.view(np.uint16))
    assert_qrot(q_gpu, q_ref)
    assert_parity(spec, out_gpu, out_ref)


@needs_gpu
def test_custom_softmax_scale():
    spec = workloads.small_variant("qwen3_0_6b_cb")
    w = cached_workload(spec)
    note("scale")
    case = GpuCase(w)
    _, out = case.step(scale=0.37)
    _, ref, _, _ = oracle_step(w, scale=0.37)
    assert_parity(spec, out, ref)


@needs_gpu
def test_empty_batch():
    note("empty batch")
    k = torch.zeros((4, 2, 16, 128), dtype=torch.bfloat16, device="cuda")
    kv = kb.PagedKV(k, k.clone(), torch.zeros((0, 4), dtype=torch.int32, device="cuda"),
                    torch.zeros((0,), dtype=torch.int32, device="cuda"), 4, 1, 1)
    q = torch.zeros((0, 1, 4, 128), device="cuda")
    kv_in = torch.zeros((0, 1, 2, 128), device="cuda")
    kb.rope_append_kv(kv, q, kv_in, kv_in)
    out = kb.decode_attention(kv, q)
    torch.cuda.synchronize()
    assert out.shape == (0, 1, 4, 128)


FAMILY_CASES = [(n, k) for n in ["llama3_8b", "qwen3_0_6b_cb", "long_ctx", "mtp_verify"]
                for k in (kb.KVD_KERNEL_VALU, kb.KVD_KERNEL_MFMA)]


@needs_gpu
@pytest.mark.parametrize("name,kernel", FAMILY_CASES,
                         ids=[f"{n}-{'valu' if k == 1 else 'mfma'}" for n, k in FAMILY_CASES])
def test_each_kernel_family(name, kernel):
    """Both attention kernels (vector ALU and matrix core) against the oracle
    on every small configuration, whichever the planner would pick."""
    spec = workloads.small_variant(name)
    w = cached_workload(spec)
    note("family", name, kernel)
    case = GpuCase(w)
    _, out = case.step(kernel=kernel)
    _, ref, _, _ = oracle_step(w)
    e = assert_parity(spec, out, ref)
    print(f"{name} kernel {kernel}: error {e:.3e}")


@needs_gpu
def test_one_workspace_across_shapes():
    """One workspace, its counter head zeroed once and the rest garbage,
    serves calls of any shape, split count and kernel in turn; repeated
    calls give identical results (the counters return to zero after every
    call and the partials are rewritten before they are read)."""
    ws = torch.full((64 << 20,), 0x7F, dtype=torch.uint8, device="cuda")
    ws[:kb.WORKSPACE_COUNTER_BYTES].zero_()
    cases = []
    for name, kernel, splits in [("llama3_8b", 2, 3), ("qwen3_0_6b_cb", 2, 4), ("llama3_8b", 1, 5),
                                 ("mtp_verify", 2, 6), ("llama3_8b", 2, 3), ("chunked_prefill", 2, 2),
                                 ("qwen3_0_6b_cb", 2, 2)]:
        spec = workloads.small_variant(name)
        w = cached_workload(spec)
        case = GpuCase(w)
        q_rot = kb.rope_append_kv(case.kv, case.q, case.k, case.v, rope_base=spec.rope_base)
        need = kb.decode_attention_workspace_size(case.kv, splits, kernel)
        assert 0 < need <= ws.numel()
        note("workspace reuse", name, kernel, splits)
        outs = []
        for _ in range(3):
            out = kb.decode_attention(case.kv, q_rot, workspace_buf=ws, num_splits=splits, kernel=kernel)
            torch.cuda.synchronize()
            outs.append(out.cpu().numpy())
        assert all(np.array_equal(outs[0], o) for o in outs[1:])
        cases.append((spec, w, outs[0]))
    for spec, w, out in cases:
        _, ref, _, _ = oracle_step(w)
        assert_parity(spec, out, ref)


@needs_gpu
@pytest.mark.parametrize("name", ["llama3_8b", "mtp_verify", "valu_f32"])
def test_step_replays_under_hip_graph_capture(name):
    """The whole step (RoPE+append, attention, split merge) captured in a HIP
    graph: every replay, with eager work and synchronisations in between,
    matches the eager result bit for bit."""
    if name == "valu_f32":
        spec = workloads.Spec("graph_valu_f32", 3, 2, 8, 2, 64, 16, "f32", (600, 5000), 10000.0,
                              "normal", "shuffled", spare_frac=0.1, seed=77)
        w = workloads.make_workload(spec)
        assert kb.decode_attention_plan(GpuCase(w).kv)[0] > 1, "want a split plan"
    else:
        spec = workloads.small_variant(name)
        w = cached_workload(spec)
    note("graph", name)
    case = GpuCase(w)
    q_rot = torch.empty_like(case.q)
    out = torch.empty_like(case.q)
    ws = kb.workspace(case.kv)
    ws = ws.clone() if ws is not None else None

    def step():
        kb.rope_append_kv(case.kv, case.q, case.k, case.v, q_rot, rope_base=spec.rope_base,
                          layout=spec.layout)
        kb.decode_attention(case.kv, q_rot, out, workspace_buf=ws)

    step()
    torch.cuda.synchronize()
    eager = out.cpu().numpy().copy()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    torch.cuda.synchronize()
    for i in range(4):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), eager), f"replay {i} differs from eager"
        step()                       # eager work between replays
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), eager)


WINDOW_CASES = [("llama3_8b", 256), ("qwen3_0_6b_cb", 100), ("mtp_verify", 64), ("long_ctx", 4096),
                ("llama3_8b", 1), ("qwen3_0_6b_cb", 100000)]


@needs_gpu
@pytest.mark.parametrize("name,window", WINDOW_CASES, ids=[f"{n}-w{w}" for n, w in WINDOW_CASES])
@pytest.mark.parametrize("kernel", [kb.KVD_KERNEL_VALU, kb.KVD_KERNEL_MFMA], ids=["valu", "mfma"])
def test_sliding_window(name, window, kernel):
    """Sliding-window attention (the query at position p sees keys
    p-W+1 .. p) against the oracle, both kernel families."""
    spec = workloads.small_variant(name)
    w = cached_workload(spec)
    note("window", name, window, kernel)
    case = GpuCase(w, window=window)
    _, out = case.step(kernel=kernel)
    _, ref, _, _ = oracle_step(w, window=window)
    assert_parity(spec, out, ref)


@needs_gpu
def test_shared_prefix_blocks():
    """Sequences whose tables point at the same physical blocks for a common
    prefix (prefix caching): reads are shared, each append lands in the
    sequence's own last block."""
    spec = workloads.Spec("shared_prefix", 6, 2, 8, 2, 128, 16, "bf16", (200, 900), 10000.0,
                          "normal", "shuffled", spare_frac=0.1, seed=31)
    w = workloads.make_workload(spec)
    shared = 10                      # 160 keys, below every context
    table = w.block_table.copy()
    table[1:, :shared] = table[0, :shared]
    note("shared prefix")
    case = GpuCase(w, block_table=table)
    _, out = case.step()
    kp, vp = case.pools()
    _, ref, kp_ref, vp_ref = oracle_step(w, block_table=table)
    assert np.array_equal(kp, kp_ref) and np.array_equal(vp, vp_ref)
    assert_parity(spec, out, ref)


@needs_gpu
def test_rollback_after_verify():
    """Verify a 4-token draft, accept 2, roll back by lowering seq_lens, then
    decode the next token into the rejected slot (the ferrox `engine` cache
    truncate, done here by the caller's seq_lens alone)."""
    spec = workloads.Spec("rollback", 4, 4, 16, 4, 128, 16, "bf16", (50, 700), 10000.0, "normal",
                          "shuffled", spare_frac=0.1, seed=41)
    w = workloads.make_workload(spec)
    note("rollback")
    case = GpuCase(w)
    case.step()                                   # verify: appends 4 draft tokens
    oc = oracle_cache(w)
    oc.rope_append_kv(w.q, w.k, w.v, spec.rope_base)
    # accept 2 drafts: the next token goes to position ctx + 2
    sl = (w.ctx_lens + 3).astype(np.int32)
    rng = np.random.default_rng(7)
    q1 = rng.standard_normal((spec.num_seqs, 1, spec.n_q_heads, spec.head_dim), dtype=np.float32)
    k1 = rng.standard_normal((spec.num_seqs, 1, spec.n_kv_heads, spec.head_dim), dtype=np.float32)
    v1 = rng.standard_normal((spec.num_seqs, 1, spec.n_kv_heads, spec.head_dim), dtype=np.float32)
    kv1 = kb.PagedKV(case.k_cache, case.v_cache, case.table, torch.from_numpy(sl).cuda(),
                     spec.n_q_heads, 1, int(sl.max()))
    q_rot = kb.rope_append_kv(kv1, torch.from_numpy(q1).cuda(), torch.from_numpy(k1).cuda(),
                              torch.from_numpy(v1).cuda(), rope_base=spec.rope_base)
    out = kb.decode_attention(kv1, q_rot).cpu().numpy()
    oc1 = oracle_cache(w, seq_lens=sl, q_tokens=1, k_pool=oc.k_pool, v_pool=oc.v_pool)
    ref = oc1.decode_attention(oc1.rope_append_kv(q1, k1, v1, spec.rope_base))
    kp, vp = case.pools()
    assert np.array_equal(kp, oc1.k_pool) and np.array_equal(vp, oc1.v_pool)
    assert_parity(spec, out, ref)
