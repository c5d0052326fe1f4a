"""GPU: the fused decode step (kvd_decode_step) against the two calls it
replaces (kvd_rope_append_kv, then kvd_decode_attention) and against the
oracle.  With the same plan the two must agree bit for bit -- the output, the
rotated queries and both cache pools -- because the fused kernel performs the
same roundings; the oracle then bounds both."""
import dataclasses

import numpy as np
import pytest
import torch

from gpu_common import GpuCase, assert_parity, assert_qrot, cached_workload, note, oracle_step
from helpers import oracle_cache
from kv_cached_decode_amd import binding as kb
from kv_cached_decode_amd import workloads

pytestmark = pytest.mark.gpu


def two_calls(case, kernel=kb.KVD_KERNEL_AUTO, num_splits=0):
    s = case.w.spec
    q_rot = kb.rope_append_kv(case.kv, case.q, case.k, case.v, torch.zeros_like(case.q),
                              rope_base=s.rope_base, layout=s.layout)
    out = kb.decode_attention(case.kv, q_rot, kernel=kernel, num_splits=num_splits)
    torch.cuda.synchronize()
    return q_rot.cpu().numpy(), out.cpu().numpy()


def fused(case, kernel=kb.KVD_KERNEL_AUTO, num_splits=0, want_q_rot=True):
    s = case.w.spec
    res = kb.decode_step(case.kv, case.q, case.k, case.v,
                         q_rot=torch.zeros_like(case.q) if want_q_rot else None,
                         rope_base=s.rope_base, layout=s.layout, kernel=kernel,
                         num_splits=num_splits)
    torch.cuda.synchronize()
    if want_q_rot:
        return res[1].cpu().numpy(), res[0].cpu().numpy()
    return None, res.cpu().numpy()


def bits(a):
    """Bit patterns, so that the NaN-poisoned slots compare equal too."""
    return a.view(np.uint32) if a.dtype == np.float32 else a


def assert_same(a_case, b_case, a, b):
    assert np.array_equal(a[1], b[1]), "attention output differs"
    if a[0] is not None and b[0] is not None:
        assert np.array_equal(a[0], b[0]), "q_rot differs"
    ka, va = a_case.pools()
    kb_, vb = b_case.pools()
    assert np.array_equal(bits(ka), bits(kb_)), "K pool differs"
    assert np.array_equal(bits(va), bits(vb)), "V pool differs"


# the bf16 configurations (matrix-core plans: one fused kernel, or the
# prefill kernel after the RoPE/append kernel) and vector-ALU plans (the two
# kernels in a row): an fp32 cache, and a bf16 cache with one query row per
# kv head with the kernel family forced (the automatic plan takes the matrix
# cores there)
SPECS = [workloads.small_variant(n) for n in workloads.CONFIG_ORDER[1:]] + [
    workloads.Spec("valu_f32", 3, 2, 8, 2, 64, 16, "f32", (600, 5000), 10000.0, "normal", "shuffled",
                   spare_frac=0.1, seed=77),
    workloads.Spec("valu_mha_bf16", 4, 1, 8, 8, 128, 16, "bf16", (100, 3000), 10000.0, "normal",
                   "shuffled", spare_frac=0.1, seed=78),
    workloads.Spec("mfma_mha_bf16", 4, 1, 8, 8, 128, 16, "bf16", (100, 3000), 10000.0, "normal",
                   "shuffled", spare_frac=0.1, seed=78),
    # matrix-core plans with more than 256 new-key pairs per kv head (the
    # append's later rounds): 16 tokens at g = 1, 8 tokens at g = 2
    workloads.Spec("mha_t16", 3, 16, 8, 8, 128, 16, "bf16", (100, 900), 10000.0, "normal", "shuffled",
                   spare_frac=0.1, seed=79),
    workloads.Spec("g2_t8", 3, 8, 16, 8, 128, 16, "bf16", (50, 700), 500000.0, "normal_scaled",
                   "shuffled", spare_frac=0.1, seed=80, layout=1),
]


@pytest.mark.parametrize("spec", SPECS, ids=lambda s: s.name)
@pytest.mark.parametrize("want_q_rot", [True, False], ids=["q_rot", "no_q_rot"])
def test_fused_equals_two_calls_small(spec, want_q_rot):
    w = cached_workload(spec)
    kernel = kb.KVD_KERNEL_VALU if spec.name.startswith("valu") else kb.KVD_KERNEL_AUTO
    note("fused vs two calls", spec.name, want_q_rot, kernel)
    ref_case, case = GpuCase(w), GpuCase(w)
    ref = two_calls(ref_case, kernel=kernel)
    got = fused(case, kernel=kernel, want_q_rot=want_q_rot)
    assert_same(ref_case, case, ref, got)
    _, out_ref, _, _ = oracle_step(w)
    assert_parity(spec, got[1], out_ref)


@pytest.mark.parametrize("name", ["llama3_8b", "qwen3_0_6b_cb", "long_ctx", "mtp_verify",
                                  "chunked_prefill"])
def test_fused_equals_two_calls_full(name):
    """Full sizes, in the launch configuration the benchmark times (the step
    without a q_rot buffer where the plan is one fused kernel, as the
    benchmark calls it): bitwise equal to the two calls, and every output
    row and both whole pools against the oracle."""
    spec = workloads.CONFIGS[name]
    w = cached_workload(spec)
    note("fused full", name)
    ref_case = GpuCase(w)
    ref = two_calls(ref_case)
    ref_pools = ref_case.pools()
    del ref_case
    torch.cuda.empty_cache()
    case = GpuCase(w)
    got_q = fused(case)
    got = fused(GpuCase(w), want_q_rot=False) if name != "chunked_prefill" else got_q
    assert np.array_equal(ref[1], got_q[1]) and np.array_equal(ref[0], got_q[0])
    assert np.array_equal(ref[1], got[1])
    kp, vp = case.pools()
    assert np.array_equal(kp, ref_pools[0]) and np.array_equal(vp, ref_pools[1])
    q_ref, out_ref, kp_ref, vp_ref = oracle_step(w)
    assert np.array_equal(kp, kp_ref) and np.array_equal(vp, vp_ref)
    assert_qrot(got_q[0], q_ref)
    assert_parity(spec, got[1], out_ref, label=f"step/{name}")


def test_draft_split_across_workgroups():
    """Verify drafts whose new tokens straddle a split boundary: each part is
    appended by the workgroup that reads it, and nothing else changes.  Five
    splits of 121 keys over contexts of 600; four sequences are shortened so
    that a boundary falls 1, 2, 3 and 1 keys into their 4-token drafts
    (lowering a length only drops allocated slots)."""
    spec = workloads.small_variant("mtp_verify").with_(name="mtp_uniform600", ctx=600)
    w = cached_workload(spec)
    T = spec.q_tokens
    sl = np.array([604, 122, 244, 366, 485], np.int32)
    assert np.all(sl <= w.seq_lens)
    note("draft across splits")
    ref_case, case = GpuCase(w, seq_lens=sl), GpuCase(w, seq_lens=sl)
    n, keys, _ = kb.decode_attention_plan(case.kv, num_splits=5, kernel=kb.KVD_KERNEL_MFMA)
    assert (n, keys) == (5, 121)
    bounds = np.arange(1, n) * keys
    assert sum(bool(((L - T < bounds) & (bounds < L)).any()) for L in sl) == 4
    ref = two_calls(ref_case, kernel=kb.KVD_KERNEL_MFMA, num_splits=5)
    got = fused(case, kernel=kb.KVD_KERNEL_MFMA, num_splits=5)
    assert_same(ref_case, case, ref, got)
    oc = oracle_cache(w, seq_lens=sl)
    out_ref = oc.decode_attention(oc.rope_append_kv(w.q, w.k, w.v, spec.rope_base))
    kp, vp = case.pools()
    assert np.array_equal(kp, oc.k_pool) and np.array_equal(vp, oc.v_pool)
    assert_parity(spec, got[1], out_ref)


@pytest.mark.parametrize("name,window", [("mtp_verify", 3), ("mtp_verify", 64), ("llama3_8b", 200),
                                         ("qwen3_0_6b_cb", 50)])
def test_fused_with_window(name, window):
    spec = workloads.small_variant(name)
    w = cached_workload(spec)
    note("fused window", name, window)
    ref_case, case = GpuCase(w, window=window), GpuCase(w, window=window)
    ref = two_calls(ref_case, kernel=kb.KVD_KERNEL_MFMA)
    got = fused(case, kernel=kb.KVD_KERNEL_MFMA)
    assert_same(ref_case, case, ref, got)
    _, out_ref, _, _ = oracle_step(w, window=window)
    assert_parity(spec, got[1], out_ref)


@pytest.mark.parametrize("name", ["llama3_8b", "mtp_verify"])
def test_fused_interleaved_layout(name):
    spec = dataclasses.replace(workloads.small_variant(name), layout=1, name=name + "_il")
    w = workloads.make_workload(spec)
    note("fused interleaved", name)
    ref_case, case = GpuCase(w), GpuCase(w)
    ref = two_calls(ref_case)
    got = fused(case)
    assert_same(ref_case, case, ref, got)
    q_ref, out_ref, kp_ref, vp_ref = oracle_step(w)
    kp, vp = case.pools()
    assert np.array_equal(kp, kp_ref) and np.array_equal(vp, vp_ref)
    assert_qrot(got[0], q_ref)
    assert_parity(spec, got[1], out_ref)


@pytest.mark.parametrize("splits", [1, 2, 7])
def test_fused_split_counts(splits):
    spec = workloads.small_variant("llama3_8b")
    w = cached_workload(spec)
    note("fused splits", splits)
    ref_case, case = GpuCase(w), GpuCase(w)
    ref = two_calls(ref_case, num_splits=splits)
    got = fused(case, num_splits=splits)
    assert_same(ref_case, case, ref, got)


def test_fused_step_replays_under_hip_graph_capture():
    spec = workloads.small_variant("mtp_verify")
    w = cached_workload(spec)
    note("fused graph")
    case = GpuCase(w)
    out = torch.empty_like(case.q)
    q_rot = torch.empty_like(case.q)
    ws = kb.workspace(case.kv)
    ws = ws.clone() if ws is not None else None

    def step():
        kb.decode_step(case.kv, case.q, case.k, case.v, out=out, q_rot=q_rot, rope_base=spec.rope_base,
                       workspace_buf=ws)

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
        step()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), eager)


def test_split_longer_than_one_piece():
    """One split of more cache blocks than the fused kernel stages at a time
    (2048): the step runs as the two kernels in a row and stays correct."""
    spec = workloads.Spec("one_long_split", 1, 1, 8, 2, 128, 16, "bf16", 33000, 10000.0, "normal",
                          "shuffled", spare_frac=0.05, seed=81)
    w = cached_workload(spec)
    note("split longer than one piece")
    ref_case, case = GpuCase(w), GpuCase(w)
    n, keys, _ = kb.decode_attention_plan(case.kv, num_splits=1, kernel=kb.KVD_KERNEL_MFMA)
    assert n == 1 and (keys + 15) // 16 > 2048
    ref = two_calls(ref_case, kernel=kb.KVD_KERNEL_MFMA, num_splits=1)
    got = fused(case, kernel=kb.KVD_KERNEL_MFMA, num_splits=1)
    assert_same(ref_case, case, ref, got)
    _, out_ref, _, _ = oracle_step(w)
    assert_parity(spec, got[1], out_ref)


@pytest.mark.parametrize("B", [64, 65, 200])
def test_longest_first_batches(B):
    """Ragged batches whose workgroups exceed the resident slots, so the
    kernel ranks the sequences longest-first: up to 64 sequences inside each
    wave, more through LDS.  Contexts of 1..400 keys, some lengths shared
    (ties go by index).  Three splits (the planner gives these short contexts
    one): the ranking then covers (sequence, split) units.  The fused step
    equals the two calls and the oracle."""
    spec = workloads.Spec(f"ranked_b{B}", B, 1, 16, 8, 128, 16, "bf16", (1, 400), 10000.0, "normal",
                          "shuffled", spare_frac=0.05, seed=90 + B)
    w = cached_workload(spec)
    note("longest-first batch", B)
    ref_case, case = GpuCase(w), GpuCase(w)
    splits, _, kern = kb.decode_attention_plan(case.kv, num_splits=3)
    assert kern == kb.KVD_KERNEL_MFMA and splits * 8 * B > 512, "expected a ranked plan"
    assert len(np.unique(w.seq_lens)) < B, "expected equal lengths"
    ref = two_calls(ref_case, num_splits=3)
    got = fused(case, num_splits=3)
    assert_same(ref_case, case, ref, got)
    _, out_ref, _, _ = oracle_step(w)
    assert_parity(spec, got[1], out_ref)
