"""GPU: the decode kernel's own merge of its splits.  With two splits, each
workgroup publishes its partial with agent-scope stores and takes a ticket;
the last of a (sequence, kv head) merges both in a fixed order (more splits
go to the combine kernel, checked the same way).  Consecutive calls run through one workspace with new queries each
time (so every call's partials differ from the previous call's, and a stale
read would show): each result equals the one-split result of the same
queries (no merge there), lse included; repeated calls are bitwise equal;
and the counters at the head of the workspace are zero after every call."""
import numpy as np
import pytest
import torch

from gpu_common import DEV, GpuCase, assert_parity, cached_workload, note, oracle_step
from kv_cached_decode_amd import binding as kb
from kv_cached_decode_amd import workloads

pytestmark = pytest.mark.gpu


def _close(a, b, tol=2e-5):
    return float((a - b).abs().max() / b.abs().max().clamp_min(1e-30)) <= tol


# two splits: the kernel merges them itself (ragged lengths give the
# continuous batch empty second splits); more: the combine kernel
@pytest.mark.parametrize("name,splits", [("llama3_8b", 2), ("qwen3_0_6b_cb", 2), ("mtp_verify", 2),
                                         ("long_ctx", 2), ("llama3_8b", 5), ("qwen3_0_6b_cb", 3),
                                         ("long_ctx", 8)])
def test_merge_under_changing_queries(name, splits):
    w = cached_workload(workloads.small_variant(name))
    note("split merge", name, splits)
    case = GpuCase(w)
    kv = case.kv
    assert kb.decode_attention_plan(kv, splits, kb.KVD_KERNEL_MFMA) [0] == splits
    n = kb.decode_attention_workspace_size(kv, splits, kb.KVD_KERNEL_MFMA)
    ws = torch.zeros(n, dtype=torch.uint8, device=DEV)
    g = torch.Generator(device=DEV).manual_seed(splits)
    for i in range(12):
        q = torch.randn(kv.q_shape(), generator=g, device=DEV) * (1.0 + 3.0 * (i % 3))
        out, lse = kb.decode_attention_lse(kv, q, workspace_buf=ws, num_splits=splits, kernel=kb.KVD_KERNEL_MFMA)
        again = kb.decode_attention(kv, q, workspace_buf=ws, num_splits=splits, kernel=kb.KVD_KERNEL_MFMA)
        one, lse1 = kb.decode_attention_lse(kv, q, num_splits=1, kernel=kb.KVD_KERNEL_MFMA)
        torch.cuda.synchronize()
        assert torch.equal(out, again), f"call {i}: not deterministic"
        assert _close(out, one), f"call {i}: merged splits differ from one split"
        assert torch.allclose(lse, lse1, rtol=1e-5, atol=1e-5), f"call {i}: lse differs"
        assert not ws[:kb.WORKSPACE_COUNTER_BYTES].any(), f"call {i}: counters left nonzero"


def test_merge_in_the_fused_step_through_graph_replays():
    """The fused decode step at 2 splits (merged in the kernel) captured in a
    HIP graph: every replay (with eager calls and new queries in between)
    merges its splits afresh."""
    spec = workloads.small_variant("llama3_8b")
    w = cached_workload(spec)
    note("split merge graph")
    case = GpuCase(w)
    n = kb.decode_attention_workspace_size(case.kv, 2)
    ws = torch.zeros(n, dtype=torch.uint8, device=DEV)
    out = torch.empty_like(case.q)
    q = case.q.clone()

    def step():
        kb.decode_step(case.kv, q, case.k, case.v, out=out, rope_base=spec.rope_base, workspace_buf=ws,
                       num_splits=2)

    step()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        step()
    torch.cuda.synchronize()
    g = torch.Generator(device=DEV).manual_seed(7)
    for i in range(4):
        q.copy_(torch.randn(q.shape, generator=g, device=DEV))
        step()
        torch.cuda.synchronize()
        eager = out.clone()
        out.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i} differs from the eager step"
        assert not ws[:kb.WORKSPACE_COUNTER_BYTES].any()


@pytest.mark.parametrize("splits", [2, 4])
def test_ranked_batch_equal_shares(splits):
    """The continuous batch at full size with more (sequence, split) units
    than resident slots: the kernel ranks them and gives each sequence's
    splits equal shares of its own key range.  With two splits it merges
    them itself (its live splits counted from that share), with four the
    combine kernel does; both equal the one-split result (an unranked plan
    over whole sequences), lse included, through repeated calls."""
    w = cached_workload(workloads.CONFIGS["qwen3_0_6b_cb"])
    note("ranked equal shares", splits)
    case = GpuCase(w)
    kv = case.kv
    assert kb.decode_attention_plan(kv, splits, kb.KVD_KERNEL_MFMA)[0] == splits
    n = kb.decode_attention_workspace_size(kv, splits, kb.KVD_KERNEL_MFMA)
    ws = torch.zeros(n, dtype=torch.uint8, device=DEV)
    g = torch.Generator(device=DEV).manual_seed(100 + splits)
    for i in range(3):
        q = torch.randn(kv.q_shape(), generator=g, device=DEV) * (1.0 + 3.0 * i)
        out, lse = kb.decode_attention_lse(kv, q, workspace_buf=ws, num_splits=splits, kernel=kb.KVD_KERNEL_MFMA)
        again = kb.decode_attention(kv, q, workspace_buf=ws, num_splits=splits, kernel=kb.KVD_KERNEL_MFMA)
        one, lse1 = kb.decode_attention_lse(kv, q, num_splits=1, kernel=kb.KVD_KERNEL_MFMA)
        torch.cuda.synchronize()
        assert torch.equal(out, again), f"call {i}: not deterministic"
        assert _close(out, one), f"call {i}: split shares differ from one split"
        assert torch.allclose(lse, lse1, rtol=1e-5, atol=1e-5), f"call {i}: lse differs"
        assert not ws[:kb.WORKSPACE_COUNTER_BYTES].any(), f"call {i}: counters left nonzero"


@pytest.mark.parametrize("splits", [2, 3])
def test_ranked_batch_equal_shares_with_window(splits):
    """The ranked continuous batch with a sliding window of 3000 keys: each
    sequence's splits share its windowed range equally.  The two-call step
    and the fused step (new K/V substituted from the split holding them)
    against the oracle, every row."""
    spec = workloads.CONFIGS["qwen3_0_6b_cb"]
    w = cached_workload(spec)
    window = 3000
    note("ranked equal shares, window", splits)
    case = GpuCase(w, window=window)
    kv = case.kv
    assert kb.decode_attention_plan(kv, splits, kb.KVD_KERNEL_MFMA)[0] == splits
    _, out = case.step(num_splits=splits)
    _, ref, _, _ = oracle_step(w, window=window)
    assert_parity(spec, out, ref, label=f"ranked window two-call/{splits}")
    fused = kb.decode_step(kv, case.q, case.k, case.v, rope_base=spec.rope_base, num_splits=splits)
    torch.cuda.synchronize()
    assert_parity(spec, fused.cpu().numpy(), ref, label=f"ranked window fused/{splits}")
