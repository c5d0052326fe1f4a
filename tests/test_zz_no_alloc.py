"""GPU: kvd_decode_step_noalloc, the decode step with its split-K partials in
the library's static per-device scratch, against kvd_decode_step with a
workspace from the caller.  Both run the same kernels with the same plan, so
the outputs, the rotated queries and both pools must agree bit for bit; the
oracle then bounds the output.  Two calls in a row on the same GPU, the second
with a smaller input, so the second reads partials the first left behind
wherever it failed to rewrite them."""
import numpy as np
import pytest
import torch

from gpu_common import GpuCase, assert_parity, assert_qrot, cached_workload, note, oracle_step
from kv_cached_decode_amd import binding as kb
from kv_cached_decode_amd import workloads

pytestmark = pytest.mark.gpu


def bits(a):
    return a.view(np.uint32) if a.dtype == np.float32 else a


def with_workspace(case, splits):
    s = case.w.spec
    n = kb.decode_attention_workspace_size(case.kv, splits)
    ws = torch.zeros(max(n, 1), dtype=torch.uint8, device=case.q.device)
    # zeroed: the rows of padding tokens (ragged chunks) are left as they are
    out, q_rot = torch.zeros_like(case.q), torch.zeros_like(case.q)
    kb.decode_step(case.kv, case.q, case.k, case.v, out=out, q_rot=q_rot, rope_base=s.rope_base,
                   layout=s.layout, workspace_buf=ws, num_splits=splits)
    torch.cuda.synchronize()
    return out.cpu().numpy(), q_rot.cpu().numpy()


def no_alloc(case, splits):
    s = case.w.spec
    # zeroed: the rows of padding tokens (ragged chunks) are left as they are
    out, q_rot = torch.zeros_like(case.q), torch.zeros_like(case.q)
    kb.decode_step_noalloc(case.kv, case.q, case.k, case.v, out, q_rot=q_rot, rope_base=s.rope_base,
                           layout=s.layout, num_splits=splits)
    torch.cuda.synchronize()
    return out.cpu().numpy(), q_rot.cpu().numpy()


def test_no_alloc_step_equals_workspace_step_twice():
    # a larger call, then a smaller one (fewer rows, another split count):
    # the full Llama-3-8B-shaped layer at its own plan (2 splits), then the
    # small continuous batch at 3 forced splits
    cases = [(workloads.CONFIGS["llama3_8b"], 0), (workloads.small_variant("qwen3_0_6b_cb"), 3)]
    sizes = []
    for spec, splits in cases:
        w = cached_workload(spec)
        note("no-alloc step", spec.name, "splits", splits)
        ref_case, case = GpuCase(w), GpuCase(w)
        n_splits = kb.decode_attention_plan(case.kv, splits)[0]
        need = kb.decode_attention_workspace_size(case.kv, splits)
        assert n_splits > 1 and 0 < need <= kb.NOALLOC_SCRATCH_BYTES, (n_splits, need)
        sizes.append(need)
        ref = with_workspace(ref_case, splits)
        got = no_alloc(case, splits)
        assert np.array_equal(bits(ref[0]), bits(got[0])), "output differs from kvd_decode_step"
        assert np.array_equal(bits(ref[1]), bits(got[1])), "rotated queries differ"
        for a, b in zip(ref_case.pools(), case.pools()):
            assert np.array_equal(bits(a), bits(b)), "cache pools differ"
        q_ref, out_ref, kp_ref, vp_ref = oracle_step(w)
        kp, vp = case.pools()
        assert np.array_equal(kp, kp_ref) and np.array_equal(vp, vp_ref)
        assert_qrot(got[1], q_ref)
        assert_parity(spec, got[0], out_ref, label=f"noalloc/{spec.name}")
        del ref_case, case
        torch.cuda.empty_cache()
    assert sizes[1] < sizes[0], "the second call should be the smaller one"


def test_no_alloc_rejects_a_plan_beyond_the_scratch():
    """A plan whose partials exceed the static scratch (the full continuous
    batch, 1024 query rows, at 20 forced splits: 10.6 MB) is refused on the
    host and nothing runs: the pools stay as they were."""
    w = cached_workload(workloads.CONFIGS["qwen3_0_6b_cb"])
    note("no-alloc oversize")
    case = GpuCase(w)
    before = case.pools()
    splits = 20
    assert kb.decode_attention_workspace_size(case.kv, splits) > kb.NOALLOC_SCRATCH_BYTES
    out = torch.empty_like(case.q)
    with pytest.raises(kb.KvdError) as e:
        kb.decode_step_noalloc(case.kv, case.q, case.k, case.v, out, rope_base=w.spec.rope_base,
                               num_splits=splits)
    assert e.value.status == kb.KVD_ERR_WORKSPACE
    torch.cuda.synchronize()
    for a, b in zip(before, case.pools()):
        assert np.array_equal(bits(a), bits(b))


def test_no_alloc_prefill_step_with_splits():
    """A chunked-prefill plan (ragged chunks, RoPE of the queries inside the
    prefill kernel) at 2 and then 3 forced splits, its partials in the static
    scratch: bit for bit the step with a workspace, then against the oracle."""
    # two sequences, ragged chunks of up to 48 tokens (192 query rows per kv
    # head: two row tiles of the prefill kernel); 3.2 and 4.8 MB of partials
    spec = workloads.small_variant("chunked_prefill").with_(name="chunked_prefill_noalloc", num_seqs=2,
                                                            q_tokens=48, chunk=(1, 48), seed=109)
    w = cached_workload(spec)
    for splits in (2, 3):
        note("no-alloc prefill step", spec.name, "splits", splits)
        ref_case, case = GpuCase(w), GpuCase(w)
        assert kb.decode_attention_plan(case.kv, splits)[0] == splits
        need = kb.decode_attention_workspace_size(case.kv, splits)
        assert 0 < need <= kb.NOALLOC_SCRATCH_BYTES, need
        ref = with_workspace(ref_case, splits)
        got = no_alloc(case, splits)
        assert np.array_equal(bits(ref[0]), bits(got[0])), "output differs from kvd_decode_step"
        assert np.array_equal(bits(ref[1]), bits(got[1])), "rotated queries differ"
        for a, b in zip(ref_case.pools(), case.pools()):
            assert np.array_equal(bits(a), bits(b)), "cache pools differ"
        q_ref, out_ref, kp_ref, vp_ref = oracle_step(w)
        kp, vp = case.pools()
        assert np.array_equal(kp, kp_ref) and np.array_equal(vp, vp_ref)
        live = np.zeros(out_ref.shape[:2], bool)
        for b, n in enumerate(w.q_lens):
            live[b, :n] = True
        assert_qrot(got[1][live], q_ref[live])
        assert_parity(spec, got[0][live], out_ref[live], label=f"noalloc/{spec.name}/{splits}")
        del ref_case, case
        torch.cuda.empty_cache()
