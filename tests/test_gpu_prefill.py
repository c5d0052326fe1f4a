"""GPU: chunked prefill and other many-row cases (more than 16 query rows
per kv head run through the prefill kernel) against the oracle, every row;
ragged chunks (q_lens), the append of exactly the real tokens, windows,
split counts, and agreement with the vector-ALU kernel."""
import numpy as np
import pytest
import torch

from gpu_common import GpuCase, assert_parity, assert_qrot, note, oracle_step
from kv_cached_decode_amd import binding as kb
from kv_cached_decode_amd import workloads

pytestmark = pytest.mark.gpu


def spec(name, B, T, Hq, Hkv, ctx, seed, chunk=None, bs=16):
    return workloads.Spec(name, B, T, Hq, Hkv, 128, bs, "bf16", ctx, 10000.0, "normal", "shuffled",
                          spare_frac=0.1, seed=seed, chunk=chunk)


CASES = [
    spec("chunk64_g4", 2, 64, 32, 8, (100, 500), 61),          # uniform chunk, 256 rows per kv head
    spec("chunk40_g8", 2, 40, 64, 8, (0, 300), 62),            # 320 rows, tile tails
    spec("chunk33_mha", 2, 33, 8, 8, (50, 200), 63),           # g = 1: 33 rows
    spec("ragged_g4", 4, 100, 32, 8, (0, 400), 64, chunk=(0, 100)),
    spec("ragged_bs64", 3, 130, 16, 8, (200, 900), 65, chunk=(17, 130), bs=64),
    spec("chunk32_g4", 3, 32, 32, 8, (0, 400), 67, chunk=(5, 32)),   # 128 rows: four-wave workgroups
]


@pytest.mark.parametrize("sp", CASES, ids=lambda s: s.name)
def test_prefill_all_rows(sp):
    w = workloads.make_workload(sp)
    note("prefill", sp.name, "q_lens", None if w.q_lens is None else w.q_lens.tolist())
    case = GpuCase(w)
    assert kb.decode_attention_plan(case.kv)[2] == kb.KVD_KERNEL_MFMA
    q_gpu, out = case.step()
    kp, vp = case.pools()
    q_ref, ref, kp_ref, vp_ref = oracle_step(w)
    assert np.array_equal(kp, kp_ref) and np.array_equal(vp, vp_ref), "append differs"
    assert_qrot(q_gpu, q_ref)
    if w.q_lens is not None:
        for b, n in enumerate(w.q_lens):
            assert np.all(out[b, n:] == 0.0), "padding rows must be 0"
    assert_parity(sp, out, ref)


def test_ragged_extremes():
    """Chunks of 0, 1 and T tokens side by side (the workload allocates every
    sequence a full chunk of T; the chunks below only lower the lengths)."""
    sp = spec("ragged_extremes", 3, 48, 32, 8, (0, 200), 66, chunk=(48, 48))
    w = workloads.make_workload(sp)
    q_lens = np.array([0, 1, 48], np.int32)
    sl = (w.ctx_lens + q_lens).astype(np.int32)
    assert np.all(sl <= w.seq_lens)
    note("ragged extremes")
    case = GpuCase(w, seq_lens=sl, q_lens=q_lens)
    q_gpu, out = case.step()
    kp, vp = case.pools()
    w2 = workloads.Workload(**{**w.__dict__, "seq_lens": sl, "q_lens": q_lens})
    q_ref, ref, kp_ref, vp_ref = oracle_step(w2)
    assert np.array_equal(kp, kp_ref) and np.array_equal(vp, vp_ref)
    assert np.all(out[0] == 0.0) and np.all(out[1, 1:] == 0.0)
    assert_parity(sp, out, ref)


@pytest.mark.parametrize("splits", [1, 3, 9])
def test_prefill_split_counts(splits):
    sp = spec("prefill_splits", 2, 64, 32, 8, (300, 700), 67)
    w = workloads.make_workload(sp)
    note("prefill splits", splits)
    case = GpuCase(w)
    _, out = case.step(num_splits=splits)
    _, ref, _, _ = oracle_step(w)
    assert_parity(sp, out, ref)


@pytest.mark.parametrize("window", [1, 20, 100])
def test_prefill_window(window):
    sp = spec("prefill_window", 2, 64, 32, 8, (100, 300), 68)
    w = workloads.make_workload(sp)
    note("prefill window", window)
    case = GpuCase(w, window=window)
    _, out = case.step()
    _, ref, _, _ = oracle_step(w, window=window)
    assert_parity(sp, out, ref)


def test_prefill_and_valu_kernels_agree():
    sp = spec("prefill_vs_valu", 2, 24, 32, 8, (0, 250), 69, chunk=(5, 24))
    w = workloads.make_workload(sp)
    note("prefill vs valu")
    outs = {}
    for kern in (kb.KVD_KERNEL_MFMA, kb.KVD_KERNEL_VALU):
        case = GpuCase(w)
        outs[kern] = case.step(kernel=kern)[1]
        del case
        torch.cuda.empty_cache()
    _, ref, _, _ = oracle_step(w)
    for kern, out in outs.items():
        assert_parity(sp, out, ref)
    # both families hold the 2e-3 bound; they also agree with each other
    assert np.max(np.abs(outs[kb.KVD_KERNEL_MFMA] - outs[kb.KVD_KERNEL_VALU])) <= 4e-3 * np.max(np.abs(ref))


@pytest.mark.parametrize("splits", [0, 2])
def test_longest_first_unit_order(splits):
    """More (sequence, row tile, split) units than resident workgroup slots,
    ragged chunks with empty tiles: the kernel takes its units longest-first
    (a permutation every workgroup derives); every row still matches."""
    sp = spec("ranked_units", 12, 256, 32, 8, (0, 300), 70, chunk=(1, 256))
    w = workloads.make_workload(sp)
    note("longest-first", splits, "q_lens", w.q_lens.tolist())
    case = GpuCase(w)
    plan = kb.decode_attention_plan(case.kv, num_splits=splits)
    # 8 row tiles x 12 sequences x splits units, 8 kv heads each: beyond the
    # 2 x 256 resident slots
    assert plan[2] == kb.KVD_KERNEL_MFMA and plan[0] == (splits or 1)
    _, out = case.step(num_splits=splits)
    _, ref, _, _ = oracle_step(w)
    for b, n in enumerate(w.q_lens):
        assert np.all(out[b, n:] == 0.0), "padding rows must be 0"
    assert_parity(sp, out, ref)


@pytest.mark.parametrize("big_first", [False, True])
def test_rows_of_very_different_scales(big_first):
    """Runs of 4 tokens (16 rows of a kv-head group at g = 4, one MFMA row
    block) whose queries are scaled by 1 or 2e4, alternately: rows with
    scores of a few hundredths beside rows whose scores spread over hundreds
    (log2 units).  Each row block keeps its own running maximum while the two
    blocks a wave holds exchange theirs together, and the large jumps of the
    maximum rescale without overflow or loss."""
    sp = spec("row_scales", 2, 64, 32, 8, (100, 400), 71)
    w = workloads.make_workload(sp)
    big = ((np.arange(sp.q_tokens) // 4) % 2 == 0) == big_first
    f = np.where(big, 2e4, 1.0).astype(np.float32)
    w = workloads.Workload(**{**w.__dict__, "q": (w.q * f[None, :, None, None]).astype(np.float32)})
    note("row scales", big_first)
    case = GpuCase(w)
    assert kb.decode_attention_plan(case.kv)[2] == kb.KVD_KERNEL_MFMA
    _, out = case.step()
    _, ref, _, _ = oracle_step(w)
    # each group of rows against its own scale (the peaky rows' outputs are
    # single values of V; the flat rows' are averages, about 20x smaller)
    for rows in (big, ~big):
        assert_parity(sp, out[:, rows], ref[:, rows])


def _scale_v(w, factor, keys_every=1):
    """The workload with V scaled by a power of two (exact in bf16 and fp32):
    the cached rows of every keys_every-th slot of the pool, and the new
    tokens' rows."""
    bits = w.v_pool.astype(np.uint32) << 16
    f = bits.view(np.float32).copy()
    sl = f[:, :, ::keys_every, :]
    sl *= np.float32(factor)
    v_pool = (f.view(np.uint32) >> 16).astype(np.uint16)
    v_pool[np.isnan(f)] = w.v_pool[np.isnan(f)]          # poisoned slots stay as they were
    return workloads.Workload(**{**w.__dict__, "v_pool": v_pool, "v": (w.v * np.float32(factor)).astype(np.float32)})


@pytest.mark.parametrize("splits", [0, 3])
@pytest.mark.parametrize("factor,every", [(2.0 ** 18, 5), (2.0 ** -20, 1)], ids=["beyond_fp16", "below_fp16"])
def test_v_outside_fp16_range(factor, every, splits):
    """V rows beyond fp16's range (2^18 x N(0,1)/sqrt(128) on every fifth
    slot) or all below its normal range (2^-20 x): the units that meet them
    are recomputed with bf16 weights and V, and every row matches the oracle."""
    sp = spec("v_range", 2, 64, 32, 8, (100, 400), 72)
    w = _scale_v(workloads.make_workload(sp), factor, every)
    note("v outside fp16", factor, every, splits)
    case = GpuCase(w)
    assert kb.decode_attention_plan(case.kv, num_splits=splits)[2] == kb.KVD_KERNEL_MFMA
    _, out = case.step(num_splits=splits)
    kp, vp = case.pools()
    _, ref, kp_ref, vp_ref = oracle_step(w)
    assert np.array_equal(vp, vp_ref)
    assert_parity(sp, out, ref)


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


def _step_vs_two_calls(w, window=0, splits=0, want_q_rot=True):
    """kvd_decode_step on a prefill plan (the RoPE/append kernel for the new
    K/V rows, then the prefill kernel rotating its own queries) against the
    two calls with the same plan: every real row bitwise, both pools bitwise,
    and the padding rows of out and q_rot left as they were (NaN sentinels).
    Returns (out, q_rot) of the step."""
    s = w.spec
    ref_case, case = GpuCase(w, window=window), GpuCase(w, window=window)
    assert kb.decode_attention_plan(case.kv, num_splits=splits)[2] == kb.KVD_KERNEL_MFMA
    q_rot_ref = torch.full_like(ref_case.q, float("nan"))
    kb.rope_append_kv(ref_case.kv, ref_case.q, ref_case.k, ref_case.v, q_rot_ref, s.rope_base, s.layout)
    out_ref = kb.decode_attention(ref_case.kv, q_rot_ref, torch.full_like(ref_case.q, float("nan")),
                                  num_splits=splits)
    out = torch.full_like(case.q, float("nan"))
    q_rot = torch.full_like(case.q, float("nan")) if want_q_rot else None
    kb.decode_step(case.kv, case.q, case.k, case.v, out=out, q_rot=q_rot, rope_base=s.rope_base,
                   layout=s.layout, num_splits=splits)
    torch.cuda.synchronize()
    out, out_ref = out.cpu().numpy(), out_ref.cpu().numpy()
    q_lens = w.q_lens if w.q_lens is not None else np.full(s.num_seqs, s.q_tokens)
    real = np.arange(s.q_tokens)[None, :] < q_lens[:, None]            # [B][T]
    assert np.array_equal(_bits(out[real]), _bits(out_ref[real])), "step differs from the two calls"
    assert np.all(np.isnan(out[~real])), "padding rows of out were written"
    for a_, b_ in zip(ref_case.pools(), case.pools()):
        assert np.array_equal(a_, b_), "pools differ"
    if want_q_rot:
        q_rot, q_rot_ref = q_rot.cpu().numpy(), q_rot_ref.cpu().numpy()
        assert np.array_equal(_bits(q_rot[real]), _bits(q_rot_ref[real])), "q_rot differs"
        assert np.all(np.isnan(q_rot[~real])), "padding rows of q_rot were written"
    return out, q_rot, case


STEP_CASES = CASES + [
    spec("ragged_g2", 3, 90, 16, 8, (0, 500), 73, chunk=(1, 90)),     # g = 2: 180 rows, 64 tokens a tile
    spec("mha_long", 2, 200, 8, 8, (0, 300), 74, chunk=(150, 200)),   # g = 1: 128 tokens a tile
]


@pytest.mark.parametrize("sp", STEP_CASES, ids=lambda s: s.name)
@pytest.mark.parametrize("want_q_rot", [True, False], ids=["q_rot", "no_q_rot"])
def test_prefill_step_rotates_its_own_queries(sp, want_q_rot):
    w = workloads.make_workload(sp)
    note("prefill step", sp.name, want_q_rot)
    out, q_rot, case = _step_vs_two_calls(w, want_q_rot=want_q_rot)
    q_ref, ref, kp_ref, vp_ref = oracle_step(w)
    kp, vp = case.pools()
    assert np.array_equal(kp, kp_ref) and np.array_equal(vp, vp_ref)
    q_lens = w.q_lens if w.q_lens is not None else np.full(sp.num_seqs, sp.q_tokens)
    real = np.arange(sp.q_tokens)[None, :] < q_lens[:, None]
    if want_q_rot:
        assert_qrot(q_rot[real], q_ref[real])
    assert_parity(sp, out[real], ref[real], label=f"prefill_step/{sp.name}")


@pytest.mark.parametrize("layout,window,splits", [(1, 0, 0), (0, 37, 0), (1, 100, 3), (0, 0, 3)])
def test_prefill_step_layouts_windows_splits(layout, window, splits):
    sp = spec("prefill_step_var", 3, 80, 32, 8, (0, 400), 75, chunk=(10, 80)).with_(layout=layout)
    w = workloads.make_workload(sp)
    note("prefill step variants", layout, window, splits)
    out, _, _ = _step_vs_two_calls(w, window=window, splits=splits)
    _, ref, _, _ = oracle_step(w, window=window)
    real = np.arange(sp.q_tokens)[None, :] < w.q_lens[:, None]
    assert_parity(sp, out[real], ref[real])
