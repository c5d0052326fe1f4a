"""GPU: a seeded sweep of small random shapes through the whole step
(kvd_decode_step) against the oracle -- batch, new tokens, ragged chunks,
head counts and group sizes, head dim and cache dtype, block size, context
lengths, sliding windows, RoPE pairing -- so that the planner's kernel
choices (vector ALU, matrix-core decode, prefill; one or several splits)
meet combinations the targeted tests do not name.  Every case also checks
the append bit for bit."""
import numpy as np
import pytest
import torch

from gpu_common import GpuCase, assert_parity, assert_qrot, note, oracle_step
from kv_cached_decode_amd import binding as kb
from kv_cached_decode_amd import workloads

pytestmark = pytest.mark.gpu


def random_case(i):
    rng = np.random.default_rng(1000 + i)
    D, dtype = [(128, "bf16"), (128, "bf16"), (64, "f32"), (128, "f32"), (256, "bf16")][rng.integers(5)]
    g = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    T = int(rng.choice([1, 1, 2, 4, 5, 17, 40]))
    B = int(rng.integers(1, 5))
    bs = int(rng.choice([16, 64]))
    lo = int(rng.integers(0, 300))
    ctx = (lo, lo + int(rng.integers(1, 700)))
    chunk = (1, T) if T > 1 and rng.random() < 0.4 else None
    window = int(rng.choice([0, 0, 0, 7, 100]))
    spec = workloads.Spec(f"rand{i}", B, T, g * Hkv, Hkv, D, bs, dtype, ctx, 10000.0, "normal", "shuffled",
                          spare_frac=0.1, seed=2000 + i, layout=int(rng.integers(2)), chunk=chunk)
    # drawn last, so the shapes above do not depend on them: a forced split
    # count (two splits merge inside the decode kernel), and whether the
    # rotated queries are asked for
    splits = int(rng.choice([0, 0, 2, 3]))
    want_q_rot = bool(rng.random() < 0.3)
    return spec, window, splits, want_q_rot


@pytest.mark.parametrize("i", range(64))
def test_random_shape(i):
    spec, window, splits, want_q_rot = random_case(i)
    w = workloads.make_workload(spec)
    note("random shape", i, spec, "window", window, "splits", splits, "q_rot", want_q_rot)
    case = GpuCase(w, window=window)
    res = kb.decode_step(case.kv, case.q, case.k, case.v, rope_base=spec.rope_base, layout=spec.layout,
                         num_splits=splits, want_q_rot=want_q_rot)
    torch.cuda.synchronize()
    out = (res[0] if want_q_rot else res).cpu().numpy()
    kp, vp = case.pools()
    q_ref, ref, kp_ref, vp_ref = oracle_step(w, window=window)
    assert np.array_equal(kp.view(np.uint8), kp_ref.view(np.uint8)), "K pool differs"
    assert np.array_equal(vp.view(np.uint8), vp_ref.view(np.uint8)), "V pool differs"
    real = np.ones(out.shape[:2], bool)
    if w.q_lens is not None:
        real = np.arange(spec.q_tokens)[None, :] < w.q_lens[:, None]
        assert np.all(out[~real] == 0.0), "padding rows of a zeroed out must stay 0"
    if want_q_rot:
        assert_qrot(res[1].cpu().numpy()[real], q_ref[real])
    assert_parity(spec, out, ref)
