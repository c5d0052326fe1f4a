"""The pages' end-to-end check at model level (ferric-core `examples/generate.rs`):
a 3-layer tiny LM decodes one token at a time through the library's paged KV
cache, and every step's logits must equal a full non-cached recompute over
the prefix so far, within the page's 2e-3 bound on the logits."""
import numpy as np
import pytest

import oracle
from gpu_common import note
from kv_cached_decode_amd import workloads
from oracle import tiny_lm

pytestmark = pytest.mark.gpu

CFG = workloads.TINY_LM
W = workloads.tiny_lm_weights(CFG)
PROMPT = list(workloads.TINY_LM_PROMPT)
STEPS = len(PROMPT) + workloads.TINY_LM_GEN_STEPS
PAGE_BOUND = 2e-3      # the page's bound on max |cached logits - recompute logits|
F32_BOUND = 1e-4       # fp32 cache and fp32 projections: rounding ~1e-6 on logits ~4


def shuffled_table(num_seqs, capacity, bs, seed):
    nb = -(-capacity // bs)
    perm = np.random.default_rng(seed).permutation(num_seqs * nb + 5).astype(np.int32)
    return perm[:num_seqs * nb].reshape(num_seqs, nb)


def gpu_model(num_seqs, capacity, bs, kv_dtype, seed=0):
    from tiny_lm_gpu import GpuTinyLM
    return GpuTinyLM(W, CFG, num_seqs, capacity, bs, kv_dtype,
                     shuffled_table(num_seqs, capacity, bs, seed))


def oracle_greedy():
    m = tiny_lm.CachedLM(W, CFG, 1, 16, 4, oracle.ORACLE_F64)
    seq = list(PROMPT)
    for pos in range(STEPS):
        lg = m.step([seq[pos]])[0]
        if pos + 1 >= len(seq):
            seq.append(int(np.argmax(lg)))
    return seq


@pytest.mark.parametrize("bs", [4, 16])
def test_generate_matches_full_recompute(bs):
    """Prompt [3, 14, 1, 15] teacher-forced, then 5 greedy steps; fp32 cache."""
    note("tiny LM generate, fp32 cache, block", bs)
    model = gpu_model(1, 16, bs, "f32", seed=bs)
    seq, worst = list(PROMPT), 0.0
    for pos in range(STEPS):
        lg = model.step([[seq[pos]]])[0, 0]
        ref = tiny_lm.full_forward(seq[:pos + 1], W, CFG)
        worst = max(worst, float(np.max(np.abs(lg - ref))))
        assert np.all(np.isfinite(lg)), f"non-finite logits at position {pos}"
        if pos + 1 >= len(seq):
            seq.append(int(np.argmax(lg)))
    print(f"generated {seq[len(PROMPT):]}, worst |logits - recompute| = {worst:.3e}")
    assert worst <= PAGE_BOUND
    assert worst <= F32_BOUND
    assert seq == oracle_greedy()


def test_continuous_batching_matches_full_recompute():
    """Four sequences with different prompts join at different steps and step
    in changing subsets (per-sequence positions in one call), fp32 cache."""
    note("tiny LM continuous batching")
    prompts = [[3, 14, 1, 15], [7], [2, 9, 30, 4, 11, 5], [0, 31]]
    start, cap = [0, 2, 1, 3], 12
    model = gpu_model(4, cap, 4, "f32", seed=7)
    seqs, fed, worst = [list(p) for p in prompts], [0] * 4, 0.0
    for step in range(12):
        active = [i for i in range(4) if step >= start[i] and fed[i] < cap]
        lg = model.step([[seqs[i][fed[i]]] for i in active], active)[:, 0]
        for r, i in enumerate(active):
            fed[i] += 1
            ref = tiny_lm.full_forward(seqs[i][:fed[i]], W, CFG)
            worst = max(worst, float(np.max(np.abs(lg[r] - ref))))
            if fed[i] >= len(seqs[i]):
                seqs[i].append(int(np.argmax(lg[r])))
    assert worst <= F32_BOUND


def test_bf16_cache_matches_oracle_with_same_rounding():
    """bf16 cache: the exact reference is the oracle's incremental decode with
    the same bf16 cache (the recompute differs by the cache rounding itself)."""
    note("tiny LM bf16 cache")
    model = gpu_model(1, 16, 4, "bf16", seed=3)
    ref_model = tiny_lm.CachedLM(W, CFG, 1, 16, 4, oracle.ORACLE_BF16)
    seq, worst = list(PROMPT), 0.0
    for pos in range(STEPS):
        lg = model.step([[seq[pos]]])[0, 0]
        ref = ref_model.step([seq[pos]])[0]
        worst = max(worst, float(np.max(np.abs(lg - ref)) / np.max(np.abs(ref))))
        if pos + 1 >= len(seq):
            seq.append(int(np.argmax(ref)))
    assert worst <= 2e-3


def test_verify_draft_then_rollback():
    """Speculative verify at model level: after the prompt, the 4-token greedy
    continuation is fed as one T=4 call (causal within the draft); each row's
    logits equal the recompute over its own prefix.  Then the last two draft
    tokens are rejected (the length is lowered) and decoding continues from
    there, again matching the recompute."""
    note("tiny LM verify + rollback")
    ref_seq = oracle_greedy()
    model = gpu_model(1, 16, 4, "f32", seed=11)
    for pos in range(len(PROMPT) - 1):
        model.step([[PROMPT[pos]]])
    draft = ref_seq[len(PROMPT) - 1:len(PROMPT) + 3]         # 4 tokens from position 3
    lg = model.step([draft])[0]
    for t in range(4):
        ref = tiny_lm.full_forward(ref_seq[:len(PROMPT) + t], W, CFG)
        assert np.max(np.abs(lg[t] - ref)) <= F32_BOUND, f"draft row {t}"
    # Keep positions 0..4 (prompt + first accepted token); feed a different token
    # at position 5 and check against the recompute of that new prefix.
    model.rollback(0, len(PROMPT) + 1)
    alt = (ref_seq[len(PROMPT) + 1] + 1) % CFG.vocab
    lg = model.step([[alt]])[0, 0]
    ref = tiny_lm.full_forward(ref_seq[:len(PROMPT) + 1] + [alt], W, CFG)
    assert np.max(np.abs(lg - ref)) <= F32_BOUND
