"""Host: the benchmark's accounting.  The algorithmic bytes and flops that
the roofline divides by the measured time, against derivations by hand from
the configurations' shapes, and the refusal of runs on more than one GPU."""
import os
import subprocess
import sys

import numpy as np

from kv_cached_decode_amd import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def lengths_only(name, seq_lens, q_lens=None):
    """A workload of configuration `name` that carries only its lengths (the
    accounting reads nothing else)."""
    e = np.zeros(0, np.float32)
    sl = np.asarray(seq_lens, np.int32)
    spec = workloads.CONFIGS[name].with_(num_seqs=sl.size)
    return workloads.Workload(spec, np.zeros(sl.size, np.int64), sl, np.zeros((sl.size, 0), np.int32),
                              e, e, e, e, e, q_lens=None if q_lens is None else np.asarray(q_lens, np.int32))


def test_kv_bytes_of_the_fixed_configurations():
    # sequences x keys after the append x 8 kv heads x 128 dims x (K and V) x 2 bytes
    assert lengths_only("llama3_8b", [4097] * 16).algorithmic_bytes()["kv_read"] == 16 * 4097 * 8 * 128 * 2 * 2
    assert lengths_only("llama3_8b", [4097] * 16).algorithmic_bytes()["kv_read"] == 268_500_992
    assert lengths_only("long_ctx", [131073] * 4).algorithmic_bytes()["kv_read"] == 2_147_500_032
    assert lengths_only("mtp_verify", [16388] * 32).algorithmic_bytes()["kv_read"] == 2_148_007_936


def test_step_bytes_llama3_8b():
    b = lengths_only("llama3_8b", [4097] * 16).algorithmic_bytes()
    q_and_out = 16 * 32 * 128 * 4 * 2        # q read and out written, fp32
    table = 16 * 65 * 4                      # 65 block ids of 64 keys cover 4097 keys
    lens = 16 * 4                            # seq_lens
    new_kv = 16 * 2 * 8 * 128 * (4 + 2)      # new K and V read as fp32, appended as bf16
    assert b["attention"] == 268_500_992 + q_and_out + table + lens
    assert b["step"] == b["attention"] + new_kv == 269_226_112


def test_ragged_lengths_and_chunks():
    # two sequences of 100 and 37 keys, blocks of 16; ragged chunks of 5 and 2
    # new tokens in a step of up to 8
    w = lengths_only("chunked_prefill", [100, 37], [5, 2])
    b = w.algorithmic_bytes()
    assert b["kv_read"] == (100 + 37) * 8 * 128 * 2 * 2
    real_rows = (5 + 2) / 2                  # per sequence, on average
    assert b["attention"] == b["kv_read"] + int(2 * real_rows * 32 * 128 * 4 * 2) + (7 + 3) * 4 + 2 * 4


def test_flops_count_every_visible_key_once():
    # verify step: token t of a sequence of L keys (T new) sees L - T + 1 + t keys
    L, T, B = 16388, 4, 32
    w = lengths_only("mtp_verify", [L] * B)
    per_seq = sum(L - T + 1 + t for t in range(T))
    assert w.algorithmic_flops() == B * per_seq * 32 * 128 * 2 * 2
    # ragged chunks, counted key by key
    seq_lens, q_lens = [100, 37, 512], [5, 2, 1]
    w = lengths_only("chunked_prefill", seq_lens, q_lens)
    pairs = 0
    for L, n in zip(seq_lens, q_lens):
        for t in range(n):
            pairs += sum(1 for key in range(L) if key <= L - n + t)
    assert w.algorithmic_flops() == pairs * 32 * 128 * 4


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
