"""GPU: kvd_check_descriptor, the optional device-side check of a
descriptor's contract.  The descriptors of every workload leave the flag word
clear; planted violations (a length past max_seq_len, a block id outside the
pool inside the visible range, a chunk longer than T, a negative shard
position, a whole cache shorter than its new tokens) set exactly their bit.
The planted descriptors go to the check only: the check reads the lengths,
positions and table rows, never past a row, and dereferences no block id."""
import numpy as np
import pytest
import torch

from gpu_common import DEV, GpuCase, cached_workload, note
from kv_cached_decode_amd import binding as kb
from kv_cached_decode_amd import workloads

pytestmark = pytest.mark.gpu


def flags_of(kv):
    f = kb.check_descriptor(kv)
    torch.cuda.synchronize()
    return int(f.cpu().item())


@pytest.mark.parametrize("name", workloads.CONFIG_ORDER)
def test_workloads_are_clean(name):
    w = cached_workload(workloads.small_variant(name))
    note("check clean", name)
    case = GpuCase(w)
    assert flags_of(case.kv) == 0


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(DEV)


def test_planted_violations_set_their_bits():
    w = cached_workload(workloads.small_variant("qwen3_0_6b_cb"))
    s = w.spec
    note("check planted")
    case = GpuCase(w)
    base = case.kv

    def variant(**kw):
        d = dict(k_cache=base.k_cache, v_cache=base.v_cache, block_table=base.block_table,
                 seq_lens=base.seq_lens, n_q_heads=base.n_q_heads, q_tokens_per_seq=base.q_tokens_per_seq,
                 max_seq_len=base.max_seq_len)
        d.update(kw)
        return kb.PagedKV(**d)

    sl = w.seq_lens.copy()
    sl[2] = base.max_seq_len + 1                            # past the host bound
    assert flags_of(variant(seq_lens=_t(sl))) & kb.KVD_CHECK_SEQ_LEN
    sl = w.seq_lens.copy()
    sl[3] = 0                                               # shorter than its new token
    assert flags_of(variant(seq_lens=_t(sl))) == kb.KVD_CHECK_SEQ_LEN

    table = w.block_table.copy()
    b = 4
    table[b, (int(w.seq_lens[b]) - 1) // s.block_size] = -1          # the new token's block
    assert flags_of(variant(block_table=_t(table))) == kb.KVD_CHECK_BLOCK_ID
    table = w.block_table.copy()
    table[1, 0] = w.num_blocks                              # one past the pool
    assert flags_of(variant(block_table=_t(table))) == kb.KVD_CHECK_BLOCK_ID

    # an unallocated block before every query's window is not read, not flagged
    b = int(np.argmax(w.seq_lens))
    assert w.seq_lens[b] > 3 * s.block_size
    table = w.block_table.copy()
    table[b, 0] = -1
    assert flags_of(variant(block_table=_t(table), window=s.block_size)) == 0
    assert flags_of(variant(block_table=_t(table))) == kb.KVD_CHECK_BLOCK_ID

    q_lens = np.ones(s.num_seqs, np.int32)
    q_lens[5] = s.q_tokens + 1                              # a chunk longer than T
    assert flags_of(variant(q_lens=_t(q_lens))) == kb.KVD_CHECK_Q_LENS

    kp0 = np.zeros(s.num_seqs, np.int32)
    kp0[6] = -3                                             # a negative shard position
    q_pos = (w.seq_lens - s.q_tokens).astype(np.int32)
    assert flags_of(variant(key_pos0=_t(kp0), q_pos=_t(q_pos))) == kb.KVD_CHECK_SHARD

    # bits accumulate in a word the caller keeps
    f = torch.zeros(1, dtype=torch.int32, device=DEV)
    kb.check_descriptor(variant(q_lens=_t(q_lens)), f)
    kb.check_descriptor(variant(key_pos0=_t(kp0), q_pos=_t(q_pos)), f)
    kb.check_descriptor(base, f)
    torch.cuda.synchronize()
    assert int(f.cpu().item()) == kb.KVD_CHECK_Q_LENS | kb.KVD_CHECK_SHARD
