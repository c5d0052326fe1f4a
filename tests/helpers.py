"""Shared test helpers: wrap a workload for the oracle, gather dense K/V."""
import numpy as np

import oracle
from kv_cached_decode_amd import workloads

ORACLE_DT = {"bf16": oracle.ORACLE_BF16, "f32": oracle.ORACLE_F32, "f64": oracle.ORACLE_F64}


def bf16_bits_to_f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def pool_as_f64(w, pool):
    if w.spec.kv_dtype == "bf16":
        return bf16_bits_to_f64(pool)
    return pool.astype(np.float64)


_WORKLOAD_Q_LENS = object()


def oracle_cache(w, seq_lens=None, q_tokens=None, k_pool=None, v_pool=None, block_table=None,
                 dtype=None, window=0, key_pos0=None, q_pos=None, q_lens=_WORKLOAD_Q_LENS):
    """An OracleCache over copies of the workload's pools (or the given ones);
    ragged chunk lengths default to the workload's."""
    if q_lens is _WORKLOAD_Q_LENS:
        q_lens = w.q_lens
    s = w.spec
    dt = dtype or s.kv_dtype
    kp = np.array(w.k_pool if k_pool is None else k_pool, copy=True)
    vp = np.array(w.v_pool if v_pool is None else v_pool, copy=True)
    if dt == "f64" and kp.dtype != np.float64:
        kp, vp = pool_as_f64(w, kp), pool_as_f64(w, vp)
    return oracle.OracleCache(
        num_seqs=s.num_seqs, q_tokens=q_tokens or s.q_tokens, n_q_heads=s.n_q_heads,
        n_kv_heads=s.n_kv_heads, head_dim=s.head_dim, block_size=s.block_size,
        k_pool=np.ascontiguousarray(kp), v_pool=np.ascontiguousarray(vp),
        block_table=np.ascontiguousarray(w.block_table if block_table is None else block_table),
        seq_lens=np.ascontiguousarray(w.seq_lens if seq_lens is None else seq_lens, dtype=np.int32),
        cache_dtype=ORACLE_DT[dt], window=window, key_pos0=key_pos0, q_pos=q_pos, q_lens=q_lens)


def gather(pool_f64, table_row, bs, kvh, n):
    """Dense [n][D] rows of one kv head of one sequence, positions 0..n-1."""
    pos = np.arange(n)
    blk = table_row[pos // bs]
    return pool_f64[blk, kvh, pos % bs, :]


def small(name):
    return workloads.make_workload(workloads.small_variant(name))
