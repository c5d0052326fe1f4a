"""ctypes access to the fp64 CPU oracle (oracle/kvd_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
benchmark's CPU-baseline leg, never by the product library.  Inputs are numpy
arrays on the host; the oracle works on host copies of the cache pools.
"""
import ctypes
import os

import numpy as np

from .build import LIB, build

ORACLE_F32, ORACLE_BF16, ORACLE_F64 = 0, 1, 2
ROPE_HALF, ROPE_INTERLEAVED = 0, 1

_DTYPES = {ORACLE_F32: np.float32, ORACLE_BF16: np.uint16, ORACLE_F64: np.float64}


class _Cache(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("q_tokens", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("cache_dtype", ctypes.c_int32),
        ("k_pool", ctypes.c_void_p),
        ("v_pool", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("seq_lens", ctypes.c_void_p),
        ("window", ctypes.c_int32),
        ("key_pos0", ctypes.c_void_p),
        ("q_pos", ctypes.c_void_p),
        ("q_lens", ctypes.c_void_p),
    ]


_lib = None
# KVD_ORACLE_LIB names another build of kvd_oracle.c (the sanitizer build)
_lib_path = os.environ.get("KVD_ORACLE_LIB") or LIB


def use_library(path=None):
    """Point the bindings at another build of kvd_oracle.c (None = the default
    one).  Used by the tests that check that planted mistakes are caught."""
    global _lib, _lib_path
    _lib_path = path or LIB
    _lib = None


def lib():
    global _lib
    if _lib is None:
        if _lib_path == LIB and not os.path.exists(LIB):
            build()
        L = ctypes.CDLL(_lib_path)
        P = ctypes.c_void_p
        L.oracle_rope.argtypes = [P, P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                  P, ctypes.c_double, ctypes.c_int32]
        L.oracle_rope_append_kv.argtypes = [ctypes.POINTER(_Cache), P, P, P, P,
                                            ctypes.c_double, ctypes.c_int32]
        L.oracle_decode_attention.argtypes = [ctypes.POINTER(_Cache), P, ctypes.c_double,
                                              P, P, P]
        L.oracle_decode_attention_rows.argtypes = [ctypes.POINTER(_Cache), P, ctypes.c_double,
                                                   P, ctypes.c_int64, P, P]
        L.oracle_bf16_from_double.argtypes = [ctypes.c_double]
        L.oracle_bf16_from_double.restype = ctypes.c_uint16
        L.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_double.restype = ctypes.c_double
        L.oracle_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _req(a, dtype):
    a = np.asarray(a)
    if a.dtype != dtype or not a.flags["C_CONTIGUOUS"]:
        raise TypeError(f"oracle expects a C-contiguous {np.dtype(dtype)} array, got {a.dtype}")
    return a


class OracleCache:
    """Host-side paged cache as the oracle sees it.

    k_pool / v_pool: [num_blocks][Hkv][bs][D] arrays (float32, uint16 bf16 bits
    or float64), modified in place by rope_append_kv.
    """

    def __init__(self, *, num_seqs, q_tokens, n_q_heads, n_kv_heads, head_dim, block_size,
                 k_pool, v_pool, block_table, seq_lens, cache_dtype, window=0, key_pos0=None,
                 q_pos=None, q_lens=None):
        self.cache_dtype = cache_dtype
        dt = _DTYPES[cache_dtype]
        self.k_pool = _req(k_pool, dt)
        self.v_pool = _req(v_pool, dt)
        self.block_table = _req(block_table, np.int32)
        self.seq_lens = _req(seq_lens, np.int32)
        self.num_seqs, self.q_tokens = int(num_seqs), int(q_tokens)
        self.n_q_heads, self.n_kv_heads, self.head_dim = int(n_q_heads), int(n_kv_heads), int(head_dim)
        self.block_size = int(block_size)
        # context-parallel shard: global position of local key 0 and of new token 0
        self.key_pos0 = None if key_pos0 is None else _req(np.ascontiguousarray(key_pos0, np.int32), np.int32)
        self.q_pos = None if q_pos is None else _req(np.ascontiguousarray(q_pos, np.int32), np.int32)
        # ragged new tokens per sequence (rows past q_lens[b] are padding)
        self.q_lens = None if q_lens is None else _req(np.ascontiguousarray(q_lens, np.int32), np.int32)
        self._c = _Cache(self.num_seqs, self.q_tokens, self.n_q_heads, self.n_kv_heads,
                         self.head_dim, self.block_size, int(self.k_pool.shape[0]),
                         int(self.block_table.shape[1]) if self.block_table.ndim == 2 else 0,
                         cache_dtype, _ptr(self.k_pool), _ptr(self.v_pool),
                         _ptr(self.block_table), _ptr(self.seq_lens), int(window),
                         _ptr(self.key_pos0), _ptr(self.q_pos), _ptr(self.q_lens))

    def rope_append_kv(self, q, k, v, base, layout=ROPE_HALF):
        q = _req(q, np.float32)
        k = _req(k, np.float32)
        v = _req(v, np.float32)
        q_rot = np.zeros(q.shape, np.float64)
        rc = lib().oracle_rope_append_kv(ctypes.byref(self._c), _ptr(q), _ptr(k), _ptr(v),
                                         _ptr(q_rot), float(base), int(layout))
        if rc:
            raise ValueError(f"oracle_rope_append_kv: bad descriptor (rc={rc})")
        return q_rot

    def decode_attention(self, q_rot, scale=None, want_lse=False, want_wsum=False):
        q_rot = _req(q_rot, np.float64)
        if scale is None:
            scale = 1.0 / np.sqrt(self.head_dim)
        rows = self.num_seqs * self.q_tokens * self.n_q_heads
        out = np.zeros((self.num_seqs, self.q_tokens, self.n_q_heads, self.head_dim), np.float64)
        lse = np.zeros(rows, np.float64) if want_lse else None
        wsum = np.zeros(rows, np.float64) if want_wsum else None
        rc = lib().oracle_decode_attention(ctypes.byref(self._c), _ptr(q_rot), float(scale),
                                           _ptr(out), _ptr(lse), _ptr(wsum))
        if rc:
            raise ValueError(f"oracle_decode_attention: bad descriptor (rc={rc})")
        res = [out]
        if want_lse:
            res.append(lse.reshape(self.num_seqs, self.q_tokens, self.n_q_heads))
        if want_wsum:
            res.append(wsum.reshape(self.num_seqs, self.q_tokens, self.n_q_heads))
        return res[0] if len(res) == 1 else tuple(res)

    def decode_attention_rows(self, q_rot, rows, scale=None):
        """Attention for selected flat rows (b*T*Hq + t*Hq + h) only."""
        q_rot = _req(q_rot, np.float64)
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        if scale is None:
            scale = 1.0 / np.sqrt(self.head_dim)
        out = np.zeros((rows.size, self.head_dim), np.float64)
        lse = np.zeros(rows.size, np.float64)
        rc = lib().oracle_decode_attention_rows(ctypes.byref(self._c), _ptr(q_rot), float(scale),
                                                _ptr(rows), rows.size, _ptr(out), _ptr(lse))
        if rc:
            raise ValueError(f"oracle_decode_attention_rows: bad descriptor (rc={rc})")
        return out, lse


def rope(x, positions, base, layout=ROPE_HALF):
    """RoPE of x[n_rows][n_heads][D] (float64) at one absolute position per row."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    pos = np.ascontiguousarray(positions, dtype=np.int64)
    n_rows, n_heads, D = x.shape
    if pos.shape != (n_rows,):
        raise ValueError("one position per row")
    y = np.empty_like(x)
    rc = lib().oracle_rope(_ptr(x), _ptr(y), n_rows, n_heads, D, _ptr(pos), float(base), int(layout))
    if rc:
        raise ValueError("oracle_rope: bad arguments")
    return y


def bf16_from_double(x: float) -> int:
    return int(lib().oracle_bf16_from_double(float(x)))


def bf16_to_double(bits: int) -> float:
    return float(lib().oracle_bf16_to_double(int(bits)))


def threads() -> int:
    return int(lib().oracle_threads())
