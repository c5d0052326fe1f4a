"""The C ABI on the host (no GPU): the library loads, exports every entry
point the header declares, and rejects bad descriptors before launching
anything."""
import ctypes
import os
import re

import pytest

from kv_cached_decode_amd import binding as kb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")

pytestmark = pytest.mark.skipif(not os.path.exists(kb.LIB_PATH), reason="libkvd.so not built")


def header_functions():
    """Every function declared in include/*.h."""
    names = set()
    for f in sorted(os.listdir(INCLUDE)):
        if f.endswith(".h"):
            text = re.sub(r"/\*.*?\*/", "", open(os.path.join(INCLUDE, f)).read(), flags=re.S)
            names |= set(re.findall(r"\b(kvd_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_header_and_binding_agree():
    assert header_functions() == sorted(kb.EXPORTED)


def test_every_declared_symbol_is_exported():
    L = ctypes.CDLL(kb.LIB_PATH)
    for name in header_functions():
        assert hasattr(L, name), name


def test_status_strings_and_version():
    assert kb.status_name(0) == "KVD_OK"
    assert kb.status_name(4) == "KVD_ERR_WORKSPACE"
    assert kb.status_name(99) == "KVD_ERR_UNKNOWN"
    assert kb.lib().kvd_abi_version() == 3


FAKE = 0x100000   # never dereferenced: every case below fails validation first


def desc(**kw):
    d = dict(num_seqs=2, q_tokens_per_seq=1, n_q_heads=8, n_kv_heads=2, head_dim=128,
             block_size=16, num_blocks=64, max_blocks_per_seq=8, max_seq_len=100,
             kv_dtype=kb.KVD_KV_BF16, window=0, k_cache=FAKE, v_cache=FAKE + 0x10000, block_table=FAKE + 0x20000,
             seq_lens=FAKE + 0x30000)
    d.update(kw)
    return kb.KvdPagedKV(**d)


BAD = [
    (dict(num_seqs=-1), kb.KVD_ERR_SHAPE),
    (dict(q_tokens_per_seq=0), kb.KVD_ERR_SHAPE),
    (dict(q_tokens_per_seq=1025), kb.KVD_ERR_UNSUPPORTED),
    (dict(n_q_heads=6, n_kv_heads=4), kb.KVD_ERR_SHAPE),
    (dict(n_kv_heads=0), kb.KVD_ERR_SHAPE),
    (dict(head_dim=96), kb.KVD_ERR_UNSUPPORTED),
    (dict(head_dim=8), kb.KVD_ERR_UNSUPPORTED),
    (dict(block_size=0), kb.KVD_ERR_UNSUPPORTED),
    (dict(block_size=24), kb.KVD_ERR_UNSUPPORTED),
    (dict(block_size=2048), kb.KVD_ERR_UNSUPPORTED),
    (dict(num_blocks=0), kb.KVD_ERR_SHAPE),
    (dict(num_blocks=2 ** 30, n_q_heads=8, n_kv_heads=2), kb.KVD_ERR_UNSUPPORTED),   # 2^31 pool rows
    (dict(max_seq_len=0), kb.KVD_ERR_SHAPE),
    (dict(q_tokens_per_seq=4, max_seq_len=3), kb.KVD_ERR_SHAPE),
    (dict(q_lens=FAKE + 0x60001), kb.KVD_ERR_SHAPE),         # misaligned chunk lengths
    (dict(max_seq_len=129), kb.KVD_ERR_SHAPE),            # > 8 blocks * 16
    (dict(kv_dtype=2), kb.KVD_ERR_UNSUPPORTED),
    (dict(window=-1), kb.KVD_ERR_SHAPE),
    (dict(k_cache=0), kb.KVD_ERR_NULL),
    (dict(block_table=0), kb.KVD_ERR_NULL),
    (dict(seq_lens=0), kb.KVD_ERR_NULL),
    (dict(k_cache=FAKE + 8), kb.KVD_ERR_SHAPE),           # misaligned
    (dict(q_pos=FAKE + 0x40002), kb.KVD_ERR_SHAPE),       # misaligned shard positions
    (dict(q_tokens_per_seq=4, max_seq_len=3, key_pos0=FAKE + 0x40000), kb.KVD_ERR_SHAPE),
]


@pytest.mark.parametrize("kw,status", BAD, ids=[str(k) for k, _ in BAD])
def test_bad_descriptor_rejected_before_launch(kw, status):
    d = desc(**kw)
    L = kb.lib()
    ws = ctypes.c_void_p(FAKE)
    st = L.kvd_decode_attention(ctypes.byref(d), FAKE, FAKE, 0.0, ws, 1 << 30, None)
    assert st == status, kb.last_error()
    assert kb.last_error()
    st = L.kvd_rope_append_kv(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 10000.0, 0, None)
    assert st == status, kb.last_error()
    st = L.kvd_decode_step(ctypes.byref(d), FAKE, FAKE, FAKE, None, FAKE, 10000.0, 0, 0.0, None, ws,
                           1 << 30, None)
    assert st == status, kb.last_error()
    st = L.kvd_decode_attention_lse(ctypes.byref(d), FAKE, FAKE, FAKE, 0.0, None, ws, 1 << 30, None)
    assert st == status, kb.last_error()
    assert L.kvd_decode_attention_workspace_size(ctypes.byref(d)) == ctypes.c_size_t(-1).value


def test_null_descriptor():
    L = kb.lib()
    assert L.kvd_decode_attention(None, FAKE, FAKE, 0.0, None, 0, None) == kb.KVD_ERR_NULL
    assert L.kvd_rope_append_kv(None, FAKE, FAKE, FAKE, FAKE, 1e4, 0, None) == kb.KVD_ERR_NULL
    assert L.kvd_decode_step(None, FAKE, FAKE, FAKE, None, FAKE, 1e4, 0, 0.0, None, None, 0,
                             None) == kb.KVD_ERR_NULL


def test_bad_call_arguments():
    L = kb.lib()
    d = desc(max_blocks_per_seq=64, max_seq_len=1000)
    assert L.kvd_rope_append_kv(ctypes.byref(d), 0, FAKE, FAKE, FAKE, 1e4, 0, None) == kb.KVD_ERR_NULL
    assert L.kvd_rope_append_kv(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, -1.0, 0, None) == kb.KVD_ERR_SHAPE
    assert L.kvd_rope_append_kv(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, float("inf"), 0, None) == kb.KVD_ERR_SHAPE
    assert L.kvd_rope_append_kv(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 1e4, 2, None) == kb.KVD_ERR_UNSUPPORTED
    assert L.kvd_decode_attention(ctypes.byref(d), 0, FAKE, 0.0, None, 0, None) == kb.KVD_ERR_NULL
    assert L.kvd_decode_attention(ctypes.byref(d), FAKE, FAKE, float("nan"), None, 0, None) == kb.KVD_ERR_SHAPE
    need = L.kvd_decode_attention_workspace_size(ctypes.byref(d))
    assert need > 0
    assert L.kvd_decode_attention(ctypes.byref(d), FAKE, FAKE, 0.0, None, 0, None) == kb.KVD_ERR_WORKSPACE
    assert L.kvd_decode_attention(ctypes.byref(d), FAKE, FAKE, 0.0, FAKE, need - 1, None) == kb.KVD_ERR_WORKSPACE
    assert L.kvd_decode_attention(ctypes.byref(d), FAKE, FAKE, 0.0, FAKE + 16, need, None) == kb.KVD_ERR_WORKSPACE
    bad_kernel = kb.KvdAttnOptions(0, 7)
    assert L.kvd_decode_attention_ex(ctypes.byref(d), FAKE, FAKE, 0.0, ctypes.byref(bad_kernel), FAKE,
                                     need, None) == kb.KVD_ERR_UNSUPPORTED


def test_decode_step_bad_arguments():
    """The fused step checks the union of the two calls' arguments; q_rot may
    be NULL, out may not."""
    L = kb.lib()
    d = desc(max_blocks_per_seq=64, max_seq_len=1000)
    need = L.kvd_decode_attention_workspace_size(ctypes.byref(d))

    def step(q=FAKE, k=FAKE, v=FAKE, q_rot=None, out=FAKE, base=1e4, layout=0, scale=0.0, opt=None,
             ws=FAKE, nbytes=need):
        return L.kvd_decode_step(ctypes.byref(d), q, k, v, q_rot, out, base, layout, scale, opt, ws,
                                 nbytes, None)

    assert step(q=0) == kb.KVD_ERR_NULL
    assert step(k=0) == kb.KVD_ERR_NULL
    assert step(out=0) == kb.KVD_ERR_NULL
    assert step(q_rot=FAKE + 2) == kb.KVD_ERR_SHAPE
    assert step(base=0.0) == kb.KVD_ERR_SHAPE
    assert step(layout=5) == kb.KVD_ERR_UNSUPPORTED
    assert step(scale=float("inf")) == kb.KVD_ERR_SHAPE
    assert step(ws=None, nbytes=0) == kb.KVD_ERR_WORKSPACE
    assert step(nbytes=need - 1) == kb.KVD_ERR_WORKSPACE
    assert step(opt=ctypes.byref(kb.KvdAttnOptions(0, 9))) == kb.KVD_ERR_UNSUPPORTED


def test_empty_batch_is_a_noop():
    L = kb.lib()
    d = desc(num_seqs=0, k_cache=0, v_cache=0, block_table=0, seq_lens=0)
    assert L.kvd_decode_attention(ctypes.byref(d), 0, 0, 0.0, None, 0, None) == kb.KVD_OK
    assert L.kvd_rope_append_kv(ctypes.byref(d), 0, 0, 0, 0, 1e4, 0, None) == kb.KVD_OK
    assert L.kvd_decode_step(ctypes.byref(d), 0, 0, 0, None, 0, 1e4, 0, 0.0, None, None, 0,
                             None) == kb.KVD_OK
    assert L.kvd_decode_attention_workspace_size(ctypes.byref(d)) == 0


def _plan(d, splits=0, kernel=0):
    s, k, kern = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    o = kb.KvdAttnOptions(splits, kernel)
    st = kb.lib().kvd_decode_attention_plan(ctypes.byref(d), ctypes.byref(o), ctypes.byref(s),
                                            ctypes.byref(k), ctypes.byref(kern))
    assert st == 0, kb.last_error()
    return s.value, k.value, kern.value


@pytest.mark.parametrize("max_len", [1, 2, 17, 255, 256, 257, 4097, 8193, 16388, 131073])
@pytest.mark.parametrize("B,T,Hq,Hkv", [(1, 1, 4, 4), (16, 1, 32, 8), (64, 1, 16, 8), (4, 1, 64, 8),
                                        (32, 4, 32, 8)])
def test_plan_covers_every_key(max_len, B, T, Hq, Hkv):
    if max_len < T:
        return
    bs = 16
    d = desc(num_seqs=B, q_tokens_per_seq=T, n_q_heads=Hq, n_kv_heads=Hkv,
             max_blocks_per_seq=(max_len + bs - 1) // bs, max_seq_len=max_len)
    for forced in (0, 1, 3, 1000):
        s, k, _ = _plan(d, forced, kernel=1)
        assert s >= 1 and k >= 1
        assert s * k >= max_len, "splits must cover every key"
        assert (s - 1) * k < max_len, "no split may start past the longest sequence"
        if forced:
            assert s <= max(forced, -(-max_len // (4094 * bs)))
        ws = kb.lib().kvd_decode_attention_workspace_size_ex(ctypes.byref(d),
                                                             ctypes.byref(kb.KvdAttnOptions(forced, 1)))
        rows = B * T * Hq
        if s == 1:
            assert ws == 0
        else:
            assert ws >= rows * s * (128 + 2) * 4


@pytest.mark.parametrize("B,T,Hq,Hkv", [(16, 1, 32, 8), (4, 1, 64, 8), (32, 4, 32, 8), (64, 1, 16, 8),
                                        (16, 1, 32, 32)])
def test_matrix_core_plan(B, T, Hq, Hkv):
    """The matrix-core kernel covers every key with its splits and is the
    automatic choice for every bf16 cache of head_dim 128, one query row per
    kv head included."""
    d = desc(num_seqs=B, q_tokens_per_seq=T, n_q_heads=Hq, n_kv_heads=Hkv, max_blocks_per_seq=1024,
             max_seq_len=16384)
    for forced in (0, 1, 3, 1000):
        s, k, kern = _plan(d, forced, kernel=2)
        assert kern == 2 and s * k >= 16384 and (s - 1) * k < 16384
        if forced:
            assert s <= forced
    _, _, kern = _plan(d, 0, 0)
    assert kern == 2, "bf16, head_dim 128: the matrix cores, whatever the rows per kv head"


def test_lse_and_merge_arguments():
    L = kb.lib()
    d = desc(max_blocks_per_seq=64, max_seq_len=1000)
    need = L.kvd_decode_attention_workspace_size(ctypes.byref(d))
    assert L.kvd_decode_attention_lse(ctypes.byref(d), FAKE, FAKE, None, 0.0, None, FAKE, need,
                                      None) == kb.KVD_ERR_NULL
    assert L.kvd_decode_attention_lse(ctypes.byref(d), FAKE, FAKE, FAKE + 2, 0.0, None, FAKE, need,
                                      None) == kb.KVD_ERR_SHAPE
    M = L.kvd_merge_partials
    assert M(0, 10, 128, FAKE, FAKE, FAKE, None, None) == kb.KVD_ERR_SHAPE
    assert M(4097, 10, 128, FAKE, FAKE, FAKE, None, None) == kb.KVD_ERR_UNSUPPORTED
    assert M(2, -1, 128, FAKE, FAKE, FAKE, None, None) == kb.KVD_ERR_SHAPE
    assert M(2, 10, 0, FAKE, FAKE, FAKE, None, None) == kb.KVD_ERR_SHAPE
    assert M(2, 10, 128, None, FAKE, FAKE, None, None) == kb.KVD_ERR_NULL
    assert M(2, 10, 128, FAKE, FAKE, FAKE + 1, None, None) == kb.KVD_ERR_SHAPE
    assert M(2, 0, 128, None, None, None, None, None) == kb.KVD_OK          # nothing to merge


def test_shard_without_new_tokens_plans():
    """A context-parallel shard may hold fewer keys than new tokens, even none
    at all; it still gets a plan and a workspace size."""
    d = desc(q_tokens_per_seq=4, max_seq_len=0, q_pos=FAKE + 0x40000, key_pos0=FAKE + 0x50000)
    s, k, kern = _plan(d)
    assert s >= 1 and k >= 1
    assert kb.lib().kvd_decode_attention_workspace_size(ctypes.byref(d)) != ctypes.c_size_t(-1).value


@pytest.mark.parametrize("T", [5, 17, 64, 512, 1024])
def test_prefill_plan(T):
    """More than 16 query rows per kv head on the matrix cores: the prefill
    kernel, whose splits cover every key; ragged chunks may leave the
    length bound below T."""
    d = desc(num_seqs=8, q_tokens_per_seq=T, n_q_heads=32, n_kv_heads=8, max_blocks_per_seq=400,
             max_seq_len=max(T, 4096 + T))
    s, k, kern = _plan(d)
    assert kern == 2 and s * k >= 4096 + T and (s - 1) * k < 4096 + T
    d = desc(num_seqs=2, q_tokens_per_seq=T, max_seq_len=1, q_lens=FAKE + 0x60000)
    assert _plan(d)[0] >= 1


def test_noalloc_step_validates_before_anything_runs():
    """kvd_decode_step_noalloc checks like kvd_decode_step, then refuses a plan
    whose split-K partials exceed its static scratch (KVD_NOALLOC_SCRATCH_BYTES)
    before it looks up the scratch or launches anything."""
    L = kb.lib()

    def step(d, splits=0):
        opt = ctypes.byref(kb.KvdAttnOptions(splits, 0)) if splits else None
        return L.kvd_decode_step_noalloc(ctypes.byref(d), FAKE, FAKE, FAKE, None, FAKE, 1e4, 0, 0.0, opt,
                                         None)

    assert L.kvd_decode_step_noalloc(None, FAKE, FAKE, FAKE, None, FAKE, 1e4, 0, 0.0, None,
                                     None) == kb.KVD_ERR_NULL
    for kw, status in BAD:
        assert step(desc(**kw)) == status, (kw, kb.last_error())
    assert step(desc(num_seqs=0, k_cache=0, v_cache=0, block_table=0, seq_lens=0)) == kb.KVD_OK
    # the full continuous batch (64 sequences x 16 q heads, up to 8193 keys)
    # at 20 splits: 1024 rows x 20 x (128 + 2) x 4 bytes = 10.6 MB > 8 MiB
    big = desc(num_seqs=64, n_q_heads=16, n_kv_heads=8, max_blocks_per_seq=513, max_seq_len=8193,
               num_blocks=40000)
    need = L.kvd_decode_attention_workspace_size_ex(ctypes.byref(big), ctypes.byref(kb.KvdAttnOptions(20, 0)))
    assert need > kb.NOALLOC_SCRATCH_BYTES
    assert step(big, 20) == kb.KVD_ERR_WORKSPACE
    assert "static scratch" in kb.last_error()


def test_check_descriptor_arguments():
    """kvd_check_descriptor validates on the host like the other calls and
    needs an aligned flag word; an empty batch launches nothing."""
    L = kb.lib()
    assert L.kvd_check_descriptor(None, FAKE, None) == kb.KVD_ERR_NULL
    for kw, status in BAD:
        assert L.kvd_check_descriptor(ctypes.byref(desc(**kw)), FAKE, None) == status, kw
    d = desc(max_blocks_per_seq=64, max_seq_len=1000)
    assert L.kvd_check_descriptor(ctypes.byref(d), None, None) == kb.KVD_ERR_NULL
    assert L.kvd_check_descriptor(ctypes.byref(d), FAKE + 2, None) == kb.KVD_ERR_SHAPE
    empty = desc(num_seqs=0, k_cache=0, v_cache=0, block_table=0, seq_lens=0)
    assert L.kvd_check_descriptor(ctypes.byref(empty), FAKE, None) == kb.KVD_OK
