"""Thin ctypes binding over libkvd.so (include/kvd.h).

Argument marshalling only: every step of the decode path runs in the HIP
kernels of libkvd.so.  PyTorch provides device memory and the stream; the
functions take torch CUDA (HIP) tensors, check their dtype, device, shape and
contiguity, and pass raw pointers plus torch's current stream to the C ABI.
There is no fallback: if the library is not built, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

# the library built next to this file; KVD_LIB_PATH names another build of it
# (the host-sanitizer build the CPU tests load)
LIB_PATH = os.environ.get("KVD_LIB_PATH") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                           "libkvd.so")

KVD_OK, KVD_ERR_NULL, KVD_ERR_SHAPE, KVD_ERR_UNSUPPORTED, KVD_ERR_WORKSPACE, KVD_ERR_LAUNCH = range(6)
KVD_KV_F32, KVD_KV_BF16 = 0, 1
KVD_ROPE_HALF, KVD_ROPE_INTERLEAVED = 0, 1
KVD_KERNEL_AUTO, KVD_KERNEL_VALU, KVD_KERNEL_MFMA = 0, 1, 2

EXPORTED = [
    "kvd_rope_append_kv", "kvd_decode_attention", "kvd_decode_attention_ex",
    "kvd_decode_attention_workspace_size", "kvd_decode_attention_workspace_size_ex",
    "kvd_decode_attention_plan", "kvd_decode_step", "kvd_decode_step_noalloc",
    "kvd_decode_attention_lse", "kvd_merge_partials", "kvd_status_string", "kvd_last_error",
    "kvd_abi_version", "kvd_probe_stream_read", "kvd_check_descriptor",
]
KVD_CHECK_SEQ_LEN, KVD_CHECK_BLOCK_ID, KVD_CHECK_Q_LENS, KVD_CHECK_SHARD = 1, 2, 4, 8

# bytes of the per-device static scratch of kvd_decode_step_noalloc (kvd.h)
NOALLOC_SCRATCH_BYTES = 8 << 20
# the arrival counters at the head of every split-K workspace (kvd.h)
WORKSPACE_COUNTER_BYTES = 16384


class KvdPagedKV(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("q_tokens_per_seq", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("max_seq_len", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("k_cache", ctypes.c_void_p),
        ("v_cache", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("seq_lens", ctypes.c_void_p),
        ("key_pos0", ctypes.c_void_p),
        ("q_pos", ctypes.c_void_p),
        ("q_lens", ctypes.c_void_p),
    ]


class KvdAttnOptions(ctypes.Structure):
    _fields_ = [("num_splits", ctypes.c_int32), ("kernel", ctypes.c_int32)]


class KvdError(RuntimeError):
    def __init__(self, status, where, detail):
        self.status = status
        super().__init__(f"{where}: {status_name(status)}: {detail}")


_lib = None


def lib():
    """The loaded libkvd.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m kv_cached_decode_amd.build` "
                               "(there is no non-HIP fallback)")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        KV = ctypes.POINTER(KvdPagedKV)
        OPT = ctypes.POINTER(KvdAttnOptions)
        L.kvd_rope_append_kv.argtypes = [KV, P, P, P, P, ctypes.c_double, I32, P]
        L.kvd_rope_append_kv.restype = I32
        L.kvd_decode_attention.argtypes = [KV, P, P, ctypes.c_float, P, SZ, P]
        L.kvd_decode_attention.restype = I32
        L.kvd_decode_attention_ex.argtypes = [KV, P, P, ctypes.c_float, OPT, P, SZ, P]
        L.kvd_decode_attention_ex.restype = I32
        L.kvd_decode_attention_workspace_size.argtypes = [KV]
        L.kvd_decode_attention_workspace_size.restype = SZ
        L.kvd_decode_attention_workspace_size_ex.argtypes = [KV, OPT]
        L.kvd_decode_attention_workspace_size_ex.restype = SZ
        L.kvd_decode_attention_plan.argtypes = [KV, OPT, ctypes.POINTER(I32), ctypes.POINTER(I32),
                                                ctypes.POINTER(I32)]
        L.kvd_decode_attention_plan.restype = I32
        L.kvd_decode_step.argtypes = [KV, P, P, P, P, P, ctypes.c_double, I32, ctypes.c_float, OPT,
                                      P, SZ, P]
        L.kvd_decode_step.restype = I32
        L.kvd_decode_step_noalloc.argtypes = [KV, P, P, P, P, P, ctypes.c_double, I32, ctypes.c_float,
                                              OPT, P]
        L.kvd_decode_step_noalloc.restype = I32
        L.kvd_decode_attention_lse.argtypes = [KV, P, P, P, ctypes.c_float, OPT, P, SZ, P]
        L.kvd_decode_attention_lse.restype = I32
        L.kvd_merge_partials.argtypes = [I32, ctypes.c_int64, I32, P, P, P, P, P]
        L.kvd_merge_partials.restype = I32
        L.kvd_status_string.argtypes = [I32]
        L.kvd_status_string.restype = ctypes.c_char_p
        L.kvd_last_error.argtypes = []
        L.kvd_last_error.restype = ctypes.c_char_p
        L.kvd_abi_version.restype = I32
        L.kvd_check_descriptor.argtypes = [KV, P, P]
        L.kvd_check_descriptor.restype = I32
        L.kvd_probe_stream_read.argtypes = [P, SZ, I32, I32, I32, P, P]
        L.kvd_probe_stream_read.restype = I32
        _lib = L
    return _lib


def status_name(status: int) -> str:
    return lib().kvd_status_string(int(status)).decode()


def last_error() -> str:
    return lib().kvd_last_error().decode()


def _check(status, where):
    if status != KVD_OK:
        raise KvdError(status, where, last_error())


def _stream_handle(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _need(t: torch.Tensor, name: str, dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


@dataclass
class PagedKV:
    """One layer's paged KV cache plus the batch it serves (kvd_paged_kv).

    k_cache, v_cache: [num_blocks][Hkv][bs][D], torch.bfloat16 or torch.float32.
    block_table:      int32 [B][max_blocks_per_seq].
    seq_lens:         int32 [B], keys per sequence including the T new tokens.
    max_seq_len:      host-side bound on seq_lens (sizes the split-K plan).
    window:           sliding window in keys (0 = the whole cache).
    key_pos0, q_pos:  int32 [B] or None: a context-parallel shard holding the
                      keys at global positions key_pos0 .. key_pos0 +
                      seq_lens - 1, with new token t at global q_pos + t.
    q_lens:           int32 [B] or None: ragged chunks, q_lens[b] <= T new
                      tokens per sequence (rows past them are padding).
    """
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    block_table: torch.Tensor
    seq_lens: torch.Tensor
    n_q_heads: int
    q_tokens_per_seq: int
    max_seq_len: int
    window: int = 0
    key_pos0: Optional[torch.Tensor] = None
    q_pos: Optional[torch.Tensor] = None
    q_lens: Optional[torch.Tensor] = None

    def __post_init__(self):
        if self.k_cache.dtype not in (torch.bfloat16, torch.float32):
            raise TypeError("cache must be bfloat16 or float32")
        _need(self.k_cache, "k_cache", self.k_cache.dtype)
        _need(self.v_cache, "v_cache", self.k_cache.dtype, self.k_cache.shape)
        _need(self.block_table, "block_table", torch.int32)
        _need(self.seq_lens, "seq_lens", torch.int32)
        if self.k_cache.dim() != 4 or self.block_table.dim() != 2 or self.seq_lens.dim() != 1:
            raise ValueError("k/v_cache must be 4-D, block_table 2-D and seq_lens 1-D")
        if self.block_table.shape[0] != self.seq_lens.shape[0]:
            raise ValueError("block_table and seq_lens disagree on the batch size")
        for name in ("key_pos0", "q_pos", "q_lens"):
            t = getattr(self, name)
            if t is not None:
                _need(t, name, torch.int32, (self.num_seqs,))

    @property
    def num_seqs(self):
        return int(self.seq_lens.shape[0])

    @property
    def n_kv_heads(self):
        return int(self.k_cache.shape[1])

    @property
    def block_size(self):
        return int(self.k_cache.shape[2])

    @property
    def head_dim(self):
        return int(self.k_cache.shape[3])

    def struct(self) -> KvdPagedKV:
        return KvdPagedKV(
            self.num_seqs, int(self.q_tokens_per_seq), int(self.n_q_heads), self.n_kv_heads,
            self.head_dim, self.block_size, int(self.k_cache.shape[0]),
            int(self.block_table.shape[1]), int(self.max_seq_len),
            KVD_KV_BF16 if self.k_cache.dtype == torch.bfloat16 else KVD_KV_F32, int(self.window),
            self.k_cache.data_ptr(), self.v_cache.data_ptr(), self.block_table.data_ptr(),
            self.seq_lens.data_ptr(),
            self.key_pos0.data_ptr() if self.key_pos0 is not None else None,
            self.q_pos.data_ptr() if self.q_pos is not None else None,
            self.q_lens.data_ptr() if self.q_lens is not None else None)

    def q_shape(self):
        return (self.num_seqs, self.q_tokens_per_seq, self.n_q_heads, self.head_dim)

    def kv_shape(self):
        return (self.num_seqs, self.q_tokens_per_seq, self.n_kv_heads, self.head_dim)


def _new_out(kv: PagedKV, like):
    """An output buffer allocated here: zeros for a batch of ragged chunks,
    whose padding rows the library leaves as they are (so they read as 0)."""
    return torch.zeros_like(like) if kv.q_lens is not None else torch.empty_like(like)


def _opts(num_splits, kernel):
    if not num_splits and not kernel:
        return None
    return ctypes.byref(KvdAttnOptions(int(num_splits), int(kernel)))


def rope_append_kv(kv: PagedKV, q, k, v, q_rot=None, rope_base=10000.0, layout=KVD_ROPE_HALF,
                   stream=None):
    """kvd_rope_append_kv: rotate q/k at each new token's position, append the
    new K/V rows to the cache.  Returns q_rot (allocated if not given)."""
    _need(q, "q", torch.float32, kv.q_shape())
    _need(k, "k", torch.float32, kv.kv_shape())
    _need(v, "v", torch.float32, kv.kv_shape())
    if q_rot is None:
        q_rot = torch.empty_like(q)
    _need(q_rot, "q_rot", torch.float32, kv.q_shape())
    d = kv.struct()
    _check(lib().kvd_rope_append_kv(ctypes.byref(d), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                    q_rot.data_ptr(), float(rope_base), int(layout),
                                    _stream_handle(stream)), "kvd_rope_append_kv")
    return q_rot


def decode_attention_workspace_size(kv: PagedKV, num_splits=0, kernel=KVD_KERNEL_AUTO) -> int:
    d = kv.struct()
    n = lib().kvd_decode_attention_workspace_size_ex(ctypes.byref(d), _opts(num_splits, kernel))
    if n == ctypes.c_size_t(-1).value:
        raise KvdError(KVD_ERR_SHAPE, "kvd_decode_attention_workspace_size", last_error())
    return int(n)


def decode_attention_plan(kv: PagedKV, num_splits=0, kernel=KVD_KERNEL_AUTO):
    """(splits, keys per split, kernel family) the library would use."""
    d = kv.struct()
    s, kps, k = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(lib().kvd_decode_attention_plan(ctypes.byref(d), _opts(num_splits, kernel),
                                           ctypes.byref(s), ctypes.byref(kps), ctypes.byref(k)),
           "kvd_decode_attention_plan")
    return s.value, kps.value, k.value


_ws_cache = {}


def workspace(kv: PagedKV, num_splits=0, kernel=KVD_KERNEL_AUTO, stream=None):
    """A cached device workspace big enough for this descriptor (None if none
    is needed), one per (device, stream): calls that share a workspace must
    not run concurrently, so work on different streams gets different
    buffers.  The buffer is allocated on that stream (torch's allocator then
    reuses a replaced one only for work ordered after it there), zeroed once
    (its head holds arrival counters that every call leaves at zero).
    Allocation happens here, outside the library."""
    n = decode_attention_workspace_size(kv, num_splits, kernel)
    if n == 0:
        return None
    dev = kv.k_cache.device
    handle = _stream_handle(stream)
    key = (dev, handle)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < n:
        s = stream if stream is not None else torch.cuda.current_stream(dev)
        with torch.cuda.stream(s) if isinstance(s, torch.cuda.Stream) else _nullcontext():
            buf = torch.zeros(n, dtype=torch.uint8, device=dev)   # the arrival counters start at zero
        _ws_cache[key] = buf
    return buf


class _nullcontext:
    def __enter__(self):
        return self

    def __exit__(self, *a):
        return False


def decode_attention(kv: PagedKV, q_rot, out=None, softmax_scale=0.0, workspace_buf=None,
                     num_splits=0, kernel=KVD_KERNEL_AUTO, stream=None):
    """kvd_decode_attention(_ex): out[b,t,h] = softmax(scale q.K^T) V over the
    keys query t of sequence b can see.  Returns out."""
    _need(q_rot, "q_rot", torch.float32, kv.q_shape())
    if out is None:
        out = _new_out(kv, q_rot)
    _need(out, "out", torch.float32, kv.q_shape())
    if workspace_buf is None:
        workspace_buf = workspace(kv, num_splits, kernel, stream)
    wptr = workspace_buf.data_ptr() if workspace_buf is not None else None
    wbytes = workspace_buf.numel() * workspace_buf.element_size() if workspace_buf is not None else 0
    d = kv.struct()
    _check(lib().kvd_decode_attention_ex(ctypes.byref(d), q_rot.data_ptr(), out.data_ptr(),
                                         float(softmax_scale), _opts(num_splits, kernel), wptr,
                                         wbytes, _stream_handle(stream)),
           "kvd_decode_attention")
    return out


def decode_step(kv: PagedKV, q, k, v, out=None, q_rot=None, want_q_rot=False, rope_base=10000.0,
                layout=KVD_ROPE_HALF, softmax_scale=0.0, workspace_buf=None, num_splits=0,
                kernel=KVD_KERNEL_AUTO, stream=None):
    """kvd_decode_step: RoPE + append + decode attention in one call (one
    kernel on matrix-core plans).  Returns out, or (out, q_rot) when q_rot is
    given or want_q_rot is set."""
    _need(q, "q", torch.float32, kv.q_shape())
    _need(k, "k", torch.float32, kv.kv_shape())
    _need(v, "v", torch.float32, kv.kv_shape())
    if out is None:
        out = _new_out(kv, q)
    _need(out, "out", torch.float32, kv.q_shape())
    if q_rot is None and want_q_rot:
        q_rot = torch.empty_like(q)
    if q_rot is not None:
        _need(q_rot, "q_rot", torch.float32, kv.q_shape())
    if workspace_buf is None:
        workspace_buf = workspace(kv, num_splits, kernel, stream)
    wptr = workspace_buf.data_ptr() if workspace_buf is not None else None
    wbytes = workspace_buf.numel() * workspace_buf.element_size() if workspace_buf is not None else 0
    d = kv.struct()
    _check(lib().kvd_decode_step(ctypes.byref(d), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                 q_rot.data_ptr() if q_rot is not None else None, out.data_ptr(),
                                 float(rope_base), int(layout), float(softmax_scale),
                                 _opts(num_splits, kernel), wptr, wbytes, _stream_handle(stream)),
           "kvd_decode_step")
    return (out, q_rot) if q_rot is not None else out


def decode_step_noalloc(kv: PagedKV, q, k, v, out, q_rot=None, rope_base=10000.0,
                        layout=KVD_ROPE_HALF, softmax_scale=0.0, num_splits=0,
                        kernel=KVD_KERNEL_AUTO, stream=None):
    """kvd_decode_step_noalloc: the whole step with the split-K partials in
    the library's static per-device scratch; the caller passes every output
    buffer (nothing is allocated here either).  Returns out."""
    _need(q, "q", torch.float32, kv.q_shape())
    _need(k, "k", torch.float32, kv.kv_shape())
    _need(v, "v", torch.float32, kv.kv_shape())
    _need(out, "out", torch.float32, kv.q_shape())
    if q_rot is not None:
        _need(q_rot, "q_rot", torch.float32, kv.q_shape())
    d = kv.struct()
    _check(lib().kvd_decode_step_noalloc(ctypes.byref(d), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                         q_rot.data_ptr() if q_rot is not None else None,
                                         out.data_ptr(), float(rope_base), int(layout),
                                         float(softmax_scale), _opts(num_splits, kernel),
                                         _stream_handle(stream)),
           "kvd_decode_step_noalloc")
    return out


def decode_attention_lse(kv: PagedKV, q_rot, out=None, lse=None, softmax_scale=0.0, workspace_buf=None,
                         num_splits=0, kernel=KVD_KERNEL_AUTO, stream=None):
    """kvd_decode_attention_lse: decode attention plus each row's natural-log
    log-sum-exp (a context-parallel shard's partial).  Returns (out, lse)."""
    _need(q_rot, "q_rot", torch.float32, kv.q_shape())
    if out is None:
        out = _new_out(kv, q_rot)
    if lse is None:
        shape = kv.q_shape()[:3]
        if kv.q_lens is not None:      # padding rows are left as they are: -inf here
            lse = torch.full(shape, float("-inf"), dtype=torch.float32, device=q_rot.device)
        else:
            lse = torch.empty(shape, dtype=torch.float32, device=q_rot.device)
    _need(out, "out", torch.float32, kv.q_shape())
    _need(lse, "lse", torch.float32, kv.q_shape()[:3])
    if workspace_buf is None:
        workspace_buf = workspace(kv, num_splits, kernel, stream)
    wptr = workspace_buf.data_ptr() if workspace_buf is not None else None
    wbytes = workspace_buf.numel() * workspace_buf.element_size() if workspace_buf is not None else 0
    d = kv.struct()
    _check(lib().kvd_decode_attention_lse(ctypes.byref(d), q_rot.data_ptr(), out.data_ptr(),
                                          lse.data_ptr(), float(softmax_scale), _opts(num_splits, kernel),
                                          wptr, wbytes, _stream_handle(stream)),
           "kvd_decode_attention_lse")
    return out, lse


def merge_partials(outs, lses, out=None, lse_out=None, stream=None):
    """kvd_merge_partials: outs fp32 [P][rows..][D], lses fp32 [P][rows..] ->
    (out [rows..][D], lse [rows..])."""
    if outs.dim() < 2 or lses.shape != outs.shape[:-1]:
        raise ValueError("outs must be [P][...][D] and lses [P][...]")
    _need(outs, "outs", torch.float32)
    _need(lses, "lses", torch.float32)
    P, D = int(outs.shape[0]), int(outs.shape[-1])
    rows = int(lses[0].numel())
    if out is None:
        out = torch.empty(outs.shape[1:], dtype=torch.float32, device=outs.device)
    if lse_out is None:
        lse_out = torch.empty(lses.shape[1:], dtype=torch.float32, device=outs.device)
    _need(out, "out", torch.float32, outs.shape[1:])
    _need(lse_out, "lse_out", torch.float32, lses.shape[1:])
    _check(lib().kvd_merge_partials(P, rows, D, outs.data_ptr(), lses.data_ptr(), out.data_ptr(),
                                    lse_out.data_ptr(), _stream_handle(stream)),
           "kvd_merge_partials")
    return out, lse_out


def check_descriptor(kv: PagedKV, flags=None, stream=None):
    """kvd_check_descriptor: the descriptor's device-side contract checked on
    the GPU; returns the flag word (a 1-element int32 device tensor, cleared
    here when allocated here) with KVD_CHECK_* bits for the violations."""
    if flags is None:
        flags = torch.zeros(1, dtype=torch.int32, device=kv.seq_lens.device)
    _need(flags, "flags", torch.int32, (1,))
    d = kv.struct()
    _check(lib().kvd_check_descriptor(ctypes.byref(d), flags.data_ptr(), _stream_handle(stream)),
           "kvd_check_descriptor")
    return flags


def probe_stream_read(buf, workgroups, threads=256, unroll=4, sink=None, stream=None):
    """kvd_probe_stream_read (include/kvd_probe.h): one read of the whole of
    `buf` (a contiguous device tensor) by a plain streaming kernel."""
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=buf.device)
    nbytes = buf.numel() * buf.element_size()
    st = lib().kvd_probe_stream_read(buf.data_ptr(), nbytes, int(workgroups), int(threads), int(unroll),
                                     sink.data_ptr(), _stream_handle(stream))
    if st != 0:
        raise RuntimeError(f"kvd_probe_stream_read failed with code {st}")
    return sink
