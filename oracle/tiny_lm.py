"""fp64 reference for the tiny decoder LM that ferric-core `examples/generate.rs`
decodes through a KV cache.

TEST INFRASTRUCTURE ONLY: imported by the tests, never by the product library.

The page builds a small Llama-style LM and decodes it one token at a time,
checking every step's logits against a full non-cached recompute over the
prefix so far (module doc comment; `forward_cpu`, `layer_cpu`, `step_gpu`).
One layer, as the page composes it:

    a   = RMSNorm(x) * wn1
    q,k = RoPE(a Wq), RoPE(a Wk) at each token's absolute position; v = a Wv
    x   = x + CausalMHA(q, k, v) Wo
    b   = RMSNorm(x) * wn2
    x   = x + (SiLU(b Wg) * (b Wu)) Wd            (SiLU(z) = z * sigmoid(z))

then logits = (RMSNorm(x) * wln) Wlm.  The page shows neither the RMSNorm
nor the RoPE body; the readings taken here are RMSNorm(x) = x / sqrt(mean(x^2)
+ eps) and RoPE as the library's HALF pairing, theta_i = base^(-2i/D).

Two forms are provided:

* `full_forward` -- the page's reference: the whole prefix at once, dense
  causal attention, no cache.  fp64 throughout.
* `CachedLM` -- the page's incremental form: per token, project it alone,
  RoPE + append into a paged cache, and attend the single query against the
  cache.  The RoPE/append/attention step is the C oracle's
  (`oracle_rope_append_kv`, `oracle_decode_attention`); everything around it
  is fp64 numpy.  With an fp64 cache it must reproduce `full_forward` up to
  rounding (the page's exactness claim); with a bf16 or fp32 cache it is the
  exact reference for a GPU decode that stores the same rounded cache.
"""
import numpy as np

from . import ORACLE_BF16, ORACLE_F32, ORACLE_F64, ROPE_HALF, OracleCache, rope

_POOL_DTYPE = {ORACLE_F32: np.float32, ORACLE_BF16: np.uint16, ORACLE_F64: np.float64}


def rmsnorm(x, w, eps):
    """x / sqrt(mean(x^2) + eps) * w over the last axis (fp64)."""
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * np.asarray(w, np.float64)


def silu(z):
    return z / (1.0 + np.exp(-z))


def causal_mha(q, k, v):
    """q, k, v: [P][H][dh] fp64 (positions 0..P-1, one kv head per q head, as
    the page's `mha_causal` is called).  Row i attends rows 0..i with scale
    1/sqrt(dh).  Dense: the full score matrix, masked, softmax per row."""
    P, H, dh = q.shape
    out = np.zeros_like(q)
    for h in range(H):
        s = q[:, h, :] @ k[:, h, :].T / np.sqrt(dh)
        s[np.triu(np.ones((P, P), bool), k=1)] = -np.inf
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ v[:, h, :]
    return out


def _f64(a):
    return np.asarray(a, np.float64)


def _proj(a, W, f32):
    y = a @ _f64(W)
    return y.astype(np.float32).astype(np.float64) if f32 else y


def layer_full(x, L, cfg, qkv_f32=False):
    """One layer over a whole prefix x [P][d] (fp64), positions 0..P-1.
    qkv_f32 rounds the q/k/v projections to float32 before RoPE, as a step
    whose RoPE/append entry point takes float32 inputs does."""
    P = x.shape[0]
    H, dh = cfg.n_heads, cfg.head_dim
    a = rmsnorm(x, L["wn1"], cfg.eps)
    pos = np.arange(P)
    q = rope(_proj(a, L["wq"], qkv_f32).reshape(P, H, dh), pos, cfg.rope_base, ROPE_HALF)
    k = rope(_proj(a, L["wk"], qkv_f32).reshape(P, H, dh), pos, cfg.rope_base, ROPE_HALF)
    v = _proj(a, L["wv"], qkv_f32).reshape(P, H, dh)
    x = x + causal_mha(q, k, v).reshape(P, H * dh) @ _f64(L["wo"])
    b = rmsnorm(x, L["wn2"], cfg.eps)
    g = b @ _f64(L["wg"])
    return x + (silu(g) * (b @ _f64(L["wu"]))) @ _f64(L["wd"])


def full_forward(ids, w, cfg, all_rows=False, qkv_f32=False):
    """Logits of the last token of `ids` (or of every position with
    all_rows=True) by the full non-cached recompute."""
    x = _f64(w["emb"])[np.asarray(ids, np.int64)]
    for L in w["layers"]:
        x = layer_full(x, L, cfg, qkv_f32)
    logits = rmsnorm(x, w["wln"], cfg.eps) @ _f64(w["wlm"])
    return logits if all_rows else logits[-1]


class CachedLM:
    """Incremental decoding of B sequences through per-layer paged caches held
    by the C oracle.  Each `step` feeds one token per sequence (its next
    position) and returns fp64 logits [B][vocab].  The cache stores rotated
    keys and values rounded to `cache_dtype`."""

    def __init__(self, w, cfg, num_seqs, capacity, block_size=4, cache_dtype=ORACLE_F64,
                 block_table=None):
        self.w, self.cfg, self.B = w, cfg, int(num_seqs)
        self.bs = int(block_size)
        self.max_blocks = -(-int(capacity) // self.bs)
        if block_table is None:
            block_table = np.arange(self.B * self.max_blocks, dtype=np.int32).reshape(self.B, -1)
        self.table = np.ascontiguousarray(block_table, dtype=np.int32)
        n_blocks = int(self.table.max()) + 1
        shape = (n_blocks, cfg.n_heads, self.bs, cfg.head_dim)
        dt = _POOL_DTYPE[cache_dtype]
        self.pools = [(np.zeros(shape, dt), np.zeros(shape, dt)) for _ in w["layers"]]
        self.cache_dtype = cache_dtype
        self.lens = np.zeros(self.B, np.int32)     # tokens cached per sequence

    def step(self, tokens, seqs=None):
        """Feed tokens[i] to sequence seqs[i] (default: every sequence, in
        order); only the listed sequences advance, as in continuous batching."""
        cfg = self.cfg
        H, dh = cfg.n_heads, cfg.head_dim
        seqs = np.arange(self.B) if seqs is None else np.asarray(seqs, np.int64)
        B = len(seqs)
        self.lens[seqs] += 1                       # the new token is appended first
        seq_lens = np.ascontiguousarray(self.lens[seqs], dtype=np.int32)
        table = np.ascontiguousarray(self.table[seqs])
        x = _f64(self.w["emb"])[np.asarray(tokens, np.int64)]
        for L, (kp, vp) in zip(self.w["layers"], self.pools):
            a = rmsnorm(x, L["wn1"], cfg.eps)
            q = (a @ _f64(L["wq"])).astype(np.float32).reshape(B, 1, H, dh)
            k = (a @ _f64(L["wk"])).astype(np.float32).reshape(B, 1, H, dh)
            v = (a @ _f64(L["wv"])).astype(np.float32).reshape(B, 1, H, dh)
            c = OracleCache(num_seqs=B, q_tokens=1, n_q_heads=H, n_kv_heads=H, head_dim=dh,
                            block_size=self.bs, k_pool=kp, v_pool=vp, block_table=table,
                            seq_lens=seq_lens, cache_dtype=self.cache_dtype)
            q_rot = c.rope_append_kv(q, k, v, cfg.rope_base, ROPE_HALF)
            att = c.decode_attention(q_rot).reshape(B, H * dh)
            x = x + att @ _f64(L["wo"])
            b = rmsnorm(x, L["wn2"], cfg.eps)
            g = b @ _f64(L["wg"])
            x = x + (silu(g) * (b @ _f64(L["wu"]))) @ _f64(L["wd"])
        return rmsnorm(x, self.w["wln"], cfg.eps) @ _f64(self.w["wlm"])
