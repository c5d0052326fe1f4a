"""Full non-cached causal recompute in numpy fp64 -- the pages' own check.

ferric-core `examples/generate.rs` (module doc comment and the `forward_cpu` /
`layer_cpu` pair) validates KV-cached decoding by recomputing the whole prefix
without a cache: RoPE every position at its own index, causal multi-head
attention over the full matrix, and take the last row(s).  This module is that
recompute, written as dense matrix algebra (complex-number RoPE, a masked score
matrix, scipy's softmax) so that it shares no formulation with the oracle's
per-key loops.  It pins the oracle; it is not itself the oracle.
"""
import numpy as np
from scipy.special import softmax


def rope_complex(x, positions, base, layout):
    """x: [P][H][D] float64; rotate each head vector at its row's position by
    multiplying the pair (a, c) viewed as a + ic with exp(i * pos * theta_i)."""
    P, H, D = x.shape
    half = D // 2
    theta = np.power(float(base), -np.arange(half, dtype=np.float64) * 2.0 / D)
    rot = np.exp(1j * np.outer(np.asarray(positions, np.float64), theta))[:, None, :]
    if layout == 0:
        z = x[..., :half] + 1j * x[..., half:]
        z = z * rot
        return np.concatenate([z.real, z.imag], axis=-1)
    z = x[..., 0::2] + 1j * x[..., 1::2]
    z = z * rot
    out = np.empty_like(x)
    out[..., 0::2] = z.real
    out[..., 1::2] = z.imag
    return out


def causal_attention(q, k, v, scale=None):
    """q: [P][Hq][D], k/v: [P][Hkv][D], positions 0..P-1, causal (a query sees
    itself and everything before it).  Returns [P][Hq][D] and the log-sum-exp."""
    P, Hq, D = q.shape
    Hkv = k.shape[1]
    g = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    kk = np.repeat(k, g, axis=1)   # query head h reads kv head h // g
    vv = np.repeat(v, g, axis=1)
    s = np.einsum("ihd,jhd->hij", q, kk) * scale
    mask = np.triu(np.ones((P, P), bool), k=1)
    s[:, mask] = -np.inf
    w = softmax(s, axis=-1)
    out = np.einsum("hij,jhd->ihd", w, vv)
    m = s.max(axis=-1, keepdims=True)
    lse = (m + np.log(np.exp(s - m).sum(axis=-1, keepdims=True)))[..., 0]
    return out, lse.T


def recompute_last_rows(q_raw, k_raw, v_raw, T, base, layout, store=None):
    """Full recompute over one sequence's raw prefix (positions 0..P-1) and
    return the last T rows.  `store` optionally rounds the rotated keys and the
    values the way the cache stores them (e.g. to float32)."""
    P = q_raw.shape[0]
    pos = np.arange(P)
    q = rope_complex(q_raw.astype(np.float64), pos, base, layout)
    k = rope_complex(k_raw.astype(np.float64), pos, base, layout)
    v = v_raw.astype(np.float64)
    if store is not None:
        k, v = store(k), store(v)
    out, lse = causal_attention(q, k, v)
    return out[P - T:], lse[P - T:]
