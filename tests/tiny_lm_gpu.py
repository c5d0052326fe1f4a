"""The tiny decoder LM of ferric-core `examples/generate.rs`, decoded on the GPU
with the library's RoPE + append and paged decode attention inside.

The layers around the attention step (RMSNorm, the q/k/v and output
projections, the SiLU-gated MLP, the LM head) run as plain torch fp32 ops on
the device: they are the model the step sits in, not part of it.  Every layer
has its own K and V pool; all layers share one block table.  Pools start
filled with NaN, so a read of a slot that was never appended shows up in the
logits.
"""
import numpy as np
import torch

from kv_cached_decode_amd import binding as kb

DEV = "cuda:0"


def _rmsnorm(x, w, eps):
    return x * torch.rsqrt((x * x).mean(dim=-1, keepdim=True) + eps) * w


class GpuTinyLM:
    def __init__(self, w, cfg, num_seqs, capacity, block_size, kv_dtype, block_table):
        self.cfg, self.B, self.capacity = cfg, int(num_seqs), int(capacity)
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(DEV)
        self.emb, self.wln, self.wlm = t(w["emb"]), t(w["wln"]), t(w["wlm"])
        self.layers = [{k: t(v) for k, v in L.items()} for L in w["layers"]]
        self.table = np.ascontiguousarray(block_table, np.int32)
        n_blocks = int(self.table.max()) + 1
        shape = (n_blocks, cfg.n_heads, int(block_size), cfg.head_dim)
        dt = torch.bfloat16 if kv_dtype == "bf16" else torch.float32
        self.pools = [(torch.full(shape, float("nan"), dtype=dt, device=DEV),
                       torch.full(shape, float("nan"), dtype=dt, device=DEV))
                      for _ in self.layers]
        self.lens = np.zeros(self.B, np.int32)

    def step(self, tokens, seqs=None):
        """tokens: [n][T] token ids for sequences `seqs` (default all, in
        order).  Appends T tokens per listed sequence and returns float64
        logits [n][T][vocab]; query t sees the cache up to its own token."""
        cfg = self.cfg
        H, dh, d = cfg.n_heads, cfg.head_dim, cfg.d_model
        seqs = np.arange(self.B) if seqs is None else np.asarray(seqs, np.int64)
        toks = np.asarray(tokens, np.int64).reshape(len(seqs), -1)
        n, T = toks.shape
        self.lens[seqs] += T
        seq_lens = torch.from_numpy(np.ascontiguousarray(self.lens[seqs], np.int32)).to(DEV)
        table = torch.from_numpy(np.ascontiguousarray(self.table[seqs])).to(DEV)
        x = self.emb[torch.from_numpy(toks.reshape(-1)).to(DEV)]            # [n*T][d]
        for L, (kp, vp) in zip(self.layers, self.pools):
            kv = kb.PagedKV(kp, vp, table, seq_lens, H, T, self.capacity)
            a = _rmsnorm(x, L["wn1"], cfg.eps)
            q = (a @ L["wq"]).view(n, T, H, dh).contiguous()
            k = (a @ L["wk"]).view(n, T, H, dh).contiguous()
            v = (a @ L["wv"]).view(n, T, H, dh).contiguous()
            q_rot = kb.rope_append_kv(kv, q, k, v, rope_base=cfg.rope_base)
            att = kb.decode_attention(kv, q_rot)
            x = x + att.view(n * T, d) @ L["wo"]
            b = _rmsnorm(x, L["wn2"], cfg.eps)
            g = b @ L["wg"]
            x = x + (g * torch.sigmoid(g) * (b @ L["wu"])) @ L["wd"]
        logits = _rmsnorm(x, self.wln, cfg.eps) @ self.wlm
        torch.cuda.synchronize()
        return logits.view(n, T, -1).double().cpu().numpy()

    def rollback(self, seq, n_keep):
        """Drop a sequence's cached tokens past n_keep (rejected draft tokens):
        only the length changes; the slots are overwritten by later appends."""
        self.lens[seq] = n_keep
