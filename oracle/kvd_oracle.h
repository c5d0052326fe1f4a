/*
 * kvd_oracle.h -- plain, slow CPU reference for KV-cached decode attention (fp64).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load or call this code.  It shares no
 * source, header, helper or table with the GPU library: it has its own cache
 * descriptor, its own bf16 rounding and its own RoPE, written from the
 * definitions on the pages:
 *
 *   - ferric-core `examples/generate.rs` (docs.rs page, module doc comment):
 *     each decode step projects only the new token, appends its K/V to a
 *     per-layer cache and attends the single query against the whole cache;
 *     RoPE uses the token's absolute position; the result must equal a full
 *     non-cached causal recompute over the prefix.
 *   - the same file, `step_gpu`: the append happens before attention and the
 *     key count is the cache length after the append; `mha_decode_t` takes
 *     separate query-head and kv-head counts.
 *   - Ferrum Infer README, "Key Optimizations": batched RoPE with per-item
 *     positions, paged KV through a block table, one launch for all batch
 *     items, split-K flash decoding.
 *
 * Everything is computed in fp64; the only roundings are into the cache dtype
 * (round-to-nearest-even, once, from the fp64 rotated value).
 *
 * Parity status: every function here is pinned by the CPU tests (closed
 * forms, invariants, the full causal recompute, library routines); none is
 * "parity unpinned".
 */
#ifndef KVD_ORACLE_H
#define KVD_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Cache element types understood by the oracle.  ORACLE_F64 exists only so
 * that the oracle can be checked against the full recompute without any
 * rounding in the cache. */
enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_F64 = 2 };

/* RoPE pairings: HALF rotates (x[i], x[i + D/2]); INTERLEAVED rotates
 * (x[2i], x[2i + 1]). */
enum { ORACLE_ROPE_HALF = 0, ORACLE_ROPE_INTERLEAVED = 1 };

typedef struct {
    int32_t num_seqs;           /* B */
    int32_t q_tokens;           /* T new tokens per sequence (1 = decode) */
    int32_t n_q_heads;          /* Hq */
    int32_t n_kv_heads;         /* Hkv, divides Hq */
    int32_t head_dim;           /* D, even */
    int32_t block_size;         /* bs, keys per cache block */
    int32_t num_blocks;         /* blocks in each pool */
    int32_t max_blocks_per_seq; /* row stride of block_table */
    int32_t cache_dtype;        /* ORACLE_F32 / ORACLE_BF16 / ORACLE_F64 */
    void *k_pool;               /* [num_blocks][Hkv][bs][D] */
    void *v_pool;               /* [num_blocks][Hkv][bs][D] */
    const int32_t *block_table; /* [B][max_blocks_per_seq] */
    const int32_t *seq_lens;    /* [B] keys per sequence, new tokens included */
    int32_t window;             /* sliding window in keys (0 = whole cache): the
                                   query at position p sees keys
                                   max(0, p - window + 1) .. p */
    /* Context-parallel shard (both may be NULL): the cache holds only the
     * keys at global positions key_pos0[b] .. key_pos0[b] + seq_lens[b] - 1
     * (local key i is global key key_pos0[b] + i), and new token t of
     * sequence b sits at global position q_pos[b] + t.  NULL means
     * key_pos0 = 0 and q_pos = seq_lens - T (the whole cache). */
    const int32_t *key_pos0;    /* [B] */
    const int32_t *q_pos;       /* [B] */
    /* Ragged new tokens (may be NULL = T for every sequence): sequence b has
     * q_lens[b] <= T new tokens; rows t >= q_lens[b] are padding, appended
     * nowhere and answered with out = 0, lse = -inf.  Without q_pos the new
     * tokens are the last q_lens[b] keys of the cache. */
    const int32_t *q_lens;      /* [B] */
} oracle_cache;

/* Return codes: 0 ok, nonzero = bad descriptor (nothing written). */

/* RoPE of `n_rows` rows of `n_heads` head vectors (length head_dim) at the
 * given absolute positions (one per row).  y may alias x. */
int oracle_rope(const double *x, double *y, int32_t n_rows, int32_t n_heads,
                int32_t head_dim, const int64_t *positions, double base,
                int32_t layout);

/* RoPE the new q and k at their global position p = q_pos[b] + t (default
 * seq_lens[b] - T + t), store round(k_rot) and round(v) into the slot of
 * local key p - key_pos0[b] that the block table names, and return the
 * rotated q in fp64.  A token whose local slot lies outside 0 .. seq_lens[b]
 * - 1 (a context-parallel shard that does not hold it) is rotated into q_rot
 * and not stored.  q: [B][T][Hq][D]; k, v: [B][T][Hkv][D]; q_rot:
 * [B][T][Hq][D]. */
int oracle_rope_append_kv(const oracle_cache *c, const float *q,
                          const float *k, const float *v, double *q_rot,
                          double base, int32_t layout);

/* Attention of every query row against the cache as it stands.  Query t of
 * sequence b, at global position p, sees the keys at global positions
 * 0 .. p (inclusive), or the last `window` of them, that the cache holds.
 * out: [B][T][Hq][D]; lse (optional, may be NULL): [B][T][Hq] natural-log
 * log-sum-exp of the scaled scores; wsum (optional): [B][T][Hq] sum of the
 * normalised softmax weights (1 up to rounding).  A row that sees no key
 * gets out = 0, lse = -inf and wsum = 0. */
int oracle_decode_attention(const oracle_cache *c, const double *q_rot,
                            double scale, double *out, double *lse,
                            double *wsum);

/* The same attention, restricted to the query rows listed in `rows` (flat
 * indices b*T*Hq + t*Hq + h); out/lse get n_rows entries, in list order. */
int oracle_decode_attention_rows(const oracle_cache *c, const double *q_rot,
                                 double scale, const int64_t *rows,
                                 int64_t n_rows, double *out, double *lse);

/* fp64 -> bf16 bits, round to nearest even, single rounding. */
uint16_t oracle_bf16_from_double(double x);
double oracle_bf16_to_double(uint16_t bits);

/* Threads the attention loops run on. */
int oracle_threads(void);

#ifdef __cplusplus
}
#endif
#endif
