/*
 * kvd.h -- C ABI of the KV-cached decode-attention library (libkvd.so),
 * hand-written HIP kernels for MI355X (gfx950).
 *
 * The operation is the single-token decode step of a decoder layer's
 * attention as the ferric-core `examples/generate.rs` page defines it (module
 * doc comment; `step_gpu`): the new token's Q and K are rotated by RoPE at the
 * token's absolute position, the new K/V rows are appended to the per-layer
 * cache, and each query attends against the whole cache (`mha_decode_t`, which
 * takes separate query-head and kv-head counts).  The Ferrum Infer README
 * ("Key Optimizations") adds what a serving batch needs: per-item positions in
 * one launch, one launch for all batch items, a paged block pool addressed
 * through a block table, and split-K flash decoding for long caches.  The
 * ferrox-models index (`speculative`) adds verifying several draft tokens per
 * sequence in one batched pass.
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers (hipMalloc'd or torch-owned
 *     memory on the current device) unless a comment says otherwise; the
 *     descriptor itself lives in host memory and is read during the call only.
 *   - The caller owns every buffer.  The library never allocates, frees or
 *     synchronises, and keeps no state between calls except caches that
 *     change no result: a per-thread error string, a per-thread copy of the
 *     last RoPE frequency table (theta_i for the last base and head_dim), a
 *     per-device cache of the compute-unit count and, for
 *     kvd_decode_step_noalloc, the per-device address of its static scratch.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream).  It launches kernels and returns.
 *   - Arguments are validated on the host first.  On any error nothing is
 *     enqueued and a non-zero kvd_status is returned; kvd_last_error() then
 *     describes it.  Device-side contract violations (a block id outside the
 *     pool, seq_lens[b] above max_seq_len) are undefined behaviour.
 */
#ifndef KVD_H
#define KVD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes (int32_t on the wire). */
enum {
    KVD_OK = 0,
    KVD_ERR_NULL = 1,        /* a required pointer is NULL */
    KVD_ERR_SHAPE = 2,       /* inconsistent sizes */
    KVD_ERR_UNSUPPORTED = 3, /* valid but not built (head_dim, dtype, ...) */
    KVD_ERR_WORKSPACE = 4,   /* workspace missing or too small */
    KVD_ERR_LAUNCH = 5       /* the HIP runtime refused a launch */
};

/* Cache element types. */
enum { KVD_KV_F32 = 0, KVD_KV_BF16 = 1 };

/* RoPE pairings (the pages name a configurable RoPE layout in the ferrox
 * `config` module without defining it): HALF rotates (x[i], x[i + D/2]),
 * INTERLEAVED rotates (x[2i], x[2i + 1]), for i < D/2. */
enum { KVD_ROPE_HALF = 0, KVD_ROPE_INTERLEAVED = 1 };

/* Attention kernel families (kvd_attn_options.kernel). */
enum { KVD_KERNEL_AUTO = 0, KVD_KERNEL_VALU = 1, KVD_KERNEL_MFMA = 2 };

/*
 * The paged KV cache of one layer plus the batch it serves.
 *
 *   num_seqs            B, sequences in the batch (>= 0; 0 is a no-op).
 *   q_tokens_per_seq    T, new tokens per sequence: 1 = decode, >1 = verify of
 *                       a T-token draft or a prefill chunk, causal within it.
 *                       1..1024 (more than 16 query rows per kv head run
 *                       through the prefill kernel).
 *   n_q_heads           Hq; n_kv_heads Hkv; Hq % Hkv == 0.  Query head h
 *                       reads kv head h / (Hq / Hkv).
 *   head_dim            D in {16, 32, 64, 128, 256}.
 *   block_size          bs, keys per cache block: a power of two, 1..1024.
 *   num_blocks          blocks in each pool; num_blocks * n_kv_heads < 2^31.
 *   max_blocks_per_seq  row stride of block_table.
 *   max_seq_len         host-side upper bound on every seq_lens[b]; it sizes
 *                       the split-K plan (no device read is needed, so a call
 *                       can be captured in a HIP graph).
 *                       T <= max_seq_len <= max_blocks_per_seq * bs.
 *   kv_dtype            KVD_KV_BF16 or KVD_KV_F32.
 *   window              sliding window in keys, 0 = attend the whole cache: the
 *                       query at position p sees keys max(0, p - window + 1)
 *                       .. p (the ferrox-models kv_budget SlidingWindow).  The
 *                       append is unaffected; keys before every query's window
 *                       are not read.
 *   k_cache, v_cache    [num_blocks][Hkv][bs][D] each, element type kv_dtype,
 *                       16-byte aligned.  Key position p of sequence b lives in
 *                       block block_table[b][p / bs], slot p % bs.
 *   block_table         int32 [B][max_blocks_per_seq], physical block ids.
 *   seq_lens            int32 [B]: keys of each sequence INCLUDING its T new
 *                       tokens (seq_lens[b] >= T unless q_pos is given).  New
 *                       token t of sequence b
 *                       sits at position seq_lens[b] - T + t and its query
 *                       sees keys 0 .. seq_lens[b] - T + t.
 *   key_pos0, q_pos     context-parallel shard (CP/DCP, one of the parallel
 *                       modes of the ferrite page), both int32 [B] device
 *                       arrays or NULL.  The cache then holds only the keys at
 *                       global positions key_pos0[b] .. key_pos0[b] +
 *                       seq_lens[b] - 1 (local key i = global key key_pos0[b]
 *                       + i), and new token t sits at global position q_pos[b]
 *                       + t: its query sees the held keys at global positions
 *                       up to q_pos[b] + t (and inside the window).  NULL
 *                       means key_pos0 = 0 and q_pos = key_pos0 +
 *                       seq_lens - T, the whole cache; with q_pos given,
 *                       seq_lens[b] may be below T (a shard without the new
 *                       tokens).  kvd_rope_append_kv (and kvd_decode_step)
 *                       rotate at the global position and store at local
 *                       slot q_pos[b] + t - key_pos0[b] when it lies in
 *                       [0, seq_lens[b]); a shard that does not hold the
 *                       slot gets the rotated query and stores nothing (the
 *                       shard holding the token appends it).  A row that
 *                       sees no key of the shard gets out = 0 (and lse =
 *                       -inf from kvd_decode_attention_lse).
 *   q_lens              int32 [B] device array or NULL (= T for every
 *                       sequence): ragged chunks, sequence b brings q_lens[b]
 *                       <= T new tokens (chunked prefill with a different
 *                       chunk per sequence, drafts of different lengths).
 *                       They are the last q_lens[b] keys (or sit at q_pos[b]
 *                       + t); rows t >= q_lens[b] are padding: not appended,
 *                       and their q_rot, out and lse rows are left as they
 *                       are (not written).  seq_lens[b] >= q_lens[b].
 */
typedef struct kvd_paged_kv {
    int32_t num_seqs;
    int32_t q_tokens_per_seq;
    int32_t n_q_heads;
    int32_t n_kv_heads;
    int32_t head_dim;
    int32_t block_size;
    int32_t num_blocks;
    int32_t max_blocks_per_seq;
    int32_t max_seq_len;
    int32_t kv_dtype;
    int32_t window;
    void *k_cache;
    void *v_cache;
    const int32_t *block_table;
    const int32_t *seq_lens;
    const int32_t *key_pos0;
    const int32_t *q_pos;
    const int32_t *q_lens;
} kvd_paged_kv;

/*
 * RoPE + append (generate.rs `step_gpu`: `rope_off_t` on q and k at the token's
 * position, then the K/V rows are appended; Ferrum README: batched RoPE with
 * per-item positions, paged KV writes).
 *
 *   q      fp32 [B][T][Hq][D]  new queries before RoPE.
 *   k, v   fp32 [B][T][Hkv][D] new keys (before RoPE) and values.
 *   q_rot  fp32 [B][T][Hq][D]  rotated queries (may alias q).
 *   rope_base  theta_i = rope_base^(-2i/D); position p turns pair i by p*theta_i.
 *   layout     KVD_ROPE_HALF or KVD_ROPE_INTERLEAVED.
 *
 * Angles and rotations are evaluated in fp64; q_rot is that value rounded to
 * fp32, the cache receives it rounded to kv_dtype (round-to-nearest-even, a
 * single rounding), and v is stored rounded to kv_dtype.  Exactly the B*T
 * target slots of each pool are written.  Only seq_lens, block_table, the
 * shard positions (if any) and the pools are read from the descriptor's
 * device memory.
 */
int32_t kvd_rope_append_kv(const kvd_paged_kv *kv, const float *q, const float *k,
                           const float *v, float *q_rot, double rope_base,
                           int32_t layout, void *stream);

/* Tuning / testing knobs for decode attention.  A NULL pointer means all
 * automatic.  num_splits: 0 = automatic, else the number of key-range
 * partitions per (sequence, kv head).  kernel: KVD_KERNEL_*. */
typedef struct kvd_attn_options {
    int32_t num_splits;
    int32_t kernel;
} kvd_attn_options;

/* The counter region at the head of every split-K workspace (see
 * kvd_decode_attention); batches of more than 4096 (sequence, kv head) pairs
 * merge their splits in a second kernel instead. */
#define KVD_WORKSPACE_COUNTER_BYTES ((size_t)16384)

/* Bytes of device workspace kvd_decode_attention needs for this descriptor on
 * the current device (0 when no split-K partials are needed).  Returns
 * (size_t)-1 for an invalid descriptor.  The Ferrum Infer README ("Key
 * Optimizations") names split-K flash decoding for long caches; the pages
 * show no interface for its scratch, so the caller owns it, sized here. */
size_t kvd_decode_attention_workspace_size(const kvd_paged_kv *kv);
size_t kvd_decode_attention_workspace_size_ex(const kvd_paged_kv *kv,
                                              const kvd_attn_options *opt);

/* The plan kvd_decode_attention would use: key-range partitions per (seq, kv
 * head), keys per partition (at most; on a ragged batch whose units the
 * matrix-core decode kernel ranks, each sequence's partitions are equal
 * shares of its own range) and kernel family.  Any out pointer may be NULL.
 * The pages define no such call (the Ferrum Infer README only says split-K
 * switches on for long caches); it reports this library's choice. */
int32_t kvd_decode_attention_plan(const kvd_paged_kv *kv, const kvd_attn_options *opt,
                                  int32_t *num_splits, int32_t *keys_per_split,
                                  int32_t *kernel);

/*
 * Decode attention over the paged cache (generate.rs `mha_decode_t`; Ferrum
 * README: one launch for every batch item, block-table indirection, split-K
 * flash decoding with an online-softmax combine; ferrox `speculative`: all
 * draft tokens verified in one pass).
 *
 *   q_rot          fp32 [B][T][Hq][D] rotated queries.
 *   out            fp32 [B][T][Hq][D]
 *                  out = sum_j softmax_j(scale * q.K_j) V_j over the visible
 *                  keys j = 0 .. seq_lens[b] - T + t.
 *   softmax_scale  scale; 0 means 1/sqrt(D).
 *   workspace      device scratch of at least kvd_decode_attention_workspace_size
 *                  bytes (may be NULL when that is 0), 256-byte aligned.  Its
 *                  first KVD_WORKSPACE_COUNTER_BYTES hold arrival counters
 *                  (on a matrix-core decode plan of two splits the last
 *                  workgroup of each (sequence, kv head) to finish merges
 *                  the two itself; other plans merge in a second kernel):
 *                  they must be zero before a workspace is first used --
 *                  allocate it zeroed -- and every call leaves them zero
 *                  again, so one workspace serves calls of any shape, eager
 *                  or replayed in a HIP graph.  The rest is clobbered
 *                  scratch.  Calls that share a workspace must not run
 *                  concurrently.
 *
 * Accumulation is fp32; the cache is read in kv_dtype.  Cache slots past
 * seq_lens (tail slots, unused blocks) are never read, whatever they hold.
 * For a fixed plan the result is bitwise deterministic: the splits are
 * merged in a fixed order whichever finishes last.
 *
 * Arithmetic.  fp32 caches, and bf16 caches on the vector-ALU kernel: fp32
 * vector arithmetic on the cached values.  bf16 caches on the matrix cores
 * (head_dim 128, two or more query rows per kv head): fp32 accumulation; q
 * enters as a bf16 hi + lo pair (about 16 significant bits),
 * the softmax weights likewise for up to 16 query rows per kv head (normwise
 * error near 1e-6); with more rows P.V runs in fp16 (normwise error near
 * 1e-4), and a (sequence, row tile, split) unit whose V leaves fp16's range
 * -- an element beyond 65504, or none at or above 2^-14 -- is recomputed
 * with bf16 V and hi + lo weights.
 */
int32_t kvd_decode_attention(const kvd_paged_kv *kv, const float *q_rot, float *out,
                             float softmax_scale, void *workspace,
                             size_t workspace_bytes, void *stream);
int32_t kvd_decode_attention_ex(const kvd_paged_kv *kv, const float *q_rot, float *out,
                                float softmax_scale, const kvd_attn_options *opt,
                                void *workspace, size_t workspace_bytes, void *stream);

/*
 * Decode attention that also exports each row's log-sum-exp, the partial a
 * context-parallel shard hands to the merge (kvd_merge_partials).
 *
 *   lse    fp32 [B][T][Hq]: log(sum_j exp(scale * q.K_j)) in natural-log
 *          units over the keys the row sees in this cache; -inf (and out = 0)
 *          for a row that sees none.
 * Everything else as kvd_decode_attention_ex (same workspace size).
 */
int32_t kvd_decode_attention_lse(const kvd_paged_kv *kv, const float *q_rot, float *out,
                                 float *lse, float softmax_scale, const kvd_attn_options *opt,
                                 void *workspace, size_t workspace_bytes, void *stream);

/*
 * Merge n_parts partial attention results of the same rows (one per
 * context-parallel shard, gathered into one buffer):
 *     LSE = log sum_p exp(lse_p),  out = sum_p exp(lse_p - LSE) * out_p.
 *
 *   n_parts   >= 1 (at most 4096).
 *   rows      query rows per part (B*T*Hq); head_dim D as for the cache.
 *   outs      fp32 [n_parts][rows][D];  lses  fp32 [n_parts][rows].
 *   out       fp32 [rows][D];  lse_out fp32 [rows] or NULL.
 * Parts with lse = -inf drop out; a row with every part at -inf gets out = 0
 * and lse -inf.  out may not alias outs.
 */
int32_t kvd_merge_partials(int32_t n_parts, int64_t rows, int32_t head_dim, const float *outs,
                           const float *lses, float *out, float *lse_out, void *stream);

/*
 * The whole decode step in one call: kvd_rope_append_kv followed by
 * kvd_decode_attention_ex (generate.rs `step_gpu`: RoPE of the new q/k at the
 * token's position, the append, then `mha_decode_t` over the cache; the
 * Ferrum Infer README counts launches saved by fusing the steps of a decode).
 *
 *   q, k, v, rope_base, layout   as for kvd_rope_append_kv (q is NOT rotated
 *                                in place).
 *   q_rot   fp32 [B][T][Hq][D] receives the rotated queries, or NULL if the
 *           caller does not want them.
 *   out, softmax_scale, opt, workspace, workspace_bytes
 *           as for kvd_decode_attention_ex (same workspace size).
 *
 * Results (out, q_rot, the cache) are bitwise those of the two calls in a
 * row with the same plan.  When the plan uses the matrix-core decode kernel
 * (at most 16 query rows per kv head), the descriptor is not a
 * context-parallel shard and a split spans at most 2048 cache blocks, one
 * kernel does all of it (plus the split combine when there are several
 * splits): each workgroup rotates its own query rows, and the workgroup whose
 * key range holds the new tokens stores their K/V rows and uses them directly.
 * When it uses the prefill kernel (more than 16 query rows per kv head), the
 * RoPE/append kernel appends the new K/V rows and the prefill kernel rotates
 * the query rows it reads (the rotated queries make no round trip through
 * memory).  On both, pass q_rot = NULL unless the rotated queries are
 * wanted: writing them is extra work.  Otherwise (the vector-ALU kernel, or a
 * context-parallel shard or long split on the decode kernel) the RoPE/append
 * kernel runs first and, if q_rot is NULL, `out` holds the rotated queries in
 * between.
 */
int32_t kvd_decode_step(const kvd_paged_kv *kv, const float *q, const float *k, const float *v,
                        float *q_rot, float *out, double rope_base, int32_t layout,
                        float softmax_scale, const kvd_attn_options *opt, void *workspace,
                        size_t workspace_bytes, void *stream);

/*
 * kvd_decode_step for callers that cannot allocate device memory: code under
 * HIP graph capture, serving loops and harnesses that forbid hipMalloc.  The
 * split-K partials go to a static device array of KVD_NOALLOC_SCRATCH_BYTES
 * that the library holds on each GPU it runs on (until the process ends)
 * instead of a caller's workspace; nothing is allocated or freed.
 *
 *   Arguments and results as for kvd_decode_step, without the workspace.
 *   A plan needing more partial storage than KVD_NOALLOC_SCRATCH_BYTES
 *   (kvd_decode_attention_workspace_size_ex reports it) returns
 *   KVD_ERR_WORKSPACE and enqueues nothing.  A plan with several splits
 *   takes (head_dim + 2) * 4 bytes per (query row, split) pair, so 8 MiB
 *   holds about 16000 pairs at head_dim 128; plans of one split need none.
 *   Every call on one GPU shares that GPU's array (zero when the library is
 *   loaded; every call rewrites the partials it reads and leaves the
 *   arrival counters at its head zero, so nothing needs clearing between
 *   calls), so calls that may overlap on one GPU -- on different streams,
 *   or from different host threads without ordering -- race and must not be
 *   issued.
 *   The first call on a device looks the array's address up (a runtime query,
 *   no allocation); a failure there returns KVD_ERR_LAUNCH.
 */
#define KVD_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
int32_t kvd_decode_step_noalloc(const kvd_paged_kv *kv, const float *q, const float *k,
                                const float *v, float *q_rot, float *out, double rope_base,
                                int32_t layout, float softmax_scale, const kvd_attn_options *opt,
                                void *stream);

/*
 * Optional debug check of the descriptor's device-side contract: the parts
 * that live in device memory and that the entry points above take on trust
 * (their violation is undefined behaviour there).  The pages report such
 * errors as values (ferric-core generate.rs returns Result and asserts its
 * shapes); a caller that cannot vouch for its batch runs this check on the
 * same stream before the step and reads the flag word.
 *
 *   flags  device pointer to one 32-bit word (4-byte aligned).  The kernel
 *          ORs in a KVD_CHECK_* bit for every kind of violation it finds and
 *          leaves the word as it was otherwise, so the caller clears it
 *          first (or keeps accumulating over calls).
 *     KVD_CHECK_SEQ_LEN   a seq_lens[b] below 0 or above max_seq_len, or,
 *                         for a whole cache, below the sequence's new tokens
 *     KVD_CHECK_BLOCK_ID  a block-table entry for a key some query sees
 *                         (from the first query's window on) outside
 *                         [0, num_blocks)
 *     KVD_CHECK_Q_LENS    a q_lens[b] below 0 or above q_tokens_per_seq
 *     KVD_CHECK_SHARD     a negative key_pos0[b] or q_pos[b]
 * Host-side validation as for the other calls first.  One workgroup per
 * sequence; it reads seq_lens, q_lens, key_pos0, q_pos and the table rows
 * (never past a row) and dereferences no block id, so it is safe on any
 * descriptor the host validation accepts.  Asynchronous on `stream`.
 */
enum {
    KVD_CHECK_SEQ_LEN = 1,
    KVD_CHECK_BLOCK_ID = 2,
    KVD_CHECK_Q_LENS = 4,
    KVD_CHECK_SHARD = 8
};
int32_t kvd_check_descriptor(const kvd_paged_kv *kv, uint32_t *flags, void *stream);

/* Human-readable name of a status code (static storage).  The error calls
 * stand for the pages' errors as values (generate.rs: Result, unwrap); the
 * pages define no C form of them. */
const char *kvd_status_string(int32_t status);

/* Detail of the last non-OK status returned on the calling thread (static or
 * thread-local storage; "" if none). */
const char *kvd_last_error(void);

/* ABI version, bumped on any incompatible change (2: kvd_paged_kv.window;
 * 3: kvd_paged_kv.key_pos0, .q_pos and .q_lens). */
int32_t kvd_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* KVD_H */
