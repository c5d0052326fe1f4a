/*
 * kvd_oracle.c -- plain fp64 CPU reference for KV-cached decode attention.
 *
 * TEST INFRASTRUCTURE ONLY (see kvd_oracle.h).  Straight loops, no blocking,
 * no fusion, no reordering beyond the definitions:
 *
 *   RoPE (ferric-core generate.rs, module doc: "RoPE uses the token's
 *   absolute position"; `rope_off_t(x, t, h, dh, base, pos)` in `step_gpu`):
 *       theta_i = base^(-2i/D),  phi = pos * theta_i,
 *       (a, c) <- (a cos phi - c sin phi,  a sin phi + c cos phi).
 *
 *   Append (generate.rs `step_gpu`: the new K/V rows are appended and the key
 *   count is taken after the append; Ferrum README "Paged KV attention": a
 *   block pool addressed through a block table):
 *       pos = seq_lens[b] - T + t,
 *       slot = pool[table[b][pos / bs]][kvh][pos % bs][:].
 *
 *   Attention (generate.rs `mha_decode_t(q, k, v, hq, hkv, dh, s)`, GQA as in
 *   the ferrox `decoder` module; the sliding window of the ferrox
 *   `kv_budget::SlidingWindow` type limits it to the last `window` keys):
 *       s_j = scale * <q_rot, K_j>, j = j0 .. p, p = seq_lens[b] - T + t,
 *       j0 = 0, or max(0, p - window + 1) with a window,
 *       out = sum_j exp(s_j - max s) V_j / sum_j exp(s_j - max s),
 *       lse = log sum_j exp(s_j),
 *       kv head of query head h = h / (Hq / Hkv).
 *
 *   Context-parallel shard (context parallelism, CP and DCP, is one of the
 *   composable parallel modes on the ferrite page): the cache holds global
 *   keys key_pos0 .. key_pos0 + seq_lens - 1 and the new tokens sit at
 *   q_pos + t; the same sums run over the held keys only, so the shards'
 *   (out, lse) pairs merge into the whole-cache result by
 *       LSE = log sum_p exp(lse_p),  out = sum_p exp(lse_p - LSE) out_p.
 */
#include "kvd_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

uint16_t oracle_bf16_from_double(double x)
{
    /* bf16: 1 sign bit, the 8 exponent bits of fp32, 7 stored significand
     * bits.  Round |x| to a multiple of its bf16 quantum, ties to even. */
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    if (isnan(x))
        return (uint16_t)(sign | 0x7FC0u);
    double a = fabs(x);
    if (a == 0.0)
        return sign;
    int e;
    frexp(a, &e);           /* a in [2^(e-1), 2^e) */
    int E = e - 1;
    if (E < -126)           /* subnormal range: fixed quantum 2^-133 */
        E = -126;
    double quantum = ldexp(1.0, E - 7);
    double n = nearbyint(a / quantum);  /* default mode: nearest, ties even */
    double r = n * quantum;
    if (r >= 0x1p128)
        return (uint16_t)(sign | 0x7F80u);  /* overflow to infinity */
    float f = (float)r;     /* exact: r has at most 8 significant bits */
    uint32_t bits;
    memcpy(&bits, &f, sizeof bits);
    return (uint16_t)(sign | (uint16_t)(bits >> 16));
}

double oracle_bf16_to_double(uint16_t b)
{
    uint32_t bits = (uint32_t)b << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Rotate one head vector x (length D) at absolute position pos. */
static void rope_one(const double *x, double *y, int32_t D, int64_t pos,
                     double base, int32_t layout)
{
    int32_t half = D / 2;
    for (int32_t i = 0; i < half; ++i) {
        double theta = pow(base, -2.0 * (double)i / (double)D);
        double phi = (double)pos * theta;
        double cs = cos(phi), sn = sin(phi);
        int32_t ia, ic;
        if (layout == ORACLE_ROPE_HALF) {
            ia = i;
            ic = i + half;
        } else {
            ia = 2 * i;
            ic = 2 * i + 1;
        }
        double a = x[ia], c = x[ic];
        y[ia] = a * cs - c * sn;
        y[ic] = a * sn + c * cs;
    }
}

int oracle_rope(const double *x, double *y, int32_t n_rows, int32_t n_heads,
                int32_t head_dim, const int64_t *positions, double base,
                int32_t layout)
{
    if (n_rows < 0 || n_heads < 1 || head_dim < 2 || (head_dim % 2) != 0)
        return 1;
    if (layout != ORACLE_ROPE_HALF && layout != ORACLE_ROPE_INTERLEAVED)
        return 1;
    double *tmp = (double *)malloc(sizeof(double) * (size_t)head_dim);
    if (!tmp)
        return 2;
    for (int32_t r = 0; r < n_rows; ++r)
        for (int32_t h = 0; h < n_heads; ++h) {
            const double *xs = x + ((size_t)r * n_heads + h) * head_dim;
            double *ys = y + ((size_t)r * n_heads + h) * head_dim;
            rope_one(xs, tmp, head_dim, positions[r], base, layout);
            memcpy(ys, tmp, sizeof(double) * (size_t)head_dim);
        }
    free(tmp);
    return 0;
}

/* New tokens of sequence b, the global position of local key 0, and that
 * of new token 0 (by default the new tokens are the last keys held). */
static int32_t n_new(const oracle_cache *c, int32_t b)
{
    return c->q_lens ? c->q_lens[b] : c->q_tokens;
}

static int64_t key_pos0(const oracle_cache *c, int32_t b)
{
    return c->key_pos0 ? (int64_t)c->key_pos0[b] : 0;
}

static int64_t q_pos0(const oracle_cache *c, int32_t b)
{
    return c->q_pos ? (int64_t)c->q_pos[b]
                    : key_pos0(c, b) + (int64_t)c->seq_lens[b] - n_new(c, b);
}

static int check_cache(const oracle_cache *c)
{
    if (!c || c->num_seqs < 0 || c->q_tokens < 1 || c->n_q_heads < 1 ||
        c->n_kv_heads < 1 || c->n_q_heads % c->n_kv_heads != 0 ||
        c->head_dim < 2 || c->head_dim % 2 != 0 || c->block_size < 1 ||
        c->num_blocks < 0 || c->max_blocks_per_seq < 0 || c->window < 0)
        return 1;
    if (c->cache_dtype != ORACLE_F32 && c->cache_dtype != ORACLE_BF16 &&
        c->cache_dtype != ORACLE_F64)
        return 1;
    for (int32_t b = 0; b < c->num_seqs; ++b) {
        int64_t L = c->seq_lens[b];
        if (c->q_lens && (c->q_lens[b] < 0 || c->q_lens[b] > c->q_tokens))
            return 1;
        if (L < (c->q_pos ? 0 : n_new(c, b)))
            return 1;
        int64_t nblk = (L + c->block_size - 1) / c->block_size;
        if (nblk > c->max_blocks_per_seq)
            return 1;
        for (int64_t i = 0; i < nblk; ++i) {
            int32_t id = c->block_table[(size_t)b * c->max_blocks_per_seq + i];
            if (id < 0 || id >= c->num_blocks)
                return 1;
        }
    }
    return 0;
}

/* Flat element index of (local key pos of sequence b, kv head, dim 0). */
static size_t slot_index(const oracle_cache *c, int32_t b, int64_t pos,
                         int32_t kvh)
{
    int32_t blk = c->block_table[(size_t)b * c->max_blocks_per_seq +
                                 pos / c->block_size];
    int64_t off = pos % c->block_size;
    return (((size_t)blk * c->n_kv_heads + kvh) * c->block_size + off) *
           c->head_dim;
}

static void store(const oracle_cache *c, void *pool, size_t idx, double x)
{
    if (c->cache_dtype == ORACLE_F32)
        ((float *)pool)[idx] = (float)x;    /* C conversion: nearest even */
    else if (c->cache_dtype == ORACLE_BF16)
        ((uint16_t *)pool)[idx] = oracle_bf16_from_double(x);
    else
        ((double *)pool)[idx] = x;
}

static double load(const oracle_cache *c, const void *pool, size_t idx)
{
    if (c->cache_dtype == ORACLE_F32)
        return (double)((const float *)pool)[idx];
    if (c->cache_dtype == ORACLE_BF16)
        return oracle_bf16_to_double(((const uint16_t *)pool)[idx]);
    return ((const double *)pool)[idx];
}

int oracle_rope_append_kv(const oracle_cache *c, const float *q,
                          const float *k, const float *v, double *q_rot,
                          double base, int32_t layout)
{
    if (check_cache(c))
        return 1;
    if (layout != ORACLE_ROPE_HALF && layout != ORACLE_ROPE_INTERLEAVED)
        return 1;
    const int32_t B = c->num_seqs, T = c->q_tokens, Hq = c->n_q_heads,
                  Hkv = c->n_kv_heads, D = c->head_dim;
    double *x = (double *)malloc(sizeof(double) * (size_t)D);
    double *y = (double *)malloc(sizeof(double) * (size_t)D);
    if (!x || !y) {
        free(x);
        free(y);
        return 2;
    }
    for (int32_t b = 0; b < B; ++b)
        for (int32_t t = 0; t < n_new(c, b); ++t) {
            int64_t pos = q_pos0(c, b) + t;              /* global: the rotation */
            int64_t local = pos - key_pos0(c, b);        /* the cache slot */
            for (int32_t h = 0; h < Hq; ++h) {
                size_t o = (((size_t)b * T + t) * Hq + h) * D;
                for (int32_t d = 0; d < D; ++d)
                    x[d] = (double)q[o + d];
                rope_one(x, q_rot + o, D, pos, base, layout);
            }
            /* a context-parallel shard that does not hold this token (its
             * slot lies outside the keys the shard keeps) needs the rotated
             * query for its partial but stores nothing: the shard holding
             * the token appends it */
            if (local < 0 || local >= c->seq_lens[b])
                continue;
            for (int32_t h = 0; h < Hkv; ++h) {
                size_t o = (((size_t)b * T + t) * Hkv + h) * D;
                size_t s = slot_index(c, b, local, h);
                for (int32_t d = 0; d < D; ++d)
                    x[d] = (double)k[o + d];
                rope_one(x, y, D, pos, base, layout);
                for (int32_t d = 0; d < D; ++d) {
                    store(c, c->k_pool, s + d, y[d]);
                    store(c, c->v_pool, s + d, (double)v[o + d]);
                }
            }
        }
    free(x);
    free(y);
    return 0;
}

/* One query row: q (D values) of sequence b at global position p, against
 * the keys it sees: global 0 .. p, or p - window + 1 .. p, of those the cache
 * holds (local keys i0 .. i1-1 below).  Writes out[D], *lse and *wsum; a row
 * that sees no key gets out = 0, lse = -inf, wsum = 0. */
static int attend_row(const oracle_cache *c, int32_t b, int32_t kvh, int64_t p,
                      const double *q, double scale, double *out, double *lse,
                      double *wsum)
{
    const int32_t D = c->head_dim;
    const int64_t k0 = key_pos0(c, b);
    int64_t g0 = (c->window > 0 && p + 1 > c->window) ? p + 1 - c->window : 0;
    int64_t i0 = g0 - k0, i1 = p + 1 - k0;
    if (i0 < 0)
        i0 = 0;
    if (i1 > c->seq_lens[b])
        i1 = c->seq_lens[b];
    for (int32_t d = 0; d < D; ++d)
        out[d] = 0.0;
    if (i1 <= i0) {
        if (lse)
            *lse = -INFINITY;
        if (wsum)
            *wsum = 0.0;
        return 0;
    }
    double *s = (double *)malloc(sizeof(double) * (size_t)(i1 - i0));
    if (!s)
        return 2;
    double m = -INFINITY;
    for (int64_t j = i0; j < i1; ++j) {
        size_t idx = slot_index(c, b, j, kvh);
        double dot = 0.0;
        for (int32_t d = 0; d < D; ++d)
            dot += q[d] * load(c, c->k_pool, idx + d);
        s[j - i0] = scale * dot;
        if (s[j - i0] > m)
            m = s[j - i0];
    }
    double denom = 0.0;
    for (int64_t j = i0; j < i1; ++j) {
        s[j - i0] = exp(s[j - i0] - m);   /* unnormalised weight */
        denom += s[j - i0];
    }
    double total = 0.0;
    for (int64_t j = i0; j < i1; ++j) {
        size_t idx = slot_index(c, b, j, kvh);
        double w = s[j - i0] / denom;
        total += w;
        for (int32_t d = 0; d < D; ++d)
            out[d] += w * load(c, c->v_pool, idx + d);
    }
    if (lse)
        *lse = m + log(denom);
    if (wsum)
        *wsum = total;
    free(s);
    return 0;
}

int oracle_decode_attention_rows(const oracle_cache *c, const double *q_rot,
                                 double scale, const int64_t *rows,
                                 int64_t n_rows, double *out, double *lse)
{
    if (check_cache(c))
        return 1;
    const int32_t T = c->q_tokens, Hq = c->n_q_heads, D = c->head_dim;
    const int32_t g = Hq / c->n_kv_heads;
    const int64_t total_rows = (int64_t)c->num_seqs * T * Hq;
    for (int64_t r = 0; r < n_rows; ++r)
        if (rows[r] < 0 || rows[r] >= total_rows)
            return 1;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
    for (int64_t r = 0; r < n_rows; ++r) {
        int64_t row = rows[r];
        int32_t h = (int32_t)(row % Hq);
        int32_t t = (int32_t)((row / Hq) % T);
        int32_t b = (int32_t)(row / ((int64_t)Hq * T));
        if (t >= n_new(c, b)) {            /* padding row */
            for (int32_t d = 0; d < D; ++d)
                out[(size_t)r * D + d] = 0.0;
            if (lse)
                lse[r] = -INFINITY;
            continue;
        }
        err |= attend_row(c, b, h / g, q_pos0(c, b) + t, q_rot + (size_t)row * D,
                          scale, out + (size_t)r * D, lse ? lse + r : NULL, NULL);
    }
    return err;
}

int oracle_decode_attention(const oracle_cache *c, const double *q_rot,
                            double scale, double *out, double *lse,
                            double *wsum)
{
    if (check_cache(c))
        return 1;
    const int32_t T = c->q_tokens, Hq = c->n_q_heads, D = c->head_dim;
    const int32_t g = Hq / c->n_kv_heads;
    const int64_t n_rows = (int64_t)c->num_seqs * T * Hq;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
    for (int64_t row = 0; row < n_rows; ++row) {
        int32_t h = (int32_t)(row % Hq);
        int32_t t = (int32_t)((row / Hq) % T);
        int32_t b = (int32_t)(row / ((int64_t)Hq * T));
        if (t >= n_new(c, b)) {            /* padding row */
            for (int32_t d = 0; d < D; ++d)
                out[(size_t)row * D + d] = 0.0;
            if (lse)
                lse[row] = -INFINITY;
            if (wsum)
                wsum[row] = 0.0;
            continue;
        }
        err |= attend_row(c, b, h / g, q_pos0(c, b) + t, q_rot + (size_t)row * D,
                          scale, out + (size_t)row * D, lse ? lse + row : NULL,
                          wsum ? wsum + row : NULL);
    }
    return err;
}
