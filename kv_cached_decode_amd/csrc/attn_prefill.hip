// attn_prefill.hip -- attention of many query rows per kv head against the
// paged cache: chunked prefill (the ferric-core generate.rs page treats
// prefill and decode as the same step; the Ferrum Infer README sends prefill
// through a flash-attention kernel) and long drafts, g*T > 16 rows, bf16
// cache, head_dim 128.  Causal within the chunk: new token t sees the keys up
// to its own position.
//
// Workgroup = WAVES wave64s (4: two workgroups per CU) over a tile of 32 *
// WAVES query rows of one (sequence, kv head) -- wave w owns rows 32w ..
// 32w+31 of the tile as two 16-row blocks, row r = t*g + hg -- and one key
// range (split).  Unlike the decode kernel, every wave needs every key, so
// the K and V tiles (32 keys) are staged in LDS once by all the threads and
// shared by the waves: the kv-head
// group's rows share the keys, which is what makes the work dense enough for
// the matrix cores.  Each K or V operand a wave reads from LDS feeds both of
// its row blocks, so LDS reads per query row are half those of one block per
// wave.  Double-buffered: while the waves consume tile i from LDS, each
// thread's registers hold its share of tile i+1 on the way from HBM (one
// barrier per tile).  Per wave, row block and tile, as in the decode kernel:
//   S^T[32 keys x 16 rows] = K . Q^T   (K from LDS, Q as bf16 hi + lo),
//   online softmax per row (the row sits in lane l%16),
//   O^T[128 x 16 rows] += V^T . P^T    (V^T read transposed from LDS; V and
//   P in fp16, or bf16 V with P as bf16 hi + lo when V leaves fp16's range).
// The loop ends at the last key any row of the tile sees.  A wave skips the
// tiles none of its rows sees (past the causal end of its last row, before
// the window of its first), and leaves out the mask on tiles every one of its
// rows sees whole; the running rescale happens only when a row's maximum
// grows (otherwise its factor is exactly 1).  Rows past the chunk take no
// part, and their outputs are left as they are.  Split ranges, windows,
// ragged chunks and context-parallel shards follow the same rules as the
// decode kernels (kvd_internal.h).
//
// RoPE of the queries (rope_q: q holds the raw queries, the RoPE/append
// kernel has appended the new K/V rows before this kernel runs): each query
// row is rotated by the workgroup that reads it, at its token's position,
// with the RoPE/append kernel's arithmetic (fp64 angle, cosine, sine and
// rotation, rounded once to fp32), so the result is bitwise that of reading
// its rotated queries.  The angles of the tile's tokens are formed once per
// workgroup, 32 tokens at a time, in the LDS of the K/V tiles before the first
// tile is staged; every lane holds both elements of each of its pairs (dims d
// and d + 64, or 2i and 2i + 1), so the rotation needs no data exchange.
#include <type_traits>

#include "kvd_internal.h"
#include "rope_math.h"

namespace kvd {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int WAVES = PREFILL_WAVES;
constexpr int THREADS = 64 * WAVES;
constexpr int D = 128;
constexpr int LOG2_ROW_BYTES = 8;         // one cached key or value row: D bf16
static_assert((1 << LOG2_ROW_BYTES) == D * 2, "row bytes");
constexpr int TILE = 32;
constexpr int RB = 2;                     // 16-row blocks per wave
constexpr int WROWS = 16 * RB;            // query rows per wave
constexpr int ROWS = WAVES * WROWS;       // query rows per workgroup
// LDS row stride of the K tile, 288 bytes as for the V tile: the tile's reads
// and writes are then free of bank conflicts (SQ_LDS_BANK_CONFLICT per
// dispatch of the chunked prefill: 51k at 288 bytes, 6.3M at 272 and 320,
// 44M at 256)
constexpr int KROWB = D * 2 + 32;
constexpr int VROWB = D * 2 + 32;         // LDS row stride of the V tile (transposed reads)
constexpr int CHUNKS = TILE * D * 2 / 16;   // 16-byte chunks of a K (or V) tile
constexpr int CPT = CHUNKS / THREADS;        // of them per thread
static_assert(CPT * THREADS == CHUNKS, "the threads split a tile evenly");
constexpr int K_BYTES = TILE * KROWB;
constexpr int V_BYTES = TILE * VROWB;
constexpr int MAX_STAGED_BLOCKS = 4096;   // block ids of a split, staged in LDS
constexpr int RANK_MAX = PREFILL_RANK_MAX;  // units ranked longest-first (their key counts and the units by rank share the block-id array)
static_assert(RANK_MAX <= THREADS, "one unit per thread in the ranking");
static_assert(RANK_MAX <= 512 && RANK_MAX % 16 == 0, "unit indices fit the sort key's 9 bits");
constexpr float M_EMPTY = -1e30f;
constexpr int HALF = D / 2;
constexpr int ANG_TOKENS = 32;            // tokens whose angles share the LDS at a time
static_assert(2 * ANG_TOKENS * HALF * sizeof(double) <= 2 * K_BYTES + 2 * V_BYTES,
              "the angle table fits in the K/V tiles");
// The running maximum of a row moves (and its sums are rescaled) only when a
// tile's scores exceed it by more than RESCALE_SLACK (log2 units); below that
// the weights exp2(s - m) stay at most 2^RESCALE_SLACK, harmless in fp32, and
// the result is the same since numerator and denominator share m.
constexpr float RESCALE_SLACK = 8.0f;
static_assert(ROWS == PREFILL_ROWS, "rows per workgroup");

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ inline bf16x8 as_bf16x8(const u32x4& u) { return __builtin_bit_cast(bf16x8, u); }

__device__ inline bf16x8 join(const s16x4& a, const s16x4& b) {
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    s16x8 v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, v);
}

__device__ inline s16x4 lds_tr(const char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(__attribute__((address_space(3))) void*)p);
}

// Two fp32 weights as bf16 hi + lo pairs (element 0 in the low half): hi is
// the rounded value, lo the rounded remainder.  One conversion rounds both
// his, and their fp32 values come back with a shift and a mask.
__device__ inline void split_pair(float a, float b, unsigned& hi, unsigned& lo) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    hi = __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){a, b}, bf16x2));
    const float ra = a - __uint_as_float(hi << 16), rb = b - __uint_as_float(hi & 0xffff0000u);
    lo = __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){ra, rb}, bf16x2));
}

// Two fp32 values as an fp16 pair (element 0 in the low half), rounded to
// nearest even.
__device__ inline unsigned f16_pair(float a, float b) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){a, b}, f16x2));
}

// A bf16 pair as an fp16 pair: exact for magnitudes in [2^-14, 65504].
__device__ inline unsigned f16_from_bf16_pair(unsigned u) {
    return f16_pair(__uint_as_float(u << 16), __uint_as_float(u & 0xffff0000u));
}

// The fast pass's weights in fp16 are scaled by 2^P_SCALE_LOG2 (they stay at
// most 2^RESCALE_SLACK = 2^8 before it, so at most 2^15 after).  The scale
// rides in the scores: they accumulate onto P_SCALE_LOG2 - m, so exp2 yields
// the scaled weights, O and the row sums carry the same factor, and the
// maximum less P_SCALE_LOG2 is what the unit exports.
constexpr float P_SCALE_LOG2 = 7.0f;

// Reductions over lanes l, l^16, l^32, l^48 (the four lane groups holding a
// row's keys).  permlane16_swap / permlane32_swap of a register with itself
// leave, in every lane, its own value and its partner's (lane ^ 16, lane ^ 32)
// in the two results, in an order that depends on the lane; the single
// addition is symmetric in them, so every lane gets the same value.
__device__ inline float xor_sum(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// Maximum of two floats in one instruction.  (fmaxf on values that come out
// of a lane exchange first quiets signalling NaNs with two more.)
__device__ inline float vmax(float a, float b) {
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// The maxima of a and b over the four 16-lane rows at once.  permlane16_swap
// (x, y) trades x's odd rows for y's even rows: it returns (x0 y0 x2 y2) and
// (x1 y1 x3 y3), so the first swap and maximum leave a's and b's row pairs
// side by side; permlane32_swap trades x's upper half for y's lower half, so
// the second folds rows 0-1 against 2-3; the third hands each lane both
// results.  Scores hold no NaN.
__device__ inline void xor_max2(float& a, float& b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    const float c = vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));   // rows: a01 b01 a23 b23
    const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(c), __float_as_uint(c), false, false);
    const float e = vmax(__uint_as_float(q[0]), __uint_as_float(q[1]));   // rows: a b a b
    const auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(e), __float_as_uint(e), false, false);
    a = __uint_as_float(t[0]);
    b = __uint_as_float(t[1]);
}

// A unit of work is (sequence b, row tile, split): the keys
// [key_begin, key_end) that rows row0 .. row0 + ROWS - 1 of the sequence's
// kv-head group see within the split; live_rows of them are real (their
// token is inside the chunk).  The same for every kv head.
struct Unit {
    int b, rtile, split;
    int qo, n_live, key_begin, key_end, live_rows;
};
static_assert(RANK_MAX * (1 + sizeof(Unit) / sizeof(int)) <= MAX_STAGED_BLOCKS,
              "ranking arrays (key counts, units by rank) share the block-id array");

__device__ inline Unit unit_of(const AttnArgs& a, int u, int n_rtiles) {
    const CacheView& c = a.c;
    Unit w;
    w.split = u % a.num_splits;
    w.rtile = n_rtiles - 1 - (u / a.num_splits) % n_rtiles;   // later (longer) row tiles first
    w.b = u / (a.num_splits * n_rtiles);
    const int L = c.seq_lens[w.b];
    const int nn = n_new(c, w.b);
    w.qo = q_local0(c, w.b, L);
    w.key_begin = range_start(c, w.qo) + w.split * a.split_keys;
    const int row0 = w.rtile * ROWS;
    w.n_live = nn * c.g;
    w.live_rows = min(ROWS, w.n_live - row0);
    // the last token of the tile inside the chunk sees keys up to its own position
    const int t_last = min(nn, (row0 + ROWS - 1) / c.g + 1) - 1;
    w.key_end = min(min(range_end(c, L, w.qo, nn), w.key_begin + a.split_keys), w.qo + t_last + 1);
    return w;
}

// The rank a grid position takes.  The dispatcher fills each XCD's CUs with
// its first 64 workgroups in a fixed pattern, workgroups j and j + 32 (in the
// XCD's order) on the same CU, and deals the rest to whichever slot frees
// first.  With the kv head fastest and 8m kv heads (an XCD per kv head
// residue), positions p and p + 32/m share a CU at the start: they take
// ranks r and 2*(32/m) - 1 - r, so a CU starts with one long and one short
// unit instead of two long ones; later positions keep the longest-first
// order.  Any other head count, or fewer than 2*(32/m) units, keeps that
// order throughout.  Only the balance depends on this.
__device__ inline int cu_paired_rank(int pos, int n_units, int Hkv) {
    if (PREFILL_WGS_PER_CU != 2 || Hkv % 8 != 0 || 32 % (Hkv / 8) != 0) return pos;
    const int P = 32 / (Hkv / 8);
    if (pos < P || pos >= 2 * P || n_units < 2 * P) return pos;
    return 3 * P - 1 - pos;
}

__global__ __launch_bounds__(THREADS, PREFILL_WGS_PER_CU) void attn_prefill_kernel(AttnArgs a) {
    // the K and V tiles (double-buffered); before the first tile, the
    // cosines and sines of the query rotation
    __shared__ __attribute__((aligned(16))) char sm_kv[2 * K_BYTES + 2 * V_BYTES];
    char (*const sm_k)[K_BYTES] = (char (*)[K_BYTES])sm_kv;
    char (*const sm_v)[V_BYTES] = (char (*)[V_BYTES])(sm_kv + 2 * K_BYTES);
    __shared__ __attribute__((aligned(16))) int sm_blk[MAX_STAGED_BLOCKS];
    __shared__ int sm_v_normal, sm_nonfinite;   // the fast pass's verdict

    const CacheView& c = a.c;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n16 = lane & 15;
    const int j = lane >> 4;
    // Grid: kv head fastest (consecutive workgroups, one per kv head, read
    // different heads' keys), then the unit position.
    const int kvh = blockIdx.x % c.Hkv;
    const int pos = blockIdx.x / c.Hkv;
    const int n_rtiles = (a.rows + ROWS - 1) / ROWS;
    const int n_units = a.num_splits * n_rtiles * c.B;
    // the rotation pair's frequency, read first: the ranking's waits cover
    // it, so the angle rounds below wait for no load
    const double theta = a.rope_q ? kernarg_double(offsetof(AttnArgs, theta), tid % HALF) : 0.0;
    Unit un;
    if (a.rank_longest && n_units <= RANK_MAX) {
        // Longest-first: position pos takes the unit of rank pos by key count
        // (ties by unit index; empty units last), so the longest units start
        // first and the short ones fill the slots at the end.  Every
        // workgroup derives the same permutation; thread v describes unit v
        // and files it under its rank.
        // The sort key packs the key count (below 2^22: a split stages at
        // most 4094 blocks of at most 1024 keys) above the unit index (a
        // lower index first among equal counts), so the keys are distinct and
        // a unit's rank is the number of larger keys: one compare per unit,
        // sixteen keys per round of four broadcast LDS reads.
        unsigned* const sm_work = (unsigned*)sm_blk;
        Unit* const sm_unit = (Unit*)(sm_blk + RANK_MAX);
        const int n_keys = (n_units + 15) & ~15;
        Unit x{};
        unsigned key = 0u;        // padding: below every unit
        if (tid < n_units) {
            x = unit_of(a, tid, n_rtiles);
            const int w = x.live_rows > 0 ? max(0, x.key_end - x.key_begin) : 0;
            key = (unsigned)(w + 1) << 9 | (unsigned)(511 - tid);
        }
        if (tid < n_keys) sm_work[tid] = key;
        __syncthreads();
        if (tid < n_units) {
            int r = 0;
            for (int i = 0; i < n_keys; i += 16) {
                const u32x4 y0 = *(const u32x4*)(sm_work + i);
                const u32x4 y1 = *(const u32x4*)(sm_work + i + 4);
                const u32x4 y2 = *(const u32x4*)(sm_work + i + 8);
                const u32x4 y3 = *(const u32x4*)(sm_work + i + 12);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    r += (y0[e] > key) + (y1[e] > key) + (y2[e] > key) + (y3[e] > key);
            }
            sm_unit[r] = x;
        }
        __syncthreads();
        un = sm_unit[cu_paired_rank(pos, n_units, c.Hkv)];
        __syncthreads();       // sm_blk is reused for block ids below
    } else {
        un = unit_of(a, pos, n_rtiles);
    }
    // theta has arrived by now (the unit's own loads were waited for); a
    // counted wait says so, so that the angle loop waits for no later load
    __builtin_amdgcn_s_waitcnt(0x0f70);     // vmcnt(0)
    const int b = un.b, split = un.split;
    const int row0 = un.rtile * ROWS;
    const int qo = un.qo, n_live = un.n_live, live_rows = un.live_rows;
    const int key_begin = un.key_begin, key_end = un.key_end;
    // a unit without keys (a context-parallel shard holding none its rows
    // see) still rotates its rows when the rotated queries are asked for
    const bool no_keys = key_begin >= key_end;
    if (live_rows <= 0 || (no_keys && !(a.rope_q && a.q_rot && split == 0))) {
        write_empty_partials(a, b, kvh, split, row0, ROWS);
        return;
    }

    // The wave's rows wrow0 .. wrow0 + 31, the live ones up to wlast: keys a
    // live row of the wave sees lie in [lo_min, vis_last]; every one of them
    // sees [lo_max, vis_first].
    const int wrow0 = row0 + WROWS * wave;
    const bool wave_live = wrow0 < n_live;
    const int wlast = min(wrow0 + WROWS, n_live) - 1;
    const int vis_first = qo + wrow0 / c.g;
    const int vis_last = qo + wlast / c.g;
    const int lo_min = vis_first - c.window + 1;
    const int lo_max = vis_last - c.window + 1;

    // this lane's query rows (row n16 of each block) and their visible keys
    bool row_ok[RB], row_live[RB];
    int vis[RB], lo[RB];
    size_t qrow[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int row = wrow0 + 16 * rb + n16;
        row_ok[rb] = row < a.rows;
        row_live[rb] = row < n_live;             // n_live <= rows
        const int t = row_ok[rb] ? row / c.g : 0;
        qrow[rb] = ((size_t)b * c.T + t) * c.Hq + kvh * c.g + (row_ok[rb] ? row - t * c.g : 0);
        vis[rb] = row_live[rb] ? qo + t : -1;
        lo[rb] = c.window > 0 ? vis[rb] - c.window + 1 : 0;
    }

    // The rotation's tokens: t_lo .. t_hi - 1 cover the tile's live rows;
    // pos0 is the global position of the sequence's token 0.
    const int t_lo = row0 / c.g;
    const int t_hi = min(n_live - 1, row0 + ROWS - 1) / c.g + 1;
    const int pos0 = a.rope_q ? qo + (c.key_pos0 ? c.key_pos0[b] : 0) : 0;
    double* const cs = (double*)sm_kv;       // the angles, before the first tile is staged
    double* const sn = cs + ANG_TOKENS * HALF;
    // the angles of tokens tb .. tb + nt - 1 into LDS (thread tid keeps pair
    // tid % HALF in every round)
    auto angles = [&](int tb, int nt) {
        for (int idx = tid; idx < nt * HALF; idx += THREADS)
            rope_angle(theta, pos0 + tb + idx / HALF, cs[idx], sn[idx]);
    };

    // This lane's query elements (dims 32kk + 8j .. +8 of each row; rows past
    // the chunk take zeros, their results are replaced below) and the
    // split's block ids are fetched together, and the first round of the
    // rotation's angles is formed while they are in flight; the first K/V
    // tile's loads go out once the block ids are in LDS.
    float4 xq[RB][4][2];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const float* qp = a.q + qrow[rb] * D;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            xq[rb][kk][0] = xq[rb][kk][1] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            if (row_live[rb]) {
                xq[rb][kk][0] = *(const float4*)(qp + 32 * kk + 8 * j);
                xq[rb][kk][1] = *(const float4*)(qp + 32 * kk + 8 * j + 4);
            }
        }
    }
    const int blk0 = key_begin >> c.log2_bs;
    const int nblk = no_keys ? 0 : ((key_end - 1) >> c.log2_bs) - blk0 + 1;
    const int* trow = c.table + (size_t)b * c.max_blocks + blk0;
    // staged as the (block, kv head) row of the pools: blk * Hkv + kvh; each
    // thread's first id is read before the angles
    const int blk_pre = tid < nblk ? trow[tid] : 0;
    if (a.rope_q) angles(t_lo, min(ANG_TOKENS, t_hi - t_lo));
    if (tid < nblk) sm_blk[tid] = blk_pre * c.Hkv + kvh;
    for (int i = tid + THREADS; i < nblk; i += THREADS) sm_blk[i] = trow[i] * c.Hkv + kvh;
    if (tid == 0) {
        sm_v_normal = 0;
        sm_nonfinite = 0;
    }
    __syncthreads();

    // Each thread moves CPT of the 512 16-byte chunks of a K tile and CPT of
    // the V tile: chunk ch = tid + THREADS*i -> key ch / 16, column ch % 16.
    // Keys past the range re-read its last key (weight 0 below).  Plain
    // loads, not streaming ones: every row tile of a (sequence, kv head)
    // reads the same keys at about the same time, and lines loaded with the
    // streaming hint leave L2 before the other tiles get to them.
    const char* kbase = (const char*)c.k;
    const char* vbase = (const char*)c.v;
    const int bs_mask = (1 << c.log2_bs) - 1;
    u32x4 kr[CPT], vr[CPT];
    // When the tiles start on 16-key boundaries of blocks of at least 16
    // keys, the 16 keys of one chunk row (THREADS / 16 keys apart for the
    // CPT rows of a thread) share a block: its id is a broadcast LDS read
    // (all CPT of them issued before the one wait), the address a scalar
    // base plus the thread's fixed offset (16 * tid), and a whole tile needs
    // no clamp.
    static_assert(THREADS / 16 * CPT == TILE, "each chunk row of a tile is THREADS / 16 keys");
    const bool aligned = c.log2_bs >= 4 && (key_begin & 15) == 0;
    auto load = [&](int base) {
        if (aligned && base + TILE <= key_end) {
            unsigned hrow[CPT];
#pragma unroll
            for (int i = 0; i < CPT; ++i) hrow[i] = sm_blk[((base + THREADS / 16 * i) >> c.log2_bs) - blk0];
#pragma unroll
            for (int i = 0; i < CPT; ++i) {
                const int kb = base + THREADS / 16 * i;
                const size_t off = ((size_t)__builtin_amdgcn_readfirstlane(hrow[i]) << (c.log2_bs + LOG2_ROW_BYTES)) +
                                   ((size_t)(kb & bs_mask) << LOG2_ROW_BYTES);
                kr[i] = *(const u32x4*)(kbase + off + (unsigned)(16 * tid));
                vr[i] = *(const u32x4*)(vbase + off + (unsigned)(16 * tid));
            }
            return;
        }
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int ch = tid + THREADS * i;
            const int key = min(base + (ch >> 4), key_end - 1);
            const unsigned hrow = sm_blk[(key >> c.log2_bs) - blk0];
            const size_t off = ((size_t)hrow << (c.log2_bs + LOG2_ROW_BYTES)) +
                               ((key & bs_mask) << LOG2_ROW_BYTES | 16 * (ch & 15));
            kr[i] = *(const u32x4*)(kbase + off);
            vr[i] = *(const u32x4*)(vbase + off);
        }
    };
    if (!no_keys) load(key_begin);

    if (a.rope_q) {
        // The queries of the tile's tokens, rotated at their positions: the
        // angles of up to ANG_TOKENS tokens at a time in LDS (the first
        // round's are there already), then each lane turns the pairs of its
        // rows whose tokens are in the round.
        int t_row[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) t_row[rb] = row_live[rb] ? (wrow0 + 16 * rb + n16) / c.g : -1;
        for (int tb = t_lo; tb < t_hi; tb += ANG_TOKENS) {
            const int nt = min(ANG_TOKENS, t_hi - tb);
            if (tb != t_lo) angles(tb, nt);
            __syncthreads();
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const int tt = t_row[rb] - tb;
                if (tt < 0 || tt >= nt) continue;
                const double* cr = cs + tt * HALF;
                const double* sr = sn + tt * HALF;
                auto turn = [&](float& x, float& y, int i) {
                    double xr, yr;
                    rope_rotate(x, y, cr[i], sr[i], xr, yr);
                    x = (float)xr;
                    y = (float)yr;
                };
                if (a.interleaved) {
                    // pairs (2i, 2i + 1) inside each float4: dims 32kk + 8j + 4h + {0,1} and {2,3}
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const int i = 16 * kk + 4 * j + 2 * h;
                            turn(xq[rb][kk][h].x, xq[rb][kk][h].y, i);
                            turn(xq[rb][kk][h].z, xq[rb][kk][h].w, i + 1);
                        }
                } else {
                    // pairs (i, i + 64): dims 8j + e with 64 + 8j + e, and 32 + 8j + e with 96 + 8j + e
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const int i = 32 * kk + 8 * j + 4 * h;
                            turn(xq[rb][kk][h].x, xq[rb][kk + 2][h].x, i);
                            turn(xq[rb][kk][h].y, xq[rb][kk + 2][h].y, i + 1);
                            turn(xq[rb][kk][h].z, xq[rb][kk + 2][h].z, i + 2);
                            turn(xq[rb][kk][h].w, xq[rb][kk + 2][h].w, i + 3);
                        }
                }
            }
            __syncthreads();          // the table is rewritten next round, then staged over
        }
        // the rotated queries, when asked for (split 0 writes them)
        if (a.q_rot && split == 0) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                if (!row_live[rb]) continue;
                float* qp = a.q_rot + qrow[rb] * D;
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    *(float4*)(qp + 32 * kk + 8 * j) = xq[rb][kk][0];
                    *(float4*)(qp + 32 * kk + 8 * j + 4) = xq[rb][kk][1];
                }
            }
        }
    }
    if (no_keys) {
        write_empty_partials(a, b, kvh, split, row0, ROWS);
        return;
    }

    // Q^T operands in log2 units, hi + lo
    bf16x8 qhi[RB][4], qlo[RB][4];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const float4 x0 = xq[rb][kk][0], x1 = xq[rb][kk][1];
            const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float v = xs[e] * a.scale_log2;
                const __bf16 hi = (__bf16)v;
                qhi[rb][kk][e] = hi;
                qlo[rb][kk][e] = (__bf16)(v - (float)hi);
            }
        }

    // running max m (log2 units), O^T and this lane's part of the row sums.
    // The scores accumulate onto off - m (onto off before the row's first
    // key; off = P_SCALE_LOG2 on the fast pass, else 0), so they come out of
    // the matrix cores relative to the running max, offset by off.
    static_assert(RB == 2, "row maxima are exchanged in pairs");
    // A row moves its maximum when a tile's relative maximum exceeds thr:
    // the slack (plus off) once it has one, -inf before its first key.
    float m[RB], lsum[RB], thr[RB];
    f32x4 o[RB][8], neg_m[RB];

    // The key loop.  The fast pass (F16) feeds P.V to the matrix cores in
    // fp16, one MFMA where bf16 hi + lo takes two: V converted as it is
    // staged (exact for magnitudes in [2^-14, 65504]), the weights scaled by
    // 2^P_SCALE_LOG2 (fp16 keeps 11 significant bits; weights below 2^-31 of a row's
    // maximum flush to zero, at most 6e-5 of the sum over 2^17 keys).  It
    // hands the unit to the exact pass -- bf16 V, weights as bf16 hi + lo --
    // when a V element lay beyond fp16's range (a result comes out
    // non-finite) or none lay in its normal range (they would keep a few
    // bits), and returns whether it stands.
    auto run = [&](auto f16_tag) -> bool {
        constexpr bool F16 = decltype(f16_tag)::value;
        constexpr float off = F16 ? P_SCALE_LOG2 : 0.0f;
        unsigned vexp = 0u;             // the staged fp16 pairs, ORed (their exponent fields tell)
        auto stage = [&](int buf, bool f16) {
#pragma unroll
            for (int i = 0; i < CPT; ++i) {
                const int ch = tid + THREADS * i;
                *(u32x4*)(sm_k[buf] + (ch >> 4) * KROWB + 16 * (ch & 15)) = kr[i];
                u32x4 vs = vr[i];
                if (f16) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        vs[q] = f16_from_bf16_pair(vs[q]);
                        vexp |= vs[q];
                    }
                }
                *(u32x4*)(sm_v[buf] + (ch >> 4) * VROWB + 16 * (ch & 15)) = vs;
            }
        };
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            m[rb] = M_EMPTY;
            lsum[rb] = 0.0f;
            thr[rb] = -INFINITY;
            neg_m[rb] = (f32x4){off, off, off, off};
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) o[rb][nt] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
        }

        stage(0, F16);
        __syncthreads();
        if (key_begin + TILE < key_end) load(key_begin + TILE);

        int buf = 0;
        for (int base = key_begin; base < key_end; base += TILE, buf ^= 1) {
            // wave-uniform: does any live row of the wave see a key of the tile,
            // and does every one see all of them?
            const bool active = wave_live && base <= vis_last && (c.window == 0 || base + TILE - 1 >= lo_min);
            if (active) {
                const bool whole = base + TILE <= key_end && base + TILE - 1 <= vis_first &&
                                   (c.window == 0 || base >= lo_max);
                const char* kt = sm_k[buf];
                const char* vt = sm_v[buf];
                // scores less the running max: S^T tiles (16 keys x 16 rows),
                // keys base + 16h + 4j + i
                f32x4 s[RB][2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb) s[rb][h] = neg_m[rb];
                    const char* kp = kt + (16 * h + n16) * KROWB + 16 * j;
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) {
                        const bf16x8 kop = as_bf16x8(*(const u32x4*)(kp + 64 * kk));
#pragma unroll
                        for (int rb = 0; rb < RB; ++rb) {
                            s[rb][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qhi[rb][kk], s[rb][h], 0, 0, 0);
                            s[rb][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qlo[rb][kk], s[rb][h], 0, 0, 0);
                        }
                    }
                }
                // (a branch, not selects: all but the last one or two tiles of
                // a unit are whole for every row of the wave)
                if (__builtin_expect(!whole, 0)) {
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                        for (int h = 0; h < 2; ++h)
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const int key = base + 16 * h + 4 * j + i;
                                if (key >= key_end || key > vis[rb] || key < lo[rb]) s[rb][h][i] = -INFINITY;
                            }
                }
                // running maxima: when one row of the wave saw its first key or
                // grew past the slack, every row moves up to its tile maximum
                // (a row without a key yet stays empty) and the tile's scores
                // follow it
                float mx[RB];
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    float x = -INFINITY;
#pragma unroll
                    for (int h = 0; h < 2; ++h)
#pragma unroll
                        for (int i = 0; i < 4; ++i) x = fmaxf(x, s[rb][h][i]);   // three-input maxima
                    mx[rb] = x;
                }
                xor_max2(mx[0], mx[1]);
                if (__builtin_expect(__builtin_amdgcn_ballot_w64(mx[0] > thr[0] || mx[1] > thr[1]) != 0, 0)) {
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb) {
                        const bool started = m[rb] != M_EMPTY;
                        const float mxr = mx[rb] - off;          // the tile's maximum less m
                        const float up = started ? fmaxf(mxr, 0.0f) : mxr;
                        const float mnew = started ? m[rb] + up : (up > -INFINITY ? up : M_EMPTY);
                        const float shift = started ? mnew - m[rb] : (mnew == M_EMPTY ? 0.0f : mnew);
                        const float alpha = started ? fast_exp2(m[rb] - mnew) : 1.0f;
                        m[rb] = mnew;
                        thr[rb] = mnew == M_EMPTY ? -INFINITY : RESCALE_SLACK + off;
                        lsum[rb] *= alpha;
#pragma unroll
                        for (int nt = 0; nt < 8; ++nt) o[rb][nt] *= alpha;
                        const float nm = (mnew == M_EMPTY ? 0.0f : -mnew) + off;
                        neg_m[rb] = (f32x4){nm, nm, nm, nm};
#pragma unroll
                        for (int h = 0; h < 2; ++h) s[rb][h] -= shift;
                    }
                }
                u32x4 phi[RB], plo[RB];      // fp16 weights (F16), or bf16 hi and lo
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                    for (int h = 0; h < 2; ++h)
#pragma unroll
                        for (int i = 0; i < 4; i += 2) {
                            const float p0 = fast_exp2(s[rb][h][i]);
                            const float p1 = fast_exp2(s[rb][h][i + 1]);
                            lsum[rb] += p0;
                            lsum[rb] += p1;
                            if constexpr (F16) {
                                phi[rb][2 * h + i / 2] = f16_pair(p0, p1);
                            } else {
                                unsigned ph, pl;
                                split_pair(p0, p1, ph, pl);
                                phi[rb][2 * h + i / 2] = ph;
                                plo[rb][2 * h + i / 2] = pl;
                            }
                        }
                // O^T += V^T . P^T; lane (n16, j) reads V rows 4j + i and 16 + 4j + i
                const char* rd = vt + (4 * j + (n16 >> 2)) * VROWB + 8 * (n16 & 3);
#pragma unroll
                for (int nt = 0; nt < 8; ++nt) {
                    const bf16x8 vop = join(lds_tr(rd + 32 * nt), lds_tr(rd + 16 * VROWB + 32 * nt));
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb) {
                        if constexpr (F16) {
                            o[rb][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                                __builtin_bit_cast(f16x8, vop), __builtin_bit_cast(f16x8, phi[rb]), o[rb][nt], 0, 0, 0);
                        } else {
                            o[rb][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, as_bf16x8(phi[rb]), o[rb][nt], 0, 0, 0);
                            o[rb][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, as_bf16x8(plo[rb]), o[rb][nt], 0, 0, 0);
                        }
                    }
                }
            }
            // the next tile into the other buffer (read two tiles ago, released
            // by the last barrier), then the one after it from HBM
            if (base + TILE < key_end) stage(buf ^ 1, F16);
            __syncthreads();
            if (base + 2 * TILE < key_end) load(base + 2 * TILE);
        }
        if constexpr (F16) {
            bool finite = __builtin_isfinite(lsum[0]) && __builtin_isfinite(lsum[1]);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int nt = 0; nt < 8; ++nt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) finite = finite && __builtin_isfinite(o[rb][nt][i]);
            if ((vexp & 0x7c007c00u) != 0u) sm_v_normal = 1;
            if (!finite) sm_nonfinite = 1;
            __syncthreads();
            if (sm_nonfinite || !sm_v_normal) {    // the same in every lane
                __syncthreads();                    // (keeps the two passes apart for the compiler)
                return false;
            }
            // O and the row sums both carry 2^off: the output stands, and the
            // maximum takes the factor out of the exported (m, l)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
                if (m[rb] != M_EMPTY) m[rb] -= off;
        }
        return true;
    };
    if (!run(std::true_type{})) {
        load(key_begin);
        run(std::false_type{});
    }

    // row n16's sum over the four lane groups; O^T element (dim 16nt + 4j + i, row n16)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) lsum[rb] = xor_sum(lsum[rb]);   // all lanes active
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        if (!row_ok[rb]) continue;
        if (!row_live[rb]) {        // a padding token: left as it is, or an empty partial
            if (a.num_splits == 1) continue;
            m[rb] = M_EMPTY;
            lsum[rb] = 0.0f;
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) o[rb][nt] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
        }
        if (a.num_splits == 1) {
            float* op = a.out + qrow[rb] * D;
#pragma unroll
            for (int nt = 0; nt < 8; ++nt)
                *(float4*)(op + 16 * nt + 4 * j) =
                    make_float4(finish_out(o[rb][nt][0], lsum[rb]), finish_out(o[rb][nt][1], lsum[rb]),
                                finish_out(o[rb][nt][2], lsum[rb]), finish_out(o[rb][nt][3], lsum[rb]));
            if (a.lse && j == 0) a.lse[qrow[rb]] = finish_lse(m[rb], lsum[rb]);
        } else {
            const size_t part = qrow[rb] * a.num_splits + split;
            float* op = a.part_o + part * D;
#pragma unroll
            for (int nt = 0; nt < 8; ++nt)
                *(float4*)(op + 16 * nt + 4 * j) = make_float4(o[rb][nt][0], o[rb][nt][1], o[rb][nt][2], o[rb][nt][3]);
            if (j == 0) {
                a.part_ml[part * 2 + 0] = m[rb];
                a.part_ml[part * 2 + 1] = lsum[rb];
            }
        }
    }
}

}  // namespace

int prefill_step_keys() { return TILE; }

hipError_t launch_attn_prefill(const AttnArgs& a, hipStream_t s) {
    const int64_t n_rtiles = (a.rows + ROWS - 1) / ROWS;
    const int64_t n = (int64_t)a.num_splits * n_rtiles * a.c.B * a.c.Hkv;
    if (n > INT32_MAX) return hipErrorInvalidConfiguration;
    dim3 grid((unsigned)n);
    hipLaunchKernelGGL(attn_prefill_kernel, grid, dim3(THREADS), 0, s, a);
    return hipGetLastError();
}

}  // namespace kvd
