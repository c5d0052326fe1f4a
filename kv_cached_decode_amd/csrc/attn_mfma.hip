// attn_mfma.hip -- decode attention on the matrix cores, for multi-token
// verify (ferrox-models `speculative`: every draft token of a sequence is
// verified in one batched pass; ferrite's MTP speculation) and any other case
// where the g*T query rows that share a kv head make Q.K^T a small dense
// contraction (g*T <= 16 rows, bf16 cache, head_dim 128).
//
// Workgroup = 4 wave64s per (split, kv head, sequence), as in the VALU path.
// Each wave streams 32-key tiles of the workgroup's key range (tiles w, w+4,
// ... of the range) and keeps its own online-softmax state; the waves merge
// through LDS at the end.  Per 32-key tile, with M = g*T <= 16 query rows:
//
//   S^T[32 keys x 16 rows] = K[32 x 128] . Q^T[128 x 16]
//       v_mfma_f32_16x16x32_bf16, two 16-key tiles x four 32-dim steps.  The
//       K operand (lane l: key l%16, 8 consecutive dims) is loaded straight
//       from the paged cache, 16 keys x 64 contiguous bytes per instruction.
//       Q is split into bf16 hi + lo parts (q = hi + lo to ~16 bits), so the
//       scores keep fp32-class accuracy: two MFMAs per step.
//   softmax: the MFMA result leaves each lane one row (l%16) and 8 keys, so
//       the row max/sum need only the xor-16/xor-32 lane exchange.
//   O^T[128 x 16 rows] += V^T[128 x 32] . P^T[32 x 16]
//       P comes straight out of the score registers (no data movement), again
//       as bf16 hi + lo.  V^T fragments are read from a row-major LDS copy of
//       the V tile with ds_read_b64_tr_b16 (each 16-lane group turns 4 key
//       rows x 16 dims into 16 lanes x 4 keys), two reads per 32-key MFMA.
//       O^T keeps the row in l%16, so the per-row rescale is lane-local.
//
// Fused decode step (FUSED): the kernel also does the RoPE + append step of
// generate.rs `step_gpu` for its own rows and keys.  Every workgroup rotates
// its query rows from the raw q (angles of the T new positions evaluated once
// in fp64 into LDS, the same arithmetic as the stand-alone RoPE kernel); the
// workgroup whose key range holds new tokens rotates and rounds their K/V
// rows, stores them into the cache and substitutes them into its own tiles
// from LDS, so it never waits for its own stores.  The rotated queries, when
// the caller wants them, are written after the key loop: stores issued with
// the first tile in flight are waited for together with it (one in-order
// memory counter).  The result is bitwise the RoPE/append kernel followed by
// the unfused attention with the same plan.
//
// Keys past the range are clamped to the range's last key for the loads and
// masked to weight 0; keys past a draft token's position, or before its
// sliding window, are masked the same way (causal within the draft).  Split
// ranges start at the first key any query can see, so keys before every
// window are not read.
#include <type_traits>

#include "bf16_round.h"
#include "kvd_internal.h"
#include "rope_math.h"

namespace kvd {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int WAVES = 4;
constexpr int D = 128;
constexpr int TILE = 32;                 // keys per wave iteration
constexpr int ROWB = D * 2 + 32;         // LDS row stride of the V tile (bytes)
constexpr int VT_BYTES = TILE * ROWB;    // one wave's V tile
constexpr float M_EMPTY = -1e30f;
constexpr int MAX_PIECE_BLOCKS = MFMA_PIECE_BLOCKS;   // block ids staged in LDS at a time
constexpr int LPT_MAX_SEQS = 256;        // batches ranked longest-first (one rank per thread)
constexpr int MAX_T = 16;                // new tokens per sequence (rows <= 16)
constexpr int HALF = D / 2;

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

// Reductions over lanes l, l^16, l^32, l^48 (the four lane groups holding a
// row's keys).  permlane16_swap / permlane32_swap of a register with itself
// leave, in every lane, its own value and its partner's (lane ^ 16, lane ^ 32)
// in the two results, in an order that depends on the lane; max and the
// single addition are symmetric in them, so every lane gets the same value.
__device__ inline float xor_max(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}

__device__ inline float xor_sum(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// Sequence order: workgroups are dispatched in blockIdx order, so when the
// grid is larger than the resident slots (the host says so), sequence slot z
// of the grid takes the z-th longest sequence (ties by index).  With a
// ragged batch the longest units start first and the short ones fill the
// gaps (longest-processing-time-first list scheduling); a uniform batch keeps
// its natural order.  Batches up to LPT_MAX_SEQS (larger ones keep their
// natural order): thread b packs sequence b's length with its index into a
// distinct key (longer first, then lower index; lengths past 2^24 - 1
// compare as equal, which only changes the order) and counts the keys above
// its own, sixteen per round of four broadcast LDS reads; the thread of
// rank z names the sequence.  Returns the sequence and, in len, its length.
__device__ inline int lpt_rank_pick(int B, int z, const int* seq_lens, unsigned* sm_key, int* sm_pick, int& len) {
    static_assert(LPT_MAX_SEQS <= 256, "sequence indices fit the key's low 8 bits");
    const int b = threadIdx.x;          // B <= LPT_MAX_SEQS <= blockDim.x
    const int n16 = (B + 15) & ~15;
    const int L = b < B ? seq_lens[b] : 0;
    const unsigned key = b < B ? (unsigned)min(max(L, 0), (1 << 24) - 1) << 8 | (unsigned)(255 - b) : 0u;
    if (b < n16) sm_key[b] = key;
    __syncthreads();
    if (b < B) {
        int rank = 0;
        for (int i = 0; i < n16; i += 16) {
            const uint4 y0 = *(const uint4*)(sm_key + i);
            const uint4 y1 = *(const uint4*)(sm_key + i + 4);
            const uint4 y2 = *(const uint4*)(sm_key + i + 8);
            const uint4 y3 = *(const uint4*)(sm_key + i + 12);
            rank += (y0.x > key) + (y0.y > key) + (y0.z > key) + (y0.w > key);
            rank += (y1.x > key) + (y1.y > key) + (y1.z > key) + (y1.w > key);
            rank += (y2.x > key) + (y2.y > key) + (y2.z > key) + (y2.w > key);
            rank += (y3.x > key) + (y3.y > key) + (y3.z > key) + (y3.w > key);
        }
        if (rank == z) {
            sm_pick[0] = b;
            sm_pick[1] = L;
        }
    }
    __syncthreads();
    len = sm_pick[1];
    const int pick = sm_pick[0];
    __syncthreads();                    // the ranking's LDS is reused next
    return pick;
}

// The same ranking for batches of at most 64 sequences inside one wave: lane
// b holds sequence b's length packed with its index into a distinct key
// (longer first, then lower index; lengths past 2^26 - 1 compare as equal,
// which only changes the order), each lane counts the keys above its own
// through lane reads, and the lane of rank z names the sequence.  Every wave
// ranks on its own: no LDS and no barrier.  Returns the sequence and, in
// len, its length.
__device__ inline int lpt_rank_pick_wave(int B, int z, const int* seq_lens, int& len) {
    const int lane = threadIdx.x & 63;
    const int L = lane < B ? seq_lens[lane] : 0;
    const unsigned key = lane < B ? (unsigned)min(max(L, 0), (1 << 26) - 1) << 6 | (63 - lane) : 0u;
    int rank = 0;
    for (int i = 0; i < B; ++i) rank += __builtin_amdgcn_readlane(key, i) > key;
    const int pick = __builtin_ctzll(__builtin_amdgcn_ballot_w64(lane < B && rank == z));
    len = __builtin_amdgcn_readlane(L, pick);
    return pick;
}

// Split s of S over the keys [rs, re) one sequence's queries see, in equal
// shares of that range (ragged batches, where the units are ranked by key
// count: a split of the plan's length, split_keys, would leave a short
// sequence one piece and empty splits beside it): [k0, k1), empty when the
// range has fewer than s + 1 keys.  A share is at most split_keys (the
// range is at most the plan's length; a sequence longer than max_seq_len,
// outside the contract, keeps the plan's split length and loses its last
// keys, as with the plan's splits).  Returns the share.
__device__ inline int equal_split(int rs, int re, int S, int s, int split_keys, int& k0, int& k1) {
    const int e = min(split_keys, max(1, (re - rs + S - 1) / S));
    k0 = rs + s * e;
    k1 = min(re, k0 + e);
    return e;
}

// Unit order, when the batch has several splits: the units are (sequence,
// split) pairs, and a split of a short sequence can hold as many keys as a
// split of a long one, so the units themselves are ranked.  Thread v (one
// per unit, up to 256) forms unit v = (v / S, v % S)'s key count exactly as
// the workgroup that runs it will, packs it with the unit index into a
// distinct key (more keys first, then lower index), files the unit under its
// rank and its sequence length beside it; grid position pos (split index
// fastest, then sequence slot) takes the unit of rank pos.  Returns the unit
// and, in len, its sequence's length.
__device__ inline int lpt_unit_pick(const AttnArgs& a, int pos, unsigned* sm_key, int* sm_unit,
                                    int* sm_len, int& len) {
    const CacheView& c = a.c;
    const int S = a.num_splits;
    const int n = c.B * S, n16 = (n + 15) & ~15;     // n <= 256
    const int v = threadIdx.x;
    unsigned key = 0u;                  // padding: below every unit
    int L = 0;
    if (v < n) {
        const int bb = v / S, s = v - bb * S;
        L = c.seq_lens[bb];
        const int qo = q_local0(c, bb, L);
        int k0, k1;
        equal_split(range_start(c, qo), range_end(c, L, qo, n_new(c, bb)), S, s, a.split_keys, k0, k1);
        const int keys = max(0, k1 - k0);
        key = ((unsigned)min(keys, (1 << 23) - 1) << 8 | (unsigned)(255 - v)) + 1u;
    }
    if (v < n16) sm_key[v] = key;
    __syncthreads();
    if (v < n) {
        // sixteen keys per round: four broadcast reads in flight
        int r = 0;
        for (int i = 0; i < n16; i += 16) {
            const uint4 y0 = *(const uint4*)(sm_key + i);
            const uint4 y1 = *(const uint4*)(sm_key + i + 4);
            const uint4 y2 = *(const uint4*)(sm_key + i + 8);
            const uint4 y3 = *(const uint4*)(sm_key + i + 12);
            r += (y0.x > key) + (y0.y > key) + (y0.z > key) + (y0.w > key);
            r += (y1.x > key) + (y1.y > key) + (y1.z > key) + (y1.w > key);
            r += (y2.x > key) + (y2.y > key) + (y2.z > key) + (y2.w > key);
            r += (y3.x > key) + (y3.y > key) + (y3.z > key) + (y3.w > key);
        }
        sm_unit[r] = v;
        sm_len[r] = L;
    }
    __syncthreads();
    const int u = sm_unit[pos];
    len = sm_len[pos];
    __syncthreads();                    // the ranking's LDS is reused next
    return u;
}

constexpr int PER_THREAD = 16 * D / 256;     // (row, dim) elements of a workgroup's 16 rows per thread

// The end of a split when the kernel merges its own splits.  Once every
// thread's partial stores have completed (agent scope, so visible to every
// workgroup from then on; an empty split stores nothing), one ticket per
// workgroup.  The workgroup that takes the last ticket of its (sequence, kv
// head) resets the counter for the next call and merges the splits with the
// combine kernel's formula and order (split 0 first): its own split from
// registers, a split that holds no key of the sequence as the neutral
// partial (running max M_EMPTY, sum 0, output 0), the others read back with
// agent-scope loads -- so the result does not depend on which split finished
// last.  Rows of padding tokens are left as they are.
__device__ __forceinline__ void merge_own_splits(const AttnArgs& a, int b, int kvh, int split, int nn, int first_key,
                                 int rend, int split_len, const float (&own_o)[PER_THREAD],
                                 const float (&own_m)[PER_THREAD], const float (&own_l)[PER_THREAD]) {
    const CacheView& c = a.c;
    __shared__ unsigned sm_ticket;
    __builtin_amdgcn_s_waitcnt(0);          // every counter at zero: this thread's stores are done
    __syncthreads();
    unsigned* const cnt = a.counters + (size_t)b * c.Hkv + kvh;
    if (threadIdx.x == 0) sm_ticket = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int S = a.num_splits;
    if (sm_ticket != (unsigned)(S - 1)) return;
    if (threadIdx.x == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // splits s >= live hold no key of the sequence
    const int live = rend > first_key ? min(S, (rend - first_key + split_len - 1) / split_len) : 0;
    constexpr int MAXS = 8;                 // up to this many splits, every load goes out at once
#pragma unroll
    for (int k = 0; k < PER_THREAD; ++k) {
        const int idx = (int)threadIdx.x + 256 * k;
        const int r = idx / D, d = idx - r * D;
        if (r >= a.rows) break;
        const int t = r / c.g;
        if (t >= nn) break;                 // padding rows (past a ragged chunk) are left as they are
        const size_t qrow = ((size_t)b * c.T + t) * c.Hq + kvh * c.g + (r - t * c.g);
        const float* ml = a.part_ml + qrow * S * 2;
        const float* po = a.part_o + qrow * S * D + d;
        auto load = [&](const float* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
        float M = -INFINITY, Ls = 0.0f, O = 0.0f;
        if (S <= MAXS) {
            float ms[MAXS], ls[MAXS], os[MAXS];
#pragma unroll
            for (int s = 0; s < MAXS; ++s) {
                ms[s] = M_EMPTY;
                ls[s] = os[s] = 0.0f;
                if (s >= S) continue;
                if (s == split) {
                    ms[s] = own_m[k];
                    ls[s] = own_l[k];
                    os[s] = own_o[k];
                } else if (s < live) {
                    ms[s] = load(ml + 2 * s);
                    ls[s] = load(ml + 2 * s + 1);
                    os[s] = load(po + (size_t)s * D);
                }
            }
#pragma unroll
            for (int s = 0; s < MAXS; ++s)
                if (s < S) M = fmaxf(M, ms[s]);
#pragma unroll
            for (int s = 0; s < MAXS; ++s)
                if (s < S) {
                    const float f = exp2f(ms[s] - M);
                    Ls += ls[s] * f;
                    O += os[s] * f;
                }
        } else {
            auto m_of = [&](int s) { return s == split ? own_m[k] : s < live ? load(ml + 2 * s) : M_EMPTY; };
            for (int s = 0; s < S; ++s) M = fmaxf(M, m_of(s));
            for (int s = 0; s < S; ++s) {
                const float f = exp2f(m_of(s) - M);
                const float l = s == split ? own_l[k] : s < live ? load(ml + 2 * s + 1) : 0.0f;
                const float o = s == split ? own_o[k] : s < live ? load(po + (size_t)s * D) : 0.0f;
                Ls += l * f;
                O += o * f;
            }
        }
        a.out[qrow * D + d] = finish_out(O, Ls);
        if (a.lse && d == 0) a.lse[qrow] = finish_lse(M, Ls);
    }
}

template <bool FUSED>
__device__ __forceinline__ void attn_mfma_body(const AttnArgs& a) {
    // the V tiles during the key loop, then the per-wave outputs
    constexpr int O_BYTES = WAVES * 16 * (D + 1) * 4;
    static_assert(O_BYTES <= WAVES * VT_BYTES, "output staging must fit in the V tiles");
    __shared__ __attribute__((aligned(16))) char sm_v[WAVES * VT_BYTES];
    __shared__ int sm_blk[MAX_PIECE_BLOCKS];
    __shared__ float sm_m[WAVES][16];
    __shared__ float sm_l[WAVES][16];
    // fused step: the rounded new K/V rows ([t][dim], bf16 bits), read by the
    // key loop; the query rows, raw then rotated (written to q_rot after the
    // loop); before the loop the V-tile
    // area holds, after the keys of the longest-first ranking,
    // the cos/sin of the new positions' angles ([t][pair])
    __shared__ __attribute__((aligned(16))) uint16_t sm_knew[FUSED ? MAX_T * D : 8];
    __shared__ __attribute__((aligned(16))) uint16_t sm_vnew[FUSED ? MAX_T * D : 8];
    __shared__ __attribute__((aligned(16))) float sm_q[FUSED ? 16 * D : 4];
    double* const sm_cs = (double*)(sm_v + LPT_MAX_SEQS * 4);   // past the ranking's keys (ranked first)
    double* const sm_sn = sm_cs + MAX_T * HALF;
    static_assert(LPT_MAX_SEQS * 4 + 2 * MAX_T * HALF * 8 <= WAVES * VT_BYTES,
                  "fused scratch must fit in the V tiles");
    float (*sm_o)[16][D + 1] = (float (*)[16][D + 1])sm_v;

    const CacheView& c = a.c;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int n16 = lane & 15;          // MFMA column / row-in-tile index
    const int j = lane >> 4;            // lane group
    // grid (kv head, split, sequence slot): the hardware deals workgroups to
    // the XCDs round-robin in this order, so the eight of one (slot, split)
    // -- equal work whatever the sequence -- spread over them, instead of
    // one split index (the first always full, the last often empty) piling
    // onto the same XCDs
    const int kvh = blockIdx.x;
    int split = blockIdx.y;
    const int z = blockIdx.z;
    const int row = n16;                // query row of this lane (rows >= M are padding)
    const bool row_ok = row < a.rows;
    const int t_row = row_ok ? row / c.g : 0;
    const int h_row = kvh * c.g + (row_ok ? row - t_row * c.g : 0);

    // Loads that depend on the sequence: this lane's q slice (in the fused
    // step only wave 0's: it lays out the rows that every wave rotates), the
    // block ids of the split's first piece (thread i: ids i, i + 256, ...)
    // and, in the fused step, this thread's first new-key pair.  Without a
    // window, and when no longest-first ranking picks the sequence, none of
    // them needs the sequence's length: they go out together with it, one
    // memory round trip for all.  Otherwise they follow the length (and the
    // ranking).
    float xq[4][8];
    int tb[MAX_PIECE_BLOCKS / 256];
    float kx = 0.0f, ky = 0.0f, vx = 0.0f, vy = 0.0f;
    // qo: local index of the position of the sequence's first new token.
    // The split's first key (set below) and its length: the plan's, or an
    // equal share of the sequence's range when the units are ranked.
    int split_key0 = 0, split_len = a.split_keys;
    auto new_pair = [&](int bb, int qo, int idx, int& ia, int& ic, size_t& src) {
        const int n0 = max(qo, split_key0);
        const int t = n0 + idx / HALF - qo;
        rope_pair(idx % HALF, HALF, a.interleaved, ia, ic);
        src = (((size_t)bb * c.T + t) * c.Hkv + kvh) * D;
    };
    auto load_q = [&](int bb) {
        if (FUSED && wave != 0) return;
        const float* qp = a.q + (((size_t)bb * c.T + t_row) * c.Hq + h_row) * D;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const float4 x0 = *(const float4*)(qp + 32 * kk + 8 * j);
            const float4 x1 = *(const float4*)(qp + 32 * kk + 8 * j + 4);
            xq[kk][0] = x0.x; xq[kk][1] = x0.y; xq[kk][2] = x0.z; xq[kk][3] = x0.w;
            xq[kk][4] = x1.x; xq[kk][5] = x1.y; xq[kk][6] = x1.z; xq[kk][7] = x1.w;
        }
    };
    // block ids from the one holding key kb0 on, inside the table row, as
    // many as a split can span
    const int span = min(MAX_PIECE_BLOCKS, ((a.split_keys + (1 << c.log2_bs) - 2) >> c.log2_bs) + 1);
    auto load_blocks = [&](int bb, int kb0) {
        const int* trow = c.table + (size_t)bb * c.max_blocks;
        const int blk0 = kb0 >> c.log2_bs;
#pragma unroll
        for (int r = 0; r < MAX_PIECE_BLOCKS / 256; ++r) {
            const int i = (int)threadIdx.x + 256 * r;
            tb[r] = i < span && blk0 + i < c.max_blocks ? trow[blk0 + i] : 0;
        }
    };
    // fused step: pair threadIdx.x % HALF of new token t0 + threadIdx.x / HALF
    auto load_new_pair = [&](int bb, int t0) {
        if constexpr (FUSED) {
            const int t = t0 + (int)threadIdx.x / HALF;
            if (t >= 0 && t < c.T) {
                int ia, ic;
                rope_pair(threadIdx.x % HALF, HALF, a.interleaved, ia, ic);
                const size_t src = (((size_t)bb * c.T + t) * c.Hkv + kvh) * D;
                const int i = threadIdx.x % HALF;
                kx = a.k_new[src + ia];
                ky = a.k_new[src + ic];
                vx = a.v_new[src + 2 * i];
                vy = a.v_new[src + 2 * i + 1];
            }
        }
    };
    // In the same case each lane also fetches the block id of one key of its
    // wave's first tile (lanes 32..63 repeat 0..31), and the first tile is
    // issued from these ids before anything else waits.  The reads stay
    // inside the table row.
    const bool ranked = a.rank_longest && c.B > 1 && c.B <= LPT_MAX_SEQS;
    const bool early = c.window == 0 && !ranked;
    const int spec_base = split * a.split_keys + wave * TILE;
    int spec_blk = 0;
    // fused step: the frequency of this thread's rotation pair (pair
    // threadIdx.x % HALF in every round of the angle loop)
    const double theta = FUSED ? kernarg_double(offsetof(AttnArgs, theta), threadIdx.x % HALF) : 0.0;
    if (early) {
        const long long skey = (long long)spec_base + (lane & 31);
        if (skey < ((long long)c.max_blocks << c.log2_bs))
            spec_blk = c.table[(size_t)z * c.max_blocks + (int)(skey >> c.log2_bs)];
        load_blocks(z, split * a.split_keys);
        load_q(z);
        load_new_pair(z, 0);
    }
    int b = z;
    int L = c.seq_lens[z];
    if (ranked && a.num_splits > 1 && c.B * a.num_splits <= 256) {
        // the ranking borrows the V-tile LDS (unused until the key loop)
        const int u = lpt_unit_pick(a, split + a.num_splits * z, (unsigned*)sm_v, (int*)sm_v + 256,
                                    (int*)sm_v + 512, L);
        b = u / a.num_splits;
        split = u - b * a.num_splits;
    } else if (ranked && c.B <= 64) {
        b = lpt_rank_pick_wave(c.B, z, c.seq_lens, L);
    } else if (ranked) {
        // the ranking borrows the V-tile LDS (unused until the key loop)
        b = lpt_rank_pick(c.B, z, c.seq_lens, (unsigned*)sm_v, (int*)sm_v + LPT_MAX_SEQS, L);
    }
    const int qo = q_local0(c, b, L);
    if (!early) load_q(b);
    const int nn = n_new(c, b);          // new tokens of this sequence (rows past them: padding)
    const int rend = range_end(c, L, qo, nn);
    int key_begin = range_start(c, qo) + split * a.split_keys;
    if (ranked && a.num_splits > 1) {
        int k1;
        split_len = equal_split(range_start(c, qo), rend, a.num_splits, split, a.split_keys, key_begin, k1);
    }
    split_key0 = key_begin;
    const bool self_merge = a.num_splits > 1 && a.counters;
    if (key_begin >= rend) {            // empty split
        if (self_merge) {
            float own_o[PER_THREAD], own_m[PER_THREAD], own_l[PER_THREAD];
#pragma unroll
            for (int k = 0; k < PER_THREAD; ++k) {
                own_o[k] = 0.0f;
                own_m[k] = M_EMPTY;
                own_l[k] = 0.0f;
            }
            merge_own_splits(a, b, kvh, split, nn, range_start(c, qo), rend, split_len, own_o, own_m, own_l);
        } else {
            write_empty_partials(a, b, kvh, split, 0, a.rows);
        }
        return;
    }
    const int key_end = min(rend, key_begin + split_len);
    if (!early) load_blocks(b, key_begin);
    // first new token this split holds (if any): the early pair assumed 0
    const int t0 = max(qo, key_begin) - qo;
    if (!early || t0 != 0) load_new_pair(b, t0);
    const bool row_live = row_ok && t_row < nn;
    const int vis = row_live ? qo + t_row : -1;            // last key this row sees
    const int lo = c.window > 0 ? vis - c.window + 1 : 0;  // first key it sees

    // Q^T operand for row n16: dims 32*kk + 8*j .. +8, scaled into log2 units
    // and split into bf16 hi + lo.  Set up while the first tile's loads are
    // in flight.
    bf16x8 qhi[4], qlo[4];
    auto prepare_q = [&]() {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float v = row_ok ? xq[kk][e] * a.scale_log2 : 0.0f;
                const __bf16 hi = (__bf16)v;
                qhi[kk][e] = hi;
                qlo[kk][e] = (__bf16)(v - (float)hi);
            }
    };

    // Fused step: the angles of the T new positions (once per workgroup, into
    // LDS); the query rows rotated one pair per thread (rounded to fp32, as
    // q_rot); the new K/V rows that fall in this split rotated, rounded to
    // bf16, stored into the cache and kept in LDS for the tiles.
    const int new0 = qo;                // first new token's key index
    auto fused_angles = [&]() {
        static_assert(256 % HALF == 0, "a thread keeps its pair in every round");
        for (int idx = threadIdx.x; idx < c.T * HALF; idx += blockDim.x)
            rope_angle(theta, new0 + idx / HALF, sm_cs[idx], sm_sn[idx]);
    };
    // wave 0's raw slices of the rows into LDS (every wave holds the same
    // rows); the rotation reads them after the barrier that follows the angles
    auto fused_stage_q = [&]() {
        if (wave == 0 && row_ok) {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                float* qs = sm_q + row * D + 32 * kk + 8 * j;
                *(float4*)qs = make_float4(xq[kk][0], xq[kk][1], xq[kk][2], xq[kk][3]);
                *(float4*)(qs + 4) = make_float4(xq[kk][4], xq[kk][5], xq[kk][6], xq[kk][7]);
            }
        }
    };
    auto fused_rotate_q = [&]() {
        // one pair per thread, then each lane takes its rotated slice back
        // (rotated per lane, the sixteen pairs' fp64 temporaries would not
        // fit beside the first loads)
        for (int idx = threadIdx.x; idx < a.rows * HALF; idx += blockDim.x) {
            const int r = idx / HALF, i = idx % HALF, t = r / c.g;
            int ia, ic;
            rope_pair(i, HALF, a.interleaved, ia, ic);
            double xr, yr;
            rope_rotate(sm_q[r * D + ia], sm_q[r * D + ic], sm_cs[t * HALF + i], sm_sn[t * HALF + i], xr, yr);
            const float x1 = (float)xr, y1 = (float)yr;
            sm_q[r * D + ia] = x1;
            sm_q[r * D + ic] = y1;
        }
        __syncthreads();
        if (row_ok) {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const float4 x0 = *(const float4*)(sm_q + row * D + 32 * kk + 8 * j);
                const float4 x1 = *(const float4*)(sm_q + row * D + 32 * kk + 8 * j + 4);
                xq[kk][0] = x0.x; xq[kk][1] = x0.y; xq[kk][2] = x0.z; xq[kk][3] = x0.w;
                xq[kk][4] = x1.x; xq[kk][5] = x1.y; xq[kk][6] = x1.z; xq[kk][7] = x1.w;
            }
        }
    };
    auto fused_append = [&]() {
        // new keys n0 .. key_end-1 of this split (none unless it holds the
        // tail): pair idx goes to key n0 + idx / HALF.  The first pair of
        // each thread was loaded with q (a later round loads its own, so the
        // first round waits for nothing).
        const int n0 = max(new0, key_begin);
        if (key_end <= n0) return;
        const int count = (key_end - n0) * HALF;
        uint16_t* kc = (uint16_t*)c.k;
        uint16_t* vc = (uint16_t*)c.v;
        auto put = [&](int idx, int ia, int ic, float x0, float x1, float w0, float w1) {
            const int key = n0 + idx / HALF, i = idx % HALF, t = key - new0;
            double xr, yr;
            rope_rotate(x0, x1, sm_cs[t * HALF + i], sm_sn[t * HALF + i], xr, yr);
            const uint16_t k0 = bf16_from_f64(xr), k1 = bf16_from_f64(yr);
            const uint16_t v0 = bf16_from_f32(w0), v1 = bf16_from_f32(w1);
            // the host fuses only splits of at most MAX_PIECE_BLOCKS blocks,
            // so the staged block ids are the whole split's
            const int kblk = sm_blk[(key >> c.log2_bs) - (key_begin >> c.log2_bs)];
            const size_t dst = ((((size_t)kblk * c.Hkv + kvh) << c.log2_bs) + (key & ((1 << c.log2_bs) - 1))) * D;
            kc[dst + ia] = k0;
            kc[dst + ic] = k1;
            vc[dst + 2 * i] = v0;
            vc[dst + 2 * i + 1] = v1;
            sm_knew[t * D + ia] = k0;
            sm_knew[t * D + ic] = k1;
            sm_vnew[t * D + 2 * i] = v0;
            sm_vnew[t * D + 2 * i + 1] = v1;
        };
        if ((int)threadIdx.x < count) {
            int ia, ic;
            rope_pair(threadIdx.x % HALF, HALF, a.interleaved, ia, ic);
            put(threadIdx.x, ia, ic, kx, ky, vx, vy);
        }
        for (int idx = threadIdx.x + blockDim.x; idx < count; idx += blockDim.x) {
            int ia, ic;
            size_t src;
            new_pair(b, qo, idx, ia, ic, src);
            const int i = idx % HALF;
            put(idx, ia, ic, a.k_new[src + ia], a.k_new[src + ic], a.v_new[src + 2 * i], a.v_new[src + 2 * i + 1]);
        }
    };

    const char* kbase = (const char*)c.k;
    const char* vbase = (const char*)c.v;
    const int bs_mask = (1 << c.log2_bs) - 1;
    char* vt = sm_v + wave * VT_BYTES;

    float m = M_EMPTY, lsum = 0.0f;
    f32x4 o[8];
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) o[nt] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};

    // K operands: tile h (16 keys), step kk: lane l reads key l%16, bytes
    // [64*kk + 16*j, +16).  V rows: load i reads key 4*i + j, chunk n16.
    // Keys past the piece end re-read its last key (weight 0 below).
    // blk_of(key) gives the block id of a key of the tile.  V goes out
    // before K: a tile first stores its V rows to LDS, which then waits for
    // V alone (the memory counter is in order), and the next tile's V loads
    // go out right after that store, before the tile's score MFMAs; the next
    // K loads follow the MFMAs that free their registers.
    u32x4 kf[8], vf[8];
    auto row_of = [&](const char* basep, int key, auto&& blk_of) -> const char* {
        const size_t slot = (((size_t)blk_of(key) * c.Hkv + kvh) << c.log2_bs) + (key & bs_mask);
        return basep + slot * (D * 2);
    };
    auto issue_v = [&](int base, int pend, auto&& blk_of) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const char* vr = row_of(vbase, min(base + 4 * i + j, pend - 1), blk_of);
            vf[i] = __builtin_nontemporal_load((const u32x4*)(vr + 16 * n16));
        }
    };
    auto issue_k = [&](int base, int pend, auto&& blk_of) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const char* kr = row_of(kbase, min(base + 16 * h + n16, pend - 1), blk_of);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                kf[4 * h + kk] = __builtin_nontemporal_load((const u32x4*)(kr + 64 * kk + 16 * j));
        }
    };
    auto issue = [&](int base, int pend, auto&& blk_of) {
        issue_v(base, pend, blk_of);
        issue_k(base, pend, blk_of);
    };
    const int first_p1 = (int)min((long long)key_end,
                                  ((long long)(key_begin >> c.log2_bs) + MAX_PIECE_BLOCKS) << c.log2_bs);
    // Every load above is taken into use before the first tile goes out: a
    // wait on one of them after that point would also wait (the counter is
    // in order) for the tile.  The first piece's block ids go to LDS; the
    // fused step's raw q rows go to LDS and its new-key pair and frequency
    // are made ready; otherwise q is converted to the MFMA operands.
    {
        const int nblk0 = ((first_p1 - 1) >> c.log2_bs) - (key_begin >> c.log2_bs) + 1;
#pragma unroll
        for (int r = 0; r < MAX_PIECE_BLOCKS / 256; ++r) {
            const int i = (int)threadIdx.x + 256 * r;
            if (i < nblk0) sm_blk[i] = tb[r];
        }
    }
    if constexpr (FUSED) {
        fused_stage_q();
        __asm__ volatile("" : : "v"(kx), "v"(ky), "v"(vx), "v"(vy), "v"(theta));
    } else {
        prepare_q();
    }
    const bool spec = early && spec_base < first_p1;
    if (spec) issue(spec_base, first_p1, [&](int key) { return __shfl(spec_blk, key - spec_base); });
    // The fused step's work runs while the first tile is in flight, before
    // the first piece (whose barriers also publish the new K/V rows in LDS).
    if constexpr (FUSED) {
        fused_angles();
        __syncthreads();                    // angles, raw q rows and block ids in LDS
        fused_rotate_q();
        fused_append();
    }

    // pieces of at most MAX_PIECE_BLOCKS cache blocks (block ids in LDS)
    for (int p0 = key_begin; p0 < key_end;) {
        const int blk0 = p0 >> c.log2_bs;
        const int p1 = (int)min((long long)key_end, ((long long)blk0 + MAX_PIECE_BLOCKS) << c.log2_bs);
        const int nblk = ((p1 - 1) >> c.log2_bs) - blk0 + 1;
        const int* trow = c.table + (size_t)b * c.max_blocks + blk0;
        __syncthreads();                      // the previous piece is done with LDS
        // (the first piece's block ids were staged before the first tile)
        if (p0 != key_begin)
            for (int i = threadIdx.x; i < nblk; i += blockDim.x) sm_blk[i] = trow[i];
        __syncthreads();

        auto staged = [&](int key) { return sm_blk[(key >> c.log2_bs) - blk0]; };

        // One buffer of K/V registers per wave: the V rows go to LDS and the
        // K rows into the score MFMAs first, then the registers take the next
        // tile's loads, which stay in flight through the softmax and P.V of
        // this tile (and behind the other wave on the SIMD).
        constexpr int STRIDE = WAVES * TILE;
        int base = p0 + wave * TILE;
        if (base < p1 && !(spec && p0 == key_begin)) issue(base, p1, staged);
        if (FUSED && p0 == key_begin) prepare_q();
        // One tile of the wave: scores, softmax, P.V, and the next tile's
        // loads.  SUBST: the tile's loaded keys may include new tokens (the
        // fused step's last tiles), whose rows are taken from LDS.
        auto tile = [&](int base, auto subst) {
            constexpr bool SUBST = decltype(subst)::value;
            if constexpr (SUBST) {
                // rows of new tokens (also where a clamped lane re-reads one)
                // come from LDS, whatever the loads returned
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int key = min(base + 16 * h + n16, p1 - 1);
                    if (key >= new0)
#pragma unroll
                        for (int kk = 0; kk < 4; ++kk)
                            kf[4 * h + kk] = *(const u32x4*)(sm_knew + (key - new0) * D + 32 * kk + 8 * j);
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int key = min(base + 4 * i + j, p1 - 1);
                    if (key >= new0) vf[i] = *(const u32x4*)(sm_vnew + (key - new0) * D + 8 * n16);
                }
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) *(u32x4*)(vt + (4 * i + j) * ROWB + 16 * n16) = vf[i];
            const bool more = base + STRIDE < p1;
            if (more) issue_v(base + STRIDE, p1, staged);

            // scores: S^T tiles (16 keys x 16 rows), keys base + 16h + 4j + i
            f32x4 s[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const bf16x8 kop = as_bf16x8(kf[4 * h + kk]);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qhi[kk], acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qlo[kk], acc, 0, 0, 0);
                }
                s[h] = acc;
            }
            if (more) issue_k(base + STRIDE, p1, staged);

            // mask, running max, weights
            float mx = m;
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = base + 16 * h + 4 * j + i;
                    if (key >= p1 || key > vis || key < lo) s[h][i] = -INFINITY;
                    mx = fmaxf(mx, s[h][i]);
                }
            mx = xor_max(mx);
            const float alpha = fast_exp2(m - mx);
            m = mx;
            lsum *= alpha;
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) o[nt] *= alpha;
            bf16x8 phi, plo;
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float p = fast_exp2(s[h][i] - m);
                    lsum += p;
                    const __bf16 hi = (__bf16)p;
                    phi[4 * h + i] = hi;
                    plo[4 * h + i] = (__bf16)(p - (float)hi);
                }
            __builtin_amdgcn_wave_barrier();
            // O^T += V^T . P^T; lane (n16, j) reads V rows 4j + i (first half
            // of the key order) and 16 + 4j + i (second half) of dim tile nt.
            const char* rd = vt + (4 * j + (n16 >> 2)) * ROWB + 8 * (n16 & 3);
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) {
                const bf16x8 vop = join(lds_tr(rd + 32 * nt), lds_tr(rd + 16 * ROWB + 32 * nt));
                o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, phi, o[nt], 0, 0, 0);
                o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, plo, o[nt], 0, 0, 0);
            }
            __builtin_amdgcn_wave_barrier();
        };
        // tiles before the first new token, then (fused step) the rest
        for (; base < p1 && (!FUSED || min(base + TILE, p1) - 1 < new0); base += STRIDE)
            tile(base, std::false_type{});
        if constexpr (FUSED)
            for (; base < p1; base += STRIDE) tile(base, std::true_type{});
        p0 = p1;
    }

    // per-wave state -> LDS: row n16's sum over the four lane groups; O^T
    // element (dim 16*nt + 4*j + i, row n16)
    lsum = xor_sum(lsum);
    __syncthreads();          // every wave is done with its V tile
    if (j == 0) {
        sm_m[wave][n16] = m;
        sm_l[wave][n16] = lsum;
    }
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) sm_o[wave][n16][16 * nt + 4 * j + i] = o[nt][i];
    __syncthreads();

    // merge the four waves; write the rows (one split) or the partial.  With
    // several splits and arrival counters, the partial is published with
    // agent-scope stores (coherent across the XCDs without a cache
    // write-back) and this thread keeps its values for a merge of its own.
    float own_o[PER_THREAD], own_m[PER_THREAD], own_l[PER_THREAD];
#pragma unroll
    for (int k = 0; k < PER_THREAD; ++k) {
        const int idx = (int)threadIdx.x + 256 * k;
        const int r = idx / D, d = idx - r * D;
        if (r >= a.rows) break;
        float M = sm_m[0][r];
#pragma unroll
        for (int w = 1; w < WAVES; ++w) M = fmaxf(M, sm_m[w][r]);
        float Ls = 0.0f, O = 0.0f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) {
            const float f = fast_exp2(sm_m[w][r] - M);
            Ls += sm_l[w][r] * f;
            O += sm_o[w][r][d] * f;
        }
        const int t = r / c.g;
        const int h = kvh * c.g + (r - t * c.g);
        const size_t qrow = ((size_t)b * c.T + t) * c.Hq + h;
        if (a.num_splits == 1) {
            if (t >= nn) break;             // padding rows (past a ragged chunk) are left as they are
            a.out[qrow * D + d] = finish_out(O, Ls);
            if (a.lse && d == 0) a.lse[qrow] = finish_lse(M, Ls);
        } else if (self_merge) {
            const size_t part = qrow * a.num_splits + split;
            __hip_atomic_store(a.part_o + part * D + d, O, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (d == 0) {
                __hip_atomic_store(a.part_ml + part * 2 + 0, M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(a.part_ml + part * 2 + 1, Ls, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            own_o[k] = O;
            own_m[k] = M;
            own_l[k] = Ls;
        } else {
            a.part_o[(qrow * a.num_splits + split) * D + d] = O;
            if (d == 0) {
                a.part_ml[(qrow * a.num_splits + split) * 2 + 0] = M;
                a.part_ml[(qrow * a.num_splits + split) * 2 + 1] = Ls;
            }
        }
    }

    // the rotated queries, when asked for (split 0 writes them): after the
    // key loop, so that the first tile's wait does not include them
    if (FUSED && a.q_rot && split == 0)
        for (int idx = threadIdx.x; idx < a.rows * D; idx += blockDim.x) {
            const int r = idx / D, d = idx - r * D, t = r / c.g;
            if (t < nn) a.q_rot[(((size_t)b * c.T + t) * c.Hq + kvh * c.g + (r - t * c.g)) * D + d] = sm_q[idx];
        }

    if (self_merge) merge_own_splits(a, b, kvh, split, nn, range_start(c, qo), rend, split_len, own_o, own_m, own_l);
}

__global__ __launch_bounds__(256, 2) void attn_mfma_kernel(AttnArgs a) { attn_mfma_body<false>(a); }

// the fused decode step (its own name, so that profiles tell the two apart)
__global__ __launch_bounds__(256, 2) void decode_step_mfma_kernel(AttnArgs a) { attn_mfma_body<true>(a); }

}  // namespace

bool mfma_supported(int D_, int kv_bf16, int rows) { return D_ == D && kv_bf16 && rows >= 1 && rows <= 16; }

int mfma_step_keys() { return WAVES * TILE; }

hipError_t launch_attn_mfma(const AttnArgs& a, hipStream_t s) {
    dim3 grid(a.c.Hkv, a.num_splits, a.c.B);
    if (a.fused)
        hipLaunchKernelGGL(decode_step_mfma_kernel, grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(attn_mfma_kernel, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace kvd
