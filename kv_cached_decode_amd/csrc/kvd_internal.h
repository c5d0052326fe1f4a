// kvd_internal.h -- launch parameters shared by the host dispatcher (kvd.cpp)
// and the kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvd {

// Everything a kernel needs about the paged cache and the batch.
struct CacheView {
    int32_t B, T, Hq, Hkv, D;
    int32_t g;              // Hq / Hkv
    int32_t log2_bs;        // block size is a power of two
    int32_t max_blocks;     // block_table row stride
    const int32_t* table;   // [B][max_blocks]
    const int32_t* seq_lens;  // [B]
    void* k;                // [num_blocks][Hkv][bs][D]
    void* v;
    int32_t window;         // sliding window in keys, 0 = none
    const int32_t* key_pos0;  // [B] context-parallel shard: global position of local key 0, or null
    const int32_t* q_pos;     // [B] global position of new token 0, or null
    const int32_t* q_lens;    // [B] new tokens per sequence (<= T), or null = T
};

// New tokens of sequence b (rows t >= n_new are padding).
__device__ inline int n_new(const CacheView& c, int b) { return c.q_lens ? c.q_lens[b] : c.T; }

// Local index of the position of a sequence's new token 0 (the last key its
// first query sees): seq_lens - n_new for a whole cache; q_pos - key_pos0 for a
// context-parallel shard, which may lie past the shard's keys (all of them
// visible) or before them (none).
__device__ inline int q_local0(const CacheView& c, int b, int L) {
    if (!c.q_pos) return L - n_new(c, b);
    return c.q_pos[b] - (c.key_pos0 ? c.key_pos0[b] : 0);
}

// Keys any query of a sequence can see: [range_start, range_end), from the
// start of the first query's window (0 without one) to the last query's
// position.  Split s covers [range_start + s*split_keys, min(range_end,
// range_start + (s+1)*split_keys)), except in the matrix-core decode kernel
// when it ranks its units, where the S splits are equal shares of the range.
__device__ inline int range_start(const CacheView& c, int qo) {
    return c.window > 0 ? max(0, qo - c.window + 1) : 0;
}
__device__ inline int range_end(const CacheView& c, int L, int qo, int nn) { return max(0, min(L, qo + nn)); }

// theta_i = rope_base^(-2i/D) for i < D/2, evaluated on the host.
struct RopeTheta {
    double v[128];
};

struct RopeAppendArgs {
    CacheView c;
    int32_t kv_bf16;
    int32_t interleaved;
    int32_t skip_q;         // rotate and append the new K/V rows only (q and q_rot unused)
    RopeTheta theta;
    const float* q;
    const float* k;
    const float* v;
    float* q_rot;
};

// One key-range partition per (b, kv head, split); rows of a (b, kv head)
// pair are the g*T query rows (t, h in group) that read it.
struct AttnArgs {
    CacheView c;
    int32_t kv_bf16;
    int32_t num_splits;     // S
    int32_t split_keys;     // keys per split (multiple of the kernel's step)
    int32_t rows;           // g*T
    int32_t row_tile;       // rows handled by one workgroup (grid.x = Hkv * row tiles)
    int32_t rank_longest;   // order work longest-first (the grid exceeds the resident slots)
    float scale_log2;       // softmax scale * log2(e)
    const float* q;         // [B][T][Hq][D]
    float* out;             // [B][T][Hq][D] (written directly when S == 1)
    float* part_o;          // [B][T][Hq][S][D]   unnormalised partial outputs
    float* part_ml;         // [B][T][Hq][S][2]   (running max in log2 units, sum)
    float* lse;             // [B][T][Hq] natural-log log-sum-exp of the row, or null
    // [B][Hkv] arrival counters (zero between calls), or null: with several
    // splits, the last workgroup of a (sequence, kv head) to finish merges
    // the partials itself instead of the combine kernel
    unsigned* counters;
    // Fused decode step (matrix-core decode kernel only): q holds the raw
    // queries; the kernel rotates them, appends the new K/V rows of its split
    // to the cache and writes the rotated queries to q_rot when that is
    // non-null.
    int32_t fused;
    // Prefill kernel: q holds the raw queries, which the kernel rotates at
    // their positions (the new K/V rows are appended by the RoPE/append
    // kernel before it); the rotated queries go to q_rot when non-null.
    int32_t rope_q;
    int32_t interleaved;
    RopeTheta theta;
    const float* k_new;     // [B][T][Hkv][D] new keys before RoPE
    const float* v_new;     // [B][T][Hkv][D] new values
    float* q_rot;           // [B][T][Hq][D] or null
};

// A split that holds no key of its sequence leaves, for its rows, a partial
// that drops out of the merge (running max -1e30, sum 0, output 0), so the
// merge combines every split without reading the sequence lengths.  With a
// single split (a context-parallel shard without a key of the sequence) the
// rows are final: output 0, lse -inf.  Rows of padding tokens past a ragged
// chunk are left as they are.
__device__ inline void write_empty_partials(const AttnArgs& a, int b, int kvh, int split, int row0,
                                            int nrows) {
    const CacheView& c = a.c;
    const int D = c.D;
    const int lq = __builtin_ctz(D) - 2;      // D / 4 float4s a row (D a power of two >= 16)
    const int live = a.num_splits == 1 ? min(a.rows, n_new(c, b) * c.g) : a.rows;
    const int n4 = max(0, min(row0 + nrows, live) - row0) << lq;
    const float4 zero = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    for (int idx = threadIdx.x; idx < n4; idx += blockDim.x) {
        const int r = row0 + (idx >> lq), e4 = idx & ((1 << lq) - 1);
        const int t = r / c.g;
        const size_t qrow = ((size_t)b * c.T + t) * c.Hq + kvh * c.g + (r - t * c.g);
        if (a.num_splits == 1) {
            *(float4*)(a.out + qrow * D + 4 * e4) = zero;
            if (e4 == 0 && a.lse) a.lse[qrow] = -INFINITY;
        } else {
            const size_t part = qrow * a.num_splits + split;
            *(float4*)(a.part_o + part * D + 4 * e4) = zero;
            if (e4 == 0) *(float2*)(a.part_ml + part * 2) = make_float2(-1e30f, 0.0f);
        }
    }
}

hipError_t launch_rope_append(const RopeAppendArgs& a, hipStream_t s);
hipError_t launch_attn_valu(const AttnArgs& a, hipStream_t s);
hipError_t launch_attn_mfma(const AttnArgs& a, hipStream_t s);
hipError_t launch_attn_combine(const AttnArgs& a, hipStream_t s);
hipError_t launch_attn_prefill(const AttnArgs& a, hipStream_t s);
hipError_t launch_check_descriptor(const CacheView& c, int max_seq_len, int num_blocks, unsigned* flags,
                                   hipStream_t s);
hipError_t launch_merge_partials(int n_parts, int64_t rows, int D, const float* outs, const float* lses,
                                 float* out, float* lse_out, hipStream_t s);

// The finished row from its running max M (log2 units), sum Ls and
// unnormalised output O: out = O / Ls, lse = (M + log2 Ls) ln 2; a row that
// saw no key (Ls = 0) gets out = 0 and lse = -inf.
__device__ inline float finish_out(float O, float Ls) { return Ls > 0.0f ? O / Ls : 0.0f; }
__device__ inline float finish_lse(float M, float Ls) {
    return Ls > 0.0f ? (M + log2f(Ls)) * 0.69314718055994531f : -INFINITY;
}

// Kernel-family properties the planner needs.
int valu_step_keys(int D, int kv_bf16);      // keys per workgroup step
int valu_max_row_tile(int D, int kv_bf16);   // rows one workgroup can hold
// Block ids of one split are staged in LDS; this bounds keys per split.
constexpr int VALU_MAX_STAGED_BLOCKS = 4096;
int valu_max_split_keys(int log2_bs);
bool mfma_supported(int D, int kv_bf16, int rows);
// Waves of one prefill workgroup (32 query rows each) and the workgroups a
// CU holds at once (two waves per SIMD either way).  Four waves and two
// workgroups per CU measured faster than eight and one (178 against 196 us
// on the chunked prefill): a workgroup's waves wait at the per-tile barrier,
// and a second workgroup on the CU fills those waits.
constexpr int PREFILL_WAVES = 4;
constexpr int PREFILL_WGS_PER_CU = PREFILL_WAVES == 4 ? 2 : 1;
// Query rows of one prefill workgroup (more rows than the decode kernel takes).
constexpr int PREFILL_ROWS = 32 * PREFILL_WAVES;
// Prefill grids of at most this many (sequence, row tile, split) units are
// ordered longest-first inside the kernel.
constexpr int PREFILL_RANK_MAX = 256;
int prefill_step_keys();
int mfma_step_keys();
// Workgroups of the decode matrix-core kernel resident on one CU.
constexpr int MFMA_WGS_PER_CU = 2;
// Shortest split the matrix-core decode kernel is planned with once the
// (sequence, kv head) units alone fill every CU's resident slots: a shorter
// split pays its set-up and its share of the merge for too little streaming,
// and only ragged batches with long sequences need the pieces to balance.
// Measured steps (1, 2 and 3 splits, one GPU), batches of 512 units:
//   multi-head 16 x 32 kv heads, 4097 keys:  164.3, 168.2, 171.4 us
//   64 x 8, uniform 2048 keys:               85.6,  97.4, 107.4 us
//   64 x 8, ragged 1..2048 keys:             63.8,  64.8,  68.4 us
//   64 x 8, ragged 1..400 keys:              18.4,  28.7,  36.5 us
//   64 x 8, ragged 129..8193 keys:          232.8, 182.2, 173.6 us
// so at least 2560 keys a split: one split for the first four, three for
// the last.
constexpr int MFMA_MIN_SPLIT_KEYS = 2560;
// Resident workgroups per CU for a kernel variant (occupancy query on the
// current device; a conservative default when there is none).
int valu_wgs_per_cu(int D, int kv_bf16, int row_tile, size_t dyn_lds);
// Query rows (g*T) from which the matrix-core kernel is the default: every
// bf16 head_dim-128 plan.  Measured (rocprof, one layer's step): the
// vector-ALU kernel reaches 57.6%, 60.6% and 35.5% of 8 TB/s at 4, 2 and 8
// rows per kv head (64.5%, 39.6% and 65.3% VALU busy: issue-bound at 4 and 8
// rows), the matrix-core kernel 72.2%, 72.5% and 81.4%; at one row per kv
// head (multi-head attention) 76.7% against 78.2%, where the fused kernel
// also saves the RoPE/append launch and the split combine.
constexpr int MFMA_MIN_ROWS = 1;
// Split count at which the decode matrix-core kernel merges its splits
// itself instead of leaving them to the combine kernel.
constexpr int SELF_MERGE_SPLITS = 2;
// Block ids the decode matrix-core kernel stages in LDS at a time (one
// piece of a split).  The fused step needs a split's blocks in one piece:
// its append takes the new keys' block ids from there.
constexpr int MFMA_PIECE_BLOCKS = 2048;

}  // namespace kvd
