// attn_prefill.hip -- attention of many query rows per kv head against the
// paged cache: chunked prefill (the ferric-core generate.rs page treats
// prefill and decode as the same step; the Ferrum Infer README sends prefill
// through a flash-attention kernel) and long drafts, g*T > 16 rows, bf16
// cache, head_dim 128.  Causal within the chunk: new token t sees the keys up
// to its own position.
//
// Workgroup = 4 wave64s over a tile of 64 query rows of one (sequence, kv
// head) -- wave w owns rows 16w .. 16w+15 of the tile, row r = t*g + hg --
// and one key range (split).  Unlike the decode kernel, every wave needs
// every key, so the K and V tiles (32 keys) are staged in LDS once by all 256
// threads and shared by the four waves: the kv-head group's rows share the
// keys, which is what makes the work dense enough for the matrix cores.
// Double-buffered: while the waves consume tile i from LDS, each thread's
// registers hold its share of tile i+1 on the way from HBM (one barrier per
// tile).  Per wave and tile, as in the decode kernel:
//   S^T[32 keys x 16 rows] = K . Q^T   (K from LDS, Q as bf16 hi + lo),
//   online softmax per row (the row sits in lane l%16),
//   O^T[128 x 16 rows] += V^T . P^T    (V^T read transposed from LDS, P as
//   bf16 hi + lo).
// The loop ends at the last key any row of the tile sees.  Split ranges,
// windows, ragged chunks and context-parallel shards follow the same rules as
// the decode kernels (kvd_internal.h).
#include "kvd_internal.h"

namespace kvd {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int WAVES = 4;
constexpr int D = 128;
constexpr int TILE = 32;
constexpr int ROWS = WAVES * 16;          // query rows per workgroup
constexpr int KROWB = D * 2 + 16;         // LDS row stride of the K tile: 16 rows read at one column hit distinct banks
constexpr int VROWB = D * 2 + 32;         // LDS row stride of the V tile (transposed reads)
constexpr int K_BYTES = TILE * KROWB;
constexpr int V_BYTES = TILE * VROWB;
constexpr int MAX_STAGED_BLOCKS = 4096;   // block ids of a split, staged in LDS
constexpr float M_EMPTY = -1e30f;
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

__device__ inline float xor_max(float x) {
    x = fmaxf(x, __shfl_xor(x, 16));
    return fmaxf(x, __shfl_xor(x, 32));
}

__device__ inline float xor_sum(float x) {
    x += __shfl_xor(x, 16);
    return x + __shfl_xor(x, 32);
}

__global__ __launch_bounds__(256, 2) void attn_prefill_kernel(AttnArgs a) {
    __shared__ __attribute__((aligned(16))) char sm_k[2][K_BYTES];
    __shared__ __attribute__((aligned(16))) char sm_v[2][V_BYTES];
    __shared__ int sm_blk[MAX_STAGED_BLOCKS];

    const CacheView& c = a.c;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int n16 = lane & 15;
    const int j = lane >> 4;
    const int split = blockIdx.x;
    const int kvh = blockIdx.y % c.Hkv;
    const int rtile = blockIdx.y / c.Hkv;
    const int b = blockIdx.z;
    const int row0 = rtile * ROWS;

    const int L = c.seq_lens[b];
    const int nn = n_new(c, b);
    const int qo = q_local0(c, b, L);
    const int key_begin = range_start(c, qo) + split * a.split_keys;
    // rows of this tile that are real (not past the chunk): t < nn
    const int live_rows = min(ROWS, nn * c.g - row0);
    // the last key a row of this tile sees
    const int t_last = min(nn, (row0 + ROWS - 1) / c.g + 1) - 1;
    const int key_end = min(min(range_end(c, L, qo, nn), key_begin + a.split_keys), qo + t_last + 1);
    if (live_rows <= 0 || key_begin >= key_end) {
        write_empty_partials(a, b, kvh, split, row0, ROWS);
        return;
    }

    // this lane's query row (within the wave's 16) and its visible keys
    const int row = row0 + 16 * wave + n16;
    const bool row_ok = row < a.rows;
    const bool row_live = row_ok && row < nn * c.g;
    const int t_row = row_ok ? row / c.g : 0;
    const int h_row = kvh * c.g + (row_ok ? row - t_row * c.g : 0);
    const int vis = row_live ? qo + t_row : -1;
    const int lo = c.window > 0 ? vis - c.window + 1 : 0;

    // Q^T operand (dims 32kk + 8j .. +8 of the row) in log2 units, hi + lo
    bf16x8 qhi[4], qlo[4];
    {
        const float* qp = a.q + (((size_t)b * c.T + t_row) * c.Hq + h_row) * D;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const float4 x0 = *(const float4*)(qp + 32 * kk + 8 * j);
            const float4 x1 = *(const float4*)(qp + 32 * kk + 8 * j + 4);
            const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float v = row_ok ? xs[e] * a.scale_log2 : 0.0f;
                const __bf16 hi = (__bf16)v;
                qhi[kk][e] = hi;
                qlo[kk][e] = (__bf16)(v - (float)hi);
            }
        }
    }

    // block ids of [key_begin, key_end)
    const int blk0 = key_begin >> c.log2_bs;
    const int nblk = ((key_end - 1) >> c.log2_bs) - blk0 + 1;
    const int* trow = c.table + (size_t)b * c.max_blocks + blk0;
    for (int i = tid; i < nblk; i += blockDim.x) sm_blk[i] = trow[i];
    __syncthreads();

    // Each thread moves 2 of the 512 16-byte chunks of a K tile and 2 of the
    // V tile: chunk ch = tid + 256*i -> key ch / 16, column ch % 16.  Keys past
    // the range re-read its last key (weight 0 below).
    const char* kbase = (const char*)c.k;
    const char* vbase = (const char*)c.v;
    const int bs_mask = (1 << c.log2_bs) - 1;
    u32x4 kr[2], vr[2];
    auto load = [&](int base) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int ch = tid + 256 * i;
            const int key = min(base + (ch >> 4), key_end - 1);
            const int blk = sm_blk[(key >> c.log2_bs) - blk0];
            const size_t slot = (((size_t)blk * c.Hkv + kvh) << c.log2_bs) + (key & bs_mask);
            kr[i] = __builtin_nontemporal_load((const u32x4*)(kbase + slot * (D * 2) + 16 * (ch & 15)));
            vr[i] = __builtin_nontemporal_load((const u32x4*)(vbase + slot * (D * 2) + 16 * (ch & 15)));
        }
    };
    auto stage = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int ch = tid + 256 * i;
            *(u32x4*)(sm_k[buf] + (ch >> 4) * KROWB + 16 * (ch & 15)) = kr[i];
            *(u32x4*)(sm_v[buf] + (ch >> 4) * VROWB + 16 * (ch & 15)) = vr[i];
        }
    };

    float m = M_EMPTY, lsum = 0.0f;
    f32x4 o[8];
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) o[nt] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};

    load(key_begin);
    stage(0);
    __syncthreads();
    if (key_begin + TILE < key_end) load(key_begin + TILE);

    int buf = 0;
    for (int base = key_begin; base < key_end; base += TILE, buf ^= 1) {
        const char* kt = sm_k[buf];
        const char* vt = sm_v[buf];
        // scores: S^T tiles (16 keys x 16 rows), keys base + 16h + 4j + i
        f32x4 s[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
            const char* kp = kt + (16 * h + n16) * KROWB + 16 * j;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const bf16x8 kop = as_bf16x8(*(const u32x4*)(kp + 64 * kk));
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qhi[kk], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qlo[kk], acc, 0, 0, 0);
            }
            s[h] = acc;
        }
        // mask, running max, weights
        float mx = m;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = base + 16 * h + 4 * j + i;
                if (key >= key_end || key > vis || key < lo) s[h][i] = -INFINITY;
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
        // O^T += V^T . P^T; lane (n16, j) reads V rows 4j + i and 16 + 4j + i
        const char* rd = vt + (4 * j + (n16 >> 2)) * VROWB + 8 * (n16 & 3);
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
            const bf16x8 vop = join(lds_tr(rd + 32 * nt), lds_tr(rd + 16 * VROWB + 32 * nt));
            o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, phi, o[nt], 0, 0, 0);
            o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, plo, o[nt], 0, 0, 0);
        }
        // the next tile into the other buffer (read two tiles ago, released
        // by the last barrier), then the one after it from HBM
        if (base + TILE < key_end) stage(buf ^ 1);
        __syncthreads();
        if (base + 2 * TILE < key_end) load(base + 2 * TILE);
    }

    // row n16's sum over the four lane groups; O^T element (dim 16nt + 4j + i, row n16)
    lsum = xor_sum(lsum);
    if (!row_ok) return;
    const int t = t_row;
    const size_t qrow = ((size_t)b * c.T + t) * c.Hq + h_row;
    if (a.num_splits == 1) {
        float* op = a.out + qrow * D;
#pragma unroll
        for (int nt = 0; nt < 8; ++nt)
            *(float4*)(op + 16 * nt + 4 * j) = make_float4(finish_out(o[nt][0], lsum), finish_out(o[nt][1], lsum),
                                                           finish_out(o[nt][2], lsum), finish_out(o[nt][3], lsum));
        if (a.lse && j == 0) a.lse[qrow] = finish_lse(m, lsum);
    } else {
        const size_t part = qrow * a.num_splits + split;
        float* op = a.part_o + part * D;
#pragma unroll
        for (int nt = 0; nt < 8; ++nt)
            *(float4*)(op + 16 * nt + 4 * j) = make_float4(o[nt][0], o[nt][1], o[nt][2], o[nt][3]);
        if (j == 0) {
            a.part_ml[part * 2 + 0] = m;
            a.part_ml[part * 2 + 1] = lsum;
        }
    }
}

}  // namespace

int prefill_step_keys() { return TILE; }

hipError_t launch_attn_prefill(const AttnArgs& a, hipStream_t s) {
    const int n_rtiles = (a.rows + ROWS - 1) / ROWS;
    dim3 grid(a.num_splits, a.c.Hkv * n_rtiles, a.c.B);
    hipLaunchKernelGGL(attn_prefill_kernel, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace kvd
