// attn_valu.hip -- decode attention on the vector ALUs (single-token decode,
// and the generic path for any row count).
//
// The operation is `mha_decode_t` of ferric-core generate.rs (`step_gpu`): the
// query rows of one sequence attend against every key of its cache; query
// head h reads kv head h / (Hq/Hkv) (GQA, ferrox `decoder` module).  The
// Ferrum Infer README ("Key Optimizations") supplies the rest of the shape:
// one launch for all batch items, block-table indirection into a paged pool,
// and split-K (flash decoding) for long caches.
//
// Work decomposition: one workgroup (4 wave64s) per (split, kv head [x row
// tile], sequence).  The workgroup streams its key range in steps; within a
// step each wave owns U "groups" of KPG keys.  A group is one 16-byte
// global_load_dwordx4 per lane: LPK = 16*D/(16 bytes) lanes share one key row
// (for bf16, D = 128: 16 lanes x 8 elements), so every load instruction reads
// KPG whole rows, contiguous and 16-byte aligned.  The same registers feed
// every query row of the GQA group (K/V are read from HBM once per group).
//
//   QK:  each lane forms the partial dot product of its 8 (bf16) or 4 (fp32)
//        elements with every query row, then an xor butterfly over the LPK
//        lanes of the key (DPP quad_perm / half_mirror / mirror, then
//        ds_swizzle-class shuffles for 32/64) leaves the full score in all of
//        them, bitwise identical.
//   softmax: online, in log2 units (scale*log2(e) folded into q).  Each lane
//        group keeps its own running max m, sum l and output o for the keys it
//        has seen, rescaled once per step (not per key).
//   PV:  the V registers are in the same lane layout, so o += p * v needs no
//        data movement.
//   memory: the block ids of the workgroup's key range are staged in LDS
//        once; the K/V loads of the next step are issued before the current
//        step is computed (two register buffers), so each wave keeps a step's
//        rows in flight while it computes.
//   merge: groups of a wave merge by shuffles, the four waves through LDS;
//        the workgroup writes either the final row (one split) or its
//        unnormalised partial (m, l, o) for the combine kernel.
//
// Keys past the sequence end are never loaded (their slots may hold NaN):
// lanes past the range re-load the range's last key and weight it 0; keys past
// a draft token's own position, or before its sliding window, get score -inf
// and weight 0.
#include "kvd_internal.h"

namespace kvd {
namespace {

constexpr int WAVES = 4;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));   // one 16-byte load
constexpr float M_EMPTY = -1e30f; // running max before any key is seen

template <int CTRL>
__device__ inline float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of LPK consecutive lanes; every lane of a group
// ends with the same bits (each butterfly stage adds the same two values).
template <int LPK>
__device__ inline float group_sum(float x) {
    if constexpr (LPK >= 2) x += dpp<0xB1>(x);    // quad_perm [1,0,3,2]: lane ^ 1
    if constexpr (LPK >= 4) x += dpp<0x4E>(x);    // quad_perm [2,3,0,1]: lane ^ 2
    if constexpr (LPK >= 8) x += dpp<0x141>(x);   // row_half_mirror: i <-> 7 - i
    if constexpr (LPK >= 16) x += dpp<0x140>(x);  // row_mirror: i <-> 15 - i
    if constexpr (LPK >= 32) x += __shfl_xor(x, 16);
    if constexpr (LPK >= 64) x += __shfl_xor(x, 32);
    return x;
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int KV, int EPL>
__device__ inline void to_f32(const u32x4& r, float (&f)[EPL]) {
    if constexpr (KV) {
        const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(w[i] << 16);
            f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
    } else {
        f[0] = __uint_as_float(r.x);
        f[1] = __uint_as_float(r.y);
        f[2] = __uint_as_float(r.z);
        f[3] = __uint_as_float(r.w);
    }
}

// Keys per wave step for a head_dim / cache type.
template <int D, int KV>
struct Geo {
    static constexpr int ESZ = KV ? 2 : 4;
    static constexpr int EPL = 16 / ESZ;     // elements per lane per key
    static constexpr int LPK = D / EPL;      // lanes per key
    static constexpr int KPG = 64 / LPK;     // keys per group (one dwordx4 per lane)
    static constexpr int U = KPG >= 8 ? 2 : 4;   // groups per wave step
    static constexpr int WAVE_KEYS = U * KPG;
};

template <int D, int KV, int RT>
__global__ __launch_bounds__(256) void attn_valu_kernel(AttnArgs a) {
    using G = Geo<D, KV>;
    constexpr int EPL = G::EPL, LPK = G::LPK, KPG = G::KPG, U = G::U, WAVE_KEYS = G::WAVE_KEYS;
    static_assert(LPK >= 1 && LPK <= 64 && (64 % LPK) == 0, "unsupported head_dim");

    extern __shared__ int sm_blk[];              // block ids of this split's key range
    __shared__ float sm_o[WAVES][RT][D];
    __shared__ float sm_m[WAVES][RT];
    __shared__ float sm_l[WAVES][RT];

    const CacheView& c = a.c;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    // grid (kv head x row tile, split, sequence): kv heads fastest, so that
    // the round-robin dealing of workgroups to XCDs spreads equal work
    const int kvh = blockIdx.x % c.Hkv;
    const int rtile = blockIdx.x / c.Hkv;
    const int split = blockIdx.y;
    const int b = blockIdx.z;

    const int L = c.seq_lens[b];
    const int qo = q_local0(c, b, L);         // local index of the first new token's position
    const int key_begin = range_start(c, qo) + split * a.split_keys;
    const int nn = n_new(c, b);               // new tokens (rows past them: padding)
    const int rend = range_end(c, L, qo, nn);
    if (key_begin >= rend) {                  // empty split
        write_empty_partials(a, b, kvh, split, rtile * RT, RT);
        return;
    }
    const int key_end = min(rend, key_begin + a.split_keys);

    // stage the block ids of [key_begin, key_end) in LDS
    const int blk0 = key_begin >> c.log2_bs;
    const int nblk = ((key_end - 1) >> c.log2_bs) - blk0 + 1;
    const int* trow = c.table + (size_t)b * c.max_blocks + blk0;
    for (int i = threadIdx.x; i < nblk; i += blockDim.x) sm_blk[i] = trow[i];

    const int kslot = lane / LPK;
    const int chunk = lane % LPK;
    const int row0 = rtile * RT;

    // q rows of this tile, pre-scaled into log2 units; row r = t*g + hg.
    float qv[RT][EPL];
    int vis[RT], lo[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        const int row = row0 + r;
        const bool ok = row < a.rows && row / c.g < nn;
        const int t = ok ? row / c.g : 0;
        const int h = kvh * c.g + (ok ? row - t * c.g : 0);
        vis[r] = ok ? qo + t : -1;            // last visible key (inclusive)
        lo[r] = c.window > 0 ? vis[r] - c.window + 1 : 0;   // first visible key
        const float4* qp = (const float4*)(a.q + (((size_t)b * c.T + t) * c.Hq + h) * D + chunk * EPL);
#pragma unroll
        for (int e4 = 0; e4 < EPL / 4; ++e4) {
            const float4 v = qp[e4];
            qv[r][4 * e4 + 0] = ok ? v.x * a.scale_log2 : 0.0f;
            qv[r][4 * e4 + 1] = ok ? v.y * a.scale_log2 : 0.0f;
            qv[r][4 * e4 + 2] = ok ? v.z * a.scale_log2 : 0.0f;
            qv[r][4 * e4 + 3] = ok ? v.w * a.scale_log2 : 0.0f;
        }
    }

    float m[RT], l[RT], o[RT][EPL];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        m[r] = M_EMPTY;
        l[r] = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[r][e] = 0.0f;
    }
    __syncthreads();

    const char* kbase = (const char*)c.k;
    const char* vbase = (const char*)c.v;
    const int bs_mask = (1 << c.log2_bs) - 1;
    constexpr size_t ROW_BYTES = (size_t)D * G::ESZ;

    // Issue the loads of one wave step.  Keys past the range are clamped to
    // the last key of the range (finite data; masked to weight 0 below), so
    // the loads need no branch.
    auto issue = [&](int base, u32x4 (&kr)[U], u32x4 (&vr)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = min(base + u * KPG + kslot, key_end - 1);
            const int blk = sm_blk[(j >> c.log2_bs) - blk0];
            const size_t slot = (((size_t)blk * c.Hkv + kvh) << c.log2_bs) + (j & bs_mask);
            const size_t off = slot * ROW_BYTES + (size_t)chunk * 16;
            kr[u] = __builtin_nontemporal_load((const u32x4*)(kbase + off));
            vr[u] = __builtin_nontemporal_load((const u32x4*)(vbase + off));
        }
    };

    auto compute = [&](int base, const u32x4 (&kr)[U], const u32x4 (&vr)[U]) {
        float s[U][RT];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = base + u * KPG + kslot;
            float kf[EPL];
            to_f32<KV, EPL>(kr[u], kf);
#pragma unroll
            for (int r = 0; r < RT; ++r) {
                float acc = 0.0f;
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc += qv[r][e] * kf[e];
                acc = group_sum<LPK>(acc);
                s[u][r] = (j >= key_end || j > vis[r] || j < lo[r]) ? -INFINITY : acc;
            }
        }
        // one rescale per step and row
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            float mx = m[r];
#pragma unroll
            for (int u = 0; u < U; ++u) mx = fmaxf(mx, s[u][r]);
            const float alpha = fast_exp2(m[r] - mx);
            m[r] = mx;
            l[r] *= alpha;
#pragma unroll
            for (int e = 0; e < EPL; ++e) o[r][e] *= alpha;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float vf[EPL];
            to_f32<KV, EPL>(vr[u], vf);
#pragma unroll
            for (int r = 0; r < RT; ++r) {
                const float p = fast_exp2(s[u][r] - m[r]);
                l[r] += p;
#pragma unroll
                for (int e = 0; e < EPL; ++e) o[r][e] += p * vf[e];
            }
        }
    };

    // software pipeline: the next step's loads are in flight while this one
    // is computed
    constexpr int STRIDE = WAVES * WAVE_KEYS;
    u32x4 kA[U], vA[U], kB[U], vB[U];
    int base = key_begin + wave * WAVE_KEYS;
    if (base < key_end) issue(base, kA, vA);
    while (base < key_end) {
        int nb = base + STRIDE;
        if (nb < key_end) issue(nb, kB, vB);
        compute(base, kA, vA);
        base = nb;
        if (base >= key_end) break;
        nb = base + STRIDE;
        if (nb < key_end) issue(nb, kA, vA);
        compute(base, kB, vB);
        base = nb;
    }

    // merge the KPG key groups of this wave (lanes chunk + LPK*kslot)
#pragma unroll
    for (int off = LPK; off < 64; off <<= 1) {
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            const float mo = __shfl_xor(m[r], off);
            const float lo = __shfl_xor(l[r], off);
            const float mn = fmaxf(m[r], mo);
            const float as = fast_exp2(m[r] - mn), bs = fast_exp2(mo - mn);
            l[r] = l[r] * as + lo * bs;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                const float oo = __shfl_xor(o[r][e], off);
                o[r][e] = o[r][e] * as + oo * bs;
            }
            m[r] = mn;
        }
    }
    if (kslot == 0) {
#pragma unroll
        for (int r = 0; r < RT; ++r) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) sm_o[wave][r][chunk * EPL + e] = o[r][e];
            if (chunk == 0) {
                sm_m[wave][r] = m[r];
                sm_l[wave][r] = l[r];
            }
        }
    }
    __syncthreads();

    // merge the four waves and write the row (one split) or the partial
    for (int idx = threadIdx.x; idx < RT * D; idx += blockDim.x) {
        const int r = idx / D, d = idx - r * D;
        const int row = row0 + r;
        if (row >= a.rows) continue;
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
        const int t = row / c.g;
        const int h = kvh * c.g + (row - t * c.g);
        const size_t qrow = ((size_t)b * c.T + t) * c.Hq + h;
        if (a.num_splits == 1) {
            if (t >= nn) continue;          // padding rows (past a ragged chunk) are left as they are
            a.out[qrow * D + d] = finish_out(O, Ls);
            if (a.lse && d == 0) a.lse[qrow] = finish_lse(M, Ls);
        } else {
            a.part_o[(qrow * a.num_splits + split) * D + d] = O;
            if (d == 0) {
                a.part_ml[(qrow * a.num_splits + split) * 2 + 0] = M;
                a.part_ml[(qrow * a.num_splits + split) * 2 + 1] = Ls;
            }
        }
    }
}

template <int D, int KV>
hipError_t launch_rt(const AttnArgs& a, dim3 grid, hipStream_t s) {
    // block ids of one split's key range: it spans at most this many blocks
    const size_t lds = sizeof(int) * (size_t)(((a.split_keys - 1) >> a.c.log2_bs) + 2);
    switch (a.row_tile) {
        case 1: hipLaunchKernelGGL((attn_valu_kernel<D, KV, 1>), grid, dim3(256), lds, s, a); break;
        case 2: hipLaunchKernelGGL((attn_valu_kernel<D, KV, 2>), grid, dim3(256), lds, s, a); break;
        case 4: hipLaunchKernelGGL((attn_valu_kernel<D, KV, 4>), grid, dim3(256), lds, s, a); break;
        case 8: hipLaunchKernelGGL((attn_valu_kernel<D, KV, 8>), grid, dim3(256), lds, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int KV>
hipError_t launch_d(const AttnArgs& a, dim3 grid, hipStream_t s) {
    switch (a.c.D) {
        case 16: return launch_rt<16, KV>(a, grid, s);
        case 32: return launch_rt<32, KV>(a, grid, s);
        case 64: return launch_rt<64, KV>(a, grid, s);
        case 128: return launch_rt<128, KV>(a, grid, s);
        case 256: return launch_rt<256, KV>(a, grid, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

int valu_step_keys(int D, int kv_bf16) {
    int wk = 0;
    switch (D * 2 + kv_bf16) {
        case 32: wk = Geo<16, 0>::WAVE_KEYS; break;
        case 33: wk = Geo<16, 1>::WAVE_KEYS; break;
        case 64: wk = Geo<32, 0>::WAVE_KEYS; break;
        case 65: wk = Geo<32, 1>::WAVE_KEYS; break;
        case 128: wk = Geo<64, 0>::WAVE_KEYS; break;
        case 129: wk = Geo<64, 1>::WAVE_KEYS; break;
        case 256: wk = Geo<128, 0>::WAVE_KEYS; break;
        case 257: wk = Geo<128, 1>::WAVE_KEYS; break;
        case 512: wk = Geo<256, 0>::WAVE_KEYS; break;
        case 513: wk = Geo<256, 1>::WAVE_KEYS; break;
        default: return 256;
    }
    return WAVES * wk;
}

int valu_max_row_tile(int, int) { return 8; }

template <int D, int KV>
static const void* valu_fn(int rt) {
    switch (rt) {
        case 1: return (const void*)attn_valu_kernel<D, KV, 1>;
        case 2: return (const void*)attn_valu_kernel<D, KV, 2>;
        case 4: return (const void*)attn_valu_kernel<D, KV, 4>;
        default: return (const void*)attn_valu_kernel<D, KV, 8>;
    }
}

int valu_wgs_per_cu(int D, int kv_bf16, int row_tile, size_t dyn_lds) {
    const void* f = nullptr;
    switch (D * 2 + kv_bf16) {
        case 32: f = valu_fn<16, 0>(row_tile); break;
        case 33: f = valu_fn<16, 1>(row_tile); break;
        case 64: f = valu_fn<32, 0>(row_tile); break;
        case 65: f = valu_fn<32, 1>(row_tile); break;
        case 128: f = valu_fn<64, 0>(row_tile); break;
        case 129: f = valu_fn<64, 1>(row_tile); break;
        case 256: f = valu_fn<128, 0>(row_tile); break;
        case 257: f = valu_fn<128, 1>(row_tile); break;
        case 512: f = valu_fn<256, 0>(row_tile); break;
        default: f = valu_fn<256, 1>(row_tile); break;
    }
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, f, 256, dyn_lds) != hipSuccess || n < 1) {
        (void)hipGetLastError();
        return 2;
    }
    return n;
}

int valu_max_split_keys(int log2_bs) { return (VALU_MAX_STAGED_BLOCKS - 2) << log2_bs; }

hipError_t launch_attn_valu(const AttnArgs& a, hipStream_t s) {
    const int n_rtiles = (a.rows + a.row_tile - 1) / a.row_tile;
    dim3 grid(a.c.Hkv * n_rtiles, a.num_splits, a.c.B);
    return a.kv_bf16 ? launch_d<1>(a, grid, s) : launch_d<0>(a, grid, s);
}

}  // namespace kvd
