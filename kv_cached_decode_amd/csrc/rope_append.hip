// rope_append.hip -- RoPE of the new q/k at each token's absolute position and
// the paged append of the new K/V rows (ferric-core generate.rs `step_gpu`:
// `rope_off_t` then the cache append; Ferrum Infer README: batched RoPE with
// per-item positions, paged KV through a block table).
//
// Grid: (new token (b, t), group of heads).  The token's position is
// seq_lens[b] - n_new + t; in a context-parallel shard it is q_pos[b] + t,
// stored at local slot q_pos[b] + t - key_pos0[b] if the shard holds that
// slot (0 .. seq_lens[b] - 1), and not stored otherwise.  The D/2 rotation angles
// pos * theta_i (theta_i = base^(-2i/D) from the host) are evaluated in fp64
// once per workgroup and shared through LDS; every head's pair is then
// rotated in fp64 and rounded once: to fp32 for q_rot and an fp32 cache, to
// bf16 (round to nearest even) for a bf16 cache.  A decode step moves little
// (B*T*(Hq + 2*Hkv)*D elements) and is latency-bound; a prefill chunk moves
// tens of MB, so a thread takes four pairs of a head with two 16-byte loads
// and stores, all its loads issued first.  Padding tokens of ragged chunks do
// nothing.  With skip_q only the K/V heads are taken (the attention kernel
// then rotates the queries itself).
#include "bf16_round.h"
#include "kvd_internal.h"
#include "rope_math.h"

namespace kvd {
namespace {

// A thread takes four rotation pairs of a head: pairs 4k .. 4k+3, whose
// elements are the float4s at 4k and D/2 + 4k (pairs (i, i + D/2)) or at 8k
// and 8k + 4 (pairs (2i, 2i+1)); D/8 threads cover a head, 256/(D/8) heads
// a round.  Heads of one token are numbered q heads, then k heads, then v
// heads (v is only rounded, through the same element split).  A workgroup
// takes `rounds` rounds of heads of one token, every load issued before the
// token's angles are formed; the host picks the rounds so that a batch of
// few tokens still spreads over many workgroups.
constexpr int MAX_ROUNDS = 4;

struct Quad {
    float4 a, b;     // the two float4s of the thread's pairs
};

__device__ inline float pick(const float4& v, int j) { return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w; }
__device__ inline void put(float4& v, int j, float x) {
    if (j == 0) v.x = x; else if (j == 1) v.y = x; else if (j == 2) v.z = x; else v.w = x;
}

// pair j of the thread (0..3): its two elements within the quad
__device__ inline void pair_get(const Quad& q, int interleaved, int j, float& x, float& y) {
    if (interleaved) {
        const float4& v = j < 2 ? q.a : q.b;
        x = pick(v, 2 * (j & 1));
        y = pick(v, 2 * (j & 1) + 1);
    } else {
        x = pick(q.a, j);
        y = pick(q.b, j);
    }
}
__device__ inline void pair_set(Quad& q, int interleaved, int j, float x, float y) {
    if (interleaved) {
        float4& v = j < 2 ? q.a : q.b;
        put(v, 2 * (j & 1), x);
        put(v, 2 * (j & 1) + 1, y);
    } else {
        put(q.a, j, x);
        put(q.b, j, y);
    }
}

__device__ inline uint2 bf16x4_from_f32(const float4& v) {
    return make_uint2((uint32_t)bf16_from_f32(v.x) | (uint32_t)bf16_from_f32(v.y) << 16,
                      (uint32_t)bf16_from_f32(v.z) | (uint32_t)bf16_from_f32(v.w) << 16);
}

__global__ __launch_bounds__(256) void rope_append_kernel(RopeAppendArgs a, int rounds) {
    __shared__ double cs[128];
    __shared__ double sn[128];
    const CacheView& c = a.c;
    const int token = blockIdx.x;
    const int b = token / c.T, t = token - b * c.T;
    if (t >= n_new(c, b)) return;      // a padding token of a ragged chunk: nothing to rotate or store
    const int D = c.D, half = D >> 1;
    const int lt = __builtin_ctz(D) - 3;            // threads a head: D / 8
    const int slots = 256 >> lt;
    const int slot = (int)threadIdx.x >> lt;
    const int k = (int)threadIdx.x & ((1 << lt) - 1);
    const int heads = c.Hq + 2 * c.Hkv;
    const int offa = a.interleaved ? 8 * k : 4 * k;
    const int offb = a.interleaved ? 8 * k + 4 : half + 4 * k;
    const int h0 = (a.skip_q ? c.Hq : 0) + blockIdx.y * rounds * slots + slot;

    // This thread's inputs first (they do not depend on the angles), so their
    // latency overlaps the fp64 angle evaluation below.
    Quad x[MAX_ROUNDS];
#pragma unroll
    for (int r = 0; r < MAX_ROUNDS; ++r) {
        x[r].a = x[r].b = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        const int hd = h0 + r * slots;
        if (r >= rounds || hd >= heads) continue;
        const float* src = hd < c.Hq ? a.q + ((size_t)token * c.Hq + hd) * D
                         : hd < c.Hq + c.Hkv ? a.k + ((size_t)token * c.Hkv + (hd - c.Hq)) * D
                                             : a.v + ((size_t)token * c.Hkv + (hd - c.Hq - c.Hkv)) * D;
        x[r].a = *(const float4*)(src + offa);
        x[r].b = *(const float4*)(src + offb);
    }
    // the token's local slot, and its global position for the rotation (they
    // differ in a context-parallel shard).  A shard whose keys do not include
    // the slot rotates the query and stores nothing (the shard holding the
    // token appends it), so neither the table nor the pools are touched.
    const int L = c.seq_lens[b];
    const int local = q_local0(c, b, L) + t;
    const int pos = local + (c.key_pos0 ? c.key_pos0[b] : 0);
    const bool held = local >= 0 && local < L;
    const int blk = held ? c.table[(size_t)b * c.max_blocks + (local >> c.log2_bs)] : 0;

    for (int p = threadIdx.x; p < half; p += blockDim.x)
        rope_angle(kernarg_double(offsetof(RopeAppendArgs, theta), p), pos, cs[p], sn[p]);
    __syncthreads();

    const int off = local & ((1 << c.log2_bs) - 1);   // the cache slot of this token
#pragma unroll
    for (int r = 0; r < MAX_ROUNDS; ++r) {
        const int hd = h0 + r * slots;
        if (r >= rounds || hd >= heads) break;
        Quad y = x[r];
        if (hd < c.Hq + c.Hkv) {
            // q or k: every pair turned in fp64, rounded once
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float x0, x1;
                pair_get(x[r], a.interleaved, j, x0, x1);
                double xr, yr;
                rope_rotate(x0, x1, cs[4 * k + j], sn[4 * k + j], xr, yr);
                if (hd < c.Hq || !a.kv_bf16) {
                    pair_set(y, a.interleaved, j, (float)xr, (float)yr);
                } else {
                    // bf16 keys round straight from fp64: keep the bits in the floats' places
                    pair_set(y, a.interleaved, j, __uint_as_float(bf16_from_f64(xr)),
                             __uint_as_float(bf16_from_f64(yr)));
                }
            }
        }
        if (hd < c.Hq) {
            // query -> q_rot (fp32); q and q_rot may alias: the elements are
            // read and written by this thread only
            float* dst = a.q_rot + ((size_t)token * c.Hq + hd) * D;
            *(float4*)(dst + offa) = y.a;
            *(float4*)(dst + offb) = y.b;
            continue;
        }
        if (!held) continue;
        const bool is_k = hd < c.Hq + c.Hkv;
        const int h = is_k ? hd - c.Hq : hd - c.Hq - c.Hkv;
        const size_t row = ((((size_t)blk * c.Hkv + h) << c.log2_bs) + off) * D;
        if (a.kv_bf16) {
            uint16_t* dst = (uint16_t*)(is_k ? c.k : c.v) + row;
            if (is_k) {
                // the rounded bits sit in the low halves of the floats
                *(uint2*)(dst + offa) = make_uint2(__float_as_uint(y.a.x) | __float_as_uint(y.a.y) << 16,
                                                   __float_as_uint(y.a.z) | __float_as_uint(y.a.w) << 16);
                *(uint2*)(dst + offb) = make_uint2(__float_as_uint(y.b.x) | __float_as_uint(y.b.y) << 16,
                                                   __float_as_uint(y.b.z) | __float_as_uint(y.b.w) << 16);
            } else {
                *(uint2*)(dst + offa) = bf16x4_from_f32(y.a);
                *(uint2*)(dst + offb) = bf16x4_from_f32(y.b);
            }
        } else {
            float* dst = (float*)(is_k ? c.k : c.v) + row;
            *(float4*)(dst + offa) = y.a;
            *(float4*)(dst + offb) = y.b;
        }
    }
}

}  // namespace

hipError_t launch_rope_append(const RopeAppendArgs& a, hipStream_t s) {
    const int tokens = a.c.B * a.c.T;
    if (tokens == 0) return hipSuccess;
    const int slots = 256 / (a.c.D / 8);
    const int heads = (a.skip_q ? 0 : a.c.Hq) + 2 * a.c.Hkv;
    const int total = (heads + slots - 1) / slots;            // rounds of heads a token
    // few tokens: one round a workgroup (more workgroups); many: up to
    // MAX_ROUNDS, so that every workgroup keeps more loads in flight
    const int rounds = tokens >= 512 ? (total < MAX_ROUNDS ? total : MAX_ROUNDS) : 1;
    dim3 grid(tokens, (total + rounds - 1) / rounds);
    hipLaunchKernelGGL(rope_append_kernel, grid, dim3(256), 0, s, a, rounds);
    return hipGetLastError();
}

}  // namespace kvd
