// rope_append.hip -- RoPE of the new q/k at each token's absolute position and
// the paged append of the new K/V rows (ferric-core generate.rs `step_gpu`:
// `rope_off_t` then the cache append; Ferrum Infer README: batched RoPE with
// per-item positions, paged KV through a block table).
//
// Grid: (new token (b, t), group of heads).  The token's position is
// seq_lens[b] - n_new + t; in a context-parallel shard it is q_pos[b] + t,
// stored at local slot q_pos[b] + t - key_pos0[b].  The D/2 rotation angles
// pos * theta_i (theta_i = base^(-2i/D) from the host) are evaluated in fp64
// once per workgroup and shared through LDS; every head's pair is then
// rotated in fp64 and rounded once: to fp32 for q_rot and an fp32 cache, to
// bf16 (round to nearest even) for a bf16 cache.  The volume is tiny
// (B*T*(Hq + 2*Hkv)*D elements), so the kernel is latency-bound: a thread
// handles one rotation pair of a few heads, with all its loads issued first.
// Padding tokens of ragged chunks do nothing.
#include "bf16_round.h"
#include "kvd_internal.h"
#include "rope_math.h"

namespace kvd {
namespace {

// Heads of one token are numbered q heads, then k heads, then v heads.  A
// workgroup takes HEADS_PER_SLOT * (256 / (D/2)) of them: thread (slot, i)
// handles pair i of heads slot, slot + slots, ... (four heads), so a token's
// angles are evaluated by few workgroups and every thread's loads and stores
// are in flight together.
constexpr int HEADS_PER_SLOT = 4;

__global__ __launch_bounds__(256) void rope_append_kernel(RopeAppendArgs a) {
    __shared__ double cs[128];
    __shared__ double sn[128];
    const CacheView& c = a.c;
    const int token = blockIdx.x;
    const int b = token / c.T, t = token - b * c.T;
    if (t >= n_new(c, b)) return;      // a padding token of a ragged chunk: nothing to rotate or store
    const int D = c.D, half = D >> 1;
    const int slots = blockDim.x / half;
    const int slot = (int)threadIdx.x / half;
    const int i = (int)threadIdx.x % half;
    const int heads = c.Hq + 2 * c.Hkv;
    int ia, ic;
    rope_pair(i, half, a.interleaved, ia, ic);

    // This thread's inputs first (they do not depend on the angles), so their
    // latency overlaps the fp64 angle evaluation below.
    float x0[HEADS_PER_SLOT], x1[HEADS_PER_SLOT];
    int head[HEADS_PER_SLOT];
#pragma unroll
    for (int r = 0; r < HEADS_PER_SLOT; ++r) {
        head[r] = (blockIdx.y * HEADS_PER_SLOT + r) * slots + slot;
        x0[r] = x1[r] = 0.0f;
        const int hd = head[r];
        if (slot >= slots || hd >= heads) continue;
        if (hd < c.Hq) {
            const size_t o = ((size_t)token * c.Hq + hd) * D;
            x0[r] = a.q[o + ia];
            x1[r] = a.q[o + ic];
        } else if (hd < c.Hq + c.Hkv) {
            const size_t o = ((size_t)token * c.Hkv + (hd - c.Hq)) * D;
            x0[r] = a.k[o + ia];
            x1[r] = a.k[o + ic];
        } else {
            const size_t o = ((size_t)token * c.Hkv + (hd - c.Hq - c.Hkv)) * D + 2 * i;
            x0[r] = a.v[o];
            x1[r] = a.v[o + 1];
        }
    }
    // the token's local slot, and its global position for the rotation (they
    // differ in a context-parallel shard)
    const int local = q_local0(c, b, c.seq_lens[b]) + t;
    const int pos = local + (c.key_pos0 ? c.key_pos0[b] : 0);
    const int blk = c.table[(size_t)b * c.max_blocks + (local >> c.log2_bs)];

    for (int p = threadIdx.x; p < half; p += blockDim.x)
        rope_angle(kernarg_double(offsetof(RopeAppendArgs, theta), p), pos, cs[p], sn[p]);
    __syncthreads();
    if (slot >= slots) return;

    const int off = local & ((1 << c.log2_bs) - 1);   // the cache slot of this token
#pragma unroll
    for (int r = 0; r < HEADS_PER_SLOT; ++r) {
        const int hd = head[r];
        if (hd >= heads) break;
        if (hd < c.Hq) {
            // query -> q_rot (fp32); q and q_rot may alias: the pair is read
            // and written by this thread only.
            const size_t o = ((size_t)token * c.Hq + hd) * D;
            double xr, yr;
            rope_rotate(x0[r], x1[r], cs[i], sn[i], xr, yr);
            a.q_rot[o + ia] = (float)xr;
            a.q_rot[o + ic] = (float)yr;
        } else if (hd < c.Hq + c.Hkv) {
            const int h = hd - c.Hq;
            const size_t dst = ((((size_t)blk * c.Hkv + h) << c.log2_bs) + off) * D;
            double xr, yr;
            rope_rotate(x0[r], x1[r], cs[i], sn[i], xr, yr);
            if (a.kv_bf16) {
                uint16_t* kc = (uint16_t*)c.k;
                kc[dst + ia] = bf16_from_f64(xr);
                kc[dst + ic] = bf16_from_f64(yr);
            } else {
                float* kc = (float*)c.k;
                kc[dst + ia] = (float)xr;
                kc[dst + ic] = (float)yr;
            }
        } else {
            const int h = hd - c.Hq - c.Hkv;
            const size_t dst = ((((size_t)blk * c.Hkv + h) << c.log2_bs) + off) * D + 2 * i;
            if (a.kv_bf16) {
                uint16_t* vc = (uint16_t*)c.v;
                vc[dst] = bf16_from_f32(x0[r]);
                vc[dst + 1] = bf16_from_f32(x1[r]);
            } else {
                float* vc = (float*)c.v;
                vc[dst] = x0[r];
                vc[dst + 1] = x1[r];
            }
        }
    }
}

}  // namespace

hipError_t launch_rope_append(const RopeAppendArgs& a, hipStream_t s) {
    const int tokens = a.c.B * a.c.T;
    if (tokens == 0) return hipSuccess;
    const int half = a.c.D / 2;
    const int heads_per_wg = HEADS_PER_SLOT * (256 / half);
    const int heads = a.c.Hq + 2 * a.c.Hkv;
    dim3 grid(tokens, (heads + heads_per_wg - 1) / heads_per_wg);
    hipLaunchKernelGGL(rope_append_kernel, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace kvd
