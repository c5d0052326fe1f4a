// check_descriptor.hip -- an optional device-side check of the parts of a
// descriptor that live in device memory (sequence lengths, block ids, chunk
// lengths, shard positions), which the host cannot see without a copy.  The
// pages report such errors as values (ferric-core generate.rs returns Result
// and asserts its shapes); the decode kernels themselves treat a violation as
// undefined behaviour, so a caller that cannot vouch for its descriptors runs
// this first and reads the flag word.
//
// One workgroup per sequence.  It reads seq_lens, q_lens, key_pos0 and q_pos
// of its sequence and the block-table entries of the blocks that the
// sequence's queries can see (bounded by the table row, never past it); it
// dereferences no block id.  Violations are ORed into the flag word with a
// vector atomic; a clean descriptor leaves the word as it was.
#include "kvd.h"
#include "kvd_internal.h"

namespace kvd {
namespace {

__global__ __launch_bounds__(256) void check_descriptor_kernel(CacheView c, int max_seq_len, int num_blocks,
                                                               unsigned* flags) {
    const int b = blockIdx.x;
    const int L = c.seq_lens[b];
    const int nn = c.q_lens ? c.q_lens[b] : c.T;
    unsigned f = 0u;
    if (L < 0 || L > max_seq_len) f |= KVD_CHECK_SEQ_LEN;
    if (nn < 0 || nn > c.T) f |= KVD_CHECK_Q_LENS;
    if (c.key_pos0 && c.key_pos0[b] < 0) f |= KVD_CHECK_SHARD;
    if (c.q_pos && c.q_pos[b] < 0) f |= KVD_CHECK_SHARD;
    // a whole cache holds its new tokens as its last keys
    if (!c.q_pos && nn >= 0 && nn <= c.T && L >= 0 && L < nn) f |= KVD_CHECK_SEQ_LEN;
    // the blocks of the keys the queries can see (from the first query's
    // window on), at most the table row
    const int Lc = min(max(L, 0), max_seq_len);
    const int qo = c.q_pos ? c.q_pos[b] - (c.key_pos0 ? c.key_pos0[b] : 0) : Lc - min(max(nn, 0), Lc);
    const int first = c.window > 0 ? max(0, min(qo, Lc) - c.window + 1) : 0;
    const int blk_lo = first >> c.log2_bs;
    const int blk_hi = min((Lc + (1 << c.log2_bs) - 1) >> c.log2_bs, c.max_blocks);
    const int* row = c.table + (size_t)b * c.max_blocks;
    bool bad = false;
    for (int i = blk_lo + (int)threadIdx.x; i < blk_hi; i += blockDim.x) {
        const int id = row[i];
        bad |= id < 0 || id >= num_blocks;
    }
    if (__builtin_amdgcn_ballot_w64(bad) && (threadIdx.x & 63) == 0) f |= KVD_CHECK_BLOCK_ID;
    if (f && (threadIdx.x & 63) == 0) atomicOr(flags, f);
}

}  // namespace

hipError_t launch_check_descriptor(const CacheView& c, int max_seq_len, int num_blocks, unsigned* flags,
                                   hipStream_t s) {
    if (c.B == 0) return hipSuccess;
    hipLaunchKernelGGL(check_descriptor_kernel, dim3(c.B), dim3(256), 0, s, c, max_seq_len, num_blocks, flags);
    return hipGetLastError();
}

}  // namespace kvd
