// kvd.cpp -- the C ABI of libkvd.so: host-side validation, split-K planning
// and kernel dispatch.  Declarations and the contract of every entry point
// are in include/kvd.h.
#include "kvd.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "kvd_internal.h"

// Split-K scratch of kvd_decode_step_noalloc: one array per device (each
// GPU that loads the library holds its own copy until the process ends).  In
// host code `scratch` is only a stand-in for the symbol; the device address
// comes from hipGetSymbolAddress, looked up once per device with that device
// current, and only that address is ever passed to a kernel or a copy.
static __device__ __align__(256) unsigned char scratch[KVD_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_err[512] = "";

int32_t fail(int32_t status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return status;
}

int32_t ok() {
    g_err[0] = '\0';
    return KVD_OK;
}

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

int ilog2(int64_t x) {
    int r = 0;
    while ((int64_t(1) << r) < x) ++r;
    return r;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Compute units of the current device, cached per device.
int num_cus() {
    static std::mutex mu;
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    std::lock_guard<std::mutex> lk(mu);
    if (cache[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cache[dev] = n;
    }
    return cache[dev];
}

int32_t check_desc(const kvd_paged_kv* kv) {
    if (!kv) return fail(KVD_ERR_NULL, "descriptor is NULL");
    if (kv->num_seqs < 0) return fail(KVD_ERR_SHAPE, "num_seqs = %d < 0", kv->num_seqs);
    if (kv->num_seqs == 0) return KVD_OK;
    if (kv->q_tokens_per_seq < 1 || kv->q_tokens_per_seq > 1024)
        return fail(kv->q_tokens_per_seq < 1 ? KVD_ERR_SHAPE : KVD_ERR_UNSUPPORTED,
                    "q_tokens_per_seq = %d (supported 1..1024)", kv->q_tokens_per_seq);
    if (kv->n_q_heads < 1 || kv->n_kv_heads < 1)
        return fail(KVD_ERR_SHAPE, "head counts must be >= 1 (Hq=%d, Hkv=%d)", kv->n_q_heads,
                    kv->n_kv_heads);
    if (kv->n_q_heads % kv->n_kv_heads != 0)
        return fail(KVD_ERR_SHAPE, "n_q_heads %% n_kv_heads != 0 (%d, %d)", kv->n_q_heads,
                    kv->n_kv_heads);
    const int D = kv->head_dim;
    if (D != 16 && D != 32 && D != 64 && D != 128 && D != 256)
        return fail(KVD_ERR_UNSUPPORTED, "head_dim = %d (supported 16, 32, 64, 128, 256)", D);
    if (!is_pow2(kv->block_size) || kv->block_size > 1024)
        return fail(KVD_ERR_UNSUPPORTED, "block_size = %d (supported powers of two 1..1024)",
                    kv->block_size);
    if (kv->num_blocks < 1 || kv->max_blocks_per_seq < 1)
        return fail(KVD_ERR_SHAPE, "num_blocks = %d, max_blocks_per_seq = %d", kv->num_blocks,
                    kv->max_blocks_per_seq);
    if ((int64_t)kv->num_blocks * kv->n_kv_heads > INT32_MAX)
        return fail(KVD_ERR_UNSUPPORTED, "num_blocks * n_kv_heads = %lld (at most 2^31 - 1)",
                    (long long)kv->num_blocks * kv->n_kv_heads);
    // a context-parallel shard may hold fewer keys than new tokens (or none),
    // and ragged chunks fewer new tokens than T
    if (kv->max_seq_len < (kv->q_pos || kv->q_lens ? 0 : kv->q_tokens_per_seq))
        return fail(KVD_ERR_SHAPE, "max_seq_len = %d < q_tokens_per_seq = %d", kv->max_seq_len,
                    kv->q_tokens_per_seq);
    if ((int64_t)kv->max_seq_len > (int64_t)kv->max_blocks_per_seq * kv->block_size)
        return fail(KVD_ERR_SHAPE, "max_seq_len = %d exceeds max_blocks_per_seq * block_size = %lld",
                    kv->max_seq_len, (long long)kv->max_blocks_per_seq * kv->block_size);
    if (kv->kv_dtype != KVD_KV_F32 && kv->kv_dtype != KVD_KV_BF16)
        return fail(KVD_ERR_UNSUPPORTED, "kv_dtype = %d", kv->kv_dtype);
    if (kv->window < 0) return fail(KVD_ERR_SHAPE, "window = %d < 0", kv->window);
    if (!kv->k_cache || !kv->v_cache || !kv->block_table || !kv->seq_lens)
        return fail(KVD_ERR_NULL, "k_cache, v_cache, block_table and seq_lens must be non-NULL");
    if (((uintptr_t)kv->k_cache | (uintptr_t)kv->v_cache) & 15)
        return fail(KVD_ERR_SHAPE, "k_cache and v_cache must be 16-byte aligned");
    if (((uintptr_t)kv->block_table | (uintptr_t)kv->seq_lens | (uintptr_t)kv->key_pos0 |
         (uintptr_t)kv->q_pos | (uintptr_t)kv->q_lens) & 3)
        return fail(KVD_ERR_SHAPE, "block_table, seq_lens, key_pos0, q_pos and q_lens must be 4-byte aligned");
    return KVD_OK;
}

kvd::CacheView view_of(const kvd_paged_kv* kv) {
    kvd::CacheView c;
    c.B = kv->num_seqs;
    c.T = kv->q_tokens_per_seq;
    c.Hq = kv->n_q_heads;
    c.Hkv = kv->n_kv_heads;
    c.D = kv->head_dim;
    c.g = kv->n_q_heads / kv->n_kv_heads;
    c.log2_bs = ilog2(kv->block_size);
    c.max_blocks = kv->max_blocks_per_seq;
    c.table = kv->block_table;
    c.seq_lens = kv->seq_lens;
    c.k = kv->k_cache;
    c.v = kv->v_cache;
    c.window = kv->window;
    c.key_pos0 = kv->key_pos0;
    c.q_pos = kv->q_pos;
    c.q_lens = kv->q_lens;
    return c;
}

struct Plan {
    int kernel;       // KVD_KERNEL_VALU / KVD_KERNEL_MFMA
    bool prefill;     // matrix cores with more than 16 query rows per kv head
    int splits;
    int split_keys;
    int rows;
    int row_tile;
};

// Split-K plan from host-known sizes only (graph-capture safe).
//
// Kernel family: the matrix-core kernel when the g*T query rows sharing a kv
// head reach MFMA_MIN_ROWS (bf16, head_dim 128: every such plan, the counters
// behind it are given with the constant), else the vector-ALU kernel (fp32
// caches, other head dims).
//
// Splits: long contiguous ranges stream best.  The matrix-core kernel runs
// one workgroup per CU when the batch has fewer (sequence, kv head) units
// than CUs; with more units (continuous batching, ragged lengths) it uses
// three splits per unit, so the longest-first ordering of the kernel has
// enough small pieces to balance the CUs, but no split shorter than
// MFMA_MIN_SPLIT_KEYS once the units alone fill the resident slots.  The VALU kernel targets one round
// of its resident workgroup slots.
int32_t make_plan(const kvd_paged_kv* kv, const kvd_attn_options* opt, Plan* p) {
    const int D = kv->head_dim;
    const int bf16 = kv->kv_dtype == KVD_KV_BF16;
    const int g = kv->n_q_heads / kv->n_kv_heads;
    p->rows = g * kv->q_tokens_per_seq;
    int kernel = opt ? opt->kernel : KVD_KERNEL_AUTO;
    if (kernel != KVD_KERNEL_AUTO && kernel != KVD_KERNEL_VALU && kernel != KVD_KERNEL_MFMA)
        return fail(KVD_ERR_UNSUPPORTED, "kernel = %d", kernel);
    // the matrix-core kernels: the decode kernel up to 16 query rows per kv
    // head, the prefill kernel (row tiles sharing LDS-staged K/V) beyond
    const bool mfma_ok = kvd::mfma_supported(D, bf16, 1);
    if (kernel == KVD_KERNEL_MFMA && !mfma_ok)
        return fail(KVD_ERR_UNSUPPORTED, "matrix-core kernels need a bf16 cache and head_dim 128");
    if (kernel == KVD_KERNEL_AUTO)
        kernel = (mfma_ok && p->rows >= kvd::MFMA_MIN_ROWS) ? KVD_KERNEL_MFMA : KVD_KERNEL_VALU;
    p->kernel = kernel;
    p->prefill = kernel == KVD_KERNEL_MFMA && !kvd::mfma_supported(D, bf16, p->rows);

    const int log2_bs = ilog2(kv->block_size);
    // keys a sequence's queries can see at most: the whole cache, or the
    // window plus the draft
    const int64_t max_len = std::max<int64_t>(1, kv->window > 0
        ? std::min<int64_t>(kv->max_seq_len, (int64_t)kv->window + kv->q_tokens_per_seq - 1)
        : kv->max_seq_len);
    int step, n_rtiles;
    int64_t max_keys = INT32_MAX, target;
    if (p->prefill) {
        // compute-leaning: about two resident workgroups per CU, each split
        // staging at most 4094 block ids
        step = kvd::prefill_step_keys();
        p->row_tile = kvd::PREFILL_ROWS;
        n_rtiles = (int)cdiv(p->rows, kvd::PREFILL_ROWS);
        max_keys = (int64_t)4094 << log2_bs;
        target = kvd::PREFILL_WGS_PER_CU * (int64_t)num_cus();
    } else if (kernel == KVD_KERNEL_MFMA) {
        step = kvd::mfma_step_keys();
        p->row_tile = 16;
        n_rtiles = 1;
        const int64_t units = (int64_t)kv->num_seqs * kv->n_kv_heads;
        target = units <= num_cus() ? num_cus() : 3 * units;
    } else {
        max_keys = kvd::valu_max_split_keys(log2_bs);
        step = kvd::valu_step_keys(D, bf16);
        const int max_rt = kvd::valu_max_row_tile(D, bf16);
        int rt = 1;
        while (rt < p->rows && rt < max_rt) rt <<= 1;
        p->row_tile = rt;
        n_rtiles = (int)cdiv(p->rows, rt);
        // about one round of the resident workgroup slots
        target = (int64_t)kvd::valu_wgs_per_cu(D, bf16, rt, sizeof(int) * 64) * num_cus();
    }
    const int64_t max_splits = cdiv(max_len, step);
    int64_t splits;
    if (opt && opt->num_splits > 0) {
        splits = opt->num_splits;
    } else {
        const int64_t units = (int64_t)kv->num_seqs * kv->n_kv_heads * n_rtiles;
        splits = cdiv(target, units);
        if (kernel == KVD_KERNEL_MFMA && !p->prefill && units >= kvd::MFMA_WGS_PER_CU * (int64_t)num_cus())
            splits = std::min<int64_t>(splits, std::max<int64_t>(1, max_len / kvd::MFMA_MIN_SPLIT_KEYS));
    }
    splits = std::min<int64_t>(splits, max_splits);
    splits = std::max<int64_t>(splits, cdiv(max_len, max_keys));   // per-split staging limit
    if (splits < 1) splits = 1;
    // equal shares (the kernels clamp a range that is not a multiple of their
    // step, so no rounding that would load the first splits more)
    int64_t keys = cdiv(max_len, splits);
    splits = cdiv(max_len, keys);
    if (splits > 65535) return fail(KVD_ERR_UNSUPPORTED, "too many splits (%lld)", (long long)splits);
    if (p->prefill) {
        if (splits * kv->n_kv_heads * n_rtiles * kv->num_seqs > INT32_MAX)
            return fail(KVD_ERR_UNSUPPORTED, "grid too large: %lld splits x %d kv heads x %d row tiles x %d sequences",
                        (long long)splits, kv->n_kv_heads, n_rtiles, kv->num_seqs);
    } else if ((int64_t)kv->n_kv_heads * n_rtiles > 65535 || kv->num_seqs > 65535)
        return fail(KVD_ERR_UNSUPPORTED, "grid too large: %d kv heads x %d row tiles, %d sequences",
                    kv->n_kv_heads, n_rtiles, kv->num_seqs);
    p->splits = (int)splits;
    p->split_keys = (int)keys;
    return KVD_OK;
}

// Partial-output region sizes (floats) of a plan: o and (m, l).
void partial_sizes(const kvd_paged_kv* kv, const Plan& p, size_t* n_o, size_t* n_ml) {
    size_t rows = 0;
    if (p.splits > 1) rows = (size_t)kv->num_seqs * kv->q_tokens_per_seq * kv->n_q_heads * p.splits;
    *n_o = rows * kv->head_dim;
    *n_ml = rows * 2;
}

// Workspace carve-up: [arrival counters | partial o | partial (m, l)], each
// 256-byte aligned.  The counters take a fixed region at the head of every
// split-K workspace, whatever the plan, so no call's partials ever land where
// another call keeps its counters: a workspace zeroed once stays ready for
// calls of any shape, since every call leaves the counters it used at zero.
// They serve the matrix-core decode kernel, which merges its own splits when
// the batch has at most COUNTER_SLOTS (sequence, kv head) pairs.
constexpr size_t COUNTER_SLOTS = KVD_WORKSPACE_COUNTER_BYTES / sizeof(unsigned);

struct Carve {
    size_t cnt, o, ml, total;
};

Carve carve(const kvd_paged_kv* kv, const Plan& p) {
    Carve c{0, 0, 0, 0};
    size_t n_o, n_ml;
    partial_sizes(kv, p, &n_o, &n_ml);
    if (n_o == 0) return c;
    c.cnt = 0;
    c.o = KVD_WORKSPACE_COUNTER_BYTES;
    c.ml = c.o + ((n_o * sizeof(float) + 255) & ~size_t(255));
    c.total = c.ml + n_ml * sizeof(float);
    return c;
}

size_t workspace_for(const kvd_paged_kv* kv, const Plan& p) { return carve(kv, p).total; }

// RoPE frequencies theta_i = base^(-2i/D), i < D/2, in fp64 (the last table
// is kept per thread: a decode loop asks for the same one every step).
void fill_theta(kvd::RopeTheta* t, double base, int D) {
    thread_local double last_base = 0.0;
    thread_local int last_D = 0;
    thread_local kvd::RopeTheta last;
    if (base != last_base || D != last_D) {
        for (int i = 0; i < 128; ++i)
            last.v[i] = i < D / 2 ? std::pow(base, -2.0 * (double)i / (double)D) : 0.0;
        last_base = base;
        last_D = D;
    }
    *t = last;
}

// Arguments of the RoPE + append step (q_rot may be null: the fused step
// makes it optional).
int32_t check_rope(const float* q, const float* k, const float* v, const float* q_rot,
                   double rope_base, int32_t layout) {
    if (!q || !k || !v) return fail(KVD_ERR_NULL, "q, k and v must be non-NULL");
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)q_rot) & 3)
        return fail(KVD_ERR_SHAPE, "q, k, v, q_rot must be 4-byte aligned");
    if (!(rope_base > 0.0) || !std::isfinite(rope_base))
        return fail(KVD_ERR_SHAPE, "rope_base must be finite and > 0");
    if (layout != KVD_ROPE_HALF && layout != KVD_ROPE_INTERLEAVED)
        return fail(KVD_ERR_UNSUPPORTED, "rope layout = %d", layout);
    return KVD_OK;
}

int32_t rope_append(const kvd_paged_kv* kv, const float* q, const float* k, const float* v,
                    float* q_rot, double rope_base, int32_t layout, void* stream, bool skip_q = false) {
    kvd::RopeAppendArgs a;
    a.c = view_of(kv);
    a.kv_bf16 = kv->kv_dtype == KVD_KV_BF16;
    a.interleaved = layout == KVD_ROPE_INTERLEAVED;
    a.skip_q = skip_q;
    fill_theta(&a.theta, rope_base, kv->head_dim);
    a.q = q;
    a.k = k;
    a.v = v;
    a.q_rot = q_rot;
    hipError_t e = kvd::launch_rope_append(a, (hipStream_t)stream);
    if (e != hipSuccess) return fail(KVD_ERR_LAUNCH, "rope_append_kv launch: %s", hipGetErrorString(e));
    return ok();
}

// Inputs of the fused step: RoPE + append inside the decode attention kernel,
// or (rope_q_only) the queries' RoPE inside the prefill kernel after the
// RoPE/append kernel has appended the new K/V rows.
struct FuseIn {
    const float* k;
    const float* v;
    float* q_rot;         // may be null
    double rope_base;
    int32_t layout;
    bool rope_q_only;
};

// Decode attention; with `fuse`, q_rot is the raw q and the matrix-core
// kernel also rotates it and appends the new K/V rows.  The descriptor has
// been checked and num_seqs > 0.
int32_t attention(const kvd_paged_kv* kv, const float* q_rot, float* out, float* lse,
                  float softmax_scale, const kvd_attn_options* opt, void* workspace,
                  size_t workspace_bytes, void* stream, const FuseIn* fuse) {
    int32_t st;
    if (!q_rot || !out) return fail(KVD_ERR_NULL, "q and out must be non-NULL");
    if (((uintptr_t)q_rot | (uintptr_t)out | (uintptr_t)lse) & 3)
        return fail(KVD_ERR_SHAPE, "q, out and lse must be 4-byte aligned");
    if (!std::isfinite(softmax_scale))
        return fail(KVD_ERR_SHAPE, "softmax_scale must be finite");
    Plan p;
    st = make_plan(kv, opt, &p);
    if (st != KVD_OK) return st;
    const size_t need = workspace_for(kv, p);
    if (need > 0) {
        if (!workspace) return fail(KVD_ERR_WORKSPACE, "workspace of %zu bytes required", need);
        if (workspace_bytes < need)
            return fail(KVD_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", workspace_bytes, need);
        if ((uintptr_t)workspace & 255) return fail(KVD_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    }
    const double scale = softmax_scale != 0.0f ? (double)softmax_scale : 1.0 / std::sqrt((double)kv->head_dim);
    kvd::AttnArgs a;
    a.c = view_of(kv);
    a.kv_bf16 = kv->kv_dtype == KVD_KV_BF16;
    a.num_splits = p.splits;
    a.split_keys = p.split_keys;
    a.rows = p.rows;
    a.row_tile = p.row_tile;
    // longest-first only pays when workgroups wait for a slot
    if (p.prefill) {
        const int64_t units = (int64_t)p.splits * cdiv(p.rows, kvd::PREFILL_ROWS) * kv->num_seqs;
        a.rank_longest = units <= kvd::PREFILL_RANK_MAX &&
                         units * kv->n_kv_heads > kvd::PREFILL_WGS_PER_CU * (int64_t)num_cus();
    } else {
        a.rank_longest = (int64_t)p.splits * kv->n_kv_heads * kv->num_seqs > (int64_t)kvd::MFMA_WGS_PER_CU * num_cus();
    }
    a.scale_log2 = (float)(scale * 1.4426950408889634);
    a.q = q_rot;
    a.out = out;
    a.part_o = nullptr;
    a.part_ml = nullptr;
    a.counters = nullptr;
    a.lse = lse;
    a.fused = fuse != nullptr && !fuse->rope_q_only;
    a.rope_q = fuse != nullptr && fuse->rope_q_only;
    a.interleaved = fuse && fuse->layout == KVD_ROPE_INTERLEAVED;
    if (fuse) fill_theta(&a.theta, fuse->rope_base, kv->head_dim);
    a.k_new = fuse ? fuse->k : nullptr;
    a.v_new = fuse ? fuse->v : nullptr;
    a.q_rot = fuse ? fuse->q_rot : nullptr;
    if (need > 0) {
        const Carve cv = carve(kv, p);
        a.part_o = (float*)((char*)workspace + cv.o);
        a.part_ml = (float*)((char*)workspace + cv.ml);
        // with two splits the decode kernel merges them itself (the last
        // workgroup of a (sequence, kv head) to finish); otherwise the
        // partials go to the combine kernel.  Measured (median step, one
        // GPU, the two alternating): two splits, Llama-3-8B-shaped layer
        // 47.6 -> 46.95 us with the merge in the kernel; three splits (the
        // continuous batch) 173.4 against 174.2 us and eight (131k context)
        // 323.9 against 326.2 us in favour of the combine kernel: the last
        // workgroup's read-back of the other splits grows with their number
        // and costs more than the second launch.
        if (p.kernel == KVD_KERNEL_MFMA && !p.prefill && p.splits == kvd::SELF_MERGE_SPLITS &&
            (size_t)kv->num_seqs * kv->n_kv_heads <= COUNTER_SLOTS)
            a.counters = (unsigned*)((char*)workspace + cv.cnt);
    }
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = p.prefill                     ? kvd::launch_attn_prefill(a, s)
                   : p.kernel == KVD_KERNEL_MFMA ? kvd::launch_attn_mfma(a, s)
                                                 : kvd::launch_attn_valu(a, s);
    if (e != hipSuccess) return fail(KVD_ERR_LAUNCH, "decode attention launch: %s", hipGetErrorString(e));
    if (p.splits > 1 && !a.counters) {
        e = kvd::launch_attn_combine(a, s);
        if (e != hipSuccess) return fail(KVD_ERR_LAUNCH, "combine launch: %s", hipGetErrorString(e));
    }
    return ok();
}

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {nullptr};

// The device address of the current device's scratch array in *ptr (the
// first call on a device looks it up with that device current).
int32_t scratch_ptr(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(KVD_ERR_LAUNCH, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= MAX_DEVICES)
        return fail(KVD_ERR_UNSUPPORTED, "device %d (at most %d devices)", dev, MAX_DEVICES);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(KVD_ERR_LAUNCH, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return KVD_OK;
}

}  // namespace

extern "C" {

int32_t kvd_abi_version(void) { return 3; }

int32_t kvd_decode_step_noalloc(const kvd_paged_kv* kv, const float* q, const float* k,
                                const float* v, float* q_rot, float* out, double rope_base,
                                int32_t layout, float softmax_scale, const kvd_attn_options* opt,
                                void* stream) {
    int32_t st = check_desc(kv);
    if (st != KVD_OK) return st;
    if (kv->num_seqs == 0) return ok();
    Plan p;
    st = make_plan(kv, opt, &p);
    if (st != KVD_OK) return st;
    const size_t need = workspace_for(kv, p);
    if (need > (size_t)KVD_NOALLOC_SCRATCH_BYTES)
        return fail(KVD_ERR_WORKSPACE,
                    "the plan needs %zu bytes of split-K scratch, above the %zu of the static scratch "
                    "(use kvd_decode_step with a workspace, or fewer splits)",
                    need, (size_t)KVD_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    if (need > 0) {
        st = scratch_ptr(&ws);
        if (st != KVD_OK) return st;
    }
    return kvd_decode_step(kv, q, k, v, q_rot, out, rope_base, layout, softmax_scale, opt, ws,
                           need > 0 ? (size_t)KVD_NOALLOC_SCRATCH_BYTES : 0, stream);
}

int32_t kvd_decode_step(const kvd_paged_kv* kv, const float* q, const float* k, const float* v,
                        float* q_rot, float* out, double rope_base, int32_t layout,
                        float softmax_scale, const kvd_attn_options* opt, void* workspace,
                        size_t workspace_bytes, void* stream) {
    int32_t st = check_desc(kv);
    if (st != KVD_OK) return st;
    if (kv->num_seqs == 0) return ok();
    if (!out) return fail(KVD_ERR_NULL, "out must be non-NULL");
    st = check_rope(q, k, v, q_rot, rope_base, layout);
    if (st != KVD_OK) return st;
    Plan p;
    st = make_plan(kv, opt, &p);
    if (st != KVD_OK) return st;
    // the fused kernel appends from the block ids of one staged piece
    const bool one_piece = (int64_t)p.split_keys + kv->block_size - 1 <=
                           (int64_t)kvd::MFMA_PIECE_BLOCKS * kv->block_size;
    if (p.kernel == KVD_KERNEL_MFMA && !p.prefill && !kv->key_pos0 && !kv->q_pos && one_piece) {
        const FuseIn f{k, v, q_rot, rope_base, layout, false};
        return attention(kv, q, out, nullptr, softmax_scale, opt, workspace, workspace_bytes, stream, &f);
    }
    if (p.prefill) {
        // the new K/V rows first (every row tile at or past them reads them),
        // then the prefill kernel rotates its own query rows
        st = rope_append(kv, q, k, v, nullptr, rope_base, layout, stream, true);
        if (st != KVD_OK) return st;
        const FuseIn f{k, v, q_rot, rope_base, layout, true};
        return attention(kv, q, out, nullptr, softmax_scale, opt, workspace, workspace_bytes, stream, &f);
    }
    // vector-ALU plans, context-parallel shards on the decode kernel and
    // splits of more blocks than one piece: the two kernels in a row; `out`
    // holds the rotated queries when the caller wants none back (each output
    // row is written only after its query row has been read)
    float* qr = q_rot ? q_rot : out;
    st = rope_append(kv, q, k, v, qr, rope_base, layout, stream);
    if (st != KVD_OK) return st;
    return attention(kv, qr, out, nullptr, softmax_scale, opt, workspace, workspace_bytes, stream, nullptr);
}

int32_t kvd_check_descriptor(const kvd_paged_kv* kv, uint32_t* flags, void* stream) {
    int32_t st = check_desc(kv);
    if (st != KVD_OK) return st;
    if (!flags) return fail(KVD_ERR_NULL, "flags must be non-NULL");
    if ((uintptr_t)flags & 3) return fail(KVD_ERR_SHAPE, "flags must be 4-byte aligned");
    if (kv->num_seqs == 0) return ok();
    hipError_t e = kvd::launch_check_descriptor(view_of(kv), kv->max_seq_len, kv->num_blocks, flags,
                                                (hipStream_t)stream);
    if (e != hipSuccess) return fail(KVD_ERR_LAUNCH, "check launch: %s", hipGetErrorString(e));
    return ok();
}

const char* kvd_status_string(int32_t s) {
    switch (s) {
        case KVD_OK: return "KVD_OK";
        case KVD_ERR_NULL: return "KVD_ERR_NULL";
        case KVD_ERR_SHAPE: return "KVD_ERR_SHAPE";
        case KVD_ERR_UNSUPPORTED: return "KVD_ERR_UNSUPPORTED";
        case KVD_ERR_WORKSPACE: return "KVD_ERR_WORKSPACE";
        case KVD_ERR_LAUNCH: return "KVD_ERR_LAUNCH";
        default: return "KVD_ERR_UNKNOWN";
    }
}

const char* kvd_last_error(void) { return g_err; }

int32_t kvd_rope_append_kv(const kvd_paged_kv* kv, const float* q, const float* k, const float* v,
                           float* q_rot, double rope_base, int32_t layout, void* stream) {
    int32_t st = check_desc(kv);
    if (st != KVD_OK) return st;
    if (kv->num_seqs == 0) return ok();
    if (!q_rot) return fail(KVD_ERR_NULL, "q_rot must be non-NULL");
    st = check_rope(q, k, v, q_rot, rope_base, layout);
    if (st != KVD_OK) return st;
    return rope_append(kv, q, k, v, q_rot, rope_base, layout, stream);
}

size_t kvd_decode_attention_workspace_size_ex(const kvd_paged_kv* kv, const kvd_attn_options* opt) {
    if (check_desc(kv) != KVD_OK) return (size_t)-1;
    if (kv->num_seqs == 0) return 0;
    Plan p;
    if (make_plan(kv, opt, &p) != KVD_OK) return (size_t)-1;
    return workspace_for(kv, p);
}

size_t kvd_decode_attention_workspace_size(const kvd_paged_kv* kv) {
    return kvd_decode_attention_workspace_size_ex(kv, nullptr);
}

int32_t kvd_decode_attention_plan(const kvd_paged_kv* kv, const kvd_attn_options* opt,
                                  int32_t* num_splits, int32_t* keys_per_split, int32_t* kernel) {
    int32_t st = check_desc(kv);
    if (st != KVD_OK) return st;
    if (kv->num_seqs == 0) {
        if (num_splits) *num_splits = 0;
        if (keys_per_split) *keys_per_split = 0;
        if (kernel) *kernel = KVD_KERNEL_VALU;
        return ok();
    }
    Plan p;
    st = make_plan(kv, opt, &p);
    if (st != KVD_OK) return st;
    if (num_splits) *num_splits = p.splits;
    if (keys_per_split) *keys_per_split = p.split_keys;
    if (kernel) *kernel = p.kernel;
    return ok();
}

int32_t kvd_decode_attention_ex(const kvd_paged_kv* kv, const float* q_rot, float* out,
                                float softmax_scale, const kvd_attn_options* opt, void* workspace,
                                size_t workspace_bytes, void* stream) {
    int32_t st = check_desc(kv);
    if (st != KVD_OK) return st;
    if (kv->num_seqs == 0) return ok();
    return attention(kv, q_rot, out, nullptr, softmax_scale, opt, workspace, workspace_bytes, stream,
                     nullptr);
}

int32_t kvd_decode_attention_lse(const kvd_paged_kv* kv, const float* q_rot, float* out, float* lse,
                                 float softmax_scale, const kvd_attn_options* opt, void* workspace,
                                 size_t workspace_bytes, void* stream) {
    int32_t st = check_desc(kv);
    if (st != KVD_OK) return st;
    if (kv->num_seqs == 0) return ok();
    if (!lse) return fail(KVD_ERR_NULL, "lse must be non-NULL");
    return attention(kv, q_rot, out, lse, softmax_scale, opt, workspace, workspace_bytes, stream,
                     nullptr);
}

int32_t kvd_merge_partials(int32_t n_parts, int64_t rows, int32_t head_dim, const float* outs,
                           const float* lses, float* out, float* lse_out, void* stream) {
    if (n_parts < 1 || n_parts > 4096)
        return fail(n_parts < 1 ? KVD_ERR_SHAPE : KVD_ERR_UNSUPPORTED, "n_parts = %d (supported 1..4096)",
                    n_parts);
    if (rows < 0 || head_dim < 1) return fail(KVD_ERR_SHAPE, "rows = %lld, head_dim = %d", (long long)rows, head_dim);
    if (rows > 0x7fffffffLL) return fail(KVD_ERR_UNSUPPORTED, "rows = %lld (at most 2^31 - 1)", (long long)rows);
    if (rows == 0) return ok();
    if (!outs || !lses || !out) return fail(KVD_ERR_NULL, "outs, lses and out must be non-NULL");
    if (((uintptr_t)outs | (uintptr_t)lses | (uintptr_t)out | (uintptr_t)lse_out) & 3)
        return fail(KVD_ERR_SHAPE, "outs, lses, out and lse_out must be 4-byte aligned");
    hipError_t e = kvd::launch_merge_partials(n_parts, rows, head_dim, outs, lses, out, lse_out,
                                              (hipStream_t)stream);
    if (e != hipSuccess) return fail(KVD_ERR_LAUNCH, "merge launch: %s", hipGetErrorString(e));
    return ok();
}

int32_t kvd_decode_attention(const kvd_paged_kv* kv, const float* q_rot, float* out,
                             float softmax_scale, void* workspace, size_t workspace_bytes,
                             void* stream) {
    return kvd_decode_attention_ex(kv, q_rot, out, softmax_scale, nullptr, workspace, workspace_bytes,
                                   stream);
}

}  // extern "C"
