// libmsa C ABI: argument validation, workspace layout and launch order.
#include <math.h>

#include <atomic>
#include <mutex>

#include "msa.h"
#include "msa_internal.hpp"

namespace msa {

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];  // 0 = not queried yet; benign race (same value)

// Scratch of msa_decode_noalloc: one copy of this array on every GPU the library
// runs on, held until the process ends. In host code `scratch` names a host-side
// stand-in, never a device address: the device address is looked up once per
// device (hipGetSymbolAddress, with that device current) and only that address
// is passed to kernels.
static __device__ __align__(256) unsigned char scratch[MSA_NOALLOC_SCRATCH_BYTES];
std::atomic<void*> g_scratch_dev[kMaxDevices];  // device address of `scratch`, per device
std::mutex g_scratch_mu;

// Device address of the current device's scratch array, or null on a HIP error.
void* scratch_address(int dev) {
    void* p = g_scratch_dev[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_dev[dev].load(std::memory_order_relaxed);
    if (p) return p;
    void* addr = nullptr;
    if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || addr == nullptr) {
        (void)hipGetLastError();
        return nullptr;
    }
    g_scratch_dev[dev].store(addr, std::memory_order_release);
    return addr;
}

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }
int log2i(int x) {
    int s = 0;
    while ((1 << s) < x) ++s;
    return s;
}

// Validates `s` and fills `d`. Host only; touches no device state.
msa_status check_shape(const msa_shape* s, Dims* d) {
    if (!s || !d) return MSA_ERR_INVALID_ARG;
    if (s->batch < 1 || s->seqlen < 1 || s->h_q < 1 || s->h_kv < 1 || s->h_idx < 1 || s->top_k < 1)
        return MSA_ERR_INVALID_ARG;
    if (s->h_q % s->h_kv != 0) return MSA_ERR_INVALID_ARG;
    if (!(s->softmax_scale > 0.0f) || !isfinite(s->softmax_scale)) return MSA_ERR_INVALID_ARG;
    if (!(s->flags & MSA_CAUSAL)) return MSA_ERR_UNSUPPORTED;
    if (s->head_dim != kDim || s->idx_dim != kDim || s->block_size != kBlock) return MSA_ERR_UNSUPPORTED;
    if (s->h_idx != s->h_kv) return MSA_ERR_UNSUPPORTED;
    const int G = s->h_q / s->h_kv;
    if (!is_pow2(G) || G > kBlock) return MSA_ERR_UNSUPPORTED;
    if (s->seqlen % kBlock != 0 || s->seqlen >= (1 << 23)) return MSA_ERR_UNSUPPORTED;
    if (s->top_k > 256) return MSA_ERR_UNSUPPORTED;
    // the combine keeps a position's output row, slot weights and selection rows in LDS (<= 64 KB);
    // the bound below is the one msa.h states
    if ((double)s->h_q * (256.0 + 4.0 * (s->top_k + 1)) + 8.0 * ((double)s->top_k * s->h_q + 4.0 * s->h_kv * s->top_k) >
        65536.0)
        return MSA_ERR_UNSUPPORTED;
    // 32-bit index arithmetic bounds used inside the kernels
    const double pairs = (double)s->batch * s->h_kv * s->seqlen * s->top_k;
    if (pairs >= 2147483647.0) return MSA_ERR_UNSUPPORTED;
    if ((double)s->seqlen * s->h_kv >= 2147483647.0) return MSA_ERR_UNSUPPORTED;
    if ((double)s->batch * s->seqlen >= 2147483647.0) return MSA_ERR_UNSUPPORTED;
    if ((double)s->batch * s->h_kv > 65535.0) return MSA_ERR_UNSUPPORTED;  // grid y / z extents
    d->B = s->batch;
    d->N = s->seqlen;
    d->Hq = s->h_q;
    d->Hkv = s->h_kv;
    d->G = G;
    d->gshift = log2i(G);
    d->nblk = s->seqlen / kBlock;
    d->top_k = s->top_k;
    d->scale = s->softmax_scale;
    d->p0 = 0;
    d->Nc = s->seqlen;
    return MSA_OK;
}

// Decode: shape->seqlen is the cache capacity C. Host only.
constexpr int kDecMaxCapacity = 1 << 21;  // keeps the selection's LDS list (8 B per block) within 160 KB

msa_status check_decode_shape(const msa_shape* s, Dims* d) {
    if (!s || !d) return MSA_ERR_INVALID_ARG;
    if (s->batch < 1 || s->seqlen < 1 || s->h_q < 1 || s->h_kv < 1 || s->h_idx < 1 || s->top_k < 1)
        return MSA_ERR_INVALID_ARG;
    if (s->h_q % s->h_kv != 0) return MSA_ERR_INVALID_ARG;
    if (!(s->softmax_scale > 0.0f) || !isfinite(s->softmax_scale)) return MSA_ERR_INVALID_ARG;
    if (!(s->flags & MSA_CAUSAL)) return MSA_ERR_UNSUPPORTED;
    if (s->head_dim != kDim || s->idx_dim != kDim || s->block_size != kBlock) return MSA_ERR_UNSUPPORTED;
    if (s->h_idx != s->h_kv) return MSA_ERR_UNSUPPORTED;
    const int G = s->h_q / s->h_kv;
    if (!is_pow2(G) || G > kBlock) return MSA_ERR_UNSUPPORTED;
    if (s->seqlen % kBlock != 0 || s->seqlen > kDecMaxCapacity) return MSA_ERR_UNSUPPORTED;
    if (s->top_k > 65) return MSA_ERR_UNSUPPORTED;  // the exact rank emits at most one block per lane
    if (s->batch > 65535 || s->h_kv > 65535) return MSA_ERR_UNSUPPORTED;  // grid y / z extents
    if ((double)s->batch * s->h_kv >= 2147483647.0) return MSA_ERR_UNSUPPORTED;
    d->B = s->batch;
    d->N = s->seqlen;
    d->Hq = s->h_q;
    d->Hkv = s->h_kv;
    d->G = G;
    d->gshift = log2i(G);
    d->nblk = s->seqlen / kBlock;
    d->top_k = s->top_k;
    d->scale = s->softmax_scale;
    d->p0 = 0;
    d->Nc = s->seqlen;
    return MSA_OK;
}

// Decode workspace: the pooled scores, then the attention's split records (if any).
size_t dec_pooled_bytes(const Dims& d) { return align_up((size_t)d.B * d.Hkv * d.nblk * sizeof(float), 256); }
size_t dec_ws_bytes(const Dims& d) { return dec_pooled_bytes(d) + dec_rec_bytes(d); }

}  // namespace

namespace {

// Reverse index and work list (cnt, off, item_off, cursor, wgoff, entries): the common
// prefix of the forward and backward workspaces.
size_t plan_ws_bytes(const Dims& d) {
    const size_t n = (size_t)d.B * d.Hkv * d.nblk;
    size_t s = 0;
    s += align_up(n * 4, 256);                                    // cnt
    s += align_up((n + 1) * 4, 256);                              // off
    s += align_up((n + 1) * 4, 256);                              // item_off
    s += align_up(n * 4, 256);                                    // cursor
    s += align_up(n * rev_groups(d.Nc) * 4, 256);                  // wgoff
    s += align_up((size_t)d.B * d.Hkv * d.Nc * d.top_k * 4, 256);  // entries
    return s;
}

SparseWs carve_plan_ws(void* base, const Dims& d) {
    const size_t n = (size_t)d.B * d.Hkv * d.nblk;
    char* p = (char*)base;
    SparseWs w;
    w.cnt = (int32_t*)p;      p += align_up(n * 4, 256);
    w.off = (int32_t*)p;      p += align_up((n + 1) * 4, 256);
    w.item_off = (int32_t*)p; p += align_up((n + 1) * 4, 256);
    w.cursor = (int32_t*)p;   p += align_up(n * 4, 256);
    w.wgoff = (int32_t*)p;    p += align_up(n * rev_groups(d.Nc) * 4, 256);
    w.entries = (int32_t*)p;
    w.part_o = nullptr;
    w.part_lse = nullptr;
    return w;
}

}  // namespace

size_t sparse_ws_bytes(const Dims& d) {
    size_t s = plan_ws_bytes(d);
    s += align_up((size_t)d.B * d.Nc * d.top_k * d.Hq * kDim * 2, 256);  // part_o
    s += align_up((size_t)d.B * d.Nc * d.top_k * d.Hq * 4, 256);         // part_lse
    return s;
}

// The largest chunk of query positions (a multiple of 128, at most N) whose sparse
// attention workspace fits in `bytes`; 0 if not even 128 positions fit.
int fwd_chunk(const Dims& d, size_t bytes) {
    Dims c = d;
    int lo = 0, hi = d.N / kBlock;  // in units of 128 positions
    while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        c.Nc = mid * kBlock;
        if (sparse_ws_bytes(c) <= bytes) lo = mid;
        else hi = mid - 1;
    }
    return lo * kBlock;
}

// Workspace the library asks for: the whole sequence in one pass when that needs at
// most this much, else the chunk that fits it (the per-slot partials grow with N).
constexpr size_t kFwdWsBudget = (size_t)64 << 30;

// The chunk the library asks a workspace for: the largest that fits `bytes`, and never
// fewer than 128 positions (the smallest chunk the forward runs, whatever its size).
Dims fwd_chunk_dims(const Dims& d, size_t bytes) {
    Dims c = d;
    const int fit = fwd_chunk(d, bytes);
    c.Nc = fit > 0 ? fit : kBlock;
    return c;
}

SparseWs carve_sparse_ws(void* base, const Dims& d) {
    SparseWs w = carve_plan_ws(base, d);
    char* p = (char*)base + plan_ws_bytes(d);
    w.part_o = (void*)p;
    p += align_up((size_t)d.B * d.Nc * d.top_k * d.Hq * kDim * 2, 256);
    w.part_lse = (float*)p;
    return w;
}

size_t bwd_ws_bytes(const Dims& d) {
    size_t s = plan_ws_bytes(d);
    s += align_up(((size_t)d.B * d.N * d.Hq + 1) * 2 * 4, 256);        // rowterm
    s += align_up((size_t)d.B * d.N * d.top_k * d.Hq * kDim * 2 + 256, 256);  // dq_part + store sink
    s += align_up(bwd_max_items(d) * 2 * kBlock * kDim * 4, 256);       // dkv_part
    return s;
}

BwdWs carve_bwd_ws(void* base, const Dims& d) {
    BwdWs w;
    w.plan = carve_plan_ws(base, d);
    char* p = (char*)base + plan_ws_bytes(d);
    w.rowterm = (float*)p;
    p += align_up(((size_t)d.B * d.N * d.Hq + 1) * 2 * 4, 256);
    w.dq_part = (void*)p;
    p += align_up((size_t)d.B * d.N * d.top_k * d.Hq * kDim * 2 + 256, 256);
    w.dkv_part = (float*)p;
    return w;
}

namespace {

size_t pooled_bytes(const Dims& d) { return (size_t)d.B * d.Hkv * d.N * d.nblk * sizeof(float); }

// the single-pass kernel needs nothing; otherwise the pooled scores
size_t index_topk_ws_bytes(const Dims& d) { return index_topk_fusable(d) ? 0 : align_up(pooled_bytes(d), 256); }

size_t index_bwd_ws_bytes(const Dims& d);

size_t ws_bytes(const Dims& d, msa_op op) {
    switch (op) {
        case MSA_OP_INDEX_SCORES: return 0;
        case MSA_OP_BLOCK_TOPK: return 0;
        case MSA_OP_SPARSE_ATTN_FWD: return sparse_ws_bytes(fwd_chunk_dims(d, kFwdWsBudget));
        case MSA_OP_FWD: return index_topk_ws_bytes(d) + sparse_ws_bytes(fwd_chunk_dims(d, kFwdWsBudget));
        case MSA_OP_SPARSE_ATTN_BWD: return bwd_ws_bytes(d);
        case MSA_OP_INDEX_TOPK: return index_topk_ws_bytes(d);
        case MSA_OP_DECODE: return dec_ws_bytes(d);
        case MSA_OP_INDEX_BWD: return index_bwd_ws_bytes(d);
    }
    return 0;
}

struct IndexBwdWs {
    SparseWs plan;     // canonical plan of the main groups
    float2* lse_part;  // [B*H_idx*N*top_k] proxy (max, sum) per (t, slot), log2 units
    float* lse_px;     // fp32 [B, H_idx, N]
    void* dz;          // bf16 [entries][128]
    void* dq_part;     // bf16 [B*H_idx*N*top_k][128]
    float* dk_part;    // fp32 [items][128][128]
};

size_t index_bwd_ws_bytes(const Dims& d) {
    const size_t rows = (size_t)d.B * d.N * d.Hkv, recs = rows * d.top_k;
    return plan_ws_bytes(d) + align_up(recs * 8, 256) + align_up(rows * 4, 256) + 2 * align_up(recs * kDim * 2, 256) +
           align_up(bwd_max_items(d) * kBlock * kDim * 4, 256);
}

IndexBwdWs carve_index_bwd_ws(void* base, const Dims& d) {
    const size_t rows = (size_t)d.B * d.N * d.Hkv, recs = rows * d.top_k;
    char* c = (char*)base;
    IndexBwdWs w;
    w.plan = carve_plan_ws(c, d);     c += plan_ws_bytes(d);
    w.lse_part = (float2*)c;          c += align_up(recs * 8, 256);
    w.lse_px = (float*)c;             c += align_up(rows * 4, 256);
    w.dz = c;                         c += align_up(recs * kDim * 2, 256);
    w.dq_part = c;                    c += align_up(recs * kDim * 2, 256);
    w.dk_part = (float*)c;
    return w;
}

// index scores and selection: one pass when the list fits the single-pass kernel
hipError_t run_index_topk(const void* q_idx, const void* k_idx, int32_t* block_idx, void* workspace, const Dims& d,
                          hipStream_t stream) {
    if (index_topk_fusable(d)) return launch_index_topk(q_idx, k_idx, block_idx, d, stream);
    float* pooled = (float*)workspace;
    hipError_t e = launch_index_pool(q_idx, k_idx, pooled, d, false, stream);
    if (e == hipSuccess) e = launch_block_topk(pooled, block_idx, d, stream);
    return e;
}

msa_status hip_status(hipError_t e) { return e == hipSuccess ? MSA_OK : MSA_ERR_HIP; }

// The decode step's kernels in a workspace of dec_ws_bytes(d): pooled scores first,
// then the attention's split records.
hipError_t run_decode(const void* q_idx, const void* k_idx, const void* q, const void* k, const void* v,
                      const int32_t* seqlens, int32_t* block_idx, void* o, float* lse, void* ws, const Dims& d,
                      hipStream_t stream) {
    float* pooled = (float*)ws;
    void* records = dec_rec_bytes(d) ? (char*)ws + dec_pooled_bytes(d) : nullptr;
    hipError_t e = launch_dec_index(q_idx, k_idx, seqlens, pooled, d, stream);
    if (e == hipSuccess) e = launch_dec_topk(pooled, seqlens, block_idx, d, stream);
    if (e == hipSuccess) e = launch_dec_attn(q, k, v, seqlens, block_idx, o, lse, records, d, stream);
    return e;
}

// Sparse attention over every query position, in chunks of `chunk` positions that
// reuse one workspace (plan, partials); each chunk's rows only read K/V and the block
// indices, so the chunks are independent.
hipError_t run_sparse_attn(const void* q, const void* k, const void* v, const int32_t* block_idx, void* o, float* lse,
                           void* workspace, const Dims& d, int chunk, hipStream_t stream) {
    Dims c = d;
    c.Nc = chunk;
    const SparseWs ws = carve_sparse_ws(workspace, c);
    hipError_t e = hipSuccess;
    for (int p0 = 0; p0 < d.N && e == hipSuccess; p0 += chunk) {
        c.p0 = p0;
        c.Nc = d.N - p0 < chunk ? d.N - p0 : chunk;
        e = launch_sparse_plan(block_idx, ws, c, false, stream);
        if (e == hipSuccess) e = launch_sparse_partial(q, k, v, ws, c, stream);
        if (e == hipSuccess) e = launch_sparse_combine(q, k, v, block_idx, o, lse, ws, c, stream);
    }
    return e;
}

}  // namespace

int device_cu_count() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    if (dev < kMaxDevices) {
        const int cached = g_cu_count[dev].load(std::memory_order_relaxed);
        if (cached > 0) return cached;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    if (dev < kMaxDevices) g_cu_count[dev].store(n, std::memory_order_relaxed);
    return n;
}

}  // namespace msa

using namespace msa;

extern "C" {

msa_status msa_workspace_size(const msa_shape* shape, msa_op op, size_t* bytes) {
    if (!bytes) return MSA_ERR_INVALID_ARG;
    if (op < MSA_OP_INDEX_SCORES || op > MSA_OP_INDEX_BWD) return MSA_ERR_INVALID_ARG;
    Dims d;
    if (op == MSA_OP_DECODE) {
        const msa_status st = check_decode_shape(shape, &d);
        if (st != MSA_OK) return st;
        *bytes = dec_ws_bytes(d);
        return MSA_OK;
    }
    const msa_status st = check_shape(shape, &d);
    if (st != MSA_OK) return st;
    *bytes = ws_bytes(d, op);
    return MSA_OK;
}

msa_status msa_index_scores(const msa_shape* shape, const void* q_idx, const void* k_idx, float* pooled,
                            hipStream_t stream) {
    Dims d;
    const msa_status st = check_shape(shape, &d);
    if (st != MSA_OK) return st;
    if (!q_idx || !k_idx || !pooled) return MSA_ERR_INVALID_ARG;
    (void)hipGetLastError();
    const bool fill_upper = !(shape->flags & MSA_POOLED_VISIBLE_ONLY);
    return hip_status(launch_index_pool(q_idx, k_idx, pooled, d, fill_upper, stream));
}

msa_status msa_block_topk(const msa_shape* shape, const float* pooled, int32_t* block_idx, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
    Dims d;
    const msa_status st = check_shape(shape, &d);
    if (st != MSA_OK) return st;
    if (!pooled || !block_idx) return MSA_ERR_INVALID_ARG;
    if (!topk_supported(d.nblk, d.top_k)) return MSA_ERR_UNSUPPORTED;
    (void)workspace;
    (void)workspace_bytes;
    (void)hipGetLastError();
    return hip_status(launch_block_topk(pooled, block_idx, d, stream));
}

msa_status msa_sparse_attn_fwd(const msa_shape* shape, const void* q, const void* k, const void* v,
                               const int32_t* block_idx, void* o, float* lse, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
    Dims d;
    const msa_status st = check_shape(shape, &d);
    if (st != MSA_OK) return st;
    if (!q || !k || !v || !block_idx || !o || !lse) return MSA_ERR_INVALID_ARG;
    const int chunk = workspace ? fwd_chunk(d, workspace_bytes) : 0;
    if (chunk == 0) return MSA_ERR_WORKSPACE;
    (void)hipGetLastError();
    return hip_status(run_sparse_attn(q, k, v, block_idx, o, lse, workspace, d, chunk, stream));
}

msa_status msa_sparse_attn_plan(const msa_shape* shape, const int32_t* block_idx, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
    Dims d;
    const msa_status st = check_shape(shape, &d);
    if (st != MSA_OK) return st;
    if (!block_idx) return MSA_ERR_INVALID_ARG;
    if (!workspace || workspace_bytes < sparse_ws_bytes(d)) return MSA_ERR_WORKSPACE;
    (void)hipGetLastError();
    return hip_status(launch_sparse_plan(block_idx, carve_sparse_ws(workspace, d), d, false, stream));
}

msa_status msa_sparse_attn_partial(const msa_shape* shape, const void* q, const void* k, const void* v,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
    Dims d;
    const msa_status st = check_shape(shape, &d);
    if (st != MSA_OK) return st;
    if (!q || !k || !v) return MSA_ERR_INVALID_ARG;
    if (!workspace || workspace_bytes < sparse_ws_bytes(d)) return MSA_ERR_WORKSPACE;
    (void)hipGetLastError();
    return hip_status(launch_sparse_partial(q, k, v, carve_sparse_ws(workspace, d), d, stream));
}

msa_status msa_sparse_attn_combine(const msa_shape* shape, const void* q, const void* k, const void* v,
                                   const int32_t* block_idx, void* o, float* lse, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream) {
    Dims d;
    const msa_status st = check_shape(shape, &d);
    if (st != MSA_OK) return st;
    if (!q || !k || !v || !block_idx || !o || !lse) return MSA_ERR_INVALID_ARG;
    if (!workspace || workspace_bytes < sparse_ws_bytes(d)) return MSA_ERR_WORKSPACE;
    (void)hipGetLastError();
    return hip_status(launch_sparse_combine(q, k, v, block_idx, o, lse, carve_sparse_ws(workspace, d), d, stream));
}

msa_status msa_fwd(const msa_shape* shape, const void* q_idx, const void* k_idx, const void* q, const void* k,
                   const void* v, int32_t* block_idx, void* o, float* lse, void* workspace, size_t workspace_bytes,
                   hipStream_t stream) {
    Dims d;
    const msa_status st = check_shape(shape, &d);
    if (st != MSA_OK) return st;
    if (!q_idx || !k_idx || !q || !k || !v || !block_idx || !o || !lse) return MSA_ERR_INVALID_ARG;
    if (!index_topk_fusable(d) && !topk_supported(d.nblk, d.top_k)) return MSA_ERR_UNSUPPORTED;
    const size_t sel_bytes = index_topk_ws_bytes(d);
    if (!workspace || workspace_bytes < sel_bytes) return MSA_ERR_WORKSPACE;
    const int chunk = fwd_chunk(d, workspace_bytes - sel_bytes);
    if (chunk == 0) return MSA_ERR_WORKSPACE;
    (void)hipGetLastError();
    hipError_t e = run_index_topk(q_idx, k_idx, block_idx, workspace, d, stream);
    if (e != hipSuccess) return MSA_ERR_HIP;
    return hip_status(run_sparse_attn(q, k, v, block_idx, o, lse, (char*)workspace + sel_bytes, d, chunk, stream));
}

msa_status msa_index_topk(const msa_shape* shape, const void* q_idx, const void* k_idx, int32_t* block_idx,
                          void* workspace, size_t workspace_bytes, hipStream_t stream) {
    Dims d;
    const msa_status st = check_shape(shape, &d);
    if (st != MSA_OK) return st;
    if (!q_idx || !k_idx || !block_idx) return MSA_ERR_INVALID_ARG;
    if (!index_topk_fusable(d) && !topk_supported(d.nblk, d.top_k)) return MSA_ERR_UNSUPPORTED;
    const size_t need = ws_bytes(d, MSA_OP_INDEX_TOPK);
    if (need > 0 && (!workspace || workspace_bytes < need)) return MSA_ERR_WORKSPACE;
    (void)hipGetLastError();
    return hip_status(run_index_topk(q_idx, k_idx, block_idx, workspace, d, stream));
}

msa_status msa_decode_index_scores(const msa_shape* shape, const void* q_idx, const void* k_idx,
                                   const int32_t* seqlens, float* pooled, hipStream_t stream) {
    Dims d;
    const msa_status st = check_decode_shape(shape, &d);
    if (st != MSA_OK) return st;
    if (!q_idx || !k_idx || !seqlens || !pooled) return MSA_ERR_INVALID_ARG;
    (void)hipGetLastError();
    return hip_status(launch_dec_index(q_idx, k_idx, seqlens, pooled, d, stream));
}

msa_status msa_decode_topk(const msa_shape* shape, const float* pooled, const int32_t* seqlens, int32_t* block_idx,
                           hipStream_t stream) {
    Dims d;
    const msa_status st = check_decode_shape(shape, &d);
    if (st != MSA_OK) return st;
    if (!pooled || !seqlens || !block_idx) return MSA_ERR_INVALID_ARG;
    (void)hipGetLastError();
    return hip_status(launch_dec_topk(pooled, seqlens, block_idx, d, stream));
}

msa_status msa_decode_attn(const msa_shape* shape, const void* q, const void* k, const void* v,
                           const int32_t* seqlens, const int32_t* block_idx, void* o, float* lse,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
    Dims d;
    const msa_status st = check_decode_shape(shape, &d);
    if (st != MSA_OK) return st;
    if (!q || !k || !v || !seqlens || !block_idx || !o || !lse) return MSA_ERR_INVALID_ARG;
    const size_t rec = dec_rec_bytes(d);
    if (workspace && workspace_bytes < rec) return MSA_ERR_WORKSPACE;
    (void)hipGetLastError();
    return hip_status(launch_dec_attn(q, k, v, seqlens, block_idx, o, lse, workspace && rec ? workspace : nullptr, d,
                                      stream));
}

msa_status msa_decode(const msa_shape* shape, const void* q_idx, const void* k_idx, const void* q, const void* k,
                      const void* v, const int32_t* seqlens, int32_t* block_idx, void* o, float* lse,
                      void* workspace, size_t workspace_bytes, hipStream_t stream) {
    Dims d;
    const msa_status st = check_decode_shape(shape, &d);
    if (st != MSA_OK) return st;
    if (!q_idx || !k_idx || !q || !k || !v || !seqlens || !block_idx || !o || !lse) return MSA_ERR_INVALID_ARG;
    if (!workspace || workspace_bytes < dec_ws_bytes(d)) return MSA_ERR_WORKSPACE;
    (void)hipGetLastError();
    return hip_status(run_decode(q_idx, k_idx, q, k, v, seqlens, block_idx, o, lse, workspace, d, stream));
}

msa_status msa_decode_noalloc(const msa_shape* shape, const void* q_idx, const void* k_idx, const void* q,
                              const void* k, const void* v, const int32_t* seqlens, int32_t* block_idx, void* o,
                              float* lse, hipStream_t stream) {
    Dims d;
    const msa_status st = check_decode_shape(shape, &d);
    if (st != MSA_OK) return st;
    if (!q_idx || !k_idx || !q || !k || !v || !seqlens || !block_idx || !o || !lse) return MSA_ERR_INVALID_ARG;
    if (dec_ws_bytes(d) > (size_t)MSA_NOALLOC_SCRATCH_BYTES) return MSA_ERR_WORKSPACE;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return MSA_ERR_HIP;
    }
    void* ws = scratch_address(dev);
    if (!ws) return MSA_ERR_HIP;
    (void)hipGetLastError();
    // every pooled entry the selection reads, and every split record the merge reads, is
    // written by this call's kernels first, so the scratch needs no clearing between calls
    return hip_status(run_decode(q_idx, k_idx, q, k, v, seqlens, block_idx, o, lse, ws, d, stream));
}

msa_status msa_sparse_attn_bwd(const msa_shape* shape, const void* q, const void* k, const void* v, const void* o,
                               const float* lse, const void* d_o, const int32_t* block_idx, void* dq, void* dk,
                               void* dv, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    Dims d;
    const msa_status st = check_shape(shape, &d);
    if (st != MSA_OK) return st;
    if (!q || !k || !v || !o || !lse || !d_o || !block_idx || !dq || !dk || !dv) return MSA_ERR_INVALID_ARG;
    // the backward indexes query rows (b, t, h) with 32-bit integers
    if ((double)d.B * d.N * d.Hq >= 2147483647.0) return MSA_ERR_UNSUPPORTED;
    if (!workspace || workspace_bytes < ws_bytes(d, MSA_OP_SPARSE_ATTN_BWD)) return MSA_ERR_WORKSPACE;
    (void)hipGetLastError();
    const BwdWs ws = carve_bwd_ws(workspace, d);
    hipError_t e = launch_sparse_plan(block_idx, ws.plan, d, true, stream);
    if (e == hipSuccess) e = launch_bwd_delta(o, d_o, lse, ws.rowterm, d, stream);
    if (e == hipSuccess) e = launch_bwd_main(q, k, v, d_o, ws, d, stream);
    if (e == hipSuccess) e = launch_bwd_dq_sum(block_idx, dq, ws, d, stream);
    if (e == hipSuccess) e = launch_bwd_dkdv_reduce(dk, dv, ws, d, stream);
    return hip_status(e);
}

msa_status msa_index_bwd(const msa_shape* shape, const void* q_idx, const void* k_idx, const void* q, const void* k,
                         const float* lse, const int32_t* block_idx, float index_scale, float kl_weight,
                         void* dq_idx, void* dk_idx, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    Dims d;
    const msa_status st = check_shape(shape, &d);
    if (st != MSA_OK) return st;
    if (!q_idx || !k_idx || !q || !k || !lse || !block_idx || !dq_idx || !dk_idx) return MSA_ERR_INVALID_ARG;
    if (!(index_scale > 0.0f) || !isfinite(index_scale) || !isfinite(kl_weight)) return MSA_ERR_INVALID_ARG;
    if (d.G > 32) return MSA_ERR_UNSUPPORTED;  // a position's heads are averaged inside one 32-lane half
    if ((double)d.B * d.N * d.Hq >= 2147483647.0) return MSA_ERR_UNSUPPORTED;
    if (!workspace || workspace_bytes < index_bwd_ws_bytes(d)) return MSA_ERR_WORKSPACE;
    (void)hipGetLastError();
    const IndexBwdWs ws = carve_index_bwd_ws(workspace, d);
    hipError_t e = launch_sparse_plan(block_idx, ws.plan, d, true, stream);
    if (e == hipSuccess) e = launch_kl_lse(q_idx, k_idx, block_idx, ws.plan, ws.lse_part, ws.lse_px, index_scale, d, stream);
    if (e == hipSuccess)
        e = launch_kl_dz(q, k, q_idx, k_idx, lse, ws.lse_px, ws.plan, ws.dz, index_scale, kl_weight, d, stream);
    if (e == hipSuccess) e = launch_kl_grad(q_idx, k_idx, ws.dz, ws.plan, ws.dq_part, ws.dk_part, d, stream);
    if (e == hipSuccess) e = launch_kl_reduce(block_idx, ws.dq_part, ws.dk_part, ws.plan, dq_idx, dk_idx, d, stream);
    return hip_status(e);
}

const char* msa_status_string(msa_status status) {
    switch (status) {
        case MSA_OK: return "MSA_OK: success";
        case MSA_ERR_INVALID_ARG: return "MSA_ERR_INVALID_ARG: null pointer or inconsistent/invalid size";
        case MSA_ERR_UNSUPPORTED: return "MSA_ERR_UNSUPPORTED: valid shape this build does not handle";
        case MSA_ERR_WORKSPACE: return "MSA_ERR_WORKSPACE: workspace missing or too small";
        case MSA_ERR_HIP: return "MSA_ERR_HIP: a HIP launch failed";
    }
    return "unknown msa_status";
}

}  // extern "C"
