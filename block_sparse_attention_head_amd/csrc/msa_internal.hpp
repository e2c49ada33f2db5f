// Host-side declarations of the kernel launchers behind the libmsa C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace msa {

constexpr int kBlock = 128;  // key block size (tokens)
constexpr int kDim = 128;    // head dim of Q/K/V and of the index heads
constexpr int kRowTilesPerItem = 16;  // 128-row query tiles per sparse-attention work item

// Problem sizes after validation (all derived from msa_shape).
struct Dims {
    int B, N, Hq, Hkv, G, gshift, nblk, top_k;
    float scale;
    // query positions [p0, p0 + Nc) handled by one pass of the sparse attention (plan,
    // partial, combine) and sized in its workspace; the whole sequence unless chunked
    int p0 = 0, Nc = 0;
};

// Index scores + causal block max-pool. Writes pooled[b,g,t,c] for c <= t/128;
// when `fill_upper` also writes -inf for c > t/128.
hipError_t launch_index_pool(const void* q_idx, const void* k_idx, float* pooled, const Dims& d,
                             bool fill_upper, hipStream_t stream);

// Decode step (one query per sequence; seqlens on the device, clamped to the
// capacity d.N, <= 0 empty): index scores + block max into pooled [B, H, nblk],
// the selection into block_idx [B, H, top_k], attention into o [B, Hq, 128] and
// lse [B, Hq]. The selection needs dec_topk_lds_bytes(d) of LDS.
size_t dec_topk_lds_bytes(const Dims& d);
hipError_t launch_dec_index(const void* q_idx, const void* k_idx, const int32_t* seqlens, float* pooled, const Dims& d,
                            hipStream_t stream);
hipError_t launch_dec_topk(const float* pooled, const int32_t* seqlens, int32_t* block_idx, const Dims& d,
                           hipStream_t stream);
// Attention over the selected blocks. With `records` (dec_rec_bytes(d) bytes, non-null
// only when that is nonzero) a group's slots are spread over dec_splits(d) workgroups
// whose (m, l, O) records a second kernel merges; with records == null one workgroup
// per (sequence, KV head, head tile) does all its slots.
int dec_splits(const Dims& d);
size_t dec_rec_bytes(const Dims& d);
hipError_t launch_dec_attn(const void* q, const void* k, const void* v, const int32_t* seqlens,
                           const int32_t* block_idx, void* o, float* lse, void* records, const Dims& d,
                           hipStream_t stream);

// Index scores + block max-pool + top-k selection in one pass with no pooled
// scores in memory and no scratch; needs index_topk_fusable(d) (top_k <= 17).
bool index_topk_fusable(const Dims& d);
hipError_t launch_index_topk(const void* q_idx, const void* k_idx, int32_t* block_idx, const Dims& d,
                             hipStream_t stream);
// Largest top_k this build's selection kernel accepts for `nblk` key blocks.
bool topk_supported(int nblk, int top_k);
hipError_t launch_block_topk(const float* pooled, int32_t* block_idx, const Dims& d, hipStream_t stream);

// Workspace of the sparse attention forward, carved from one caller buffer.
struct SparseWs {
    int32_t* cnt;       // [B*Hkv*nblk]    queries per (b, g, c) tile
    int32_t* off;       // [B*Hkv*nblk+1]  exclusive prefix of cnt
    int32_t* item_off;  // [B*Hkv*nblk+1]  exclusive prefix of work items per tile
    int32_t* cursor;    // [B*Hkv*nblk]    next free place per tile (unordered scatter)
    int32_t* wgoff;     // [B*Hkv, rev_groups(N), nblk] per position range: entries, then first entry
    int32_t* entries;   // [B*Hkv*N*top_k] (t << 8 | slot), grouped by tile
    void* part_o;       // bf16 [B, N, top_k, Hkv, 16, G, 8] normalised partial outputs (lane order)
    float* part_lse;    // fp32 [B, N, top_k, Hq]      partial log-sum-exp
};
// Position ranges (workgroups) per (b, g) of the reverse-index scatter.
int rev_groups(int N);
size_t sparse_ws_bytes(const Dims& d);
SparseWs carve_sparse_ws(void* base, const Dims& d);

// Whether the forward's combine computes the (row, own block) pairs itself (then the
// unordered plan leaves them out and the partial kernel never sees them).
bool combine_folds_local(const Dims& d);
// Reverse index and work list. `canonical`: the entry order inside a tile is a
// function of block_idx alone and every valid entry is listed (the backward needs
// both); otherwise it is unordered and leaves out the local block when
// combine_folds_local(d).
hipError_t launch_sparse_plan(const int32_t* block_idx, const SparseWs& ws, const Dims& d, bool canonical,
                              hipStream_t stream);
hipError_t launch_sparse_partial(const void* q, const void* k, const void* v, const SparseWs& ws, const Dims& d,
                                 hipStream_t stream);
// Dynamic LDS bytes of the records-only combine kernel (must stay within 64 KB).
size_t combine_lds_bytes(const Dims& d);
// The combine; reads q, k and v when combine_folds_local(d) (the local block's attention).
hipError_t launch_sparse_combine(const void* q, const void* k, const void* v, const int32_t* block_idx, void* o,
                                 float* lse, const SparseWs& ws, const Dims& d, hipStream_t stream);

// Workspace of the sparse attention backward: the forward's plan (reverse index
// and work items, part_o / part_lse unused) followed by the backward's buffers.
struct BwdWs {
    SparseWs plan;
    float* rowterm;   // fp32 [2][B*N*Hq + 1]          LSE*log2(e), then D = rowsum(dO * O); + a pad row
    void* dq_part;    // bf16 [B, N, top_k, 16, Hq, 8] unscaled dQ per (t, slot, head), chunk-major,
                      // then a 256-byte sink for stores of padding rows
    float* dkv_part;  // fp32 [items, 2, 128, 128]     dK (scaled), dV per work item
};
size_t bwd_max_items(const Dims& d);
size_t bwd_ws_bytes(const Dims& d);
BwdWs carve_bwd_ws(void* base, const Dims& d);

hipError_t launch_bwd_delta(const void* o, const void* d_o, const float* lse, float* rowterm, const Dims& d,
                            hipStream_t stream);
hipError_t launch_bwd_main(const void* q, const void* k, const void* v, const void* d_o, const BwdWs& ws,
                           const Dims& d, hipStream_t stream);
hipError_t launch_bwd_dq_sum(const int32_t* block_idx, void* dq, const BwdWs& ws, const Dims& d,
                             hipStream_t stream);
hipError_t launch_bwd_dkdv_reduce(void* dk, void* dv, const BwdWs& ws, const Dims& d, hipStream_t stream);

// Compute-unit count of the current device (cached per device).
// Index-branch gradient from the KL alignment loss (k_index_bwd.hip).
hipError_t launch_kl_lse(const void* q_idx, const void* k_idx, const int32_t* block_idx, const SparseWs& plan,
                         float2* lse_part, float* lse_px, float index_scale, const Dims& d, hipStream_t stream);
hipError_t launch_kl_dz(const void* q, const void* k, const void* q_idx, const void* k_idx, const float* lse,
                        const float* lse_px, const SparseWs& plan, void* dz, float index_scale, float kl_weight,
                        const Dims& d, hipStream_t stream);
hipError_t launch_kl_grad(const void* q_idx, const void* k_idx, const void* dz, const SparseWs& plan, void* dq_part,
                          float* dk_part, const Dims& d, hipStream_t stream);
hipError_t launch_kl_reduce(const int32_t* block_idx, const void* dq_part, const float* dk_part, const SparseWs& plan,
                            void* dq_idx, void* dk_idx, const Dims& d, hipStream_t stream);

int device_cu_count();

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace msa
