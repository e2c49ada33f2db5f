/*
 * libmsa -- MiniMax Sparse Attention (MSA) forward on AMD Instinct MI355X (gfx950).
 *
 * C ABI. Every entry point takes plain device pointers, sizes in a shape
 * struct, a caller-owned workspace and a HIP stream. The library never
 * allocates, frees or synchronises: all work is enqueued on `stream` and runs
 * asynchronously. Arguments are validated on the host before anything is
 * enqueued; on any error nothing is enqueued and no output is touched.
 * No C++ exception crosses this boundary. The only global state is a
 * per-device cache of the compute-unit count (filled on first use; every
 * thread writes the same value), so calls from several host threads on
 * different streams are safe.
 *
 * The method (cited from the web pages that describe it, by title and section):
 *   [MSA summary] "MiniMax Sparse Attention (MSA): Turning Theoretical Sparse
 *       Attention Gains into Real GPU Speedups", section "Architecture:
 *       two-stage block-sparse attention": an index branch (one index query
 *       head per GQA group, one shared index key head) scores the visible key
 *       tokens, aggregates the scores into 128-token blocks and keeps the top-k
 *       blocks (the query's own block always kept); the main branch runs exact
 *       softmax attention over the selected blocks only.
 *   [Flash-MSA] "Flash-MSA: Accelerating Million-Token Training with Sparse
 *       Attention Kernels", sections "About MSA" (blocks chosen by max-pooling
 *       the index scores), "Forward" (index branch, then sparse main
 *       attention; block indices and the main LSE are kept) and "Proxy
 *       attention" (causal max inside the local block; local block forced).
 *   [flash-msa pkg] "flash-msa 0.1.0", sections "Usage" (the call takes index
 *       queries, index keys, Q, K, V, top_k and the softmax scale) and
 *       "Caveats" (head dim 128 and block size 128 only; no quantised inputs;
 *       no attention temperature or softmax bias; index heads tied to KV
 *       groups).
 *
 * Tensor layouts (all dense, row-major, contiguous; bf16 = bfloat16 passed as void*):
 *   q_idx    bf16  [B, N, H_idx, 128]   index queries
 *   k_idx    bf16  [B, N, 128]          shared index key head
 *   q        bf16  [B, N, H_q, 128]
 *   k, v     bf16  [B, N, H_kv, 128]
 *   pooled   fp32  [B, H_idx, N, nblk]  nblk = N / 128
 *   block_idx int32 [B, H_idx, N, top_k] selected blocks, ascending, -1 padded
 *   o        bf16  [B, N, H_q, 128]
 *   lse      fp32  [B, H_q, N]          natural log
 * Query head h belongs to group g = h / G (G = H_q / H_kv); group g uses KV
 * head g and index head g.
 */
#ifndef MSA_H
#define MSA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* In C++ the enums get a fixed 32-bit underlying type, so any int a C caller
 * passes is a valid value (the checks below then reject it); C's enums are
 * int-sized, so the layout is the same in both languages. */
#ifdef __cplusplus
#define MSA_ENUM_INT32 : int32_t
#else
#define MSA_ENUM_INT32
#endif

typedef enum msa_status MSA_ENUM_INT32 {
    MSA_OK = 0,
    MSA_ERR_INVALID_ARG = 1, /* null pointer, non-positive size, inconsistent heads, size overflow */
    MSA_ERR_UNSUPPORTED = 2, /* a valid shape this build does not handle (see msa_shape) */
    MSA_ERR_WORKSPACE = 3,   /* workspace pointer null or smaller than msa_workspace_size() */
    MSA_ERR_HIP = 4          /* a HIP launch failed; work before it may have been enqueued */
} msa_status;

/* flags */
#define MSA_CAUSAL 1u               /* required: the method is causal */
#define MSA_POOLED_VISIBLE_ONLY 2u  /* msa_index_scores: leave pooled[.., c > t/128] unwritten */

typedef struct msa_shape {
    int32_t batch;       /* B >= 1 */
    int32_t seqlen;      /* N >= 1, a multiple of block_size, N < 2^23 */
    int32_t h_q;         /* query heads, a multiple of h_kv; the combine keeps one position's output row,
                            slot weights and selection rows in 64 KB of LDS, which needs
                            h_q*(256 + 4*(top_k+1)) + 8*(top_k*h_q + 4*h_kv*top_k) <= 65536 */
    int32_t h_kv;        /* KV heads; G = h_q / h_kv must be a power of two <= 128 */
    int32_t h_idx;       /* index query heads; must equal h_kv */
    int32_t head_dim;    /* must be 128 */
    int32_t idx_dim;     /* must be 128 */
    int32_t block_size;  /* must be 128 */
    int32_t top_k;       /* 1 <= top_k <= 256; counts the forced local block. msa_block_topk and
                            msa_fwd also need top_k >= nblk, or top_k <= 65 with
                            (top_k-1)*ceil((nblk-1)/64) <= 1024 */
    float softmax_scale; /* > 0 and finite, usually head_dim^-0.5 */
    uint32_t flags;      /* MSA_CAUSAL must be set */
} msa_shape;

typedef enum msa_op MSA_ENUM_INT32 {
    MSA_OP_INDEX_SCORES = 0,
    MSA_OP_BLOCK_TOPK = 1,
    MSA_OP_SPARSE_ATTN_FWD = 2,
    MSA_OP_FWD = 3,
    MSA_OP_SPARSE_ATTN_BWD = 4,
    MSA_OP_INDEX_TOPK = 5,
    MSA_OP_DECODE = 6,
    MSA_OP_INDEX_BWD = 7
} msa_op;

/* Bytes of device workspace `op` needs for `shape` (0 is a valid answer).
 * The workspace is scratch owned by the caller, needs no initialisation, and
 * must not be used by anything else while the call's work runs.
 * MSA_OP_SPARSE_ATTN_FWD and MSA_OP_FWD: the per-slot partial results grow with
 * seqlen * top_k * h_q, so the answer is the size for one pass over all query
 * positions when that is at most 64 GiB, and otherwise the size for the largest
 * chunk of positions (a multiple of 128) that fits in 64 GiB, or for 128
 * positions when not even those fit (the smallest chunk the forward runs). */
msa_status msa_workspace_size(const msa_shape* shape, msa_op op, size_t* bytes);

/* Index scores with causal block max-pool ([MSA summary] "Architecture";
 * [Flash-MSA] "About MSA" item 1 and "Proxy attention"):
 *   pooled[b,g,t,c] = max_{j in block c, j <= t} sum_e q_idx[b,t,g,e] * k_idx[b,j,e]
 * for c <= t/128, and -inf for c > t/128. Raw dot products (no scale),
 * bf16 products accumulated in fp32. Writes every element of `pooled`, or only
 * the visible part (c <= t/128) when shape->flags has MSA_POOLED_VISIBLE_ONLY. */
msa_status msa_index_scores(const msa_shape* shape, const void* q_idx, const void* k_idx,
                            float* pooled, hipStream_t stream);

/* Top-k block selection with the local block forced ([MSA summary]
 * "Architecture" and "GPU kernel co-design": selection on raw scores;
 * [Flash-MSA] "Proxy attention": local block forced). For query t with
 * c_loc = t/128: if c_loc + 1 <= top_k every visible block is selected;
 * otherwise c_loc plus the top_k - 1 largest pooled[.., c] over c < c_loc,
 * larger score first, lower block first among equal scores (-0.0 == +0.0).
 * Only the visible part (c <= c_loc) of `pooled` is read. Output ascending,
 * padded with -1. Deterministic; no workspace is needed today (pass NULL, 0). */
msa_status msa_block_topk(const msa_shape* shape, const float* pooled, int32_t* block_idx,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/* msa_index_scores followed by msa_block_topk, writing only `block_idx`
 * (same layout and result, bit for bit). For top_k <= 17 one kernel does
 * both in a single pass with no pooled scores in memory: each row keeps its
 * best top_k - 1 earlier blocks in registers as the key blocks stream past
 * ([Flash-MSA] "Proxy attention": the selection is kept inside the proxy
 * kernel; [MSA summary] "GPU kernel co-design": exp-free selection on the raw
 * pooled scores). That path needs no workspace (size 0; workspace may be NULL).
 * For larger top_k the two kernels run in turn with the pooled scores (visible
 * part only) in the workspace; ask msa_workspace_size(MSA_OP_INDEX_TOPK).
 * msa_fwd uses this step. */
msa_status msa_index_topk(const msa_shape* shape, const void* q_idx, const void* k_idx, int32_t* block_idx,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Exact causal softmax attention of every query head over the blocks its
 * group selected ([MSA summary] "Architecture" main branch; [Flash-MSA]
 * "Main attention" and "Forward": O and the main LSE are produced):
 *   z_j = softmax_scale * q[b,t,h] . k[b,j,g]  for j in a selected block, j <= t
 *   o[b,t,h] = sum_j softmax(z)_j v[b,j,g];   lse[b,h,t] = log sum_j exp(z_j)
 * block_idx entries outside [0, t/128] are ignored (treated as padding);
 * a block listed twice in a row counts twice (the selections msa_fwd makes
 * never repeat a block). A row
 * with no valid entry gives o = 0 and lse = -inf. Runs KV-outer: each
 * (key block, KV head) tile gathers the queries that selected it ([MSA summary]
 * "GPU kernel co-design"), writes per-slot partial results into the workspace,
 * and a combine pass merges them; with top_k <= 16 the combine itself computes
 * each query's attention to its own block (the causal block every position of
 * a block shares). Deterministic (no floating-point atomics).
 * Any workspace that holds the partials of at least 128 query positions is
 * accepted: the positions are then processed in as many chunks as it takes
 * (each chunk reads only its rows' block indices; all K/V stay where they are),
 * with results identical to one pass. */
msa_status msa_sparse_attn_fwd(const msa_shape* shape, const void* q, const void* k, const void* v,
                               const int32_t* block_idx, void* o, float* lse,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The three phases of msa_sparse_attn_fwd, for callers that schedule or time
 * them separately. They process the whole sequence in one pass, so all three
 * need the one-pass workspace (MSA_ERR_WORKSPACE otherwise; msa_workspace_size
 * gives it whenever it is at most 64 GiB), and must be enqueued in this order
 * on one stream with the same shape and workspace:
 *   plan:    reverse sparse index ([Flash-MSA] "Backward": the map from
 *            (query, slot) to key block is inverted into key block -> queries;
 *            [MSA summary] "GPU kernel co-design": reverse sparse indexing)
 *            and the tile work list, from block_idx;
 *   partial: per (key block, KV head) tile, softmax attention of the gathered
 *            queries over that block, written to per-slot partial outputs;
 *   combine: merge of the partials into o and lse ([MSA summary] "GPU kernel
 *            co-design": two-phase forward with a global softmax combine).
 * With top_k <= 16 the combine also computes each query's attention to its own
 * (local) block, the causal block that every position of a block shares, from
 * q, k and v: the plan then leaves those (query, block) pairs out of the
 * partial phase. q, k and v are the tensors msa_sparse_attn_fwd takes (device,
 * not modified); the combine requires them non-null for every top_k
 * (MSA_ERR_INVALID_ARG otherwise). */
msa_status msa_sparse_attn_plan(const msa_shape* shape, const int32_t* block_idx, void* workspace,
                                size_t workspace_bytes, hipStream_t stream);
msa_status msa_sparse_attn_partial(const msa_shape* shape, const void* q, const void* k, const void* v,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream);
msa_status msa_sparse_attn_combine(const msa_shape* shape, const void* q, const void* k, const void* v,
                                   const int32_t* block_idx, void* o, float* lse, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream);

/* The whole forward: msa_index_topk into `block_idx`, then msa_sparse_attn_fwd
 * into `o` and `lse` ([Flash-MSA] "Forward": index branch
 * first, then sparse main attention; block indices and LSE are kept). The
 * workspace holds msa_index_topk's (0 bytes for top_k <= 17) followed by the
 * sparse attention's, which may be a chunk's (see msa_sparse_attn_fwd). */
msa_status msa_fwd(const msa_shape* shape, const void* q_idx, const void* k_idx, const void* q,
                   const void* k, const void* v, int32_t* block_idx, void* o, float* lse,
                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Backward of msa_sparse_attn_fwd over the cached block indices ([Flash-MSA]
 * "Kernel Design": the block indices are kept until the backward so that the
 * whole step after the index branch is linear in N; "Backward": the map from
 * (query, slot) to key block is inverted into key block -> queries, tasks are
 * scheduled per key block and each streams chunks of gathered query rows
 * against the resident K/V block, computing dQ, dK and dV). With z_j and the
 * attended set as in msa_sparse_attn_fwd, P_j = exp(z_j - lse[b,h,t]) and
 * D = sum_d d_o[b,t,h,d] * o[b,t,h,d]:
 *   dq[b,t,h] = softmax_scale * sum_j P_j (d_o[b,t,h] . v[b,j,g] - D) k[b,j,g]
 *   dk[b,j,g] = softmax_scale * sum_{(t,h) attending j} P_j (d_o . v_j - D) q[b,t,h]
 *   dv[b,j,g] = sum_{(t,h) attending j} P_j d_o[b,t,h]
 * Inputs: q, k, v, block_idx as given to the forward; o and lse as the forward
 * returned them; d_o bf16 [B, N, H_q, 128] (the gradient of o). Outputs (bf16,
 * every element written): dq [B, N, H_q, 128], dk and dv [B, N, H_kv, 128]
 * (zero for keys no query attends). The index branch has no gradient here.
 * Products are bf16 with fp32 accumulation (P and dS are rounded to bf16 before
 * their products, as in the forward). Per-slot dQ partials and per-task dK/dV
 * partials in the workspace (MSA_OP_SPARSE_ATTN_BWD) are summed by separate
 * passes: deterministic, no floating-point atomics. Rows with no valid entry
 * get dq = 0. Also needs batch * seqlen * h_q < 2^31 (else MSA_ERR_UNSUPPORTED). */
msa_status msa_sparse_attn_bwd(const msa_shape* shape, const void* q, const void* k, const void* v,
                               const void* o, const float* lse, const void* d_o,
                               const int32_t* block_idx, void* dq, void* dk, void* dv,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Gradient of the index (proxy) branch from the KL alignment loss, over the
 * forward's cached block indices ([MSA summary] "Training stability": the
 * top-k has no gradient, so the index projections learn from a KL loss whose
 * teacher averages the group's query heads' softmax over the selected tokens,
 * the main branch detached; [Flash-MSA] "KL Divergence Loss": the gradient to
 * a proxy logit is the proxy probability minus the teacher's, so the loss is
 * never formed; "Backward": the proxy LSE is recomputed over the selected
 * blocks). For group g, position t and each attended key j (as in
 * msa_sparse_attn_fwd: selected blocks, j <= t, a repeated entry twice):
 *   p_j  = (1/G) sum_{h in g} exp(softmax_scale q[b,t,h] . k[b,j,g] - lse[b,h,t])
 *   px_j = softmax_j(index_scale q_idx[b,t,g] . k_idx[b,j])
 *   dz_j = kl_weight * (px_j - p_j)
 *   dq_idx[b,t,g] = index_scale sum_j dz_j k_idx[b,j]
 *   dk_idx[b,j]   = index_scale sum_{(t,g) attending j} dz_j q_idx[b,t,g]
 * lse is the forward's main LSE; index_scale > 0 (the main softmax scale is the
 * plain choice: the call of the pages takes one scale) and kl_weight is the
 * gradient of the caller's total loss with respect to the KL term. Outputs
 * (bf16, every element written): dq_idx [B, N, H_idx, 128], dk_idx [B, N, 128]
 * (summed over the groups: one shared index key head). With a selection of every
 * visible block (top_k >= nblk) this is the dense warmup mode's gradient.
 * Deterministic (canonical plan, no floating-point atomics). Also needs
 * G = h_q / h_kv <= 32 and batch * seqlen * h_q < 2^31 (else MSA_ERR_UNSUPPORTED).
 * Workspace: msa_workspace_size(MSA_OP_INDEX_BWD). */
msa_status msa_index_bwd(const msa_shape* shape, const void* q_idx, const void* k_idx, const void* q,
                         const void* k, const float* lse, const int32_t* block_idx, float index_scale,
                         float kl_weight, void* dq_idx, void* dk_idx, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);

/* ---- Decode: one new query per sequence against its KV cache ----
 * [MSA summary] "Why long context is the bottleneck" (decoding adds one token
 * at a time against a cache that grows with the context) and "Experimental
 * results" (the same sparse attention serves decoding). The step for a
 * sequence of length L computes what msa_fwd computes for its last position
 * t = L - 1, over cache rows 0..t; rows at or past L are never read.
 * For these calls shape->seqlen is the cache capacity C (a multiple of 128,
 * C <= 2^21); 1 <= top_k <= 65; batch and h_kv <= 65535; other fields as for
 * the forward (the combine bound does not apply).
 *   q_idx    bf16  [B, H_idx, 128]      the new token's index queries
 *   q        bf16  [B, H_q, 128]        its queries
 *   k_idx    bf16  [B, C, 128]          index-key cache
 *   k, v     bf16  [B, C, H_kv, 128]    KV cache
 *   seqlens  int32 [B] (device)         L per sequence; L > C is read as C, L <= 0 as
 *                                        an empty sequence (block_idx -1, o 0, lse -inf)
 *   pooled   fp32  [B, H_idx, C/128]    block maxima; -inf for blocks past t/128
 *   block_idx int32 [B, H_idx, top_k]   ascending, local block last, -1 padded
 *   o        bf16  [B, H_q, 128];  lse fp32 [B, H_q] (natural log) */

/* Index scores of the new token against every cached index key, max-pooled per block. */
msa_status msa_decode_index_scores(const msa_shape* shape, const void* q_idx, const void* k_idx,
                                   const int32_t* seqlens, float* pooled, hipStream_t stream);

/* Selection per (sequence, index head) with the same rule as msa_block_topk, on rows of
 * any length up to the capacity. */
msa_status msa_decode_topk(const msa_shape* shape, const float* pooled, const int32_t* seqlens,
                           int32_t* block_idx, hipStream_t stream);

/* Softmax attention of each query head over its group's selected blocks (entries
 * outside [0, t/128] ignored; a repeated entry counts twice, as in the forward).
 * workspace may be NULL: then one workgroup per (sequence, KV head, 16 query
 * heads) walks all of its group's blocks. With a workspace of at least
 * msa_workspace_size(MSA_OP_DECODE) bytes (MSA_ERR_WORKSPACE if smaller), a step
 * with few sequences spreads each group's blocks over several workgroups, whose
 * per-split (max, sum, output) records a second kernel merges; the results agree
 * within rounding. msa_decode always passes its workspace. */
msa_status msa_decode_attn(const msa_shape* shape, const void* q, const void* k, const void* v,
                           const int32_t* seqlens, const int32_t* block_idx, void* o, float* lse,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The three steps in turn; the pooled scores and the attention's split records
 * live in the workspace (MSA_OP_DECODE). */
msa_status msa_decode(const msa_shape* shape, const void* q_idx, const void* k_idx, const void* q,
                      const void* k, const void* v, const int32_t* seqlens, int32_t* block_idx,
                      void* o, float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* msa_decode without a workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, serving loops and harnesses that forbid
 * hipMalloc). The step's scratch (the pooled block scores, B * H_idx * C/128 * 4
 * bytes, and with few sequences the attention's split records: the size
 * msa_workspace_size(MSA_OP_DECODE) gives) lives in a static device array of
 * MSA_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on, from
 * the first call on that GPU until the process ends; this call allocates nothing.
 * A step that needs more scratch than that returns MSA_ERR_WORKSPACE (nothing is
 * enqueued; use msa_decode). All calls on one GPU share its array: calls whose
 * work overlaps in time on the same GPU (other streams, other host threads) race
 * and must be ordered by the caller. Same arguments, outputs and results as
 * msa_decode (bit for bit); the first call on each device looks up the array's
 * device address (MSA_ERR_HIP if that fails). */
#define MSA_NOALLOC_SCRATCH_BYTES (32u * 1024u * 1024u)
msa_status msa_decode_noalloc(const msa_shape* shape, const void* q_idx, const void* k_idx, const void* q,
                              const void* k, const void* v, const int32_t* seqlens, int32_t* block_idx,
                              void* o, float* lse, hipStream_t stream);

/* Static, never-NULL description of a status code. */
const char* msa_status_string(msa_status status);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H */
