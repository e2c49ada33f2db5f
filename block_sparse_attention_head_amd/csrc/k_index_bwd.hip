// Gradient of the index (proxy) branch from the KL alignment loss, over the
// forward's cached block indices.
//
// [MSA summary] "Training stability": the top-k has no gradient, so the index
// projections learn from a KL alignment loss whose teacher averages each query
// head's softmax over the selected tokens (the main branch detached).
// [Flash-MSA] "KL Divergence Loss": with teacher p and proxy distribution p_px
// over the same tokens, dL/dz_px,j = p_px,j - p_j, so the loss is never formed;
// "Backward": the proxy LSE comes from a cheap sparse recompute, and the work is
// scheduled per key block over the inverted index. For group g, position t and
// an attended key j (scaled by the caller's weight w and the proxy scale s):
//   p_j  = (1/G) sum_h exp(scale q_h . k_j - lse_h(t))      main, from the forward's LSE
//   px_j = exp(s q_idx(t) . k_idx_j - lse_px(t))           proxy
//   dZ_j = w s (px_j - p_j)
//   dq_idx(t) = sum_j dZ_j k_idx_j;  dk_idx_j = sum_(t,g) dZ_j q_idx(t)
// Passes (all per work item of the backward's canonical plan, so every sum runs
// in a fixed order and the result is bitwise reproducible):
//   k_kl_lse_part, k_kl_lse_combine  the proxy LSE: per (t, slot) the max and the
//               sum of exponentials of the proxy logits over the block's attended
//               keys (MFMA), then merged over the slots;
//   k_kl_dz     per 128-row tile (positions x G heads): S^T = K Q^T and the proxy
//               Z^T = K_idx Q_idx^T on MFMA, p averaged over the G heads of a
//               position by lane exchanges, dZ rows to the workspace in bf16
//               (G <= 2); k_kl_dz_shared for G >= 4: each wave its own 32 rows,
//               S = Q K^T so the head average is in-lane, the proxy logits once
//               per position in the same layout, no workgroup barrier;
//   k_kl_grad   per chunk of 32 entries: dq_idx^T = K_idx^T dZ^T (one record per
//               (t, slot)) and dk_idx += dZ^T Q_idx (per item), on MFMA;
//   k_kl_dq_sum, k_kl_dk_reduce  the sums over slots, and over items and groups
//               (one index key head serves every group).
#include "msa_device.hpp"
#include "msa_internal.hpp"

namespace msa {

// One step of the xor butterfly that sums x over aligned groups of lanes, through
// the DPP lane crossbar instead of LDS permutes. After the steps for 1 and 2 (quad
// permutations) every quad holds its sum; the half-row mirror then pairs each lane
// with the other quad of its 8 lanes and the row mirror with the other 8 of its 16,
// so each lane adds the same two partial sums, in the same order (its own first),
// as the xor-4 and xor-8 steps would.
template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
    return x + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
// Sum of the 32 values of v over each aligned group of G lanes (G a power of two <= 32),
// left in every lane of the group: the xor butterfly 1, 2, ..., G/2.
__device__ __forceinline__ void group_sum32(f32x16 (&v)[2], int G) {
    if (G >= 2)
#pragma unroll
        for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
            for (int i = 0; i < 16; ++i) v[m2][i] = dpp_add<0xB1>(v[m2][i]);  // quad_perm [1,0,3,2]: xor 1
    if (G >= 4)
#pragma unroll
        for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
            for (int i = 0; i < 16; ++i) v[m2][i] = dpp_add<0x4E>(v[m2][i]);  // quad_perm [2,3,0,1]: xor 2
    if (G >= 8)
#pragma unroll
        for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
            for (int i = 0; i < 16; ++i) v[m2][i] = dpp_add<0x141>(v[m2][i]);  // row_half_mirror
    if (G >= 16)
#pragma unroll
        for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
            for (int i = 0; i < 16; ++i) v[m2][i] = dpp_add<0x140>(v[m2][i]);  // row_mirror
    if (G >= 32)
#pragma unroll
        for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
            for (int i = 0; i < 16; ++i) v[m2][i] += __shfl_xor(v[m2][i], 16, 64);
}

typedef __attribute__((address_space(3))) bf16x4* kl_lds_bf16x4_ptr;

constexpr int kKlMaxItemEntries = kRowTilesPerItem * kBlock;  // entries of one item when G = 1
constexpr int kKlChunk = 32;                                  // entries per k_kl_grad step

// Row-major 128-element rows with chunk ch (8 elements) of row r at slot ch ^ rsw(r):
// rows read together by one transposing load fall on distinct slots.
__device__ __forceinline__ int kl_rsw(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int kl_row_off(int row, int ch) { return row * kDim + ((ch ^ kl_rsw(row)) << 3); }

// ds_read_b64_tr_b16 on such a tile: inside each 16-lane group, lane li addresses
// row r0 + li/4, columns c0 + 4(li%4) .. +3, and receives column c0 + li of rows
// r0 .. r0+3. c0 is a multiple of 16.
__device__ __forceinline__ bf16x4 kl_tr4(const __bf16* tile, int r0, int c0, int li) {
    const int row = r0 + (li >> 2), col = c0 + 4 * (li & 3);
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((kl_lds_bf16x4_ptr)(tile + kl_row_off(row, col >> 3) + (col & 7)));
}
__device__ __forceinline__ bf16x8 kl_cat8(bf16x4 a, bf16x4 b) {
    return (bf16x8){a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// The work item's tile: the last index with item_off[tile] <= item.
__device__ __forceinline__ int kl_item_tile(const int32_t* __restrict__ item_off, int n_tiles, int item) {
    int lo = 0, hi = n_tiles;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (item_off[mid] <= item) lo = mid;
        else hi = mid;
    }
    return lo;
}

// A 128 x 128 tile with row stride `stride` into LDS at swz_chunk_offset.
__device__ __forceinline__ void kl_stage_rows(const __bf16* __restrict__ src, int stride, __bf16* dst, int tid) {
    const int row0 = tid >> 4, ch = tid & 15;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = row0 + 16 * i;
        *(uint4*)(dst + swz_chunk_offset(row, ch)) = *(const uint4*)(src + (size_t)row * stride + ch * 8);
    }
}

// Proxy logits of an item's entries, 128 at a time (lane l32 of wave w holds entry
// 32 w + l32, keys mt*32 + mfma32_row(i, h)): per entry the max of the logits
// over the block's attended keys and the sum of 2^(logit - max), both in log2
// units, to the (t, slot) record.
__global__ __launch_bounds__(256, 4) void k_kl_lse_part(
    const __bf16* __restrict__ q_idx, const __bf16* __restrict__ k_idx, const int32_t* __restrict__ off,
    const int32_t* __restrict__ item_off, const int32_t* __restrict__ entries, float2* __restrict__ lse_part,
    int N, int Hkv, int gshift, int nblk, int top_k, int n_tiles, float c_idx) {
    __shared__ __attribute__((aligned(16))) __bf16 kis[kBlock * kDim];  // K_idx[key][dim], swizzled
    __shared__ int32_t ent[kKlMaxItemEntries];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
    const int P = kBlock >> gshift;
    const int total_items = item_off[n_tiles];

    for (int item = blockIdx.x; item < total_items; item += gridDim.x) {
        const int tile = kl_item_tile(item_off, n_tiles, item);
        const int c = tile % nblk, bg = tile / nblk, g = bg % Hkv, b = bg / Hkv;
        const int e0 = off[tile], npos = off[tile + 1] - e0;
        const int n_rt = (npos + P - 1) / P;
        const int rt0 = (item - item_off[tile]) * kRowTilesPerItem;
        const int rt1 = min(rt0 + kRowTilesPerItem, n_rt);
        const int ne = min(rt1 * P, npos) - rt0 * P;
        const int ebase = e0 + rt0 * P;

        __syncthreads();
        for (int i = tid; i < ne; i += 256) ent[i] = entries[ebase + i];
        kl_stage_rows(k_idx + ((size_t)b * N + (size_t)c * kBlock) * kDim, kDim, kis, tid);
        __syncthreads();

        for (int cb = 0; cb < ne; cb += kBlock) {
            const int li = cb + wave * 32 + l32;
            const bool valid = li < ne;
            const int en = ent[valid ? li : 0], t = en >> 8;
            bf16x8 qf[8];
            const __bf16* qirow = q_idx + (((size_t)b * N + t) * Hkv + g) * kDim + 8 * h;
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) qf[kk] = *(const bf16x8*)(qirow + kk * 16);
            // the keys in two halves of 64 (half the accumulators live, so four workgroups fit a
            // CU), merged as a running max and sum
            const int lim = ((t >> 7) == c ? t - c * kBlock : kBlock - 1);
            float m = -INFINITY, l = 0.0f;
#pragma unroll
            for (int mh = 0; mh < 2; ++mh) {
                asm volatile("" ::: "memory");
                f32x16 zacc[2];
#pragma unroll
                for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
                    for (int i = 0; i < 16; ++i) zacc[m2][i] = 0.0f;
#pragma unroll
                for (int kk = 0; kk < 8; ++kk)
#pragma unroll
                    for (int m2 = 0; m2 < 2; ++m2) {
                        const bf16x8 a =
                            *(const bf16x8*)(kis + swz_chunk_offset((2 * mh + m2) * 32 + l32, 2 * kk + h));
                        zacc[m2] = mfma32(a, qf[kk], zacc[m2]);
                    }
                float mx = -INFINITY;
#pragma unroll
                for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const float zz =
                            (2 * mh + m2) * 32 + mfma32_row(i, h) <= lim ? zacc[m2][i] * c_idx : -INFINITY;
                        zacc[m2][i] = zz;
                        mx = fmaxf(mx, zz);
                    }
                mx = wave_max_xor32(mx);  // half 0 holds key 128 c <= t, always attended: finite from there on
                const float mnew = fmaxf(m, mx);
                float lh = 0.0f;
#pragma unroll
                for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
                    for (int i = 0; i < 16; ++i) lh += __builtin_amdgcn_exp2f(zacc[m2][i] - mnew);
                l = (mh == 0 ? 0.0f : l * __builtin_amdgcn_exp2f(m - mnew)) + wave_sum_xor32(lh);
                m = mnew;
            }
            if (valid && h == 0)
                lse_part[(((size_t)b * Hkv + g) * N + t) * top_k + (en & 255)] = make_float2(m, l);
        }
    }
}

// lse_px[b, g, t] (natural log) from the records of the slots whose block is attended:
// 16 lanes per row, each taking every 16th slot, merged by lane exchanges.
__global__ __launch_bounds__(256) void k_kl_lse_combine(const int32_t* __restrict__ block_idx,
                                                        const float2* __restrict__ lse_part,
                                                        float* __restrict__ lse_px, int N, int top_k,
                                                        long long rows) {
    const long long row = (long long)blockIdx.x * 16 + (threadIdx.x >> 4);  // (b, g, t)
    const int sl = threadIdx.x & 15;
    const bool live = row < rows;
    const int t = live ? (int)(row % N) : 0;
    float M = -INFINITY, L = 0.0f;
    for (int s = sl; live && s < top_k; s += 16) {
        const int c = block_idx[row * top_k + s];
        if (c < 0 || c > (t >> 7)) continue;
        const float2 r = lse_part[row * top_k + s];
        const float m2 = fmaxf(M, r.x);
        L = L * __builtin_amdgcn_exp2f(M - m2) + r.y * __builtin_amdgcn_exp2f(r.x - m2);
        M = m2;
    }
#pragma unroll
    for (int sft = 1; sft < 16; sft <<= 1) {
        const float Mo = __shfl_xor(M, sft, 64), Lo = __shfl_xor(L, sft, 64);
        const float m2 = fmaxf(M, Mo);
        L = (M == -INFINITY ? 0.0f : L * __builtin_amdgcn_exp2f(M - m2)) +
            (Mo == -INFINITY ? 0.0f : Lo * __builtin_amdgcn_exp2f(Mo - m2));
        M = m2;
    }
    if (live && sl == 0) lse_px[row] = L > 0.0f ? (M + __log2f(L)) * 0.69314718055994531f : -INFINITY;
}

__global__ __launch_bounds__(256, 2) void k_kl_dz(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ q_idx,
    const __bf16* __restrict__ k_idx, const float* __restrict__ lse, const float* __restrict__ lse_px,
    const int32_t* __restrict__ off, const int32_t* __restrict__ item_off, const int32_t* __restrict__ entries,
    __bf16* __restrict__ dz, int N, int Hq, int Hkv, int gshift, int nblk, int n_tiles, float c_main,
    float c_idx, float dz_scale) {
    __shared__ __attribute__((aligned(16))) __bf16 ks[kBlock * kDim];   // K[key][dim], swizzled
    __shared__ __attribute__((aligned(16))) __bf16 kis[kBlock * kDim];  // K_idx[key][dim], swizzled
    __shared__ int32_t ent[kKlMaxItemEntries];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
    const int G = 1 << gshift;
    const int P = kBlock >> gshift;  // positions per 128-row tile
    const int r = wave * 32 + l32;   // this lane's row: position slot r / G, head r % G
    const int pslot = r >> gshift, hh = r & (G - 1);
    const float log2e = 1.4426950408889634f, invG = 1.0f / (float)G;
    const int total_items = item_off[n_tiles];

    for (int item = blockIdx.x; item < total_items; item += gridDim.x) {
        const int tile = kl_item_tile(item_off, n_tiles, item);
        const int c = tile % nblk, bg = tile / nblk, g = bg % Hkv, b = bg / Hkv;
        const int e0 = off[tile], npos = off[tile + 1] - e0;
        const int n_rt = (npos + P - 1) / P;
        const int rt0 = (item - item_off[tile]) * kRowTilesPerItem;
        const int rt1 = min(rt0 + kRowTilesPerItem, n_rt);
        const int ne = min(rt1 * P, npos) - rt0 * P;
        const int ebase = e0 + rt0 * P;  // entry index of this item's first entry

        __syncthreads();  // the previous item's LDS reads are done
        for (int i = tid; i < ne; i += 256) ent[i] = entries[ebase + i];
        kl_stage_rows(k + (((size_t)b * N + (size_t)c * kBlock) * Hkv + g) * kDim, Hkv * kDim, ks, tid);
        kl_stage_rows(k_idx + ((size_t)b * N + (size_t)c * kBlock) * kDim, kDim, kis, tid);
        __syncthreads();

        // Rows of tile rt: this lane's entry and its query rows. Rows past the item's
        // entries reuse a valid row and are never written. The next tile's rows are
        // loaded while the current one computes.
        const int head = g * G + hh;
        auto row_t = [&](int rt, bool& valid) {
            const int li = (rt - rt0) * P + pslot;
            valid = li < ne;
            return ent[valid ? li : 0] >> 8;
        };
        auto load_q = [&](int t, bf16x8 (&buf)[8]) {
            const __bf16* row = q + (((size_t)b * N + t) * Hq + head) * kDim + 8 * h;
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) buf[kk] = *(const bf16x8*)(row + kk * 16);
        };
        auto load_qi = [&](int t, bf16x8 (&buf)[8]) {
            const __bf16* row = q_idx + (((size_t)b * N + t) * Hkv + g) * kDim + 8 * h;
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) buf[kk] = *(const bf16x8*)(row + kk * 16);
        };
        bool valid;
        int t = row_t(rt0, valid);
        bf16x8 qf[8], qif[8];
        load_q(t, qf);
        load_qi(t, qif);
        for (int rt = rt0; rt < rt1; ++rt) {
            const int li = (rt - rt0) * P + pslot;
            bool nvalid = false;
            const int tn = rt + 1 < rt1 ? row_t(rt + 1, nvalid) : t;
            const float lm = lse[((size_t)b * Hq + head) * N + t] * log2e;
            const float lp = lse_px[((size_t)b * Hkv + g) * N + t] * log2e;
            const int lim = ((t >> 7) == c ? t - c * kBlock : kBlock - 1);  // keys <= lim are attended
            // Every step is elementwise in the key (P uses the forward's LSE), so the 128 keys
            // go in two halves of 64 and only half of the accumulators are live.
#pragma unroll 1
            for (int mh = 0; mh < 2; ++mh) {
                asm volatile("" ::: "memory");
                f32x16 sacc[2], zacc[2];
#pragma unroll
                for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
                    for (int i = 0; i < 16; ++i) sacc[m2][i] = zacc[m2][i] = 0.0f;
#pragma unroll
                for (int kk = 0; kk < 8; ++kk)
#pragma unroll
                    for (int m2 = 0; m2 < 2; ++m2) {
                        const bf16x8 a = *(const bf16x8*)(ks + swz_chunk_offset((2 * mh + m2) * 32 + l32, 2 * kk + h));
                        sacc[m2] = mfma32(a, qf[kk], sacc[m2]);
                    }
                if (mh == 1 && rt + 1 < rt1) load_q(tn, qf);
#pragma unroll
                for (int kk = 0; kk < 8; ++kk)
#pragma unroll
                    for (int m2 = 0; m2 < 2; ++m2) {
                        const bf16x8 a = *(const bf16x8*)(kis + swz_chunk_offset((2 * mh + m2) * 32 + l32, 2 * kk + h));
                        zacc[m2] = mfma32(a, qif[kk], zacc[m2]);
                    }
                if (mh == 1 && rt + 1 < rt1) load_qi(tn, qif);
                // main probabilities, averaged over the position's G rows (lanes l32 ^ 1 .. G/2)
#pragma unroll
                for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int key = (2 * mh + m2) * 32 + mfma32_row(i, h);
                        sacc[m2][i] =
                            key <= lim ? __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[m2][i], c_main, -lm)) : 0.0f;
                    }
                group_sum32(sacc, G);
                if (valid && hh == 0) {
                    __bf16* dst = dz + (size_t)(ebase + li) * kBlock;
#pragma unroll
                    for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
                        for (int i0 = 0; i0 < 16; i0 += 4) {
                            const int k0 = (2 * mh + m2) * 32 + mfma32_row(i0, h);
                            bf16x4 w;
#pragma unroll
                            for (int j = 0; j < 4; ++j) {
                                const float px = k0 + j <= lim ? __builtin_amdgcn_exp2f(
                                                                     __builtin_fmaf(zacc[m2][i0 + j], c_idx, -lp))
                                                               : 0.0f;
                                w[j] = (__bf16)(dz_scale * (px - sacc[m2][i0 + j] * invG));
                            }
                            *(bf16x4*)(dst + k0) = w;
                        }
                }
            }
            t = tn;
            valid = nvalid;
        }
    }
}

// The same result for G >= 4 with the proxy logits computed once per position and
// no workgroup barrier inside an item: every wave finishes its own 32 head rows
// (32 / G positions) alone.
//  - S = Q K^T on v_mfma_f32_16x16x32_bf16 with the query rows as the A operand,
//    so a lane holds one key and four consecutive head rows per 16-row tile; the G
//    rows of a position are then in-lane (G = 4) or at most two lane exchanges away,
//    and p-bar (position, key) ends in the lanes of that key.
//  - The wave's proxy logits Z = Q_idx K_idx^T use the same layout: row 4 g + i of
//    the 16-row proxy tile carries the position of head row 16 i + 4 g (i < 2), so
//    dZ = w s (px - p-bar) is formed in-lane. A 16-row proxy tile holds 32 / G <= 8
//    positions: the unused rows are the price of needing no exchange.
//  - The rows' LSE * log2 e, causal limits and proxy LSE go through a small
//    per-wave LDS block (written and read by the same wave).
constexpr int kKlSharedPos = 32;  // positions of a 128-row tile when G >= 4

__global__ __launch_bounds__(256, 2) void k_kl_dz_shared(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ q_idx,
    const __bf16* __restrict__ k_idx, const float* __restrict__ lse, const float* __restrict__ lse_px,
    const int32_t* __restrict__ off, const int32_t* __restrict__ item_off, const int32_t* __restrict__ entries,
    __bf16* __restrict__ dz, int N, int Hq, int Hkv, int gshift, int nblk, int n_tiles, float c_main,
    float c_idx, float dz_scale) {
    __shared__ __attribute__((aligned(16))) __bf16 ks[kBlock * kDim];   // K[key][dim], swizzled
    __shared__ __attribute__((aligned(16))) __bf16 kis[kBlock * kDim];  // K_idx[key][dim], swizzled
    __shared__ int32_t ent[kRowTilesPerItem * kKlSharedPos];
    __shared__ __attribute__((aligned(16))) float rterm[4][3][32];  // per wave and row: LSE*log2e, limit, proxy LSE*log2e

    const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int G = 1 << gshift;
    const int P = kBlock >> gshift;  // <= 32
    const float log2e = 1.4426950408889634f, invG = 1.0f / (float)G;
    // head row (of the 128-row tile) whose position the proxy tile's A row l16 carries
    const int zrow = 32 * wave + 16 * ((l16 & 3) < 2 ? (l16 & 3) : 0) + 4 * (l16 >> 2);
    const int total_items = item_off[n_tiles];

    for (int item = blockIdx.x; item < total_items; item += gridDim.x) {
        const int tile = kl_item_tile(item_off, n_tiles, item);
        const int c = tile % nblk, bg = tile / nblk, g = bg % Hkv, b = bg / Hkv;
        const int e0 = off[tile], npos = off[tile + 1] - e0;
        const int n_rt = (npos + P - 1) / P;
        const int rt0 = (item - item_off[tile]) * kRowTilesPerItem;
        const int rt1 = min(rt0 + kRowTilesPerItem, n_rt);
        const int ne = min(rt1 * P, npos) - rt0 * P;
        const int ebase = e0 + rt0 * P;

        __syncthreads();  // the previous item's LDS reads are done
        for (int i = tid; i < ne; i += 256) ent[i] = entries[ebase + i];
        kl_stage_rows(k + (((size_t)b * N + (size_t)c * kBlock) * Hkv + g) * kDim, Hkv * kDim, ks, tid);
        kl_stage_rows(k_idx + ((size_t)b * N + (size_t)c * kBlock) * kDim, kDim, kis, tid);
        __syncthreads();

        const int head0 = g * G;
        // query position of head row r (0..127) of row tile rt; rows past the item's
        // entries read entry 0 and are never written
        auto pos_of = [&](int rt, int r, bool& valid) {
            const int li = (rt - rt0) * P + (r >> gshift);
            valid = li < ne;
            return ent[valid ? li : 0] >> 8;
        };
        // A operands: head rows 32 wave + 16 mt + l16 (S) and the proxy rows (Z), dims 32 kk + 8 g4 .. +7
        bf16x8 qf[2][4], qif[4];
        auto load_q = [&](int rt) {
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                const int r = 32 * wave + 16 * mt + l16;
                bool v;
                const int t = pos_of(rt, r, v);
                const __bf16* p = q + (((size_t)b * N + t) * Hq + head0 + (r & (G - 1))) * kDim + 8 * g4;
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) qf[mt][kk] = *(const bf16x8*)(p + 32 * kk);
            }
        };
        auto load_qi = [&](int rt) {
            bool v;
            const int t = pos_of(rt, zrow, v);
            const __bf16* p = q_idx + (((size_t)b * N + t) * Hkv + g) * kDim + 8 * g4;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) qif[kk] = *(const bf16x8*)(p + 32 * kk);
        };
        load_q(rt0);
        load_qi(rt0);
        for (int rt = rt0; rt < rt1; ++rt) {
            // the K and K_idx operands are read from LDS in every row tile (not hoisted out of
            // the loop into registers)
            asm volatile("" ::: "memory");
            if (lane < 32) {  // the row terms of head row 32 wave + lane
                const int r = 32 * wave + lane;
                bool v;
                const int t = pos_of(rt, r, v);
                rterm[wave][0][lane] = lse[((size_t)b * Hq + head0 + (r & (G - 1))) * N + t] * log2e;
                rterm[wave][1][lane] = __int_as_float((t >> 7) == c ? t - c * kBlock : kBlock - 1);
                rterm[wave][2][lane] = lse_px[((size_t)b * Hkv + g) * N + t] * log2e;
            }
            // S: acc[mt][nt] register i = row 16 mt + 4 g4 + i (of the wave's 32), key 16 nt + l16
            f32x4 acc[2][8];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int nt = 0; nt < 8; ++nt) acc[mt][nt] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                for (int nt = 0; nt < 8; ++nt) {
                    const bf16x8 bk = *(const bf16x8*)(ks + swz_chunk_offset(16 * nt + l16, 4 * kk + g4));
#pragma unroll
                    for (int mt = 0; mt < 2; ++mt) acc[mt][nt] = mfma16(qf[mt][kk], bk, acc[mt][nt]);
                }
            if (rt + 1 < rt1) load_q(rt + 1);
            // P = 2^(s scale log2e - LSE log2e), causal-masked on the diagonal block
            f32x4 lm4[2], lim4[2];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                lm4[mt] = *(const f32x4*)&rterm[wave][0][16 * mt + 4 * g4];
                lim4[mt] = *(const f32x4*)&rterm[wave][1][16 * mt + 4 * g4];
            }
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int nt = 0; nt < 8; ++nt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int key = 16 * nt + l16;
                        acc[mt][nt][i] = key <= __float_as_int(lim4[mt][i])
                                             ? __builtin_amdgcn_exp2f(__builtin_fmaf(acc[mt][nt][i], c_main, -lm4[mt][i]))
                                             : 0.0f;
                    }
            // p-bar: the sum over a position's G head rows (in-lane for four, then across the
            // lanes 16 and 32 apart, then across the two row tiles), over G
            float pb[2][8];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int nt = 0; nt < 8; ++nt)
                    pb[mt][nt] = (acc[mt][nt][0] + acc[mt][nt][1]) + (acc[mt][nt][2] + acc[mt][nt][3]);
            if (G >= 8)
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int nt = 0; nt < 8; ++nt) pb[mt][nt] += __shfl_xor(pb[mt][nt], 16, 64);
            if (G >= 16)
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int nt = 0; nt < 8; ++nt) pb[mt][nt] += __shfl_xor(pb[mt][nt], 32, 64);
            if (G >= 32)
#pragma unroll
                for (int nt = 0; nt < 8; ++nt) pb[0][nt] = pb[1][nt] = pb[0][nt] + pb[1][nt];
            // Z: z[nt] register i = proxy row 4 g4 + i, i.e. the position of head row 16 i + 4 g4
            f32x4 z[8];
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) z[nt] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                for (int nt = 0; nt < 8; ++nt) {
                    const bf16x8 bk = *(const bf16x8*)(kis + swz_chunk_offset(16 * nt + l16, 4 * kk + g4));
                    z[nt] = mfma16(qif[kk], bk, z[nt]);
                }
            if (rt + 1 < rt1) load_qi(rt + 1);
            // dZ rows, written by the lane group that holds a position's first head row
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int r0 = 32 * wave + 16 * i + 4 * g4;
                bool v;
                (void)pos_of(rt, r0, v);
                if (v && (r0 & (G - 1)) == 0) {
                    const float lp = rterm[wave][2][16 * i + 4 * g4];
                    const int limz = __float_as_int(rterm[wave][1][16 * i + 4 * g4]);
                    __bf16* dst = dz + (size_t)(ebase + (rt - rt0) * P + (r0 >> gshift)) * kBlock;
#pragma unroll
                    for (int nt = 0; nt < 8; ++nt) {
                        const int key = 16 * nt + l16;
                        const float px =
                            key <= limz ? __builtin_amdgcn_exp2f(__builtin_fmaf(z[nt][i], c_idx, -lp)) : 0.0f;
                        dst[key] = (__bf16)(dz_scale * (px - pb[i][nt] * invG));
                    }
                }
            }
        }
    }
}

__global__ __launch_bounds__(256, 2) void k_kl_grad(
    const __bf16* __restrict__ q_idx, const __bf16* __restrict__ k_idx, const __bf16* __restrict__ dz,
    const int32_t* __restrict__ off, const int32_t* __restrict__ item_off, const int32_t* __restrict__ entries,
    __bf16* __restrict__ dq_part, float* __restrict__ dk_part, int N, int Hkv, int gshift, int nblk, int top_k,
    int n_tiles) {
    __shared__ __attribute__((aligned(16))) __bf16 kit[kDim * kBlock];   // K_idx^T[dim][key], swizzled
    __shared__ __attribute__((aligned(16))) __bf16 dzs[kKlChunk * kDim];  // dZ rows [entry][key]
    __shared__ __attribute__((aligned(16))) __bf16 qis[kKlChunk * kDim];  // q_idx rows [entry][dim]
    __shared__ int32_t ent[kKlMaxItemEntries];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
    const int li16 = lane & 15, hi16 = (lane >> 4) & 1;  // lane inside its 16-lane group, and which half of 32
    const int P = kBlock >> gshift;
    const int total_items = item_off[n_tiles];

    for (int item = blockIdx.x; item < total_items; item += gridDim.x) {
        const int tile = kl_item_tile(item_off, n_tiles, item);
        const int c = tile % nblk, bg = tile / nblk, g = bg % Hkv, b = bg / Hkv;
        const int e0 = off[tile], npos = off[tile + 1] - e0;
        const int n_rt = (npos + P - 1) / P;
        const int rt0 = (item - item_off[tile]) * kRowTilesPerItem;
        const int rt1 = min(rt0 + kRowTilesPerItem, n_rt);
        const int ne = min(rt1 * P, npos) - rt0 * P;
        const int ebase = e0 + rt0 * P;

        __syncthreads();
        for (int i = tid; i < ne; i += 256) ent[i] = entries[ebase + i];
        {
            // K_idx transposed: thread takes keys 4 key0 + 64 i .. +3, dims 8 ch .. +7
            const __bf16* kb = k_idx + ((size_t)b * N + (size_t)c * kBlock) * kDim;
            const int key0 = tid >> 4, ch = tid & 15;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int kq = 4 * key0 + 64 * i;
                bf16x8 rows[4];
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) rows[rr] = *(const bf16x8*)(kb + (size_t)(kq + rr) * kDim + ch * 8);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    bf16x4 w;
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) w[rr] = rows[rr][e];
                    *(bf16x4*)(kit + swz_chunk_offset(ch * 8 + e, kq >> 3) + (kq & 7)) = w;
                }
            }
        }
        f32x16 dk[4];  // dK_idx[key 32 wave + row][dim 32 dt + l32]
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int i = 0; i < 16; ++i) dk[dt][i] = 0.0f;

        // A chunk's dZ and proxy rows (thread: rows tid / 16 and + 16, chunk tid % 16) are
        // loaded into registers one chunk ahead and stored into LDS at the chunk's start.
        u32x4 pz[2], pq[2];
        auto load_chunk = [&](int cb0) {
#pragma unroll
            for (int it = 0; it < 2; ++it) {
                const int row = (tid >> 4) + 16 * it, ch = tid & 15;
                pz[it] = (u32x4){0u, 0u, 0u, 0u};
                pq[it] = (u32x4){0u, 0u, 0u, 0u};
                if (cb0 + row < ne) {
                    const int t = ent[cb0 + row] >> 8;
                    pz[it] = *(const u32x4*)(dz + (size_t)(ebase + cb0 + row) * kBlock + ch * 8);
                    pq[it] = *(const u32x4*)(q_idx + (((size_t)b * N + t) * Hkv + g) * kDim + ch * 8);
                }
            }
        };
        __syncthreads();  // kit and ent are written
        load_chunk(0);
        for (int cb = 0; cb < ne; cb += kKlChunk) {
            if (cb > 0) __syncthreads();  // the previous chunk's reads are done
#pragma unroll
            for (int it = 0; it < 2; ++it) {
                const int row = (tid >> 4) + 16 * it, ch = tid & 15;
                *(u32x4*)(dzs + kl_row_off(row, ch)) = pz[it];
                *(u32x4*)(qis + kl_row_off(row, ch)) = pq[it];
            }
            if (cb + kKlChunk < ne) load_chunk(cb + kKlChunk);
            __syncthreads();
            // dq_idx^T for dims 32 wave .. +31 and the chunk's 32 entries, over the 128 keys
            {
                f32x16 acc;
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
#pragma unroll
                for (int kk = 0; kk < 8; ++kk) {
                    const bf16x8 a = *(const bf16x8*)(kit + swz_chunk_offset(wave * 32 + l32, 2 * kk + h));
                    const bf16x8 bb = *(const bf16x8*)(dzs + kl_row_off(l32, 2 * kk + h));
                    acc = mfma32(a, bb, acc);
                }
                if (cb + l32 < ne) {
                    const int en = ent[cb + l32], t = en >> 8, slot = en & 255;
                    __bf16* dst = dq_part + ((((size_t)b * Hkv + g) * N + t) * top_k + slot) * kDim + wave * 32;
#pragma unroll
                    for (int i0 = 0; i0 < 16; i0 += 4) {
                        const bf16x4 w = {(__bf16)acc[i0], (__bf16)acc[i0 + 1], (__bf16)acc[i0 + 2], (__bf16)acc[i0 + 3]};
                        *(bf16x4*)(dst + mfma32_row(i0, h)) = w;
                    }
                }
            }
            // dk_idx += dZ^T Q_idx over the chunk's entries (rows of both tiles, read transposed)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const int r0 = 16 * kk + 8 * h;
                const bf16x8 a = kl_cat8(kl_tr4(dzs, r0, wave * 32 + 16 * hi16, li16),
                                         kl_tr4(dzs, r0 + 4, wave * 32 + 16 * hi16, li16));
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) {
                    const bf16x8 bb = kl_cat8(kl_tr4(qis, r0, dt * 32 + 16 * hi16, li16),
                                              kl_tr4(qis, r0 + 4, dt * 32 + 16 * hi16, li16));
                    dk[dt] = mfma32(a, bb, dk[dt]);
                }
            }
        }
        float* dst = dk_part + (size_t)item * kBlock * kDim;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                dst[(size_t)(wave * 32 + mfma32_row(i, h)) * kDim + dt * 32 + l32] = dk[dt][i];
    }
}

// dq_idx[b, t, g] = sum of the (t, slot) records over the slots whose block is attended.
__global__ __launch_bounds__(256) void k_kl_dq_sum(const int32_t* __restrict__ block_idx,
                                                   const __bf16* __restrict__ dq_part, __bf16* __restrict__ dq_idx,
                                                   int N, int Hkv, int top_k, long long rows) {
    const long long row = (long long)blockIdx.x * 16 + (threadIdx.x >> 4);  // (b, g, t)
    if (row >= rows) return;
    const int ch = threadIdx.x & 15;
    const int t = (int)(row % N);
    const long long bg = row / N;
    const int g = (int)(bg % Hkv);
    const long long b = bg / Hkv;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    // eight slots at a time: their block indices and records are all requested before any
    // is used (a record of a slot that is not attended is read but not added), then added
    // in slot order
    for (int s0 = 0; s0 < top_k; s0 += 8) {
        int c[8];
        bf16x8 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int s = s0 + u < top_k ? s0 + u : top_k - 1;
            c[u] = block_idx[row * top_k + s];
            v[u] = *(const bf16x8*)(dq_part + (row * top_k + s) * kDim + ch * 8);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (s0 + u < top_k && c[u] >= 0 && c[u] <= (t >> 7))
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] += (float)v[u][e];
    }
    bf16x8 out;
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = (__bf16)acc[e];
    *(bf16x8*)(dq_idx + ((b * N + t) * Hkv + g) * kDim + ch * 8) = out;
}

// dk_idx of key block c = the partials of every item of the tiles (b, g, c), over g.
__global__ __launch_bounds__(256) void k_kl_dk_reduce(const float* __restrict__ dk_part,
                                                      const int32_t* __restrict__ item_off, __bf16* __restrict__ dk_idx,
                                                      int N, int Hkv, int nblk) {
    const int c = blockIdx.x % nblk, b = blockIdx.x / nblk;
    const size_t part = (size_t)kBlock * kDim;
    // a quarter of the block's 128 x 128 values per workgroup (blockIdx.y)
    const int e_end = (blockIdx.y + 1) * (kBlock * kDim / 16);
    for (int e = blockIdx.y * (kBlock * kDim / 16) + threadIdx.x; e < e_end; e += 256) {
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int g = 0; g < Hkv; ++g) {
            const int tile = (b * Hkv + g) * nblk + c;
            const int i0 = item_off[tile], i1 = item_off[tile + 1];
            int it = i0;
            // four items' partials requested at once, added in item order
            for (; it + 4 <= i1; it += 4) {
                f32x4 x[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) x[u] = *(const f32x4*)(dk_part + (size_t)(it + u) * part + e * 4);
#pragma unroll
                for (int u = 0; u < 4; ++u) acc += x[u];
            }
            for (; it < i1; ++it) acc += *(const f32x4*)(dk_part + (size_t)it * part + e * 4);
        }
        const bf16x4 w = {(__bf16)acc[0], (__bf16)acc[1], (__bf16)acc[2], (__bf16)acc[3]};
        *(bf16x4*)(dk_idx + ((size_t)b * N + (size_t)c * kBlock) * kDim + e * 4) = w;
    }
}

// ---------------------------------------------------------------------------
hipError_t launch_kl_lse(const void* q_idx, const void* k_idx, const int32_t* block_idx, const SparseWs& plan,
                         float2* lse_part, float* lse_px, float index_scale, const Dims& d, hipStream_t stream) {
    const int n = d.B * d.Hkv * d.nblk;
    hipLaunchKernelGGL(k_kl_lse_part, dim3(4 * device_cu_count()), dim3(256), 0, stream, (const __bf16*)q_idx,
                       (const __bf16*)k_idx, plan.off, plan.item_off, plan.entries, lse_part, d.N, d.Hkv, d.gshift,
                       d.nblk, d.top_k, n, index_scale * 1.4426950408889634f);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long long rows = (long long)d.B * d.Hkv * d.N;
    hipLaunchKernelGGL(k_kl_lse_combine, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, stream, block_idx,
                       lse_part, lse_px, d.N, d.top_k, rows);
    return hipGetLastError();
}

hipError_t launch_kl_dz(const void* q, const void* k, const void* q_idx, const void* k_idx, const float* lse,
                        const float* lse_px, const SparseWs& plan, void* dz, float index_scale, float kl_weight,
                        const Dims& d, hipStream_t stream) {
    const int n = d.B * d.Hkv * d.nblk;
    const float log2e = 1.4426950408889634f;
    auto kernel = d.G >= 4 ? k_kl_dz_shared : k_kl_dz;  // G >= 4: proxy logits once per position
    hipLaunchKernelGGL(kernel, dim3(2 * device_cu_count()), dim3(256), 0, stream, (const __bf16*)q,
                       (const __bf16*)k, (const __bf16*)q_idx, (const __bf16*)k_idx, lse, lse_px, plan.off,
                       plan.item_off, plan.entries, (__bf16*)dz, d.N, d.Hq, d.Hkv, d.gshift, d.nblk, n,
                       d.scale * log2e, index_scale * log2e, kl_weight * index_scale);
    return hipGetLastError();
}

hipError_t launch_kl_grad(const void* q_idx, const void* k_idx, const void* dz, const SparseWs& plan, void* dq_part,
                          float* dk_part, const Dims& d, hipStream_t stream) {
    const int n = d.B * d.Hkv * d.nblk;
    hipLaunchKernelGGL(k_kl_grad, dim3(2 * device_cu_count()), dim3(256), 0, stream, (const __bf16*)q_idx,
                       (const __bf16*)k_idx, (const __bf16*)dz, plan.off, plan.item_off, plan.entries,
                       (__bf16*)dq_part, dk_part, d.N, d.Hkv, d.gshift, d.nblk, d.top_k, n);
    return hipGetLastError();
}

hipError_t launch_kl_reduce(const int32_t* block_idx, const void* dq_part, const float* dk_part, const SparseWs& plan,
                            void* dq_idx, void* dk_idx, const Dims& d, hipStream_t stream) {
    const long long rows = (long long)d.B * d.Hkv * d.N;
    hipLaunchKernelGGL(k_kl_dq_sum, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, stream, block_idx,
                       (const __bf16*)dq_part, (__bf16*)dq_idx, d.N, d.Hkv, d.top_k, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_kl_dk_reduce, dim3((unsigned)(d.B * d.nblk), 4), dim3(256), 0, stream, dk_part, plan.item_off,
                       (__bf16*)dk_idx, d.N, d.Hkv, d.nblk);
    return hipGetLastError();
}

}  // namespace msa
