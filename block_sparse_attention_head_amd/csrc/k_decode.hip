// Decode step: one new query per sequence against its KV cache.
//
// [MSA summary] "Why long context is the bottleneck": decoding adds one token
// at a time against a cache that grows with the context; "Architecture" and
// "Experimental results": the same index branch and selection (k blocks of
// 128, local block kept) serve decoding. The step for a sequence of length L
// computes what the forward computes for its last position t = L - 1, over
// cache rows 0..t. Every stage streams from HBM with little reuse, so the
// kernels are laid out for bandwidth:
//   k_dec_index  scores of the H_idx index heads against every cached index key,
//                max-pooled per 128-key block (one wave per block);
//   k_dec_topk   the selection per (sequence, index head) row;
//   k_dec_attn   softmax attention of each query head over its group's blocks.
#include "msa_device.hpp"
#include "msa_internal.hpp"
#include "msa_topk.hpp"

namespace msa {

typedef __attribute__((address_space(3))) void* lds_ptr;
typedef __attribute__((address_space(3))) bf16x4* lds_bf16x4_ptr;

// s_waitcnt vmcnt(0) only (gfx9 encoding), after a compiler barrier so no LDS read moves above it
#define MSA_DEC_WAIT_VMCNT0()                  \
    do {                                       \
        asm volatile("" ::: "memory");         \
        __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8)); \
    } while (0)

constexpr int kDecIdxWaves = 4;   // key blocks per index workgroup (one per wave)
constexpr int kDecAttnSlices = 4;  // 32-key slices of a block, one per wave of a slot group

// Sequence length as the kernels use it: clamped to the cache capacity; <= 0 is empty.
__device__ __forceinline__ int dec_len(const int32_t* __restrict__ seqlens, int b, int C) {
    return min(seqlens[b], C);
}

// ---------------------------------------------------------------------------
// Index scores + block max. A wave owns key block c of sequence b: the block's
// 128 index keys are the A operand of v_mfma_f32_16x16x32_bf16 (16 keys x 32
// dims per tile, lane l reading key l % 16, dims 32kk + 8(l/16) .. +7 straight
// from memory), the index queries of up to 16 heads the B operand. The result
// holds keys 4(l/16) + i of head l % 16 in lane l, so the block max is an
// in-lane max plus two exchanges. Keys past t are masked (and never loaded:
// their rows are clamped to t). Blocks after the sequence's own get -inf.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_dec_index(const __bf16* __restrict__ q_idx, const __bf16* __restrict__ k_idx,
                                                   const int32_t* __restrict__ seqlens, float* __restrict__ pooled,
                                                   int C, int H, int nblk) {
    const int b = blockIdx.y;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c = blockIdx.x * kDecIdxWaves + wave;
    if (c >= nblk) return;
    const int L = dec_len(seqlens, b, C);
    const int t = L - 1;
    const int cl = L > 0 ? t / kBlock : -1;
    float* prow = pooled + (size_t)b * H * nblk + c;
    if (c > cl) {
        for (int g = lane; g < H; g += 64) prow[(size_t)g * nblk] = -INFINITY;
        return;
    }
    const int q4 = lane >> 4, n = lane & 15;
    const int rmax = t - c * kBlock;  // last valid key of the block (>= 0)
    const __bf16* kb = k_idx + ((size_t)b * C + (size_t)c * kBlock) * kDim;
    bf16x8 kf[8][4];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
        const int row = min(16 * mt + n, rmax);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) kf[mt][kk] = *(const bf16x8*)(kb + (size_t)row * kDim + 32 * kk + 8 * q4);
    }
    for (int ht = 0; ht < H; ht += 16) {
        const int h = ht + n;
        bf16x8 qf[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            if (h < H) {
                qf[kk] = *(const bf16x8*)(q_idx + ((size_t)b * H + h) * kDim + 32 * kk + 8 * q4);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) qf[kk][e] = (__bf16)0.0f;
            }
        }
        float m = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) acc = mfma16(kf[mt][kk], qf[kk], acc);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (16 * mt + 4 * q4 + i <= rmax) m = fmaxf(m, acc[i]);
        }
        m = fmaxf(m, __shfl_xor(m, 16, 64));
        m = wave_max_xor32(m);
        if (q4 == 0 && h < H) prow[(size_t)h * nblk] = m;
    }
}

// ---------------------------------------------------------------------------
// Selection per (sequence, index head) row, one workgroup of four waves each:
// the forward selection kernel's steps on a row of any length, spread over 256
// threads. Thread i takes blocks i, i + 256, ... (so wave w holds the blocks
// with (c / 64) % 4 == w).
//   1. each thread takes the max of its 32-bit score keys;
//   2. each wave finds T_w, the (top_k-1)-th largest of its 64 thread maxima,
//      bit by bit (0 when fewer lanes hold a block). At least top_k-1 keys of the
//      row are >= T_w, so T = max_w T_w is at most the row's (top_k-1)-th
//      largest key and every key of the exact selection is >= T;
//   3. each wave puts its keys >= T, as 64-bit (score, block) keys, in its own
//      LDS segment in ascending block order (sized for all its blocks, so any
//      tie pattern fits);
//   4. each candidate is ranked by counting larger candidates in all segments;
//      ranks below top_k-1 are the selection (the keys are unique);
//   5. the chosen blocks are written in ascending order, the local block last.
// ---------------------------------------------------------------------------
constexpr int kDecTopkWaves = 4;
constexpr int kDecTopkThreads = 64 * kDecTopkWaves;

__device__ __forceinline__ int dec_topk_segment(int nblk) {
    return (nblk + kDecTopkThreads - 1) / kDecTopkThreads * 64;  // blocks one wave can hold
}

__global__ __launch_bounds__(kDecTopkThreads) void k_dec_topk(const float* __restrict__ pooled,
                                                              const int32_t* __restrict__ seqlens,
                                                              int32_t* __restrict__ block_idx, int C, int H, int nblk,
                                                              int top_k) {
    extern __shared__ __attribute__((aligned(16))) uint64_t dec_list[];  // kDecTopkWaves segments
    __shared__ uint32_t wave_t[kDecTopkWaves];
    __shared__ int wave_n[kDecTopkWaves];
    __shared__ int32_t chosen[64];  // by rank; top_k <= 65
    const int row = blockIdx.x, b = row / H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int L = dec_len(seqlens, b, C);
    int32_t* dst = block_idx + (size_t)row * top_k;
    // the early exits depend on the row alone, so the whole workgroup takes them
    if (L <= 0) {
        for (int s = tid; s < top_k; s += kDecTopkThreads) dst[s] = -1;
        return;
    }
    const int cl = (L - 1) / kBlock;
    if (cl + 1 <= top_k) {  // every visible block
        for (int s = tid; s < top_k; s += kDecTopkThreads) dst[s] = s <= cl ? s : -1;
        return;
    }
    const int need = top_k - 1;
    if (need == 0) {
        if (tid == 0) dst[0] = cl;
        return;
    }
    const float* src = pooled + (size_t)row * nblk;

    // 1, 2. thread maxima, then each wave's bound
    uint32_t tmax = 0u;  // below every real key
    for (int c = tid; c < cl; c += kDecTopkThreads) {
        const uint32_t k = order_key(src[c]);
        tmax = k > tmax ? k : tmax;
    }
    uint32_t T = 0u;
#pragma unroll
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand_t = T | (1u << bit);
        if (__popcll(__ballot(tmax >= cand_t)) >= need) T = cand_t;
    }
    if (lane == 0) wave_t[wave] = T;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kDecTopkWaves; ++w) T = wave_t[w] > T ? wave_t[w] : T;

    // 3. this wave's candidates, ascending block order
    const int seg = dec_topk_segment(nblk);
    uint64_t* list = dec_list + (size_t)wave * seg;
    const uint64_t lt = (1ull << lane) - 1ull;
    int n = 0;
    for (int c0 = 64 * wave; c0 < cl; c0 += kDecTopkThreads) {
        const int c = c0 + lane;
        const uint32_t k = c < cl ? order_key(src[c]) : 0u;
        const bool take = c < cl && k >= T;
        const uint64_t mask = __ballot(take);
        if (take) list[n + __popcll(mask & lt)] = ((uint64_t)k << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)c);
        n += __popcll(mask);
    }
    if (lane == 0) wave_n[wave] = n;
    __syncthreads();

    // 4. rank every candidate against all of them
    for (int w = 0; w < kDecTopkWaves; ++w) {
        const int nw = wave_n[w];
        for (int i = tid; i < nw; i += kDecTopkThreads) {
            const uint64_t mine = dec_list[(size_t)w * seg + i];
            int r = 0;
            for (int w2 = 0; w2 < kDecTopkWaves; ++w2) {
                const uint64_t* l2 = dec_list + (size_t)w2 * seg;
                const int n2 = wave_n[w2];
                for (int j = 0; j < n2; ++j) r += l2[j] > mine ? 1 : 0;
            }
            if (r < need) chosen[r] = key_block(mine);
        }
    }
    __syncthreads();

    // 5. ascending output: a chosen block's place is the number of smaller chosen blocks
    if (tid < need) {
        const int blk = chosen[tid];
        int slot = 0;
        for (int j = 0; j < need; ++j) slot += chosen[j] < blk ? 1 : 0;
        dst[slot] = blk;
    }
    if (tid == 0) dst[need] = cl;
}

// ---------------------------------------------------------------------------
// Attention over the selected blocks. A workgroup owns (sequence b, KV head g,
// a tile of up to 16 of the group's query heads). Its NW waves form NW / 4 slot
// groups: wave w takes keys 32(w % 4) .. +31 of the selected blocks in slots
// w / 4, w / 4 + NW / 4, ... and keeps an online softmax over them (NW = 4 when
// the grid fills the chip, 16 when there are fewer groups than CUs).
//   S^T = K Q^T: K rows are the A operand, read from memory (rows past t clamped
//   to t and masked), Q the B operand; lane l holds keys 16mt + 4(l/16) + i of
//   head l % 16.
//   O += P V: those P values, rounded to bf16, are the A operand as they sit in
//   the registers (lane l: head l % 16; slot e of the 8 goes to key
//   16(e/4) + 4(l/16) + e%4); the V rows of the same keys come from the wave's
//   LDS tile (filled by global->LDS loads) through ds_read_b64_tr_b16, which
//   hands each lane one dim of 4 consecutive keys.
// The waves' (m, l, O) are merged in LDS at the end.
//
// Split mode (splits > 1; blockIdx.z = b * splits + split): when there are few
// (sequence, KV head) groups, the selected slots of one group are dealt over
// `splits` workgroups, so more CUs stream the blocks at once. Each workgroup
// then writes its heads' (M, L) and unnormalised O (relative to M, log2 units)
// to a record [b, head, split] instead of O and LSE, and k_dec_merge combines
// the records: M* = max M_s, L* = sum L_s 2^(M_s - M*), O = sum O_s 2^(M_s - M*) / L*.
// ---------------------------------------------------------------------------
__device__ __forceinline__ bf16x4 dec_tr_rows4(const __bf16* tile, int r0, int c0, int li) {
    const int row = r0 + (li >> 2), col = c0 + 4 * (li & 3);
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_ptr)(tile + row * kDim + col));
}

template <int NW>
__global__ __launch_bounds__(64 * NW) void k_dec_attn(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                                                  const __bf16* __restrict__ v, const int32_t* __restrict__ seqlens,
                                                  const int32_t* __restrict__ block_idx, __bf16* __restrict__ o,
                                                  float* __restrict__ lse, int C, int Hq, int Hkv, int G, int top_k,
                                                  float scale_log2, int splits, float2* __restrict__ rec_ml,
                                                  float* __restrict__ rec_o) {
    const int ht = blockIdx.x, g = blockIdx.y, b = blockIdx.z / splits, split = blockIdx.z - b * splits;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, q4 = lane >> 4, n = lane & 15;
    const int L = dec_len(seqlens, b, C);
    const int t = L - 1;
    const int cl = L > 0 ? t / kBlock : -1;
    const int h0 = g * G + ht * 16;
    const int hn = min(16, G - ht * 16);

    __shared__ __attribute__((aligned(16))) __bf16 vs[NW][32 * kDim];  // 8 KB of V rows per wave
    __shared__ float sm[NW][16], sl[NW][16];
    __bf16* vw = vs[wave];

    bf16x8 qf[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        if (n < hn) {
            qf[kk] = *(const bf16x8*)(q + ((size_t)b * Hq + h0 + n) * kDim + 32 * kk + 8 * q4);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) qf[kk][e] = (__bf16)0.0f;
        }
    }
    float m_run = -INFINITY, l_run = 0.0f;  // of head n, over this wave's keys so far
    f32x4 oacc[8];                          // O[head 4(l/16) + i][dim 16dt + l % 16]
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) oacc[dt] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};

    const int32_t* sel = block_idx + ((size_t)b * Hkv + g) * top_k;
    const size_t kv_row = (size_t)Hkv * kDim;  // elements between consecutive cache rows
    const __bf16* kseq = k + ((size_t)b * C * Hkv + g) * kDim;
    const __bf16* vseq = v + ((size_t)b * C * Hkv + g) * kDim;
    // wave w takes slice w % 4 of its slot group's slots: group split * NW/4 + w/4 of
    // the splits * NW/4 groups, slots group, group + splits * NW/4, ...
    constexpr int kGroups = NW / kDecAttnSlices;
    for (int s = split * kGroups + wave / kDecAttnSlices; s < top_k; s += splits * kGroups) {
        const int c = sel[s];
        if (c < 0 || c > cl) continue;  // padding or not visible
        const int kbase = c * kBlock + 32 * (wave % kDecAttnSlices);
        const int rmax = t - kbase;  // last valid key of this wave's 32
        if (rmax < 0) continue;      // the whole slice lies after t
        // V rows kbase .. kbase+31 (clamped to t) into LDS, row-major: instruction i
        // fills rows 4i .. 4i+3, lane l row 4i + l/16, dims 8(l%16) .. +7. Each
        // instruction reads whole rows (whole cache lines) that this step does not
        // read again, so the loads are nontemporal (cache policy 2 = nt): 8% faster.
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = min(4 * i + (lane >> 4), rmax);
            __builtin_amdgcn_global_load_lds((const void*)(vseq + (size_t)(kbase + r) * kv_row + 8 * (lane & 15)),
                                             (lds_ptr)(vw + 4 * i * kDim), 16, 0, 2);
        }
        bf16x8 kf[2][4];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            const int r = min(16 * mt + n, rmax);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                kf[mt][kk] = *(const bf16x8*)(kseq + (size_t)(kbase + r) * kv_row + 32 * kk + 8 * q4);
        }
        f32x4 sacc[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            sacc[mt] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) sacc[mt] = mfma16(kf[mt][kk], qf[kk], sacc[mt]);
        }
        float mb = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float sv = (16 * mt + 4 * q4 + i <= rmax) ? sacc[mt][i] * scale_log2 : -INFINITY;
                sacc[mt][i] = sv;
                mb = fmaxf(mb, sv);
            }
        mb = fmaxf(mb, __shfl_xor(mb, 16, 64));
        mb = wave_max_xor32(mb);
        const float m_new = fmaxf(m_run, mb);  // finite: key kbase <= t is valid
        const float alpha = exp2f(m_run - m_new);
        float ps = 0.0f;
        bf16x8 pa;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p = exp2f(sacc[mt][i] - m_new);
                ps += p;
                pa[4 * mt + i] = (__bf16)p;
            }
        ps += __shfl_xor(ps, 16, 64);
        ps = wave_sum_xor32(ps);
        l_run = l_run * alpha + ps;
        m_run = m_new;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float a = __shfl(alpha, 4 * q4 + i, 64);
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) oacc[dt][i] *= a;
        }
        MSA_DEC_WAIT_VMCNT0();  // this wave's V rows have landed in LDS
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            const bf16x4 lo = dec_tr_rows4(vw, 4 * q4, 16 * dt, n);
            const bf16x4 hi = dec_tr_rows4(vw, 16 + 4 * q4, 16 * dt, n);
            const bf16x8 vb = (bf16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            oacc[dt] = mfma16(pa, vb, oacc[dt]);
        }
    }

    // merge the waves: weights 2^(m_w - M) per head, O and l summed
    __syncthreads();  // every wave is done with its V tile; the tiles become the merge buffer
    float* red = (float*)&vs[0][0];  // [wave][16 heads][128 dims] fp32, 8 KB per wave
    if (q4 == 0) {
        sm[wave][n] = m_run;
        sl[wave][n] = l_run;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int h = 4 * q4 + i;
        float M = sm[0][h];
#pragma unroll
        for (int w = 1; w < NW; ++w) M = fmaxf(M, sm[w][h]);
        const float mw = sm[wave][h];
        const float wt = mw == -INFINITY ? 0.0f : exp2f(mw - M);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) red[(wave * 16 + h) * kDim + 16 * dt + n] = oacc[dt][i] * wt;
    }
    __syncthreads();
    const int h = tid >> 4, d0 = (tid & 15) * 8;
    if (h >= hn) return;
    float M = sm[0][h];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, sm[w][h]);
    float Lsum = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) Lsum += sm[w][h] == -INFINITY ? 0.0f : exp2f(sm[w][h] - M) * sl[w][h];
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        acc[e] = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) acc[e] += red[(w * 16 + h) * kDim + d0 + e];
    }
    if (splits > 1) {  // this split's record; M = -inf, L = 0, O = 0 when it saw no key
        const size_t rr = ((size_t)b * Hq + h0 + h) * splits + split;
        float4* dst = (float4*)(rec_o + rr * kDim + d0);
        dst[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
        dst[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
        if ((tid & 15) == 0) rec_ml[rr] = make_float2(M, Lsum);
        return;
    }
    const float inv = Lsum > 0.0f ? 1.0f / Lsum : 0.0f;
    bf16x8 out;
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = (__bf16)(acc[e] * inv);
    *(bf16x8*)(o + ((size_t)b * Hq + h0 + h) * kDim + d0) = out;
    if ((tid & 15) == 0)
        lse[(size_t)b * Hq + h0 + h] = Lsum > 0.0f ? (M + log2f(Lsum)) * 0.69314718055994531f : -INFINITY;
}

// Merge of the split records, 16 threads (8 dims each) per (sequence, query head) row.
// Every split writes its record (zeros and M = -inf when it saw no key), so all
// records are loaded at once, with no load behind a data-dependent branch.
constexpr int kDecMaxSplits = 16;

__global__ __launch_bounds__(256) void k_dec_merge(const float2* __restrict__ rec_ml, const float* __restrict__ rec_o,
                                                   __bf16* __restrict__ o, float* __restrict__ lse, int rows,
                                                   int splits) {
    const int r = blockIdx.x * 16 + (threadIdx.x >> 4), d0 = (threadIdx.x & 15) * 8;
    if (r >= rows) return;
    const float2* ml = rec_ml + (size_t)r * splits;
    float2 x[kDecMaxSplits];
    float4 a[kDecMaxSplits], c[kDecMaxSplits];
#pragma unroll
    for (int s = 0; s < kDecMaxSplits; ++s) {
        if (s < splits) {
            x[s] = ml[s];
            const float4* src = (const float4*)(rec_o + ((size_t)r * splits + s) * kDim + d0);
            a[s] = src[0];
            c[s] = src[1];
        }
    }
    float M = -INFINITY;
#pragma unroll
    for (int s = 0; s < kDecMaxSplits; ++s)
        if (s < splits) M = fmaxf(M, x[s].x);
    float L = 0.0f, acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
#pragma unroll
    for (int s = 0; s < kDecMaxSplits; ++s) {
        // a split that saw no key has M = -inf: weight 0 (its O is 0)
        const float w = (s < splits && x[s].x != -INFINITY) ? exp2f(x[s].x - M) : 0.0f;
        if (s < splits) {
            L += w * x[s].y;
            acc[0] += w * a[s].x;
            acc[1] += w * a[s].y;
            acc[2] += w * a[s].z;
            acc[3] += w * a[s].w;
            acc[4] += w * c[s].x;
            acc[5] += w * c[s].y;
            acc[6] += w * c[s].z;
            acc[7] += w * c[s].w;
        }
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    bf16x8 out;
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = (__bf16)(acc[e] * inv);
    *(bf16x8*)(o + (size_t)r * kDim + d0) = out;
    if ((threadIdx.x & 15) == 0) lse[r] = L > 0.0f ? (M + log2f(L)) * 0.69314718055994531f : -INFINITY;
}

// ---------------------------------------------------------------------------
size_t dec_topk_lds_bytes(const Dims& d) {
    return (size_t)kDecTopkWaves * ((d.nblk + kDecTopkThreads - 1) / kDecTopkThreads * 64) * 8;
}

hipError_t launch_dec_index(const void* q_idx, const void* k_idx, const int32_t* seqlens, float* pooled, const Dims& d,
                            hipStream_t stream) {
    dim3 grid((unsigned)((d.nblk + kDecIdxWaves - 1) / kDecIdxWaves), (unsigned)d.B);
    hipLaunchKernelGGL(k_dec_index, grid, dim3(64 * kDecIdxWaves), 0, stream, (const __bf16*)q_idx,
                       (const __bf16*)k_idx, seqlens, pooled, d.N, d.Hkv, d.nblk);
    return hipGetLastError();
}

hipError_t launch_dec_topk(const float* pooled, const int32_t* seqlens, int32_t* block_idx, const Dims& d,
                           hipStream_t stream) {
    const size_t lds = dec_topk_lds_bytes(d);
    if (lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute((const void*)k_dec_topk, hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_dec_topk, dim3((unsigned)(d.B * d.Hkv)), dim3(kDecTopkThreads), lds, stream, pooled, seqlens, block_idx,
                       d.N, d.Hkv, d.nblk, d.top_k);
    return hipGetLastError();
}

// Workgroups the attention wants in flight before it spreads a group's slots over
// several of them: four per CU of a 256-CU part. A constant (not the device's CU
// count) so that the split, and so the rounding of the result, depends on the shape
// alone.
constexpr long long kDecAttnWantGroups = 1024;

int dec_splits(const Dims& d) {
    const long long base = (long long)((d.G + 15) / 16) * d.Hkv * d.B;
    if (base * 2 >= kDecAttnWantGroups) return 1;
    long long s = (kDecAttnWantGroups + base - 1) / base;
    if (s > d.top_k) s = d.top_k;
    return (int)(s < kDecMaxSplits ? s : kDecMaxSplits);
}

size_t dec_rec_bytes(const Dims& d) {
    const int S = dec_splits(d);
    if (S <= 1) return 0;
    const size_t recs = (size_t)d.B * d.Hq * S;
    return align_up(recs * sizeof(float2), 256) + align_up(recs * kDim * sizeof(float), 256);
}

hipError_t launch_dec_attn(const void* q, const void* k, const void* v, const int32_t* seqlens,
                           const int32_t* block_idx, void* o, float* lse, void* records, const Dims& d,
                           hipStream_t stream) {
    const float sl2 = d.scale * 1.4426950408889634f;
    const int S = records ? dec_splits(d) : 1;
    if (S > 1) {
        // split mode: four-wave workgroups, the group's slots dealt over S of them, then the merge
        const size_t recs = (size_t)d.B * d.Hq * S;
        float2* rec_ml = (float2*)records;
        float* rec_o = (float*)((char*)records + align_up(recs * sizeof(float2), 256));
        dim3 grid((unsigned)((d.G + 15) / 16), (unsigned)d.Hkv, (unsigned)(d.B * S));
        hipLaunchKernelGGL(k_dec_attn<kDecAttnSlices>, grid, dim3(64 * kDecAttnSlices), 0, stream, (const __bf16*)q,
                           (const __bf16*)k, (const __bf16*)v, seqlens, block_idx, (__bf16*)o, lse, d.N, d.Hq, d.Hkv,
                           d.G, d.top_k, sl2, S, rec_ml, rec_o);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int rows = d.B * d.Hq;
        hipLaunchKernelGGL(k_dec_merge, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, stream, rec_ml, rec_o,
                           (__bf16*)o, lse, rows, S);
        return hipGetLastError();
    }
    dim3 grid((unsigned)((d.G + 15) / 16), (unsigned)d.Hkv, (unsigned)d.B);
    // Few (sequence, KV head, head tile) groups would leave most CUs idle: then four slot
    // groups of four waves share a group's selected blocks (16 waves, 130 KB of LDS).
    if ((long long)grid.x * grid.y * grid.z < device_cu_count()) {
        hipLaunchKernelGGL(k_dec_attn<4 * kDecAttnSlices>, grid, dim3(64 * 4 * kDecAttnSlices), 0, stream,
                           (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, seqlens, block_idx, (__bf16*)o, lse,
                           d.N, d.Hq, d.Hkv, d.G, d.top_k, sl2, 1, (float2*)nullptr, (float*)nullptr);
    } else {
        hipLaunchKernelGGL(k_dec_attn<kDecAttnSlices>, grid, dim3(64 * kDecAttnSlices), 0, stream, (const __bf16*)q,
                           (const __bf16*)k, (const __bf16*)v, seqlens, block_idx, (__bf16*)o, lse, d.N, d.Hq, d.Hkv,
                           d.G, d.top_k, sl2, 1, (float2*)nullptr, (float*)nullptr);
    }
    return hipGetLastError();
}

}  // namespace msa
