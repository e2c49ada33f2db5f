// Per-row top-k building blocks of the selection kernel (wave64, gfx950): one
// wave selects one row whose scores sit in registers, 16 per lane.
//
// [MSA summary] "GPU kernel co-design": exp-free selection on the raw pooled
// scores. [MSA summary] "Architecture" / [Flash-MSA] "Proxy attention": the
// query's own block is always kept; top_k - 1 blocks are chosen among the
// earlier ones, larger score first, lower block first among equal scores.
#pragma once

#include "msa_device.hpp"

namespace msa {

constexpr int kTopkRegVals = 16;

// Unconditional loads (index clamped into the row, so no branch per load); entries at or
// past cl are masked by the caller.
__device__ __forceinline__ void topk_load_row(const float* __restrict__ src, int cl, int lane,
                                              float (&v)[kTopkRegVals]) {
    const int last = cl - 1;
#pragma unroll
    for (int i = 0; i < kTopkRegVals; ++i) v[i] = src[min(lane + 64 * i, last)];
}

// Rank of `mine` among list[0..n4): how many listed keys are larger. n4 is a multiple
// of 4 and list[n..n4) holds zero keys, below every real key. Four keys per step
// with two 16-byte broadcast reads.
__device__ __forceinline__ int rank_in_list(const uint64_t* list, int n4, uint64_t mine) {
    int r = 0;
    for (int j = 0; j < n4; j += 4) {
        const ulonglong2 a = *(const ulonglong2*)(list + j);
        const ulonglong2 b = *(const ulonglong2*)(list + j + 2);
        r += (a.x > mine ? 1 : 0) + (a.y > mine ? 1 : 0) + (b.x > mine ? 1 : 0) + (b.y > mine ? 1 : 0);
    }
    return r;
}

// Steps 4 and 5 for one wave: rank the n listed keys, keep ranks below `need`,
// write the chosen blocks ascending to dst[0..need) and the local block after them.
__device__ __forceinline__ void rank_and_emit(uint64_t* list, int32_t* chosen, int n, int need, int cl,
                                              int32_t* __restrict__ dst, int lane) {
    const int n4 = (n + 3) & ~3;
    if (lane < n4 - n) list[n + lane] = 0ull;
    if (lane >= need && lane < ((need + 3) & ~3)) chosen[lane] = 0x7fffffff;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int i = lane; i < n; i += 64) {
        const uint64_t mine = list[i];
        const int r = rank_in_list(list, n4, mine);
        if (r < need) chosen[r] = key_block(mine);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // ascending block order; the local block is larger than every chosen one
    if (lane < need) {
        const int mine = chosen[lane];
        const int need4 = (need + 3) & ~3;
        int pos = 0;
        for (int j = 0; j < need4; j += 4) {
            const int4 c4 = *(const int4*)(chosen + j);
            pos += (c4.x < mine ? 1 : 0) + (c4.y < mine ? 1 : 0) + (c4.z < mine ? 1 : 0) + (c4.w < mine ? 1 : 0);
        }
        dst[pos] = mine;
    }
    if (lane == 0) dst[need] = cl;
}

// A row with more candidates than the list holds (many equal scores): exact
// without a list. T = the need-th largest score key of the row, counted with
// multiplicity, found bit by bit; every key above T is chosen (fewer than
// `need`), then the lowest blocks among the keys equal to T fill the rest
// (equal scores go to the lower block). Blocks are lane + 64 i, so ascending
// block order is (i, lane) order and ballot prefix counts place each one.
__device__ __forceinline__ void topk_row_ties(const uint32_t (&k32)[kTopkRegVals], int cl, int need,
                                              int32_t* __restrict__ dst, int lane) {
    const uint64_t lt = (1ull << lane) - 1ull;
    uint32_t T = 0u;
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand_t = T | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int i = 0; i < kTopkRegVals; ++i) cnt += __popcll(__ballot(k32[i] >= cand_t));
        if (cnt >= need) T = cand_t;
    }
    int above = 0;
#pragma unroll
    for (int i = 0; i < kTopkRegVals; ++i) above += __popcll(__ballot(k32[i] > T));
    const int rem = need - above;  // >= 1 keys equal to T are taken, lowest blocks first
    int eq_before = 0, base = 0;
#pragma unroll
    for (int i = 0; i < kTopkRegVals; ++i) {
        const uint64_t eq = __ballot(k32[i] == T);
        const bool take = k32[i] > T || (k32[i] == T && eq_before + __popcll(eq & lt) < rem);
        eq_before += __popcll(eq);
        const uint64_t tm = __ballot(take);
        if (take) dst[base + __popcll(tm & lt)] = lane + 64 * i;
        base += __popcll(tm);
    }
    if (lane == 0) dst[need] = cl;
}

// Steps 1-5 for one row whose non-local scores (blocks lane + 64 i < cl) are in
// registers: the threshold works on 32-bit score keys. The need-th largest lane
// maximum of the score keys, T32, is the high word of the need-th largest
// 64-bit lane maximum, so every key of the exact selection has a score key
// >= T32. Only those candidates get 64-bit (score, block) keys, ranked exactly;
// more than kTopkListCap of them (ties) take topk_row_ties instead.
// `list` holds kTopkListCap + 4 keys, `chosen` 64 ints; both per wave.
constexpr int kTopkListCap = 128;

__device__ __forceinline__ void topk_row_from_regs(const float (&cur)[kTopkRegVals], int cl, int need,
                                                   uint64_t* list, int32_t* chosen, int32_t* __restrict__ dst,
                                                   int lane) {
    uint32_t k32[kTopkRegVals];
    uint32_t lmax = 0u;
#pragma unroll
    for (int i = 0; i < kTopkRegVals; ++i) {
        k32[i] = lane + 64 * i < cl ? order_key(cur[i]) : 0u;
        lmax = k32[i] > lmax ? k32[i] : lmax;
    }
    uint32_t T = 0u;
#pragma unroll
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand_t = T | (1u << bit);
        if (__popcll(__ballot(lmax >= cand_t)) >= need) T = cand_t;
    }
    uint64_t masks[kTopkRegVals];
    int n = 0;
#pragma unroll
    for (int i = 0; i < kTopkRegVals; ++i) {
        masks[i] = __ballot(k32[i] >= T);
        n += __popcll(masks[i]);
    }
    if (n > kTopkListCap) {
        topk_row_ties(k32, cl, need, dst, lane);
        return;
    }
    int base = 0;
#pragma unroll
    for (int i = 0; i < kTopkRegVals; ++i) {
        if (masks[i] != 0ull) {
            if (k32[i] >= T)
                list[base + __popcll(masks[i] & ((1ull << lane) - 1ull))] =
                    ((uint64_t)k32[i] << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)(lane + 64 * i));
            base += __popcll(masks[i]);
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    rank_and_emit(list, chosen, n, need, cl, dst, lane);
}

}  // namespace msa
