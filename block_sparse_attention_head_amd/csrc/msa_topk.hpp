// Per-row top-k building blocks of the selection kernels (wave64, gfx950): one
// wave selects one row.
//
// [MSA summary] "GPU kernel co-design": exp-free selection on the raw pooled
// scores. [MSA summary] "Architecture" / [Flash-MSA] "Proxy attention": the
// query's own block is always kept; top_k - 1 blocks are chosen among the
// earlier ones, larger score first, lower block first among equal scores.
#pragma once

#include "msa_device.hpp"

namespace msa {

constexpr int kTopkRowMax = 1024;  // non-local blocks the register path holds per row

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

// Steps 4 and 5 for one wave. The n listed keys are in ascending block order;
// each is ranked by counting the larger ones, and those ranked below `need`
// (exactly `need`, since keys are unique) go to dst[0..need) in list order, so
// ascending, each placed by a ballot prefix count; the local block follows.
// `list` holds at least n + 4 keys.
__device__ __forceinline__ void rank_and_emit(uint64_t* list, int n, int need, int cl, int32_t* __restrict__ dst,
                                              int lane) {
    const int n4 = (n + 3) & ~3;
    if (lane < n4 - n) list[n + lane] = 0ull;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const uint64_t lt = (1ull << lane) - 1ull;
    int base = 0;
    for (int i0 = 0; i0 < n; i0 += 64) {
        const int i = i0 + lane;
        bool take = false;
        uint64_t mine = 0ull;
        if (i < n) {
            mine = list[i];
            take = rank_in_list(list, n4, mine) < need;
        }
        const uint64_t tm = __ballot(take);
        if (take) dst[base + __popcll(tm & lt)] = key_block(mine);
        base += __popcll(tm);
    }
    if (lane == 0) dst[need] = cl;
}

// `list` holds kTopkListCap + 4 keys per wave. The bound is searched on the top
// kTopkBoundBits bits of the key only (sign, exponent and 7 mantissa bits: within
// 2^-7 relative below the need-th lane maximum): a lower bound admits a few more
// candidates and leaves the exact ranking unchanged.
constexpr int kTopkListCap = 128;
constexpr int kTopkBoundBits = 16;

// Buffer resource word 3 for raw 32-bit accesses on gfx9-family targets.
constexpr int kRawBufferWord3 = 0x00020000;

__device__ __forceinline__ uint64_t positive_key(float x, uint32_t block) {
    return ((uint64_t)__float_as_uint(x) << 32) | (0xFFFFFFFFu - block);
}
__device__ __forceinline__ uint32_t lanes_below(uint64_t m, uint32_t acc) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, acc));
}

// Exact selection streamed from memory, for the rare rows the register path
// cannot take (a bound not above zero, or more candidates than the list holds:
// many equal scores); it holds no scores in registers. T = the need-th largest
// score key of blocks 0 .. cl - 1, counted with multiplicity, found bit by bit;
// every key above T is chosen (fewer than `need`), then the lowest blocks among
// the keys equal to T fill the rest (equal scores go to the lower block).
// Blocks c0 + lane in ascending c0 are ascending block order, so ballot prefix
// counts place each one.
__device__ __forceinline__ uint32_t exact_key(const float* __restrict__ src, int c, int cl) {
    return c < cl ? order_key(src[c]) : 0u;  // 0 is below every real key
}

__device__ __forceinline__ void topk_row_exact(const float* __restrict__ src, int cl, int need,
                                               int32_t* __restrict__ dst, int lane) {
    const uint64_t lt = (1ull << lane) - 1ull;
    uint32_t T = 0u;
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand_t = T | (1u << bit);
        int cnt = 0;
        for (int c0 = 0; c0 < cl; c0 += 64) cnt += __popcll(__ballot(exact_key(src, c0 + lane, cl) >= cand_t));
        if (cnt >= need) T = cand_t;
    }
    int above = 0;
    for (int c0 = 0; c0 < cl; c0 += 64) above += __popcll(__ballot(exact_key(src, c0 + lane, cl) > T));
    const int rem = need - above;  // >= 1 keys equal to T are taken, lowest blocks first
    int eq_before = 0, base = 0;
    for (int c0 = 0; c0 < cl; c0 += 64) {
        const uint32_t k = exact_key(src, c0 + lane, cl);
        const uint64_t eq = __ballot(k == T);
        const bool take = k > T || (k == T && eq_before + __popcll(eq & lt) < rem);
        eq_before += __popcll(eq);
        const uint64_t tm = __ballot(take);
        if (take) dst[base + __popcll(tm & lt)] = c0 + lane;
        base += __popcll(tm);
    }
    if (lane == 0) dst[need] = cl;
}

// One row of at most kTopkRowMax non-local blocks, 1 <= need < cl: steps 1-5.
//  - Loads: lane l reads blocks 256 j + 4 l .. + 3 (j = 0..3) with one 16-byte
//    buffer load each, from a buffer resource that ends at the last whole quad
//    below cl, and the up to three blocks from there to cl with one 4-byte
//    load per lane from a second one. The hardware range check returns 0 for
//    every position at or past the end of a resource and reads nothing there,
//    so no address outside blocks 0 .. cl - 1 is touched.
//  - Step 1: each lane takes the max of its scores; T = the need-th largest of
//    the lanes' score keys (or a lower bound of it: kTopkBoundBits), found bit
//    by bit with ballots. The maxima may include those zeros; T is used only
//    when its score is above zero: then no zero reaches it, at least `need` real
//    scores do, and every candidate is positive, so its raw fp32 bits already
//    order it.
//  - Steps 2-3: the scores >= T are compacted into the wave's list per 256-block
//    chunk in (lane, slot) order, which is ascending block order, each lane's
//    first slot placed by the mbcnt of the chunk's four ballots. The stores are
//    unconditional (no exec-mask branch per value): a value below T is written
//    to slot kTopkListCap + 3, past every slot the ranking reads.
//  - Steps 4-5: rank_and_emit.
// A bound not above zero, or more than kTopkListCap candidates, takes
// topk_row_exact.
__device__ __forceinline__ void topk_row_quads(const float* __restrict__ src, int cl, int need, uint64_t* list,
                                               int32_t* __restrict__ dst, int lane) {
    const int cl4 = cl & ~3;
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, cl4 * 4, kRawBufferWord3);
    const __amdgpu_buffer_rsrc_t rt =
        __builtin_amdgcn_make_buffer_rsrc((void*)(src + cl4), (short)0, (cl - cl4) * 4, kRawBufferWord3);
    float v[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        // the whole 16-byte result is reinterpreted at once (element access on the builtin's
        // own vector type does not yield the four loaded words)
        const f32x4 q = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, lane * 16 + 1024 * j, 0, 0));
        v[j][0] = q.x;
        v[j][1] = q.y;
        v[j][2] = q.z;
        v[j][3] = q.w;
    }
    const float vt = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rt, lane * 4, 0, 0));
    float m = vt;
#pragma unroll
    for (int j = 0; j < 4; ++j) m = fmaxf(fmaxf(m, fmaxf(v[j][0], v[j][1])), fmaxf(v[j][2], v[j][3]));
    const uint32_t lk = order_key(m);
    uint32_t T = 0u;
#pragma unroll
    for (int bit = 31; bit >= 32 - kTopkBoundBits; --bit) {
        const uint32_t cand_t = T | (1u << bit);
        if (__popcll(__ballot(lk >= cand_t)) >= need) T = cand_t;
    }
    if (T <= 0x80000000u) {
        topk_row_exact(src, cl, need, dst, lane);
        return;
    }
    const float tf = key_score(T);
    uint64_t mk[4][4];
    int n = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            mk[j][e] = __ballot(v[j][e] >= tf);
            n += __popcll(mk[j][e]);
        }
    const uint64_t mt = __ballot(vt >= tf);
    n += __popcll(mt);
    if (n > kTopkListCap) {
        topk_row_exact(src, cl, need, dst, lane);
        return;
    }
    int base = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if ((mk[j][0] | mk[j][1] | mk[j][2] | mk[j][3]) != 0ull) {
            uint32_t pos = lanes_below(mk[j][3], lanes_below(mk[j][2], lanes_below(mk[j][1],
                                                                                   lanes_below(mk[j][0], base))));
            const uint32_t blk = 256u * j + 4u * lane;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                // branch-free: a value below the bound goes to a slot past the list that is never read
                const bool take = v[j][e] >= tf;
                list[take ? pos : (uint32_t)(kTopkListCap + 3)] = positive_key(v[j][e], blk + e);
                pos += take ? 1u : 0u;
            }
            base += __popcll(mk[j][0]) + __popcll(mk[j][1]) + __popcll(mk[j][2]) + __popcll(mk[j][3]);
        }
    }
    if (mt != 0ull) {
        if (vt >= tf) list[lanes_below(mt, base)] = positive_key(vt, cl4 + lane);
    }
    rank_and_emit(list, n, need, cl, dst, lane);
}

}  // namespace msa
