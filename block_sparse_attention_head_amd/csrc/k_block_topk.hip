// Exp-free top-k block selection with the local block forced.
//
// [MSA summary] "GPU kernel co-design": softmax keeps the order of the
// scores, so the selection runs on the raw pooled scores with no exp.
// [MSA summary] "Architecture" / [Flash-MSA] "Proxy attention": the query's
// own block is always kept, so only top_k - 1 blocks are chosen among the
// earlier ones.
//
// One wavefront per (batch, index head, query) row. Each candidate carries a
// 64-bit key (order-preserving score bits, then the complemented block index)
// so one unsigned compare orders by (score desc, block asc) and keys are
// unique. Steps:
//   1. each lane takes the max key of its strided share of the row;
//   2. a bitonic sort of the 64 lane maxima across the wave gives T, the
//      need-th largest of them (need = top_k - 1). At least `need` keys are
//      >= T, so T is a lower bound on the need-th largest key of the row, and
//      only lanes whose max is >= T (exactly `need` of them) hold keys >= T;
//   3. the keys >= T are compacted into an LDS list with wave ballots (at most
//      need * ceil(c_loc / 64) entries);
//   4. each listed key is ranked by counting larger listed keys; ranks below
//      `need` are the selection;
//   5. the chosen blocks are put in ascending order, the local block last.
#include "msa_device.hpp"
#include "msa_internal.hpp"

namespace msa {

constexpr int kTopkWaves = 4;
constexpr int kTopkCap = 1024;  // LDS candidate slots per wave (plus 4 of padding)

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

bool topk_supported(int nblk, int top_k) {
    // Rows with c_loc + 1 <= top_k take every visible block and need no ranking.
    if (top_k >= nblk) return true;
    const int need = top_k - 1;
    if (need > 64) return false;
    const int per_lane = (nblk - 1 + 63) / 64;
    return need * per_lane <= kTopkCap;
}

__global__ __launch_bounds__(256) void k_block_topk(const float* __restrict__ pooled, int32_t* __restrict__ block_idx,
                                                    int N, int nblk, int top_k, long long rows) {
    __shared__ __attribute__((aligned(16))) uint64_t cand[kTopkWaves][kTopkCap + 4];
    __shared__ __attribute__((aligned(16))) int32_t chosen[kTopkWaves][64];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const long long row = (long long)blockIdx.x * kTopkWaves + wave;
    if (row >= rows) return;  // wave-uniform; no workgroup barrier is used below
    const int t = (int)(row % N);
    const int cl = t >> 7;
    const float* src = pooled + row * nblk;
    int32_t* dst = block_idx + row * top_k;

    if (cl + 1 <= top_k) {  // every visible block
        for (int s = lane; s < top_k; s += 64) dst[s] = s <= cl ? s : -1;
        return;
    }
    const int need = top_k - 1;
    if (need == 0) {
        if (lane == 0) dst[0] = cl;
        return;
    }

    // 1. lane maxima over blocks lane, lane+64, ... < cl
    uint64_t lmax = 0;  // below every real key
    for (int c = lane; c < cl; c += 64) {
        const uint64_t kk = select_key(src[c], c);
        lmax = kk > lmax ? kk : lmax;
    }

    // 2. bitonic sort of the lane maxima, descending: lane i ends with the (i+1)-th largest
    uint64_t x = lmax;
#pragma unroll
    for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
            const uint64_t y = shfl_xor_u64(x, j);
            const bool up = (lane & k) == 0;
            const bool lower = (lane & j) == 0;
            const bool keep_big = (lower == up);
            const uint64_t big = x > y ? x : y, small = x > y ? y : x;
            x = keep_big ? big : small;
        }
    }
    const uint32_t thi = __shfl((uint32_t)(x >> 32), need - 1, 64);
    const uint32_t tlo = __shfl((uint32_t)x, need - 1, 64);
    const uint64_t T = ((uint64_t)thi << 32) | tlo;

    // 3. compact keys >= T into the wave's LDS list
    uint64_t* list = cand[wave];
    int n = 0;
    for (int c0 = 0; c0 < cl; c0 += 64) {
        const int c = c0 + lane;
        uint64_t kk = 0;
        if (c < cl) kk = select_key(src[c], c);
        const bool take = (c < cl) && kk >= T;
        const uint64_t mask = __ballot(take);
        if (take) list[n + __popcll(mask & ((1ull << lane) - 1ull))] = kk;
        n += __popcll(mask);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // 4, 5. rank the listed keys; ascending output, local block last
    rank_and_emit(list, chosen[wave], n, need, cl, dst, lane);
}

// Rows of at most 64 * kTopkRegVals non-local blocks: each wave walks a strided
// sequence of rows, keeps the current row's scores in registers (one load per
// score) and issues the next row's loads before ranking the current one. The
// threshold works on 32-bit score keys: the need-th largest lane maximum of the
// score keys, T32, is the high word of the need-th largest 64-bit lane maximum,
// so every key of the exact selection has a score key >= T32. Only those
// candidates get 64-bit (score, block) keys and are ranked exactly.
constexpr int kTopkRegVals = 16;

__device__ __forceinline__ void topk_load_row(const float* __restrict__ src, int cl, int lane,
                                              float (&v)[kTopkRegVals]) {
#pragma unroll
    for (int i = 0; i < kTopkRegVals; ++i) {
        const int c = lane + 64 * i;
        v[i] = c < cl ? src[c] : 0.0f;
    }
}

__global__ __launch_bounds__(256) void k_block_topk_reg(const float* __restrict__ pooled,
                                                        int32_t* __restrict__ block_idx, int N, int nblk, int top_k,
                                                        long long rows) {
    __shared__ __attribute__((aligned(16))) uint64_t cand[kTopkWaves][64 * kTopkRegVals + 4];
    __shared__ __attribute__((aligned(16))) int32_t chosen[kTopkWaves][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const long long stride = (long long)gridDim.x * kTopkWaves;
    const int need = top_k - 1;
    uint64_t* list = cand[wave];

    long long row = (long long)blockIdx.x * kTopkWaves + wave;
    float v[kTopkRegVals];
    if (row < rows) {
        const int cl = (int)(row % N) >> 7;
        if (cl + 1 > top_k) topk_load_row(pooled + row * nblk, cl, lane, v);
    }
    for (; row < rows; row += stride) {
        const int t = (int)(row % N);
        const int cl = t >> 7;
        int32_t* dst = block_idx + row * top_k;
        const bool rank_row = cl + 1 > top_k;
        float cur[kTopkRegVals];
#pragma unroll
        for (int i = 0; i < kTopkRegVals; ++i) cur[i] = v[i];
        const long long nrow = row + stride;  // prefetch the next row's scores
        if (nrow < rows) {
            const int ncl = (int)(nrow % N) >> 7;
            if (ncl + 1 > top_k) topk_load_row(pooled + nrow * nblk, ncl, lane, v);
        }
        if (!rank_row) {  // every visible block
            for (int s = lane; s < top_k; s += 64) dst[s] = s <= cl ? s : -1;
            continue;
        }
        if (need == 0) {
            if (lane == 0) dst[0] = cl;
            continue;
        }
        // 1. 32-bit score keys (0 for blocks outside the row) and their lane maximum
        uint32_t k32[kTopkRegVals];
        uint32_t lmax = 0u;
#pragma unroll
        for (int i = 0; i < kTopkRegVals; ++i) {
            k32[i] = lane + 64 * i < cl ? order_key(cur[i]) : 0u;
            lmax = k32[i] > lmax ? k32[i] : lmax;
        }
        // 2. bitonic sort of the lane maxima, descending; T32 = the need-th largest (a real
        // key: at least need + 1 lanes hold a block, since cl >= top_k)
        uint32_t x = lmax;
#pragma unroll
        for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
            for (int j = k >> 1; j > 0; j >>= 1) {
                const uint32_t y = __shfl_xor(x, j, 64);
                const bool keep_big = ((lane & j) == 0) == ((lane & k) == 0);
                x = keep_big ? (x > y ? x : y) : (x > y ? y : x);
            }
        }
        const uint32_t T = __shfl(x, need - 1, 64);
        // 3. candidates: score key >= T, as 64-bit (score, block) keys
        int n = 0;
#pragma unroll
        for (int i = 0; i < kTopkRegVals; ++i) {
            const bool take = k32[i] >= T;
            const uint64_t mask = __ballot(take);
            if (take)
                list[n + __popcll(mask & ((1ull << lane) - 1ull))] =
                    ((uint64_t)k32[i] << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)(lane + 64 * i));
            n += __popcll(mask);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // 4, 5. exact rank among the candidates; ascending output, local block last
        rank_and_emit(list, chosen[wave], n, need, cl, dst, lane);
        // the next row reuses this wave's LDS lists
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

hipError_t launch_block_topk(const float* pooled, int32_t* block_idx, const Dims& d, hipStream_t stream) {
    const long long rows = (long long)d.B * d.Hkv * d.N;
    if (d.nblk - 1 <= 64 * kTopkRegVals && d.top_k <= 65) {
        // as many workgroups as are resident at once: each wave then walks its rows with
        // no second round of workgroups waiting for a slot
        static int per_cu = 0;
        if (per_cu <= 0) {
            int n = 0;
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_block_topk_reg, 256, 0) != hipSuccess || n <= 0)
                n = 2;
            per_cu = n;
        }
        const long long want = (rows + kTopkWaves - 1) / kTopkWaves;
        const long long cap = (long long)per_cu * device_cu_count();
        const unsigned blocks = (unsigned)(want < cap ? want : cap);
        hipLaunchKernelGGL(k_block_topk_reg, dim3(blocks), dim3(256), 0, stream, pooled, block_idx, d.N, d.nblk,
                           d.top_k, rows);
    } else {
        const long long blocks = (rows + kTopkWaves - 1) / kTopkWaves;
        hipLaunchKernelGGL(k_block_topk, dim3((unsigned)blocks), dim3(256), 0, stream, pooled, block_idx, d.N,
                           d.nblk, d.top_k, rows);
    }
    return hipGetLastError();
}

}  // namespace msa
