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
//   2. T, the need-th largest of the 64 lane maxima (need = top_k - 1), bounds
//      the need-th largest key of the row from below (at least `need` keys are
//      >= T), and only the lanes whose max is >= T hold keys >= T;
//   3. the keys >= T are compacted into an LDS list with wave ballots (at most
//      need * ceil(c_loc / 64) entries);
//   4. each listed key is ranked by counting larger listed keys; ranks below
//      `need` are the selection;
//   5. the chosen blocks are put in ascending order, the local block last.
// Rows of up to 1025 blocks keep their scores in registers (msa_topk.hpp):
// four 16-byte buffer loads per lane, a 16-bit bound on the lane maxima, a
// 128-entry candidate list in ascending block order and ballot-placed output;
// rows it cannot take (bound not above zero, or many equal scores) are
// selected exactly from memory. Longer rows use k_block_topk below.
#include <atomic>

#include "msa_device.hpp"
#include "msa_internal.hpp"
#include "msa_topk.hpp"

namespace msa {

constexpr int kTopkWaves = 4;
constexpr int kTopkCap = 1024;  // LDS candidate slots per wave (plus 4 of padding)

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
    rank_and_emit(list, n, need, cl, dst, lane);
}

// Rows of at most kTopkRowMax non-local blocks: each wave walks a strided
// sequence of rows (the row index is wave-uniform, so the row's scalars and
// branches stay scalar) and selects each with topk_row_quads. No row is
// prefetched: 68 registers give seven waves per SIMD, which hide the loads.
// The grid holds as many workgroups as are resident at once.
__global__ __launch_bounds__(256) void k_block_topk_reg(
    const float* __restrict__ pooled, int32_t* __restrict__ block_idx, int N, int nblk, int top_k, long long rows) {
    __shared__ __attribute__((aligned(16))) uint64_t cand[kTopkWaves][kTopkListCap + 4];
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const long long stride = (long long)gridDim.x * kTopkWaves;
    const int need = top_k - 1;
    uint64_t* list = cand[wave];
    const long long row0 = (long long)blockIdx.x * kTopkWaves + wave;
    // the query position row % N is stepped along with the row: no division per row
    const int dt = (int)(stride % N);
    int t = (int)(row0 % N);
    // row pointers advance by a fixed stride: no 64-bit multiply per row (after the last
    // row they point past the arrays and are not used). Advancing integer offsets instead
    // measured 20% slower (0.396 against 0.327 ms at 128K), from the code layout alone.
    const float* src = pooled + row0 * nblk;
    int32_t* dst = block_idx + row0 * top_k;
    const long long src_step = stride * nblk, dst_step = stride * top_k;
    for (long long row = row0; row < rows;
         row += stride, t = t + dt >= N ? t + dt - N : t + dt, src += src_step, dst += dst_step) {
        const int cl = t >> 7;
        if (cl + 1 <= top_k) {  // every visible block
            for (int s = lane; s < top_k; s += 64) dst[s] = s <= cl ? s : -1;
            continue;
        }
        if (need == 0) {
            if (lane == 0) dst[0] = cl;
            continue;
        }
        topk_row_quads(src, cl, need, list, dst, lane);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

hipError_t launch_block_topk(const float* pooled, int32_t* block_idx, const Dims& d, hipStream_t stream) {
    const long long rows = (long long)d.B * d.Hkv * d.N;
    if (d.nblk - 1 <= kTopkRowMax && d.top_k <= 65) {
        // as many workgroups as are resident at once: each wave then walks its rows with
        // no second round of workgroups waiting for a slot
        // resident workgroups per CU: a property of the kernel, the same on every device of this build;
        // computed once (a racing first call computes the same value)
        static std::atomic<int> cached_per_cu{0};
        int per_cu = cached_per_cu.load(std::memory_order_relaxed);
        if (per_cu <= 0) {
            int n = 0;
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_block_topk_reg, 256, 0) != hipSuccess || n <= 0)
                n = 2;
            per_cu = n;
            cached_per_cu.store(n, std::memory_order_relaxed);
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
