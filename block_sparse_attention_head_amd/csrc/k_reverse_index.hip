// Reverse sparse index and tile work list for the KV-outer sparse attention.
//
// [Flash-MSA] "Backward": the map (batch, index head, query, slot) -> key block
// is inverted into (batch, index head, key block) -> the queries that use it.
// [MSA summary] "GPU kernel co-design": reverse sparse indexing of queries and
// pre-scheduled tile chunks for the persistent grid.
//
// count: queries per (b, g, c) tile (LDS histogram per workgroup);
// scan:  exclusive prefix of the counts and of the work items per tile
//        (a tile of n queries is ceil(n / (128/G)) row tiles of 128 rows, cut
//        into items of up to kRowTilesPerItem row tiles);
// scatter: (t << 8 | slot) entries grouped by tile. Each workgroup reserves one
//        range per tile it touches with a single global atomic and fills it
//        from LDS counters. The order inside a tile is not fixed, and nothing
//        downstream depends on it: every query row is computed on its own.
#include "msa_device.hpp"
#include "msa_internal.hpp"

namespace msa {

constexpr int kRevThreads = 256;
constexpr int kRevLdsBins = 8192;  // LDS histogram bins; larger nblk counts straight into global memory

__global__ __launch_bounds__(256) void k_fill_i32(int32_t* __restrict__ p, int32_t v, long long n) {
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256) p[i] = v;
}

constexpr int kRevPosPerGroup = 1024;  // query positions per workgroup (4 per thread)

__device__ __forceinline__ bool valid_entry(int c, int t) { return c >= 0 && c <= (t >> 7); }

// cnt[(b*Hkv + g)*nblk + c] += number of queries t whose row selects block c (valid entries only).
__global__ __launch_bounds__(kRevThreads) void k_rev_count(const int32_t* __restrict__ block_idx,
                                                           int32_t* __restrict__ cnt, int N, int nblk, int top_k) {
    __shared__ int32_t hist[kRevLdsBins];
    const bool use_lds = nblk <= kRevLdsBins;
    const int bg = blockIdx.y;
    if (use_lds) {
        for (int i = threadIdx.x; i < nblk; i += kRevThreads) hist[i] = 0;
        __syncthreads();
    }
    for (int q = 0; q < kRevPosPerGroup / kRevThreads; ++q) {
        const int t = blockIdx.x * kRevPosPerGroup + q * kRevThreads + threadIdx.x;
        if (t >= N) break;
        const int32_t* row = block_idx + ((size_t)bg * N + t) * top_k;
        for (int s = 0; s < top_k; ++s) {
            const int c = row[s];
            if (!valid_entry(c, t)) continue;
            if (use_lds) atomicAdd(&hist[c], 1);
            else atomicAdd(&cnt[(size_t)bg * nblk + c], 1);
        }
    }
    if (use_lds) {
        __syncthreads();
        for (int i = threadIdx.x; i < nblk; i += kRevThreads)
            if (hist[i]) atomicAdd(&cnt[(size_t)bg * nblk + i], hist[i]);
    }
}

// One workgroup: exclusive scans of the tile counts and of the work items per tile.
__global__ __launch_bounds__(1024) void k_rev_scan(const int32_t* __restrict__ cnt, int32_t* __restrict__ off,
                                                   int32_t* __restrict__ item_off, int32_t* __restrict__ cursor,
                                                   int n, int pos_per_tile) {
    __shared__ int32_t s_a[1024];
    __shared__ int32_t s_b[1024];
    const int tid = threadIdx.x;
    const int per = (n + 1023) / 1024;
    const int lo = min(n, tid * per), hi = min(n, lo + per);
    int sa = 0, sb = 0;
    for (int i = lo; i < hi; ++i) {
        const int c = cnt[i];
        const int rt = (c + pos_per_tile - 1) / pos_per_tile;
        sa += c;
        sb += (rt + kRowTilesPerItem - 1) / kRowTilesPerItem;
    }
    s_a[tid] = sa;
    s_b[tid] = sb;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {  // inclusive Hillis-Steele scan
        const int va = tid >= d ? s_a[tid - d] : 0;
        const int vb = tid >= d ? s_b[tid - d] : 0;
        __syncthreads();
        s_a[tid] += va;
        s_b[tid] += vb;
        __syncthreads();
    }
    int ra = s_a[tid] - sa, rb = s_b[tid] - sb;  // exclusive base of this thread's range
    for (int i = lo; i < hi; ++i) {
        const int c = cnt[i];
        const int rt = (c + pos_per_tile - 1) / pos_per_tile;
        off[i] = ra;
        cursor[i] = ra;
        item_off[i] = rb;
        ra += c;
        rb += (rt + kRowTilesPerItem - 1) / kRowTilesPerItem;
    }
    if (tid == 1023) {
        off[n] = s_a[1023];
        item_off[n] = s_b[1023];
    }
}

// Each workgroup counts its entries per tile in LDS, reserves one contiguous
// range per touched tile with a single global atomic, then hands out slots in
// that range from LDS counters.
__global__ __launch_bounds__(kRevThreads) void k_rev_scatter(const int32_t* __restrict__ block_idx,
                                                             int32_t* __restrict__ cursor,
                                                             int32_t* __restrict__ entries, int N, int nblk,
                                                             int top_k) {
    __shared__ int32_t bins[kRevLdsBins];
    const bool use_lds = nblk <= kRevLdsBins;
    const int bg = blockIdx.y;
    int32_t* cur = cursor + (size_t)bg * nblk;
    if (use_lds) {
        for (int i = threadIdx.x; i < nblk; i += kRevThreads) bins[i] = 0;
        __syncthreads();
        for (int q = 0; q < kRevPosPerGroup / kRevThreads; ++q) {
            const int t = blockIdx.x * kRevPosPerGroup + q * kRevThreads + threadIdx.x;
            if (t >= N) break;
            const int32_t* row = block_idx + ((size_t)bg * N + t) * top_k;
            for (int s = 0; s < top_k; ++s) {
                const int c = row[s];
                if (valid_entry(c, t)) atomicAdd(&bins[c], 1);
            }
        }
        __syncthreads();
        for (int i = threadIdx.x; i < nblk; i += kRevThreads) {
            const int n = bins[i];
            bins[i] = n ? atomicAdd(&cur[i], n) : 0;
        }
        __syncthreads();
    }
    for (int q = 0; q < kRevPosPerGroup / kRevThreads; ++q) {
        const int t = blockIdx.x * kRevPosPerGroup + q * kRevThreads + threadIdx.x;
        if (t >= N) break;
        const int32_t* row = block_idx + ((size_t)bg * N + t) * top_k;
        for (int s = 0; s < top_k; ++s) {
            const int c = row[s];
            if (!valid_entry(c, t)) continue;
            const int p = use_lds ? atomicAdd(&bins[c], 1) : atomicAdd(&cur[c], 1);
            entries[p] = (t << 8) | s;
        }
    }
}

hipError_t launch_sparse_plan(const int32_t* block_idx, const SparseWs& ws, const Dims& d, hipStream_t stream) {
    const int n = d.B * d.Hkv * d.nblk;
    hipLaunchKernelGGL(k_fill_i32, dim3((n + 255) / 256), dim3(256), 0, stream, ws.cnt, 0, (long long)n);
    const dim3 rgrid((d.N + kRevPosPerGroup - 1) / kRevPosPerGroup, d.B * d.Hkv);
    hipLaunchKernelGGL(k_rev_count, rgrid, dim3(kRevThreads), 0, stream, block_idx, ws.cnt, d.N, d.nblk, d.top_k);
    hipLaunchKernelGGL(k_rev_scan, dim3(1), dim3(1024), 0, stream, ws.cnt, ws.off, ws.item_off, ws.cursor, n,
                       kBlock >> d.gshift);
    hipLaunchKernelGGL(k_rev_scatter, rgrid, dim3(kRevThreads), 0, stream, block_idx, ws.cursor, ws.entries, d.N,
                       d.nblk, d.top_k);
    return hipGetLastError();
}

}  // namespace msa
