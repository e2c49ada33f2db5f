// Reverse sparse index and tile work list for the KV-outer sparse attention.
//
// [Flash-MSA] "Backward": the map (batch, index head, query, slot) -> key block
// is inverted into (batch, index head, key block) -> the queries that use it.
// [MSA summary] "GPU kernel co-design": reverse sparse indexing of queries and
// pre-scheduled tile chunks for the persistent grid.
//
// The query positions of each (b, g) are cut into nwg consecutive ranges, one
// workgroup each. Entries (t << 8 | slot) are grouped by tile in a fixed order
// (position range, then position chunk of 256, then slot, then position), so
// the plan is a pure function of block_idx: the backward sums over a tile's
// rows in this order and is bitwise reproducible.
//   count:   per range, entries per tile (LDS histogram) -> wgcnt[bg][w][c];
//            the tile totals cnt[bg][c] by integer atomics;
//   scan:    exclusive prefix of the counts and of the work items per tile
//            (a tile of n queries is ceil(n / (128/G)) row tiles of 128 rows,
//            cut into items of up to kRowTilesPerItem row tiles);
//   wgoff:   in place, wgcnt[bg][w][c] -> off[tile] + sum over w' < w;
//   scatter: each range writes its entries from its own offsets, ranking equal
//            tiles inside a chunk by thread index (no atomics decide a slot): a
//            popcount of per-tile bit masks of thread indices up to kRevMaskBins
//            tiles, a scan over the lower threads' choices beyond (same order).
// Bins beyond the LDS capacity are handled in chunks of kRevLdsBins tiles.
//
// The forward does not need that order (every query row of a tile is computed
// on its own, so its results do not depend on where the row sits), and uses a
// cheaper unordered scatter: each range reserves one sub-range per touched tile
// with a single global atomic and hands out places from LDS counters. When the
// forward's combine computes each query's own block (combine_folds_local), the
// forward plan leaves those entries out.
#include "msa_device.hpp"
#include "msa_internal.hpp"

namespace msa {

constexpr int kRevThreads = 256;
constexpr int kRevLdsBins = 8192;  // tiles per LDS pass
constexpr int kRevMaxGroups = 256;  // position ranges per (b, g) at most

__global__ __launch_bounds__(256) void k_fill_i32(int32_t* __restrict__ p, int32_t v, long long n) {
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256) p[i] = v;
}

__device__ __forceinline__ bool valid_entry(int c, int t) { return c >= 0 && c <= (t >> 7); }
// With skip = 1 the query's own block is left out (the combine computes it).
__device__ __forceinline__ bool valid_entry(int c, int t, int skip) { return c >= 0 && c <= (t >> 7) - skip; }

int rev_positions_per_group(int N) {
    // 1024 positions per range, or more so that ranges <= 256 (at least one range)
    const int units = N > 0 ? (N + 1023) / 1024 : 1;
    return 1024 * ((units + kRevMaxGroups - 1) / kRevMaxGroups);
}
int rev_groups(int N) { return (N + rev_positions_per_group(N) - 1) / rev_positions_per_group(N); }

// wgcnt[(bg*nwg + w)*nblk + c] = entries of range w selecting tile c; cnt[bg*nblk + c] += the same.
__global__ __launch_bounds__(kRevThreads) void k_rev_count(const int32_t* __restrict__ block_idx,
                                                           int32_t* __restrict__ cnt, int32_t* __restrict__ wgcnt,
                                                           int N, int p0, int Nc, int nblk, int top_k, int ppw,
                                                           int skip) {
    __shared__ int32_t hist[kRevLdsBins];
    const int bg = blockIdx.y, w = blockIdx.x, nwg = gridDim.x;
    const int t0 = p0 + w * ppw, t1 = min(p0 + Nc, t0 + ppw);
    int32_t* mine = wgcnt + ((size_t)bg * nwg + w) * nblk;
    for (int c0 = 0; c0 < nblk; c0 += kRevLdsBins) {
        const int nb = min(kRevLdsBins, nblk - c0);
        for (int i = threadIdx.x; i < nb; i += kRevThreads) hist[i] = 0;
        __syncthreads();
        for (int t = t0 + threadIdx.x; t < t1; t += kRevThreads) {
            const int32_t* row = block_idx + ((size_t)bg * N + t) * top_k;
            for (int s = 0; s < top_k; ++s) {
                const int c = row[s];
                if (valid_entry(c, t, skip) && c >= c0 && c < c0 + nb) atomicAdd(&hist[c - c0], 1);
            }
        }
        __syncthreads();
        for (int i = threadIdx.x; i < nb; i += kRevThreads) {
            const int n = hist[i];
            mine[c0 + i] = n;
            if (n) atomicAdd(&cnt[(size_t)bg * nblk + c0 + i], n);
        }
        __syncthreads();
    }
}

// One workgroup: exclusive scans of the tile counts and of the work items per tile.
__global__ __launch_bounds__(1024) void k_rev_scan(const int32_t* __restrict__ cnt, int32_t* __restrict__ off,
                                                   int32_t* __restrict__ item_off, int32_t* __restrict__ cursor, int n,
                                                   int pos_per_tile) {
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

// In place: wgcnt[bg][w][c] becomes the first entry index of range w in tile (bg, c).
__global__ __launch_bounds__(256) void k_rev_wgoff(const int32_t* __restrict__ off, int32_t* __restrict__ wgcnt,
                                                   int n_tiles, int nblk, int nwg) {
    const int tile = blockIdx.x * 256 + threadIdx.x;
    if (tile >= n_tiles) return;
    const int bg = tile / nblk, c = tile - bg * nblk;
    int run = off[tile];
    for (int w = 0; w < nwg; ++w) {
        int32_t* p = wgcnt + ((size_t)bg * nwg + w) * nblk + c;
        const int k = *p;
        *p = run;
        run += k;
    }
}

// Range w of (b, g) writes its entries. Chunks of 256 positions are taken in
// order, slots in order inside a chunk; an entry's place in its tile is the
// tile's running offset plus the number of lower threads of the same chunk
// and slot that selected the same tile.
__global__ __launch_bounds__(kRevThreads) void k_rev_scatter(const int32_t* __restrict__ block_idx,
                                                             const int32_t* __restrict__ wgoff,
                                                             int32_t* __restrict__ entries, int N, int p0, int Nc,
                                                             int nblk, int top_k, int ppw) {
    __shared__ int32_t bins[kRevLdsBins];
    __shared__ __attribute__((aligned(16))) int32_t keys[kRevThreads];
    const int tid = threadIdx.x;
    const int bg = blockIdx.y, w = blockIdx.x, nwg = gridDim.x;
    const int t0 = p0 + w * ppw, t1 = min(p0 + Nc, t0 + ppw);
    const int32_t* base_off = wgoff + ((size_t)bg * nwg + w) * nblk;
    for (int c0 = 0; c0 < nblk; c0 += kRevLdsBins) {
        const int nb = min(kRevLdsBins, nblk - c0);
        __syncthreads();  // the previous bin chunk is done
        for (int i = tid; i < nb; i += kRevThreads) bins[i] = base_off[c0 + i];
        __syncthreads();
        for (int cb = t0; cb < t1; cb += kRevThreads) {  // uniform trip count
            const int t = cb + tid;
            const bool in = t < t1;
            const int32_t* row = block_idx + ((size_t)bg * N + (in ? t : t0)) * top_k;
            for (int s = 0; s < top_k; ++s) {
                const int c = in ? row[s] : -1;
                const bool ok = in && valid_entry(c, t) && c >= c0 && c < c0 + nb;
                keys[tid] = ok ? c : -1;
                __syncthreads();
                if (ok) {
                    int r = 0;
                    for (int j = 0; j < (tid & ~3); j += 4) {
                        const int4 kv = *(const int4*)(keys + j);
                        r += (kv.x == c) + (kv.y == c) + (kv.z == c) + (kv.w == c);
                    }
                    for (int j = tid & ~3; j < tid; ++j) r += keys[j] == c;
                    entries[bins[c - c0] + r] = (t << 8) | s;
                }
                __syncthreads();  // every place of this slot is taken from the old offsets
                if (ok) atomicAdd(&bins[c - c0], 1);
            }
        }
    }
}

// Unordered scatter (forward): places inside a tile come from atomics.
__global__ __launch_bounds__(kRevThreads) void k_rev_scatter_any(const int32_t* __restrict__ block_idx,
                                                                 int32_t* __restrict__ cursor,
                                                                 int32_t* __restrict__ entries, int N, int p0,
                                                                 int Nc, int nblk, int top_k, int ppw, int skip) {
    __shared__ int32_t bins[kRevLdsBins];
    const bool use_lds = nblk <= kRevLdsBins;
    const int bg = blockIdx.y, w = blockIdx.x;
    const int t0 = p0 + w * ppw, t1 = min(p0 + Nc, t0 + ppw);
    int32_t* cur = cursor + (size_t)bg * nblk;
    if (use_lds) {
        for (int i = threadIdx.x; i < nblk; i += kRevThreads) bins[i] = 0;
        __syncthreads();
        for (int t = t0 + threadIdx.x; t < t1; t += kRevThreads) {
            const int32_t* row = block_idx + ((size_t)bg * N + t) * top_k;
            for (int s = 0; s < top_k; ++s) {
                const int c = row[s];
                if (valid_entry(c, t, skip)) atomicAdd(&bins[c], 1);
            }
        }
        __syncthreads();
        for (int i = threadIdx.x; i < nblk; i += kRevThreads) {
            const int n = bins[i];
            bins[i] = n ? atomicAdd(&cur[i], n) : 0;
        }
        __syncthreads();
    }
    for (int t = t0 + threadIdx.x; t < t1; t += kRevThreads) {
        const int32_t* row = block_idx + ((size_t)bg * N + t) * top_k;
        for (int s = 0; s < top_k; ++s) {
            const int c = row[s];
            if (!valid_entry(c, t, skip)) continue;
            const int p = use_lds ? atomicAdd(&bins[c], 1) : atomicAdd(&cur[c], 1);
            entries[p] = (t << 8) | s;
        }
    }
}

// The same placement for key blocks up to kRevMaskBins (nblk <= 1024): a thread's rank
// among the chunk's threads that chose the same block for the same slot is the
// popcount of a per-block bit mask of thread indices below its own (set with LDS
// atomics, read after a barrier, cleared after the next one), instead of a scan over
// the lower threads' choices. Same order, so the same entries.
constexpr int kRevMaskBins = 1024;
__global__ __launch_bounds__(kRevThreads) void k_rev_scatter_mask(const int32_t* __restrict__ block_idx,
                                                                  const int32_t* __restrict__ wgoff,
                                                                  int32_t* __restrict__ entries, int N, int p0, int Nc,
                                                                  int nblk, int top_k, int ppw) {
    __shared__ int32_t bins[kRevMaskBins];
    __shared__ __attribute__((aligned(16))) uint32_t tmask[kRevMaskBins][kRevThreads / 32];
    const int tid = threadIdx.x;
    const int bg = blockIdx.y, w = blockIdx.x, nwg = gridDim.x;
    const int t0 = p0 + w * ppw, t1 = min(p0 + Nc, t0 + ppw);
    const int32_t* base_off = wgoff + ((size_t)bg * nwg + w) * nblk;
    for (int i = tid; i < nblk; i += kRevThreads) bins[i] = base_off[i];
    for (int i = tid; i < nblk * (kRevThreads / 32); i += kRevThreads) (&tmask[0][0])[i] = 0u;
    __syncthreads();
    const int word = tid >> 5;
    const uint32_t bit = 1u << (tid & 31);
    for (int cb = t0; cb < t1; cb += kRevThreads) {  // uniform trip count
        const int t = cb + tid;
        const bool in = t < t1;
        const int32_t* row = block_idx + ((size_t)bg * N + (in ? t : t0)) * top_k;
        for (int s = 0; s < top_k; ++s) {
            const int c = in ? row[s] : -1;
            const bool ok = in && valid_entry(c, t);
            if (ok) atomicOr(&tmask[c][word], bit);
            __syncthreads();
            if (ok) {
                int r = __popc(tmask[c][word] & (bit - 1u));
                for (int j = 0; j < word; ++j) r += __popc(tmask[c][j]);
                entries[bins[c] + r] = (t << 8) | s;
            }
            __syncthreads();  // every rank of this slot is taken from the old offsets and masks
            if (ok) {
                atomicAdd(&bins[c], 1);
                tmask[c][word] = 0u;
            }
            __syncthreads();  // the masks are clear for the next slot
        }
    }
}

hipError_t launch_sparse_plan(const int32_t* block_idx, const SparseWs& ws, const Dims& d, bool canonical,
                              hipStream_t stream) {
    const int n = d.B * d.Hkv * d.nblk;
    const int skip = (!canonical && combine_folds_local(d)) ? 1 : 0;  // the forward combine computes the local block
    const int ppw = rev_positions_per_group(d.Nc), nwg = rev_groups(d.Nc);
    hipLaunchKernelGGL(k_fill_i32, dim3((n + 255) / 256), dim3(256), 0, stream, ws.cnt, 0, (long long)n);
    const dim3 rgrid(nwg, d.B * d.Hkv);
    hipLaunchKernelGGL(k_rev_count, rgrid, dim3(kRevThreads), 0, stream, block_idx, ws.cnt, ws.wgoff, d.N, d.p0, d.Nc,
                       d.nblk, d.top_k, ppw, skip);
    hipLaunchKernelGGL(k_rev_scan, dim3(1), dim3(1024), 0, stream, ws.cnt, ws.off, ws.item_off, ws.cursor, n,
                       kBlock >> d.gshift);
    if (canonical) {
        hipLaunchKernelGGL(k_rev_wgoff, dim3((n + 255) / 256), dim3(256), 0, stream, ws.off, ws.wgoff, n, d.nblk,
                           nwg);
        if (d.nblk <= kRevMaskBins)
            hipLaunchKernelGGL(k_rev_scatter_mask, rgrid, dim3(kRevThreads), 0, stream, block_idx, ws.wgoff,
                               ws.entries, d.N, d.p0, d.Nc, d.nblk, d.top_k, ppw);
        else
            hipLaunchKernelGGL(k_rev_scatter, rgrid, dim3(kRevThreads), 0, stream, block_idx, ws.wgoff, ws.entries,
                               d.N, d.p0, d.Nc, d.nblk, d.top_k, ppw);
    } else {
        hipLaunchKernelGGL(k_rev_scatter_any, rgrid, dim3(kRevThreads), 0, stream, block_idx, ws.cursor, ws.entries,
                           d.N, d.p0, d.Nc, d.nblk, d.top_k, ppw, skip);
    }
    return hipGetLastError();
}

}  // namespace msa
