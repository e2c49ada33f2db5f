// Sparse main attention, KV-outer, in three phases.
//
// [MSA summary] "Architecture": every query head attends, with exact softmax,
// to the keys of the blocks its group selected (causal inside the local
// block). [MSA summary] "GPU kernel co-design": iterate over (key block,
// KV head) tiles rather than over queries, gather the queries that chose each
// tile (reverse sparse index), pack their positions x G heads into 128-row
// score tiles (query concatenation), run a persistent grid, write partial
// results into preallocated per-slot outputs (no atomic accumulation), and
// merge them in a second, global softmax-combine pass.
//
// Phase 1 (reverse index): count the queries per (b, g, c) tile, scan, and
//   scatter (t << 8 | slot) entries grouped by tile. A tile's work is cut into
//   items of up to kRowTilesPerItem row tiles of 128 rows.
// Phase 2 (k_sparse_partial): a persistent workgroup takes an item, stages K
//   and V^T of the tile in LDS once, and for each 128-row tile of gathered
//   queries computes S^T = K Q^T (one lane per query row), the row max, P in
//   bf16, O^T = V^T P^T, and writes O/l (bf16) and m*scale + ln l (fp32) to the
//   (t, slot, head) partial slot.
// Phase 3 (k_combine): per (b, t, head), merge the slot partials with the
//   online-softmax rule: M = max lse_s, w_s = exp(lse_s - M), L = sum w_s,
//   O = sum w_s O_s / L, LSE = M + ln L.
#include "msa_device.hpp"
#include "msa_internal.hpp"

namespace msa {

constexpr int kRowTilesPerItem = 16;
constexpr int kRevThreads = 256;
constexpr int kRevLdsBins = 8192;  // LDS histogram bins; larger nblk counts straight into global memory

__global__ __launch_bounds__(256) void k_fill_i32(int32_t* __restrict__ p, int32_t v, long long n) {
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256) p[i] = v;
}

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
    const int t = blockIdx.x * kRevThreads + threadIdx.x;
    if (t < N) {
        const int32_t* row = block_idx + ((size_t)bg * N + t) * top_k;
        const int cl = t >> 7;
        for (int s = 0; s < top_k; ++s) {
            const int c = row[s];
            if (c >= 0 && c <= cl) {
                if (use_lds) atomicAdd(&hist[c], 1);
                else atomicAdd(&cnt[(size_t)bg * nblk + c], 1);
            }
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

__global__ __launch_bounds__(kRevThreads) void k_rev_scatter(const int32_t* __restrict__ block_idx,
                                                             int32_t* __restrict__ cursor,
                                                             int32_t* __restrict__ entries, int N, int nblk,
                                                             int top_k) {
    const int bg = blockIdx.y;
    const int t = blockIdx.x * kRevThreads + threadIdx.x;
    if (t >= N) return;
    const int32_t* row = block_idx + ((size_t)bg * N + t) * top_k;
    const int cl = t >> 7;
    for (int s = 0; s < top_k; ++s) {
        const int c = row[s];
        if (c >= 0 && c <= cl) {
            const int p = atomicAdd(&cursor[(size_t)bg * nblk + c], 1);
            entries[p] = (t << 8) | s;
        }
    }
}

// Position p of a key inside a V^T row in LDS: bits 2 and 3 of the key index
// are swapped, so that the 8 keys a lane feeds to one PV MFMA step (the keys
// its S^T registers hold) sit in one 16-byte chunk. The map is its own inverse.
__device__ __forceinline__ int vt_pos(int key) {
    return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
}

__global__ __launch_bounds__(256, 2) void k_sparse_partial(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const int32_t* __restrict__ off, const int32_t* __restrict__ item_off, const int32_t* __restrict__ entries,
    __bf16* __restrict__ part_o, float* __restrict__ part_lse, int N, int Hq, int Hkv, int gshift, int nblk,
    int top_k, int n_tiles, float scale, float scale_log2) {
    __shared__ __attribute__((aligned(16))) __bf16 ks[kBlock * kDim];   // K[key][dim], swizzled
    __shared__ __attribute__((aligned(16))) __bf16 vts[kDim * kBlock];  // V^T[dim][vt_pos(key)], swizzled

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
    const int G = 1 << gshift;
    const int pos_per_tile = kBlock >> gshift;
    const int total_items = item_off[n_tiles];

    for (int item = blockIdx.x; item < total_items; item += gridDim.x) {
        // tile = the last index with item_off[tile] <= item
        int lo = 0, hi = n_tiles;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (item_off[mid] <= item) lo = mid;
            else hi = mid;
        }
        const int tile = lo;
        const int c = tile % nblk, bg = tile / nblk, g = bg % Hkv, b = bg / Hkv;
        const int e0 = off[tile], npos = off[tile + 1] - e0;
        const int n_rt = (npos + pos_per_tile - 1) / pos_per_tile;
        const int rt0 = (item - item_off[tile]) * kRowTilesPerItem;
        const int rt1 = min(rt0 + kRowTilesPerItem, n_rt);

        __syncthreads();  // the previous item's LDS reads are done
        {
            const __bf16* kbase = k + (((size_t)b * N + (size_t)c * kBlock) * Hkv + g) * kDim;
            const __bf16* vbase = v + (((size_t)b * N + (size_t)c * kBlock) * Hkv + g) * kDim;
            const size_t kstride = (size_t)Hkv * kDim;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int idx = tid + i * 256, key = idx >> 4, ch = idx & 15;
                *(uint4*)(ks + swz_chunk_offset(key, ch)) = *(const uint4*)(kbase + key * kstride + ch * 8);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int u = tid + i * 256, dc = u & 15, kg = u >> 4;  // 8 dims x 4 keys per unit
                bf16x8 rows[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) rows[r] = *(const bf16x8*)(vbase + (kg * 4 + r) * kstride + dc * 8);
                const int p0 = vt_pos(kg * 4);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int dim = dc * 8 + e;
                    bf16x4 w;
#pragma unroll
                    for (int r = 0; r < 4; ++r) w[r] = rows[r][e];
                    *(bf16x4*)(vts + swz_chunk_offset(dim, p0 >> 3) + (p0 & 7)) = w;
                }
            }
        }
        __syncthreads();

        for (int rt = rt0; rt < rt1; ++rt) {
            // Re-read the K / V^T operands from LDS in every row tile rather than
            // letting the compiler hoist all 64 of them into registers.
            asm volatile("" ::: "memory");
            const int r = wave * 32 + l32;  // row inside the 128-row tile
            const int pidx = rt * pos_per_tile + (r >> gshift);
            const int hh = r & (G - 1);
            const bool valid = pidx < npos;
            const int ent = valid ? entries[e0 + pidx] : 0;
            const int t = ent >> 8, slot = ent & 255;
            const int head = g * G + hh;

            bf16x8 qf[8];
            const __bf16* qrow = q + (((size_t)b * N + t) * Hq + head) * kDim;
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                if (valid) {
                    qf[kk] = *(const bf16x8*)(qrow + kk * 16 + 8 * h);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) qf[kk][e] = (__bf16)0.0f;
                }
            }

            f32x16 sacc[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int i = 0; i < 16; ++i) sacc[mt][i] = 0.0f;
#pragma unroll
            for (int kk = 0; kk < 8; ++kk)
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    const bf16x8 a = *(const bf16x8*)(ks + swz_chunk_offset(mt * 32 + l32, 2 * kk + h));
                    sacc[mt] = mfma32(a, qf[kk], sacc[mt]);
                }

            // causal mask inside the query's own block
            const bool diag = valid && (t >> 7) == c;
            if (__any(diag)) {
                const int lim = diag ? t - c * kBlock : kBlock - 1;
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        if (mt * 32 + mfma32_row(i, h) > lim) sacc[mt][i] = -INFINITY;
            }

            float m = -INFINITY;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int i = 0; i < 16; ++i) m = fmaxf(m, sacc[mt][i]);
            m = wave_max_xor32(m);

            // P = exp(scale * (s - m)) rounded to bf16 for the PV product. The LSE
            // uses the fp32 sum l; O is normalised by lb, the sum of the rounded
            // values, so the partial O is a convex combination of V rows.
            bf16x8 pf[8];
            float l = 0.0f, lb = 0.0f;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int half = 0; half < 2; ++half)
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float p = exp2f((sacc[mt][half * 8 + e] - m) * scale_log2);
                        const __bf16 pb = (__bf16)p;
                        l += p;
                        lb += (float)pb;
                        pf[mt * 2 + half][e] = pb;
                    }
            l += __shfl_xor(l, 32, 64);
            lb += __shfl_xor(lb, 32, 64);

            f32x16 oacc[4];
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int i = 0; i < 16; ++i) oacc[dt][i] = 0.0f;
#pragma unroll
            for (int kk = 0; kk < 8; ++kk)
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) {
                    const bf16x8 a = *(const bf16x8*)(vts + swz_chunk_offset(dt * 32 + l32, 2 * kk + h));
                    oacc[dt] = mfma32(a, pf[kk], oacc[dt]);
                }

            if (valid) {
                const float inv = 1.0f / lb;
                const size_t rec = (((size_t)b * N + t) * top_k + slot) * Hq + head;
                __bf16* dst = part_o + rec * kDim + h * 64;
#pragma unroll
                for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                    for (int i0 = 0; i0 < 16; i0 += 8) {
                        bf16x8 w;
#pragma unroll
                        for (int e = 0; e < 8; ++e) w[e] = (__bf16)(oacc[dt][i0 + e] * inv);
                        *(bf16x8*)(dst + dt * 16 + i0) = w;
                    }
                if (h == 0) part_lse[rec] = m * scale + logf(l);
            }
        }
    }
}

// Partial record layout: element q = hf*64 + dt*16 + i of a record holds
// dim 32*dt + 8*(i/4) + 4*hf + i%4 (the order the MFMA result registers are in).
__global__ __launch_bounds__(256) void k_combine(const __bf16* __restrict__ part_o, const float* __restrict__ part_lse,
                                                 const int32_t* __restrict__ block_idx, __bf16* __restrict__ o,
                                                 float* __restrict__ lse, int N, int Hq, int Hkv, int gshift,
                                                 int top_k) {
    const int bt = blockIdx.x;
    const int b = bt / N, t = bt - b * N;
    const int cl = t >> 7;
    for (int j = threadIdx.x; j < Hq * 16; j += 256) {
        const int head = j >> 4, ch = j & 15;
        const int g = head >> gshift;
        const int32_t* bi = block_idx + (((size_t)b * Hkv + g) * N + t) * top_k;
        const size_t rec0 = ((size_t)b * N + t) * top_k;
        float M = -INFINITY;
        for (int s = 0; s < top_k; ++s) {
            const int c = bi[s];
            if (c >= 0 && c <= cl) M = fmaxf(M, part_lse[(rec0 + s) * Hq + head]);
        }
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
        float L = 0.0f;
        if (M != -INFINITY) {
            for (int s = 0; s < top_k; ++s) {
                const int c = bi[s];
                if (c < 0 || c > cl) continue;
                const size_t rec = (rec0 + s) * Hq + head;
                const float w = expf(part_lse[rec] - M);
                L += w;
                const bf16x8 x = *(const bf16x8*)(part_o + rec * kDim + ch * 8);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] += w * (float)x[e];
            }
        }
        const float inv = L > 0.0f ? 1.0f / L : 0.0f;
        const int hf = ch >> 3, dt = (ch & 7) >> 1, i0 = (ch & 1) * 8;
        const int dim_a = 32 * dt + 2 * i0 + 4 * hf;  // elements 0..3 -> dim_a.., 4..7 -> dim_a+8..
        __bf16* orow = o + (((size_t)b * N + t) * Hq + head) * kDim;
        bf16x4 wa, wb;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            wa[e] = (__bf16)(acc[e] * inv);
            wb[e] = (__bf16)(acc[4 + e] * inv);
        }
        *(bf16x4*)(orow + dim_a) = wa;
        *(bf16x4*)(orow + dim_a + 8) = wb;
        if (ch == 0) lse[((size_t)b * Hq + head) * N + t] = M + logf(L);
    }
}

size_t sparse_ws_bytes(const Dims& d) {
    const size_t n = (size_t)d.B * d.Hkv * d.nblk;
    size_t s = 0;
    s += align_up(n * 4, 256);                                      // cnt
    s += align_up((n + 1) * 4, 256);                                // off
    s += align_up((n + 1) * 4, 256);                                // item_off
    s += align_up(n * 4, 256);                                      // cursor
    s += align_up((size_t)d.B * d.Hkv * d.N * d.top_k * 4, 256);    // entries
    s += align_up((size_t)d.B * d.N * d.top_k * d.Hq * kDim * 2, 256);  // part_o
    s += align_up((size_t)d.B * d.N * d.top_k * d.Hq * 4, 256);     // part_lse
    return s;
}

SparseWs carve_sparse_ws(void* base, const Dims& d) {
    const size_t n = (size_t)d.B * d.Hkv * d.nblk;
    char* p = (char*)base;
    SparseWs w;
    w.cnt = (int32_t*)p;      p += align_up(n * 4, 256);
    w.off = (int32_t*)p;      p += align_up((n + 1) * 4, 256);
    w.item_off = (int32_t*)p; p += align_up((n + 1) * 4, 256);
    w.cursor = (int32_t*)p;   p += align_up(n * 4, 256);
    w.entries = (int32_t*)p;  p += align_up((size_t)d.B * d.Hkv * d.N * d.top_k * 4, 256);
    w.part_o = (void*)p;      p += align_up((size_t)d.B * d.N * d.top_k * d.Hq * kDim * 2, 256);
    w.part_lse = (float*)p;
    return w;
}

hipError_t launch_sparse_plan(const int32_t* block_idx, const SparseWs& ws, const Dims& d, hipStream_t stream) {
    const int n = d.B * d.Hkv * d.nblk;
    hipLaunchKernelGGL(k_fill_i32, dim3((n + 255) / 256), dim3(256), 0, stream, ws.cnt, 0, (long long)n);
    const dim3 rgrid((d.N + kRevThreads - 1) / kRevThreads, d.B * d.Hkv);
    hipLaunchKernelGGL(k_rev_count, rgrid, dim3(kRevThreads), 0, stream, block_idx, ws.cnt, d.N, d.nblk, d.top_k);
    hipLaunchKernelGGL(k_rev_scan, dim3(1), dim3(1024), 0, stream, ws.cnt, ws.off, ws.item_off, ws.cursor, n,
                       kBlock >> d.gshift);
    hipLaunchKernelGGL(k_rev_scatter, rgrid, dim3(kRevThreads), 0, stream, block_idx, ws.cursor, ws.entries, d.N,
                       d.nblk, d.top_k);
    return hipGetLastError();
}

hipError_t launch_sparse_partial(const void* q, const void* k, const void* v, const SparseWs& ws, const Dims& d,
                                 hipStream_t stream) {
    const int n = d.B * d.Hkv * d.nblk;
    const int grid = 2 * device_cu_count();
    const float log2e = 1.4426950408889634f;
    hipLaunchKernelGGL(k_sparse_partial, dim3(grid), dim3(256), 0, stream, (const __bf16*)q, (const __bf16*)k,
                       (const __bf16*)v, ws.off, ws.item_off, ws.entries, (__bf16*)ws.part_o, ws.part_lse, d.N, d.Hq,
                       d.Hkv, d.gshift, d.nblk, d.top_k, n, d.scale, d.scale * log2e);
    return hipGetLastError();
}

hipError_t launch_sparse_combine(const int32_t* block_idx, void* o, float* lse, const SparseWs& ws, const Dims& d,
                                 hipStream_t stream) {
    hipLaunchKernelGGL(k_combine, dim3(d.B * d.N), dim3(256), 0, stream, (const __bf16*)ws.part_o, ws.part_lse,
                       block_idx, (__bf16*)o, lse, d.N, d.Hq, d.Hkv, d.gshift, d.top_k);
    return hipGetLastError();
}

}  // namespace msa
