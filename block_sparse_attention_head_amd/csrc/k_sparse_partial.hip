// Sparse main attention, phase 1: KV-outer partial attention.
//
// [MSA summary] "Architecture": every query head attends, with exact softmax,
// to the keys of the blocks its group selected (causal inside the local
// block). [MSA summary] "GPU kernel co-design": iterate over (key block,
// KV head) tiles rather than over queries, gather the queries that chose each
// tile, pack their positions x G heads into 128-row score tiles (query
// concatenation), run a persistent grid, and write partial results into
// preallocated per-slot outputs (no atomic accumulation).
//
// A persistent workgroup takes a work item, stages K and V^T of the tile in LDS
// once, and for each 128-row tile of gathered queries computes S^T = K Q^T (one
// lane per query row), the row max, P in bf16, O^T = V^T P^T, and writes
// O/sum(P) (bf16) and m*scale + ln(sum exp) (fp32) to the (t, slot, head) slot.
#include "msa_device.hpp"
#include "msa_internal.hpp"

namespace msa {


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

}  // namespace msa
