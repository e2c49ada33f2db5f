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
// A persistent workgroup takes a work item, stages K, V^T and the item's query
// entries in LDS once, and for each 128-row tile of gathered queries computes
// S^T = K Q^T (one lane per query row), the row max, P in bf16,
// O^T = V^T P^T, and writes O / sum(P) (bf16) and m*scale + ln(sum P) (fp32)
// to the (t, slot, head) slot. A partial record stores chunk-major over heads
// ([t, slot][16 chunks][H_q][8 dims]) so one store instruction writes G heads'
// chunks contiguously and the combine reads whole runs. Queries are loaded one row tile ahead.
#include "msa_device.hpp"
#include "msa_internal.hpp"

namespace msa {


// Position p of a key inside a V^T row in LDS: bits 2 and 3 of the key index
// are swapped, so that the 8 keys a lane feeds to one PV MFMA step (the keys
// its S^T registers hold) sit in one 16-byte chunk. The map is its own inverse.
__device__ __forceinline__ int vt_pos(int key) {
    return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
}

constexpr int kMaxItemEntries = kRowTilesPerItem * kBlock;  // positions of one item when G = 1

struct RowInfo {
    int t, slot;
    bool valid;
};

__global__ __launch_bounds__(256, 2) void k_sparse_partial(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const int32_t* __restrict__ off, const int32_t* __restrict__ item_off, const int32_t* __restrict__ entries,
    __bf16* __restrict__ part_o, float* __restrict__ part_lse, int N, int p0, int Nc, int Hq, int Hkv, int gshift,
    int nblk,
    int top_k, int n_tiles, float scale_log2) {
    __shared__ __attribute__((aligned(16))) __bf16 ks[kBlock * kDim];   // K[key][dim], swizzled
    __shared__ __attribute__((aligned(16))) __bf16 vts[kDim * kBlock];  // V^T[dim][vt_pos(key)], swizzled
    __shared__ int32_t ent[kMaxItemEntries];                            // this item's (t << 8 | slot)

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
    const int G = 1 << gshift;
    const int P = kBlock >> gshift;   // query positions per 128-row tile
    const int r = wave * 32 + l32;    // this lane's row inside a 128-row tile
    const int pslot = r >> gshift, hh = r & (G - 1);
    const int total_items = item_off[n_tiles];
    const float ln2 = 0.69314718055994531f;

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
        const int n_rt = (npos + P - 1) / P;
        const int rt0 = (item - item_off[tile]) * kRowTilesPerItem;
        const int rt1 = min(rt0 + kRowTilesPerItem, n_rt);
        const int ne = min(rt1 * P, npos) - rt0 * P;  // entries of this item

        __syncthreads();  // the previous item's LDS reads are done
        {
            // K rows go to ks[key][dim] (swizzled); V goes transposed to vts[dim][vt_pos(key)].
            // Per-thread offsets are one 32-bit base plus a per-step constant.
            const size_t tile_off = (((size_t)b * N + (size_t)c * kBlock) * Hkv + g) * kDim;
            const __bf16* kbase = k + tile_off;
            const __bf16* vbase = v + tile_off;
            const int kstride = Hkv * kDim;
            for (int i = tid; i < ne; i += 256) ent[i] = entries[e0 + rt0 * P + i];
            const int key0 = tid >> 4, ch = tid & 15;
            const int koff = key0 * kstride + ch * 8;
#pragma unroll
            for (int i = 0; i < 8; ++i) {  // keys key0 + 16 i
                const uint4 val = *(const uint4*)(kbase + koff + i * 16 * kstride);
                *(uint4*)(ks + swz_chunk_offset(key0 + 16 * i, ch)) = val;
            }
            const int voff = key0 * 4 * kstride + ch * 8;  // 4 keys 4*key0 + 64 i .. +3, dims 8 ch .. +7
            const int p0 = vt_pos(key0 * 4);               // < 64, a multiple of 4
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                bf16x8 rows[4];
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) rows[rr] = *(const bf16x8*)(vbase + voff + (64 * i + rr) * kstride);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    bf16x4 w;
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) w[rr] = rows[rr][e];
                    *(bf16x4*)(vts + swz_chunk_offset(ch * 8 + e, (p0 >> 3) + 8 * i) + (p0 & 7)) = w;
                }
            }
        }
        __syncthreads();

        // Row of row tile `rt` held by this lane. Rows past the item's last
        // entry read a valid query row (the item's first) and are never written.
        const size_t qhead = (size_t)g * G + hh;
        auto load_tile = [&](int rt, bf16x8 (&buf)[8], RowInfo& ri) {
            const int li = (rt - rt0) * P + pslot;
            ri.valid = li < ne;
            const int en = ent[ri.valid ? li : 0];
            ri.t = en >> 8;
            ri.slot = en & 255;
            const __bf16* qrow = q + (((size_t)b * N + ri.t) * Hq + qhead) * kDim + 8 * h;
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) buf[kk] = *(const bf16x8*)(qrow + kk * 16);
        };

        // One 128-row tile from `buf`; once S is computed, `buf` is refilled with
        // the next tile's queries, which land while this tile finishes.
        auto row_tile = [&](int rt, bf16x8 (&buf)[8], RowInfo& ri) {
            // Re-read the K / V^T operands from LDS in every row tile rather than
            // letting the compiler hoist all 64 of them into registers.
            asm volatile("" ::: "memory");
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
                    sacc[mt] = mfma32(a, buf[kk], sacc[mt]);
                }
            const RowInfo cur = ri;
            if (rt + 1 < rt1) load_tile(rt + 1, buf, ri);

            // causal mask inside the query's own block
            const bool diag = (cur.t >> 7) == c;
            if (__any(diag)) {
                // key = mt*32 + mfma32_row(i, h) > lim  <=>  mt*32 + mfma32_row(i, 0) > lim - 4h
                const int lim = (diag ? cur.t - c * kBlock : kBlock - 1) - 4 * h;
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        if (mt * 32 + mfma32_row(i, 0) > lim) sacc[mt][i] = -INFINITY;
            }

            float m = -INFINITY;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int i = 0; i < 16; ++i) m = fmaxf(m, sacc[mt][i]);
            m = wave_max_xor32(m);
            const float mb = m * scale_log2;

            // P = 2^(s*scale*log2e - m*scale*log2e): fp32 for the sum, bf16 for PV
            bf16x8 pf[8];
            float l = 0.0f;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int half = 0; half < 2; ++half)
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[mt][half * 8 + e], scale_log2, -mb));
                        l += pv;
                        pf[mt * 2 + half][e] = (__bf16)pv;
                    }
            l += __shfl_xor(l, 32, 64);
            const float inv = 1.0f / l;
            // partial O record layout: [(b*Nc + t - p0)*top_k + slot][chunk][head][8 dims], chunk = h*8 + dt*2 + i0/8
            const size_t rec2 = ((size_t)b * Nc + (cur.t - p0)) * top_k + cur.slot;
            __bf16* dst = part_o + ((rec2 * 16 + h * 8) * Hq + qhead) * 8;
            const size_t chunk_stride = (size_t)Hq * 8;

            // O^T = V^T P^T, 64 dims at a time: 128 dims x 32 rows per wave
#pragma unroll
            for (int dh = 0; dh < 2; ++dh) {
                f32x16 oacc[2];
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int i = 0; i < 16; ++i) oacc[j][i] = 0.0f;
#pragma unroll
                for (int kk = 0; kk < 8; ++kk)
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const int dt = dh * 2 + j;
                        const bf16x8 a = *(const bf16x8*)(vts + swz_chunk_offset(dt * 32 + l32, 2 * kk + h));
                        oacc[j] = mfma32(a, pf[kk], oacc[j]);
                    }
                if (cur.valid) {
#pragma unroll
                    for (int j = 0; j < 2; ++j)
#pragma unroll
                        for (int i0 = 0; i0 < 16; i0 += 8) {
                            bf16x8 w;
#pragma unroll
                            for (int e = 0; e < 8; ++e) w[e] = (__bf16)(oacc[j][i0 + e] * inv);
                            *(bf16x8*)(dst + ((dh * 2 + j) * 2 + i0 / 8) * chunk_stride) = w;
                        }
                }
            }
            if (cur.valid && h == 0) part_lse[rec2 * Hq + qhead] = (mb + __builtin_amdgcn_logf(l)) * ln2;
        };

        bf16x8 qa[8];
        RowInfo ra;
        load_tile(rt0, qa, ra);
        for (int rt = rt0; rt < rt1; ++rt) row_tile(rt, qa, ra);
    }
}

hipError_t launch_sparse_partial(const void* q, const void* k, const void* v, const SparseWs& ws, const Dims& d,
                                 hipStream_t stream) {
    const int n = d.B * d.Hkv * d.nblk;
    const int grid = 2 * device_cu_count();
    const float log2e = 1.4426950408889634f;
    hipLaunchKernelGGL(k_sparse_partial, dim3(grid), dim3(256), 0, stream, (const __bf16*)q, (const __bf16*)k,
                       (const __bf16*)v, ws.off, ws.item_off, ws.entries, (__bf16*)ws.part_o, ws.part_lse, d.N, d.p0,
                       d.Nc, d.Hq,
                       d.Hkv, d.gshift, d.nblk, d.top_k, n, d.scale * log2e);
    return hipGetLastError();
}

}  // namespace msa
