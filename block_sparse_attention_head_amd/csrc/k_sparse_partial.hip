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
// A persistent workgroup takes one contiguous run of work items (items of one
// tile are consecutive), stages K and V^T in LDS whenever the run enters a new
// tile, and for each 128-row tile of gathered queries computes S^T = K Q^T (one
// lane per query row), the row max, P in bf16, O^T = V^T P^T, and writes
// O / sum(P) (bf16) and m*scale + ln(sum P) (fp32) to the (t, slot, head) slot.
// A partial record stores each group's heads chunk-major ([t, slot][H_kv][16
// chunks][G][8 dims]): one store instruction writes G heads' chunks contiguously,
// and a group's part of a record is one contiguous G x 256-byte run for the
// combine. Queries are loaded one row tile ahead (across item and tile
// boundaries), their entries two row tiles ahead. When the combine folds in the
// query's own block, the plan leaves those (row, block) pairs out of this kernel.
#include "msa_device.hpp"
#include "msa_internal.hpp"

namespace msa {


struct RowInfo {
    int t, slot;
    bool valid;
};

// Where a workgroup is in its run of row tiles. All fields are wave-uniform.
struct Cursor {
    int item, tile, rt, rt1;  // work item, its (b, g, c) tile, row tile and the item's end
    int e0, npos;             // the tile's first entry and entry count
};

__global__ __launch_bounds__(256, 2) void k_sparse_partial(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const int32_t* __restrict__ off, const int32_t* __restrict__ item_off, const int32_t* __restrict__ entries,
    __bf16* __restrict__ part_o, float* __restrict__ part_lse, int N, int p0, int Nc, int Hq, int Hkv, int gshift,
    int nblk,
    int top_k, int n_tiles, int ipc, float scale_log2) {
    __shared__ __attribute__((aligned(16))) __bf16 ks[kBlock * kDim];   // K[key][dim], swizzled
    __shared__ __attribute__((aligned(16))) __bf16 vts[kDim * kBlock];  // V^T[dim][vt_pos(key)], swizzled

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
    const int G = 1 << gshift;
    const int P = kBlock >> gshift;   // query positions per 128-row tile
    const int r = wave * 32 + l32;    // this lane's row inside a 128-row tile
    const int pslot = r >> gshift, hh = r & (G - 1);
    const float ln2 = 0.69314718055994531f;

    // Work items are dealt to workgroups in runs of `ipc` consecutive items,
    // run j to workgroup j mod gridDim.x. Items of one tile are consecutive, so
    // K and V are staged only when a workgroup enters a new tile, and its row
    // tiles form one stream that is prefetched across item boundaries.
    const int it_end = item_off[n_tiles];
    const int it_begin = (int)blockIdx.x * ipc;
    auto seek = [&](int item, Cursor& cs) {
        cs.item = item;
        if (item >= it_end) return;
        // tile = the last index with item_off[tile] <= item
        int lo = 0, hi = n_tiles;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (item_off[mid] <= item) lo = mid;
            else hi = mid;
        }
        cs.tile = lo;
        cs.e0 = off[lo];
        cs.npos = off[lo + 1] - cs.e0;
        const int n_rt = (cs.npos + P - 1) / P;
        cs.rt = (item - item_off[lo]) * kRowTilesPerItem;
        cs.rt1 = min(cs.rt + kRowTilesPerItem, n_rt);
    };
    auto advance = [&](Cursor& cs) {
        if (cs.item >= it_end) return;
        if (++cs.rt < cs.rt1) return;
        const int nxt = cs.item + 1;
        seek(nxt % ipc ? nxt : nxt + ((int)gridDim.x - 1) * ipc, cs);
    };
    // This lane's entry (t << 8 | slot) in the cursor's row tile, or -1 past the end.
    auto fetch_entry = [&](const Cursor& cs) -> int {
        if (cs.item >= it_end) return -1;
        const int li = cs.rt * P + pslot;
        return li < cs.npos ? entries[cs.e0 + li] : -1;
    };
    // Stage K (row-major) and V^T of a tile in LDS; the caller has synchronised.
    auto stage_kv = [&](int tile) {
        const int c = tile % nblk, bg = tile / nblk, g = bg % Hkv, b = bg / Hkv;
        stage_kv_tile(k, v, ks, vts, b, g, c, N, Hkv, tid);
    };
    // Queries of one row tile: row t of the lane's head. Rows past the tile's
    // last entry read position c*128 (a valid row) and are never written.
    auto load_rows = [&](const Cursor& cs, int en, bf16x8 (&buf)[8], RowInfo& ri) {
        if (cs.item >= it_end) return;
        const int c = cs.tile % nblk, bg = cs.tile / nblk, g = bg % Hkv, b = bg / Hkv;
        ri.valid = en >= 0;
        ri.t = ri.valid ? (en >> 8) : c * kBlock;
        ri.slot = en & 255;
        const __bf16* qrow = q + (((size_t)b * N + ri.t) * Hq + (size_t)g * G + hh) * kDim + 8 * h;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) buf[kk] = *(const bf16x8*)(qrow + kk * 16);
    };

    Cursor cur, nx, nx2;
    seek(it_begin, cur);
    if (cur.item >= it_end) return;
    nx = cur;
    advance(nx);
    nx2 = nx;
    advance(nx2);
    bf16x8 qa[8];
    RowInfo ra;
    load_rows(cur, fetch_entry(cur), qa, ra);
    int en_next = fetch_entry(nx);  // entry of the next row tile; the one after is loaded a tile ahead
    int staged = -1;

    while (cur.item < it_end) {
        if (cur.tile != staged) {
            __syncthreads();  // the previous tile's LDS reads are done
            stage_kv(cur.tile);
            __syncthreads();
            staged = cur.tile;
        }
        const int c = cur.tile % nblk, bg = cur.tile / nblk, g = bg % Hkv, b = bg / Hkv;
        const size_t qhead = (size_t)g * G + hh;

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
                sacc[mt] = mfma32(a, qa[kk], sacc[mt]);
            }
        // The next row tile's queries land while this one finishes; its entry
        // was loaded a tile ago, and the entry after it is requested now.
        const RowInfo ri = ra;
        load_rows(nx, en_next, qa, ra);
        en_next = fetch_entry(nx2);

        // causal mask inside the query's own block
        const bool diag = (ri.t >> 7) == c;
        if (__any(diag)) {
            // key = mt*32 + mfma32_row(i, h) > lim  <=>  mt*32 + mfma32_row(i, 0) > lim - 4h
            const int lim = (diag ? ri.t - c * kBlock : kBlock - 1) - 4 * h;
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
        l = wave_sum_xor32(l);
        const float inv = 1.0f / l;
        // partial O record layout: [(b*Nc + t - p0)*top_k + slot][g][chunk][G heads][8 dims],
        // chunk = h*8 + dt*2 + i0/8
        const size_t rec2 = ((size_t)b * Nc + (ri.t - p0)) * top_k + ri.slot;
        __bf16* dst = part_o + rec2 * 16 * Hq * 8 + ((size_t)(g * 16 + h * 8) * G + hh) * 8;
        const size_t chunk_stride = (size_t)G * 8;

        // O^T = V^T P^T, 64 dims at a time: 128 dims x 32 rows per wave. The records
        // are read once, by the combine after this kernel, so they are written with
        // nontemporal stores that do not displace the K/V tiles other workgroups are
        // still reading (8% faster than plain stores at 128K tokens).
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
            if (ri.valid) {
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int i0 = 0; i0 < 16; i0 += 8) {
                        bf16x8 w;
#pragma unroll
                        for (int e = 0; e < 8; ++e) w[e] = (__bf16)(oacc[j][i0 + e] * inv);
                        __builtin_nontemporal_store(w, (bf16x8*)(dst + ((dh * 2 + j) * 2 + i0 / 8) * chunk_stride));
                    }
            }
        }
        if (ri.valid && h == 0)
            __builtin_nontemporal_store((mb + __builtin_amdgcn_logf(l)) * ln2, part_lse + rec2 * Hq + qhead);

        cur = nx;
        nx = nx2;
        advance(nx2);
    }
}

// Work items per run dealt to one workgroup: 4 measured a little faster than 1
// (a run per item) and than 16, and clearly faster than one run per workgroup,
// which leaves the concurrently running workgroups spread over far-apart tiles.
constexpr int kItemsPerRun = 4;

hipError_t launch_sparse_partial(const void* q, const void* k, const void* v, const SparseWs& ws, const Dims& d,
                                 hipStream_t stream) {
    const int n = d.B * d.Hkv * d.nblk;
    const int grid = 2 * device_cu_count();
    const float log2e = 1.4426950408889634f;
    hipLaunchKernelGGL(k_sparse_partial, dim3(grid), dim3(256), 0, stream, (const __bf16*)q, (const __bf16*)k,
                       (const __bf16*)v, ws.off, ws.item_off, ws.entries, (__bf16*)ws.part_o, ws.part_lse, d.N, d.p0,
                       d.Nc, d.Hq,
                       d.Hkv, d.gshift, d.nblk, d.top_k, n, kItemsPerRun, d.scale * log2e);
    return hipGetLastError();
}

}  // namespace msa
