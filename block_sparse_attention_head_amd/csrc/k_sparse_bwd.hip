// Backward of the main-branch sparse attention over cached block indices.
//
// [Flash-MSA] "Kernel Design" and "Backward": the block indices kept from the
// forward are reused, so the backward is linear in the sequence length; the
// map (query, slot) -> key block is inverted into key block -> queries and the
// work is scheduled by key block, each task streaming chunks of gathered query
// rows against one resident K/V block and producing dQ, dK and dV. [MSA
// summary] "GPU kernel co-design": per-slot preallocated outputs instead of
// atomic accumulation. Here the reverse index and work items are the
// forward's. With z = scale * q.k, P = exp(z - LSE) (LSE from the forward) and
// D = rowsum(dO * O):
//   dP = dO . v,  dS = P (dP - D),  dV = sum P dO,  dK = scale sum dS q,  dQ = scale sum dS k.
//
// Kernels:
//   k_bwd_delta       D for every (b, t, h) row.
//   k_bwd_main        one persistent workgroup per work item (a chunk of the
//                     rows gathered for one (key block, KV head) tile). Wave w
//                     owns keys 32w .. 32w+31 of the block and keeps their K, V
//                     as MFMA operands in registers. Per 32 gathered rows:
//                       S = Q K^T, dP = dO V^T    (rows x own keys, one lane per key)
//                       P, dS                      (bf16, dS also into LDS)
//                       dV += P^T dO, dK += dS^T Q (Q, dO staged transposed in LDS)
//                       dQ^T = K^T dS^T            (all 128 keys, own 32 dims)
//                     dQ rows go to bf16 per-(t, slot, head) partials (the
//                     forward's chunk-major record layout); dK, dV to one fp32
//                     partial per work item.
//   k_bwd_dq_sum      dQ = scale * sum of the valid slots' partials, to bf16.
//   k_bwd_dkdv_reduce dK, dV of each key block = sum of its items' partials, to
//                     bf16 (zero for blocks no query selected).
#include <utility>

#include "msa_device.hpp"
#include "msa_internal.hpp"

namespace msa {

// Position of index x inside a 32-wide transposed LDS line: bits 2 and 3
// swapped, so that the 8 rows one lane feeds to an MFMA k-step (the rows its
// score registers hold) are one 16-byte chunk. The map is its own inverse.
__device__ __forceinline__ int tpos(int x) { return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1); }

// ---------------------------------------------------------------------------
// D[row] = sum_d dO[row, d] * O[row, d], row = (b*N + t)*Hq + h; 16 lanes per row.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_bwd_delta(const __bf16* __restrict__ o, const __bf16* __restrict__ d_o,
                                                   float* __restrict__ delta, long long rows) {
    const long long row = (long long)blockIdx.x * 16 + (threadIdx.x >> 4);
    const int part = threadIdx.x & 15;
    float s = 0.0f;
    if (row < rows) {
        const bf16x8 a = *(const bf16x8*)(o + row * kDim + part * 8);
        const bf16x8 g = *(const bf16x8*)(d_o + row * kDim + part * 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) s += (float)a[e] * (float)g[e];
    }
#pragma unroll
    for (int m = 8; m > 0; m >>= 1) s += __shfl_xor(s, m, 16);
    if (row < rows && part == 0) delta[row] = s;
}

// ---------------------------------------------------------------------------
// Fused main backward.
//
// Per work item: the lane's own K and V rows go to registers; the block's K
// tile is staged row-major in LDS once and the lane's K^T fragments (A
// operands of dQ^T) are read from it with transposing LDS loads. Gathered
// rows go 32 at a time ("steps") through a ring of kBwdRing row-major LDS
// stages filled by direct global->LDS loads issued kBwdRing - 1 steps ahead
// (no registers held while they fly). The transposed Q^T / dO^T operands of
// dK, dV come from the same row-major stage through ds_read_b64_tr_b16. Step s:
//   (a) issue the loads of step s+3
//   (c) S = Q K^T, dP = dO V^T; P, dS (dS -> LDS)
//   (d) dV += P^T dO, dK += dS^T Q
//   (e) wait for step s+1's loads; barrier
//   (f) dQ^T rows = K^T dS^T -> bf16 partials
// ---------------------------------------------------------------------------
constexpr int kBwdRows = 32;                                   // gathered rows per step
constexpr int kBwdRing = 4;                                    // row-major stages
constexpr int kBwdMaxItemEntries = kRowTilesPerItem * kBlock;  // entries of one item when G = 1

typedef __attribute__((address_space(3))) void* lds_ptr;
typedef __attribute__((address_space(3))) bf16x4* lds_bf16x4_ptr;

// Row-major tiles with 128-element rows filled by global->LDS loads: chunk ch
// (8 elements) of row r sits at chunk slot ch ^ (r & 7). Eight consecutive rows
// read at one chunk fall into distinct banks, and most of the per-lane address
// stays independent of the chunk, so unrolled reads share base registers.
__device__ __forceinline__ int ring_off(int row, int ch) { return row * kDim + ((ch ^ (row & 7)) << 3); }

// dS rows [32][128] padded to 136 elements (272 bytes): consecutive rows shift by
// four banks, and every offset is a per-lane base plus a constant.
constexpr int kDsRow = kBlock + 8;

struct BwdRowStage {             // written by global->LDS loads
    __bf16 q[kBwdRows * kDim];   // Q rows [row][dim] (ring_off)
    __bf16 d[kBwdRows * kDim];   // dO rows
    float lse[kBwdRows];         // LSE of the row (natural log)
    float dlt[kBwdRows];         // D of the row; must follow lse
};

// ds_read_b64_tr_b16 on a row-major tile with 128-element rows (ring_off):
// inside each 16-lane group, lane li addresses row r0 + li/4, columns
// c0 + 4(li%4) .. +3, and receives column c0 + li of rows r0 .. r0+3 (checked
// on the device). c0 is a multiple of 16.
__device__ __forceinline__ bf16x4 tr_rows4(const __bf16* tile, int r0, int c0, int li) {
    const int row = r0 + (li >> 2), col = c0 + 4 * (li & 3);
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (lds_bf16x4_ptr)(tile + ring_off(row, col >> 3) + (col & 7)));
}
__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b) {
    return (bf16x8){a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// s_waitcnt with vmcnt <= n (n < 16) and no wait on the other counters (gfx9 encoding)
#define MSA_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (15 << 8))
// s_waitcnt lgkmcnt(0) only
#define MSA_WAIT_LGKM0() __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (3 << 14))

// Workgroup barrier for LDS data the caller has already waited for (lgkmcnt
// for its own LDS stores, vmcnt for its own global->LDS loads). A fenced
// barrier (__syncthreads, or a fence on LDS alone) waits for every outstanding
// vector-memory operation, because global->LDS loads write LDS; that would
// drain the row loads issued steps ahead. The memory clobber keeps the
// compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

// A 16-bit LDS store the compiler's wait insertion does not see. A plain LDS
// store made after global->LDS loads are issued makes the compiler wait for all
// of them (it cannot tell the destinations apart), which would drain the row
// prefetch every step. These stores go to a buffer no such load writes; the
// caller waits on lgkmcnt(0) before the barrier that publishes them.
template <int OFF>
__device__ __forceinline__ void lds_store_b16(uint32_t addr, uint32_t bits) {
    asm volatile("ds_write_b16 %0, %1 offset:%2" ::"v"(addr), "v"(bits), "i"(OFF) : "memory");
}
// The 16 dS values of a lane (score register i holds row mfma32_row(i, h)) into
// padded dS rows: byte address base + row(i, 0) * 2 * kDsRow, base covering the
// lane's key and its 4h row offset.
template <int... I>
__device__ __forceinline__ void store_ds16(uint32_t base, const uint32_t (&bits)[16], std::integer_sequence<int, I...>) {
    (lds_store_b16<(8 * (I >> 2) + (I & 3)) * 2 * kDsRow>(base, bits[I]), ...);
}

__global__ __launch_bounds__(256, 1) void k_bwd_main(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ d_o, const float* __restrict__ lse, const float* __restrict__ delta,
    const int32_t* __restrict__ off, const int32_t* __restrict__ item_off, const int32_t* __restrict__ entries,
    __bf16* __restrict__ dq_part, float* __restrict__ dkv_part, int N, int Hq, int Hkv, int gshift, int nblk,
    int top_k, int n_tiles, float scale, float scale_log2) {
    __shared__ __attribute__((aligned(16))) BwdRowStage ring[kBwdRing];         // also holds the K tile at item start
    __shared__ __attribute__((aligned(16))) __bf16 dsl[2][kBwdRows * kDsRow];  // dS [row][key], padded rows
    __shared__ int32_t ent[kBwdMaxItemEntries];                                 // this item's (t << 8 | slot)
    __shared__ __attribute__((aligned(16))) int32_t lims[2][kBwdRows];          // per step: last attended key per row
    static_assert(2 * sizeof(BwdRowStage) >= kBlock * kDim * sizeof(__bf16), "K tile must fit in two stages");

    const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in a scalar register
    const int li = lane & 15, dhalf = (lane >> 4) & 1;  // 16-lane group: lane in group, which 16 columns
    const int G = 1 << gshift;
    const int P = kBlock >> gshift;
    const int my_key = wave * 32 + l32;  // key of this lane inside the block
    const int total_items = item_off[n_tiles];
    const float log2e = 1.4426950408889634f;
    __bf16* ktile = ring[0].q;           // K [key][dim] during the item prologue

    for (int item = blockIdx.x; item < total_items; item += gridDim.x) {
        int lo = 0, hi = n_tiles;  // tile = last index with item_off[tile] <= item
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
        const int ne = min(rt1 * P, npos) - rt0 * P;  // entries of this item (>= 1)
        const int nrows = ne * G;
        const int nsteps = (nrows + kBwdRows - 1) / kBwdRows;
        const size_t tile_off = (((size_t)b * N + (size_t)c * kBlock) * Hkv + g) * kDim;
        const int kstride = Hkv * kDim;

        __syncthreads();  // the previous item's LDS reads are done
        for (int i = tid; i < ne; i += 256) ent[i] = entries[e0 + rt0 * P + i];
        // K tile -> LDS (row-major, swizzled through the source chunk): 8 x 4 rows per wave
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int row = 16 * i + 4 * wave + (lane >> 4);  // 128 rows over 8 x 4 waves x 4 rows
            const int ch = (lane & 15) ^ (row & 7);
            __builtin_amdgcn_global_load_lds((const void*)(k + tile_off + (size_t)row * kstride + ch * 8),
                                             (lds_ptr)(ktile + (16 * i + 4 * wave) * kDim), 16, 0, 0);
        }
        // own keys as B operands: lane holds K[my_key][16 kk + 8 h + e], same for V
        bf16x8 kf[8], vf[8];
        {
            const size_t krow = tile_off + (size_t)my_key * kstride + 8 * h;
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                kf[kk] = *(const bf16x8*)(k + krow + kk * 16);
                vf[kk] = *(const bf16x8*)(v + krow + kk * 16);
            }
            // keep these loop-invariant MFMA operands in accumulation registers (MFMA reads them
            // from there directly), leaving the vector registers to the step loop
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) asm volatile("" : "+a"(kf[kk]), "+a"(vf[kk]));
        }
        f32x16 dk[4], dv[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int i = 0; i < 16; ++i) dk[nt][i] = dv[nt][i] = 0.0f;
        MSA_WAIT_VMCNT(0);
        __syncthreads();  // ent, K tile
        // K^T fragments, A operands of dQ^T: lane holds K[16 kk + 8 h + e][32 wave + l32]
        bf16x8 ktf[8];
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
            ktf[kk] = cat8(tr_rows4(ktile, 16 * kk + 8 * h, 32 * wave + 16 * dhalf, li),
                           tr_rows4(ktile, 16 * kk + 8 * h + 4, 32 * wave + 16 * dhalf, li));
        __syncthreads();  // the K tile is read; the ring may be refilled

        // entry and head of gathered row r of this item (rows past the end read entry 0)
        auto row_src = [&](int r, bool& ok, int& t, int& slot, int& head) {
            ok = r < nrows;
            const int en = ent[ok ? (r >> gshift) : 0];
            t = en >> 8;
            slot = en & 255;
            head = g * G + (ok ? (r & (G - 1)) : 0);
        };
        // Step j's rows into ring[j % kBwdRing]: wave w loads rows 16u + 4w .. 16u + 4w + 3
        // of Q (u = 0, 1) and of dO, one 16-byte chunk per lane, the swizzle applied
        // through the source chunk; wave 0 then loads the rows' LSE and D.
        // Every wave issues exactly 4 vector-memory operations here, wave 0 one more.
        auto issue_step = [&](int j) {
            BwdRowStage& R = ring[j % kBwdRing];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rr = 16 * (i & 1) + 4 * wave + (lane >> 4);
                bool ok;
                int t, slot, head;
                row_src(j * kBwdRows + rr, ok, t, slot, head);
                const int ch = (lane & 15) ^ (rr & 7);
                const __bf16* src = (i >> 1 ? d_o : q) + (((size_t)b * N + t) * Hq + head) * kDim + ch * 8;
                __bf16* dst = (i >> 1 ? R.d : R.q) + (16 * (i & 1) + 4 * wave) * kDim;
                __builtin_amdgcn_global_load_lds((const void*)src, (lds_ptr)dst, 16, 0, 0);
            }
            if (wave == 0) {
                bool ok;
                int t, slot, head;
                row_src(j * kBwdRows + l32, ok, t, slot, head);
                const float* src = h == 0 ? lse + ((size_t)b * Hq + head) * N + t
                                          : delta + ((size_t)b * N + t) * Hq + head;
                __builtin_amdgcn_global_load_lds((const void*)src, (lds_ptr)R.lse, 4, 0, 0);
            }
        };

        // last key offset of the block that row j*32 + tid attends: its own position in its
        // own block, 127 elsewhere, -1 for rows past the end
        auto fill_lims = [&](int j) {
            if (tid < kBwdRows) {
                bool ok;
                int t, slot, head;
                row_src(j * kBwdRows + tid, ok, t, slot, head);
                lims[j & 1][tid] = !ok ? -1 : ((t >> 7) == c ? t - c * kBlock : kBlock - 1);
            }
        };

        const int ahead = min(kBwdRing - 1, nsteps);
        for (int j = 0; j < ahead; ++j) issue_step(j);
        fill_lims(0);
        MSA_WAIT_VMCNT(0);
        __syncthreads();

        for (int s = 0; s < nsteps; ++s) {
            const bool more = s + kBwdRing - 1 < nsteps;
            if (more) issue_step(s + kBwdRing - 1);  // (a)
            if (s + 1 < nsteps) fill_lims(s + 1);

            // (c) S = Q K^T, dP = dO V^T: 32 rows x this wave's 32 keys; register i holds row mfma32_row(i, h)
            const BwdRowStage& R = ring[s % kBwdRing];
            __bf16* ds_s = dsl[s & 1];
            f32x16 sa, pa;
#pragma unroll
            for (int i = 0; i < 16; ++i) sa[i] = pa[i] = 0.0f;
            {
                // all 16 operand loads in flight before the MFMA chain starts
                bf16x8 aq[8], ad[8];
#pragma unroll
                for (int kk = 0; kk < 8; ++kk) {
                    const int o2 = ring_off(l32, 2 * kk + h);
                    aq[kk] = *(const bf16x8*)(R.q + o2);
                    ad[kk] = *(const bf16x8*)(R.d + o2);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int kk = 0; kk < 8; ++kk) {
                    sa = mfma32(aq[kk], kf[kk], sa);
                    pa = mfma32(ad[kk], vf[kk], pa);
                }
            }
            bf16x8 pb[2], db[2];
            uint32_t dsbits[16];
#pragma unroll
            for (int j = 0; j < 4; ++j) {  // rows 8j + 4h + u
                const f32x4 l4 = *(const f32x4*)(R.lse + 8 * j + 4 * h);
                const f32x4 d4 = *(const f32x4*)(R.dlt + 8 * j + 4 * h);
                const int4 m4 = *(const int4*)(lims[s & 1] + 8 * j + 4 * h);
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int i = 4 * j + u;
                    const int lim = u == 0 ? m4.x : u == 1 ? m4.y : u == 2 ? m4.z : m4.w;
                    float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[i], scale_log2, -l4[u] * log2e));
                    if (my_key > lim) p = 0.0f;
                    const __bf16 dsv = (__bf16)(p * (pa[i] - d4[u]));
                    pb[i >> 3][i & 7] = (__bf16)p;
                    db[i >> 3][i & 7] = dsv;
                    dsbits[i] = (uint32_t)__builtin_bit_cast(uint16_t, dsv);
                }
            }
            store_ds16((uint32_t)(uintptr_t)(lds_ptr)(ds_s + 4 * h * kDsRow + my_key), dsbits,
                       std::make_integer_sequence<int, 16>{});
            // (d) dV += P^T dO, dK += dS^T Q: own keys x 128 dims, k = the 32 rows in the order
            // tpos(16 hs + 8 h + e) of the score registers, i.e. rows 16 hs + 4 h + {0..3} and
            // 16 hs + 8 + 4 h + {0..3}, read transposed from the row-major stage
#pragma unroll
            for (int hs = 0; hs < 2; ++hs) {
                bf16x8 bd[4], bq[4];
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
                    const int c0 = nt * 32 + 16 * dhalf;
                    bd[nt] = cat8(tr_rows4(R.d, 16 * hs + 4 * h, c0, li), tr_rows4(R.d, 16 * hs + 8 + 4 * h, c0, li));
                    bq[nt] = cat8(tr_rows4(R.q, 16 * hs + 4 * h, c0, li), tr_rows4(R.q, 16 * hs + 8 + 4 * h, c0, li));
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
                    dv[nt] = mfma32(pb[hs], bd[nt], dv[nt]);
                    dk[nt] = mfma32(db[hs], bq[nt], dk[nt]);
                }
            }
            // (e) step s+1's rows have landed: every memory operation before the loads of steps
            // s+2 and s+3 (issued in the last two (a) phases) is complete; then the barrier makes
            // all waves' LDS writes visible
            {
                const int per = wave == 0 ? 5 : 4;
                const int after = (s + kBwdRing - 2 < nsteps && s >= 1 ? per : 0) + (more ? per : 0);
                if (after == 0) MSA_WAIT_VMCNT(0);
                else if (after == 4) MSA_WAIT_VMCNT(4);
                else if (after == 5) MSA_WAIT_VMCNT(5);
                else if (after == 8) MSA_WAIT_VMCNT(8);
                else MSA_WAIT_VMCNT(10);
            }
            MSA_WAIT_LGKM0();  // this lane's dS stores (not tracked by the compiler) are done
            lds_barrier();

            // (f) dQ^T rows (unscaled) = K^T dS^T for dims 32 wave .. +31; lane l32 holds row l32
            f32x16 qa;
#pragma unroll
            for (int i = 0; i < 16; ++i) qa[i] = 0.0f;
            {
                bf16x8 bs[8];
#pragma unroll
                for (int kk = 0; kk < 8; ++kk) bs[kk] = *(const bf16x8*)(ds_s + l32 * kDsRow + (2 * kk + h) * 8);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int kk = 0; kk < 8; ++kk) qa = mfma32(ktf[kk], bs[kk], qa);
            }
            {
                bool ok;
                int t, slot, head;
                row_src(s * kBwdRows + l32, ok, t, slot, head);
                if (ok) {
                    // chunk-major partial record: [(b*N + t)*top_k + slot][16 chunks][Hq][8 dims]
                    __bf16* dst = dq_part + ((((size_t)b * N + t) * top_k + slot) * 16 * Hq + head) * 8 + 4 * h;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {  // dims 32 wave + 8 j + 4 h + u = chunk 4 wave + j
                        bf16x4 w;
#pragma unroll
                        for (int u = 0; u < 4; ++u) w[u] = (__bf16)qa[4 * j + u];
                        *(bf16x4*)(dst + (size_t)(4 * wave + j) * Hq * 8) = w;
                    }
                }
            }
        }

        // item partials [item][dK, dV][key][dim], fp32; dK carries the softmax scale
        float* pk = dkv_part + (size_t)item * 2 * kBlock * kDim;
        float* pv = pk + (size_t)kBlock * kDim;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = wave * 32 + mfma32_row(i, h), dim = nt * 32 + l32;
                pk[key * kDim + dim] = dk[nt][i] * scale;
                pv[key * kDim + dim] = dv[nt][i];
            }
    }
}

// ---------------------------------------------------------------------------
// dQ[b, t, h] = scale * sum over the valid slots of the partials; one workgroup per (b, t).
// A thread takes (chunk, head) pairs, so the reads of one slot's record are contiguous.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_bwd_dq_sum(const __bf16* __restrict__ dq_part,
                                                    const int32_t* __restrict__ block_idx, __bf16* __restrict__ dq,
                                                    int N, int Hq, int Hkv, int gshift, int top_k, float scale) {
    extern __shared__ int32_t sel[];  // [Hkv][top_k]
    const int tid = threadIdx.x, bt = blockIdx.x;
    const int b = bt / N, t = bt - b * N, cl = t >> 7;
    for (int i = tid; i < Hkv * top_k; i += 256) {
        const int g = i / top_k, s = i - g * top_k;
        sel[i] = block_idx[(((size_t)b * Hkv + g) * N + t) * top_k + s];
    }
    __syncthreads();
    const size_t slot_stride = (size_t)16 * Hq * 8;
    const __bf16* base = dq_part + (size_t)bt * top_k * slot_stride;
    for (int j = tid; j < Hq * 16; j += 256) {
        const int chunk = j / Hq, head = j - chunk * Hq;
        const int32_t* sg = sel + (head >> gshift) * top_k;
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
        for (int s = 0; s < top_k; ++s) {
            const int cc = sg[s];
            if (cc < 0 || cc > cl) continue;
            const bf16x8 a = *(const bf16x8*)(base + s * slot_stride + (size_t)j * 8);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += (float)a[e];
        }
        bf16x8 w;
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] = (__bf16)(acc[e] * scale);
        *(bf16x8*)(dq + ((size_t)bt * Hq + head) * kDim + chunk * 8) = w;
    }
}

// ---------------------------------------------------------------------------
// dK, dV of key block c (b, g): the sum of its items' partials; zero when no query selected it.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_bwd_dkdv_reduce(const float* __restrict__ dkv_part,
                                                         const int32_t* __restrict__ item_off,
                                                         __bf16* __restrict__ dk, __bf16* __restrict__ dv, int N,
                                                         int Hkv, int nblk) {
    const int tile = blockIdx.x;
    const int c = tile % nblk, bg = tile / nblk, g = bg % Hkv, b = bg / Hkv;
    const int i0 = item_off[tile], i1 = item_off[tile + 1];
    const size_t part = (size_t)kBlock * kDim;
    for (int e = threadIdx.x; e < kBlock * kDim / 4; e += 256) {  // 4 elements per unit
        f32x4 ak = {0.0f, 0.0f, 0.0f, 0.0f}, av = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int it = i0; it < i1; ++it) {
            ak += *(const f32x4*)(dkv_part + (size_t)it * 2 * part + e * 4);
            av += *(const f32x4*)(dkv_part + (size_t)it * 2 * part + part + e * 4);
        }
        const int key = (e * 4) / kDim, dim = (e * 4) % kDim;
        const size_t o = (((size_t)b * N + (size_t)c * kBlock + key) * Hkv + g) * kDim + dim;
        bf16x4 wk, wv;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            wk[u] = (__bf16)ak[u];
            wv[u] = (__bf16)av[u];
        }
        *(bf16x4*)(dk + o) = wk;
        *(bf16x4*)(dv + o) = wv;
    }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
size_t bwd_max_items(const Dims& d) {
    // an item holds up to kRowTilesPerItem row tiles of P = 128/G entries, so a
    // tile of cnt entries has ceil(ceil(cnt/P)/16) <= cnt/(16 P) + 1 items
    const size_t entries = (size_t)d.B * d.Hkv * d.N * d.top_k;
    const size_t per_item = (size_t)kRowTilesPerItem * (kBlock >> d.gshift);
    return (entries + per_item - 1) / per_item + (size_t)d.B * d.Hkv * d.nblk;
}

hipError_t launch_bwd_delta(const void* o, const void* d_o, float* delta, const Dims& d, hipStream_t stream) {
    const long long rows = (long long)d.B * d.N * d.Hq;
    hipLaunchKernelGGL(k_bwd_delta, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, stream, (const __bf16*)o,
                       (const __bf16*)d_o, delta, rows);
    return hipGetLastError();
}

hipError_t launch_bwd_main(const void* q, const void* k, const void* v, const void* d_o, const float* lse,
                           const BwdWs& ws, const Dims& d, hipStream_t stream) {
    const int n = d.B * d.Hkv * d.nblk;
    const int grid = device_cu_count();
    const float log2e = 1.4426950408889634f;
    hipLaunchKernelGGL(k_bwd_main, dim3(grid), dim3(256), 0, stream, (const __bf16*)q, (const __bf16*)k,
                       (const __bf16*)v, (const __bf16*)d_o, lse, ws.delta, ws.plan.off, ws.plan.item_off,
                       ws.plan.entries, (__bf16*)ws.dq_part, ws.dkv_part, d.N, d.Hq, d.Hkv, d.gshift, d.nblk, d.top_k, n,
                       d.scale, d.scale * log2e);
    return hipGetLastError();
}

hipError_t launch_bwd_dq_sum(const int32_t* block_idx, void* dq, const BwdWs& ws, const Dims& d,
                             hipStream_t stream) {
    const size_t lds = (size_t)d.Hkv * d.top_k * sizeof(int32_t);
    hipLaunchKernelGGL(k_bwd_dq_sum, dim3((unsigned)(d.B * d.N)), dim3(256), lds, stream, (const __bf16*)ws.dq_part, block_idx,
                       (__bf16*)dq, d.N, d.Hq, d.Hkv, d.gshift, d.top_k, d.scale);
    return hipGetLastError();
}

hipError_t launch_bwd_dkdv_reduce(void* dk, void* dv, const BwdWs& ws, const Dims& d, hipStream_t stream) {
    const int n = d.B * d.Hkv * d.nblk;
    hipLaunchKernelGGL(k_bwd_dkdv_reduce, dim3(n), dim3(256), 0, stream, ws.dkv_part, ws.plan.item_off,
                       (__bf16*)dk, (__bf16*)dv, d.N, d.Hkv, d.nblk);
    return hipGetLastError();
}

}  // namespace msa
