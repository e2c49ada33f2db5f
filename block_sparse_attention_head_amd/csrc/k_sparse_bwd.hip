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
//   k_bwd_delta       per (b, t, h) row: D and LSE * log2(e).
//   k_bwd_main        one persistent workgroup of 8 waves per CU walks the
//                     work items (a chunk of the rows gathered for one
//                     (key block, KV head) tile). Wave w owns keys 16w .. 16w+15
//                     of the block and keeps their K, V as MFMA operands in
//                     registers (16x16x32 bf16 MFMA throughout). Per 32
//                     gathered rows (a "step", staged row-major in an LDS ring
//                     by global->LDS loads three steps ahead):
//                       S = Q K^T, dP = dO V^T    (rows x own keys)
//                       P, dS                      (bf16, dS also into LDS)
//                       dV += P^T dO, dK += dS^T Q (transposed operands read from
//                                                   the row-major tiles with
//                                                   ds_read_b64_tr_b16)
//                       dQ^T = K^T dS^T            (all 128 keys, own 16 dims)
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
// Per-row terms of the main kernel, row = (b*N + t)*Hq + h, two planes of
// rows + 1 floats: plane 0 holds LSE * log2(e) (the LSE read from its [B, Hq, N]
// layout), plane 1 holds D = sum_d dO * O. Index `rows` of each plane is a pad
// row (+inf, 0) that padded step rows load: their P = exp2(-inf) = 0 exactly.
// 16 lanes per row.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_bwd_delta(const __bf16* __restrict__ o, const __bf16* __restrict__ d_o,
                                                   const float* __restrict__ lse, float* __restrict__ rowterm,
                                                   int N, int Hq, long long rows) {
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
    if (row < rows && part == 0) {
        const long long bt = row / Hq;
        const int h = (int)(row - bt * Hq);
        const long long b = bt / N;
        const int t = (int)(bt - b * N);
        rowterm[row] = lse[(b * Hq + h) * N + t] * 1.4426950408889634f;
        rowterm[rows + 1 + row] = s;
    }
    if (row == 0 && part == 0) {
        rowterm[rows] = __builtin_inff();
        rowterm[rows + 1 + rows] = 0.0f;
    }
}

// ---------------------------------------------------------------------------
// Fused main backward.
//
// One workgroup of 8 waves (two per SIMD) per work item; wave w owns keys
// 16w .. 16w+15 of the block, keeps their K and V rows as MFMA operands in
// registers, and accumulates their dK, dV. The block's K tile is staged
// row-major in LDS once per item and each wave reads its K^T fragments (A
// operands of dQ^T for dims 16w .. 16w+15) from it with transposing LDS loads.
// Gathered rows go 32 at a time ("steps") through a ring of kBwdRing row-major
// LDS stages filled by direct global->LDS loads issued kBwdRing - 1 steps
// ahead (no registers held while they fly). Step s:
//   (a) issue the loads of step s+3
//   (c) S = Q K^T, dP = dO V^T (32 rows x 16 keys); P, dS (dS -> LDS)
//   (d) dV += P^T dO, dK += dS^T Q, with dO^T, Q^T read transposed from the stage
//   (e) wait for step s+1's loads; barrier
//   (f) dQ^T (16 dims x 32 rows) = K^T dS^T over the block's 128 keys -> partials
// All MFMAs are 16x16x32.
// ---------------------------------------------------------------------------
constexpr int kBwdRows = 32;                                   // gathered rows per step
constexpr int kBwdRing = 4;                                    // row-major stages
constexpr int kBwdMaxItemEntries = kRowTilesPerItem * kBlock;  // entries of one item when G = 1

typedef __attribute__((address_space(3))) void* lds_ptr;
typedef __attribute__((address_space(3))) bf16x4* lds_bf16x4_ptr;

// Row-major tiles with 128-element rows filled by global->LDS loads: chunk ch
// (8 elements) of row r sits at chunk slot ch ^ rsw(r), rsw(r) = x ^ (2x & 14)
// for x = r & 15 (a bijection of 0..15). Chosen by measuring both read patterns
// of this kernel on the device, eight waves per CU: the 16-byte operand loads
// (sixteen rows at one chunk per 16 lanes) reach 186 B/clk per CU and the
// transposing loads 126 B/clk, against 109 and 107 B/clk with the two 2-bit
// halves of r & 15 swapped.
__device__ __forceinline__ int rsw(int r) { return (r & 15) ^ ((r << 1) & 14); }
__device__ __forceinline__ int ring_off(int row, int ch) { return row * kDim + ((ch ^ rsw(row)) << 3); }

// dS rows [32][128] padded to 136 elements (272 bytes): consecutive rows shift by
// four banks, and every offset is a per-lane base plus a constant.
constexpr int kDsRow = kBlock + 8;

struct BwdRowStage {             // written by global->LDS loads
    __bf16 q[kBwdRows * kDim];   // Q rows [row][dim] (ring_off)
    __bf16 d[kBwdRows * kDim];   // dO rows
    float lse[kBwdRows];         // LSE * log2(e) of the row (+inf for padding rows)
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
// The 8 dS values of a lane (register 4mt + i holds row 16mt + 4g + i) into
// padded dS rows: byte address base + (16mt + i) * 2 * kDsRow, base covering the
// lane's key and its 4g row offset.
template <int... I>
__device__ __forceinline__ void store_ds8(uint32_t base, const uint32_t (&bits)[8], std::integer_sequence<int, I...>) {
    (lds_store_b16<(16 * (I >> 2) + (I & 3)) * 2 * kDsRow>(base, bits[I]), ...);
}

__global__ __launch_bounds__(512, 1) void k_bwd_main(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ d_o, const float* __restrict__ rowterm, long long rows,
    const int32_t* __restrict__ off, const int32_t* __restrict__ item_off, const int32_t* __restrict__ entries,
    __bf16* __restrict__ dq_part, __bf16* __restrict__ dq_sink, float* __restrict__ dkv_part, int N, int Hq,
    int Hkv, int gshift, int nblk, int top_k, int n_tiles, float scale, float scale_log2) {
    __shared__ __attribute__((aligned(16))) BwdRowStage ring[kBwdRing];         // also holds the K tile at item start
    __shared__ __attribute__((aligned(16))) __bf16 dsl[2][kBwdRows * kDsRow];  // dS [row][key], padded rows
    __shared__ int32_t ent_row[kBwdMaxItemEntries];  // per entry: (b*N + t)*Hq + g*G, the row of its first head
    __shared__ int32_t ent_rec[kBwdMaxItemEntries];  // per entry: (b*N + t)*top_k + slot, its dQ partial record
    __shared__ __attribute__((aligned(16))) int32_t lims[2][kBwdRows];          // per step: last attended key per row
    __shared__ int32_t diagf[2];                                                // per step: some row is on the diagonal
    static_assert(2 * sizeof(BwdRowStage) >= kBlock * kDim * sizeof(__bf16), "K tile must fit in two stages");

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in a scalar register
    const int l16 = lane & 15, g4 = lane >> 4;                   // MFMA lane in its 16-lane group, group
    const int G = 1 << gshift;
    const int P = kBlock >> gshift;
    const int kw0 = 16 * wave;       // this wave's first key (and first dQ dim)
    const int my_key = kw0 + l16;    // key of this lane's S column
    const int total_items = item_off[n_tiles];
    __bf16* ktile = ring[0].q;       // K [key][dim] during the item prologue

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
        for (int i = tid; i < ne; i += 512) {
            const int en = entries[e0 + rt0 * P + i], t = en >> 8;
            ent_row[i] = (b * N + t) * Hq + g * G;
            ent_rec[i] = (b * N + t) * top_k + (en & 255);
        }
        // K tile -> LDS (row-major, swizzled through the source chunk): 4 x 4 rows per wave
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 32 * i + 4 * wave + (lane >> 4);
            const int ch = (lane & 15) ^ rsw(row);
            __builtin_amdgcn_global_load_lds((const void*)(k + tile_off + (size_t)row * kstride + ch * 8),
                                             (lds_ptr)(ktile + (32 * i + 4 * wave) * kDim), 16, 0, 0);
        }
        // own keys as B operands of S, dP: lane holds K[my_key][32 kk + 8 g4 + e], same for V
        bf16x8 kf[4], vf[4];
        {
            const size_t krow = tile_off + (size_t)my_key * kstride + 8 * g4;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                kf[kk] = *(const bf16x8*)(k + krow + kk * 32);
                vf[kk] = *(const bf16x8*)(v + krow + kk * 32);
            }
        }
        f32x4 dk[8], dv[8];
#pragma unroll
        for (int nt = 0; nt < 8; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) dk[nt][i] = dv[nt][i] = 0.0f;
        MSA_WAIT_VMCNT(0);
        __syncthreads();  // ent, K tile
        // K^T fragments, A operands of dQ^T: lane holds K[32 kk + 8 g4 + e][16 wave + l16]
        bf16x8 ktf[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            ktf[kk] = cat8(tr_rows4(ktile, 32 * kk + 8 * g4, kw0, l16), tr_rows4(ktile, 32 * kk + 8 * g4 + 4, kw0, l16));
        __syncthreads();  // the K tile is read; the ring may be refilled

        // Gathered row r of this item: its (b, t, head) row index into Q, dO and the row terms
        // (rows past the end read entry 0's first row), and its entry
        auto row_index = [&](int r, bool& ok) -> int {
            ok = r < nrows;
            return ok ? ent_row[r >> gshift] + (r & (G - 1)) : ent_row[0];
        };
        // Step j's rows into ring[j % kBwdRing]: wave w loads rows 4w .. 4w+3 of Q and of
        // dO, one 16-byte chunk per lane, the swizzle applied through the source chunk;
        // wave 0 then loads the rows' LSE * log2(e) and D. Every wave issues exactly 2
        // vector-memory operations here, wave 0 one more.
        auto issue_step = [&](int j) {
            BwdRowStage& R = ring[j % kBwdRing];
            const int rr = 4 * wave + (lane >> 4);
            bool ok;
            const int ri = row_index(j * kBwdRows + rr, ok);
            const int ch = (lane & 15) ^ rsw(rr);
            const size_t src = ((size_t)(uint32_t)ri << 7) + ch * 8;
            __builtin_amdgcn_global_load_lds((const void*)(q + src), (lds_ptr)(R.q + 4 * wave * kDim), 16, 0, 0);
            __builtin_amdgcn_global_load_lds((const void*)(d_o + src), (lds_ptr)(R.d + 4 * wave * kDim), 16, 0, 0);
            if (wave == 0) {
                const int ri2 = row_index(j * kBwdRows + (lane & 31), ok);
                const long long rt2 = ok ? (long long)ri2 : rows;  // padded rows: the pad row
                __builtin_amdgcn_global_load_lds((const void*)(rowterm + (lane >> 5) * (rows + 1) + rt2),
                                                 (lds_ptr)R.lse, 4, 0, 0);
            }
        };
        // Last key offset of the block that row j*32 + lane attends: its own position when the
        // row's query lies in this block (the causal diagonal), 127 otherwise (padding rows
        // need no limit: their P is 0). diagf[j & 1] says whether any row of step j is diagonal.
        auto fill_lims = [&](int j) {
            if (wave == 0) {
                int lim = kBlock - 1;
                if (lane < kBwdRows) {
                    const int r = j * kBwdRows + lane;
                    if (r < nrows) {
                        const int t = ent_row[r >> gshift] / Hq - b * N;
                        if ((t >> 7) == c) lim = t - c * kBlock;
                    }
                    lims[j & 1][lane] = lim;
                }
                const uint64_t m = __ballot(lim < kBlock - 1);
                if (lane == 0) diagf[j & 1] = m != 0ull;
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

            // (c) S = Q K^T, dP = dO V^T: 32 rows x this wave's 16 keys;
            // register 4 mt + i holds row 16 mt + 4 g4 + i, column key my_key
            const BwdRowStage& R = ring[s % kBwdRing];
            __bf16* ds_s = dsl[s & 1];
            f32x4 sa[2], pa[2];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) sa[mt][i] = pa[mt][i] = 0.0f;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                bf16x8 aq[4], ad[4];
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const int o2 = ring_off(16 * mt + l16, 4 * kk + g4);
                    aq[kk] = *(const bf16x8*)(R.q + o2);
                    ad[kk] = *(const bf16x8*)(R.d + o2);
                }
                __builtin_amdgcn_sched_barrier(0);  // all operand loads in flight before the MFMAs
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    sa[mt] = mfma16(aq[kk], kf[kk], sa[mt]);
                    pa[mt] = mfma16(ad[kk], vf[kk], pa[mt]);
                }
            }
            float pv[8];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                const f32x4 l4 = *(const f32x4*)(R.lse + 16 * mt + 4 * g4);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    pv[4 * mt + i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[mt][i], scale_log2, -l4[i]));
            }
            if (__builtin_amdgcn_readfirstlane(diagf[s & 1])) {  // causal mask on the diagonal rows
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) {
                    const int4 m4 = *(const int4*)(lims[s & 1] + 16 * mt + 4 * g4);
                    if (my_key > m4.x) pv[4 * mt + 0] = 0.0f;
                    if (my_key > m4.y) pv[4 * mt + 1] = 0.0f;
                    if (my_key > m4.z) pv[4 * mt + 2] = 0.0f;
                    if (my_key > m4.w) pv[4 * mt + 3] = 0.0f;
                }
            }
            // P^T, dS^T as A operands of dV, dK: k index 8 g4 + e is row 4 g4 + e (e < 4)
            // and row 16 + 4 g4 + e - 4 (e >= 4), exactly the rows this lane holds
            bf16x8 pb, db;
            uint32_t dsbits[8];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                const f32x4 d4 = *(const f32x4*)(R.dlt + 16 * mt + 4 * g4);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const __bf16 dsv = (__bf16)(pv[4 * mt + i] * (pa[mt][i] - d4[i]));
                    pb[4 * mt + i] = (__bf16)pv[4 * mt + i];
                    db[4 * mt + i] = dsv;
                    dsbits[4 * mt + i] = (uint32_t)__builtin_bit_cast(uint16_t, dsv);
                }
            }
            store_ds8((uint32_t)(uintptr_t)(lds_ptr)(ds_s + 4 * g4 * kDsRow + my_key), dsbits,
                      std::make_integer_sequence<int, 8>{});
            // (d) dV += P^T dO, dK += dS^T Q: own 16 keys x 128 dims; B operands are the rows
            // 4 g4 .. +3 and 16 + 4 g4 .. +3 of dO / Q at dim 16 nt + l16, read transposed
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                bf16x8 bd[4], bq[4];
#pragma unroll
                for (int n4 = 0; n4 < 4; ++n4) {
                    const int c0 = 16 * (4 * half + n4);
                    bd[n4] = cat8(tr_rows4(R.d, 4 * g4, c0, l16), tr_rows4(R.d, 16 + 4 * g4, c0, l16));
                    bq[n4] = cat8(tr_rows4(R.q, 4 * g4, c0, l16), tr_rows4(R.q, 16 + 4 * g4, c0, l16));
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int n4 = 0; n4 < 4; ++n4) {
                    dv[4 * half + n4] = mfma16(pb, bd[n4], dv[4 * half + n4]);
                    dk[4 * half + n4] = mfma16(db, bq[n4], dk[4 * half + n4]);
                }
            }
            // (e) step s+1's rows have landed: every memory operation before the loads of steps
            // s+2 and s+3 (issued in the last two (a) phases) is complete; then the barrier makes
            // all waves' LDS writes visible
            // Issued after those loads: the loads of (a) of step s-1, the two dQ stores of (f) of
            // step s-1, the loads of (a) of step s; they may stay in flight. The empty asm keeps the
            // compiler from sinking any of them below the wait.
            asm volatile("" ::: "memory");
            {
                const int per = wave == 0 ? 3 : 2;
                const int after = (s >= 1 && s + kBwdRing - 2 < nsteps ? per : 0) + (s >= 1 ? 2 : 0) + (more ? per : 0);
                switch (after) {
                    case 0: MSA_WAIT_VMCNT(0); break;
                    case 2: MSA_WAIT_VMCNT(2); break;
                    case 3: MSA_WAIT_VMCNT(3); break;
                    case 4: MSA_WAIT_VMCNT(4); break;
                    case 5: MSA_WAIT_VMCNT(5); break;
                    case 6: MSA_WAIT_VMCNT(6); break;
                    case 7: MSA_WAIT_VMCNT(7); break;
                    default: MSA_WAIT_VMCNT(8); break;
                }
            }
            MSA_WAIT_LGKM0();  // this lane's dS stores (not tracked by the compiler) are done
            lds_barrier();

            // (f) dQ^T (unscaled) = K^T dS^T for dims 16 wave .. +15 and the 32 rows;
            // register i holds dim 16 wave + 4 g4 + i of row 16 rt + l16
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                f32x4 qa = {0.0f, 0.0f, 0.0f, 0.0f};
                bf16x8 bs[4];
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    bs[kk] = *(const bf16x8*)(ds_s + (16 * rt + l16) * kDsRow + 32 * kk + 8 * g4);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) qa = mfma16(ktf[kk], bs[kk], qa);
                // chunk-major partial record: [(b*N + t)*top_k + slot][16 chunks][Hq][8 dims]. Rows
                // past the end store to the sink, so every step issues exactly two stores per lane
                // and the vmcnt accounting above stays exact.
                const int r = s * kBwdRows + 16 * rt + l16;
                const int dim = kw0 + 4 * g4;
                const int head = g * G + (r & (G - 1));
                __bf16* dst = r < nrows ? dq_part + ((size_t)ent_rec[r >> gshift] * 16 + (dim >> 3)) * Hq * 8 +
                                              head * 8 + (dim & 7)
                                        : dq_sink;
                bf16x4 w4;
#pragma unroll
                for (int i = 0; i < 4; ++i) w4[i] = (__bf16)qa[i];
                __builtin_nontemporal_store(w4, (bf16x4*)dst);  // read once, by k_bwd_dq_sum
            }
        }

        // item partials [item][dK, dV][key][dim], fp32; dK carries the softmax scale;
        // register i of tile nt holds key kw0 + 4 g4 + i, dim 16 nt + l16. Like the dQ
        // partials they are read once, by a later kernel: nontemporal stores.
        float* pk = dkv_part + (size_t)item * 2 * kBlock * kDim;
        float* pv2 = pk + (size_t)kBlock * kDim;
#pragma unroll
        for (int nt = 0; nt < 8; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = kw0 + 4 * g4 + i, dim = 16 * nt + l16;
                __builtin_nontemporal_store(dk[nt][i] * scale, pk + key * kDim + dim);
                __builtin_nontemporal_store(dv[nt][i], pv2 + key * kDim + dim);
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
            const bf16x8 a = __builtin_nontemporal_load((const bf16x8*)(base + s * slot_stride + (size_t)j * 8));
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
    // a quarter of the block's values per workgroup (blockIdx.y), 4 elements per unit
    const int e_end = (blockIdx.y + 1) * (kBlock * kDim / 16);
    for (int e = blockIdx.y * (kBlock * kDim / 16) + threadIdx.x; e < e_end; e += 256) {
        f32x4 ak = {0.0f, 0.0f, 0.0f, 0.0f}, av = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int it = i0; it < i1; ++it) {
            ak += __builtin_nontemporal_load((const f32x4*)(dkv_part + (size_t)it * 2 * part + e * 4));
            av += __builtin_nontemporal_load((const f32x4*)(dkv_part + (size_t)it * 2 * part + part + e * 4));
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

hipError_t launch_bwd_delta(const void* o, const void* d_o, const float* lse, float* rowterm, const Dims& d,
                            hipStream_t stream) {
    const long long rows = (long long)d.B * d.N * d.Hq;
    hipLaunchKernelGGL(k_bwd_delta, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, stream, (const __bf16*)o,
                       (const __bf16*)d_o, lse, rowterm, d.N, d.Hq, rows);
    return hipGetLastError();
}

hipError_t launch_bwd_main(const void* q, const void* k, const void* v, const void* d_o, const BwdWs& ws,
                           const Dims& d, hipStream_t stream) {
    const int n = d.B * d.Hkv * d.nblk;
    const int grid = device_cu_count();
    const float log2e = 1.4426950408889634f;
    hipLaunchKernelGGL(k_bwd_main, dim3(grid), dim3(512), 0, stream, (const __bf16*)q, (const __bf16*)k,
                       (const __bf16*)v, (const __bf16*)d_o, ws.rowterm, (long long)d.B * d.N * d.Hq, ws.plan.off,
                       ws.plan.item_off,
                       ws.plan.entries, (__bf16*)ws.dq_part,
                       (__bf16*)ws.dq_part + (size_t)d.B * d.N * d.top_k * d.Hq * kDim, ws.dkv_part, d.N, d.Hq, d.Hkv, d.gshift, d.nblk, d.top_k, n,
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
    hipLaunchKernelGGL(k_bwd_dkdv_reduce, dim3(n, 4), dim3(256), 0, stream, ws.dkv_part, ws.plan.item_off,
                       (__bf16*)dk, (__bf16*)dv, d.N, d.Hkv, d.nblk);
    return hipGetLastError();
}

}  // namespace msa
