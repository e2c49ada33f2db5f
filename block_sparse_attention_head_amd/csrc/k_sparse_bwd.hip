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
//   k_bwd_main        one persistent workgroup of 4 waves (one per SIMD) per
//                     CU walks the work items (a chunk of the rows gathered
//                     for one (key block, KV head) tile). Wave w owns keys
//                     32w .. 32w+31 of the block and keeps their K, V as MFMA
//                     operands in registers (16x16x32 bf16 MFMA throughout).
//                     Per 32 gathered rows (a "step", fetched into registers a
//                     step ahead and stored row-major into an LDS ring):
//                       S = Q K^T, dP = dO V^T    (rows x own keys)
//                       P, dS                      (bf16, dS also into LDS)
//                       dV += P^T dO, dK += dS^T Q (transposed operands read from
//                                                   the row-major tiles with
//                                                   ds_read_b64_tr_b16)
//                       dQ^T = K^T dS^T            (all 128 keys, own 32 dims)
//                     dQ rows go to bf16 per-(t, slot, head) partials, grouped
//                     by KV head; dK, dV to one fp32 partial per work item.
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
// One workgroup of 4 waves (one per SIMD, up to 512 registers each) per work
// item; wave w owns keys 32w .. 32w+31 of the block, keeps their K and V rows
// as MFMA operands in registers, and accumulates their dK, dV. Each wave reads
// the gathered rows once for its 32 keys, half the LDS traffic per key of 16.
// The block's K tile is staged row-major in LDS once per item and each wave
// reads its K^T fragments (A operands of dQ^T for dims 32w .. 32w+31) from it
// with transposing LDS loads. Gathered rows go 32 at a time ("steps"): step
// j's rows are fetched into registers late in step j - 2 and stored into
// ring[j % kBwdRing] late in step j - 1, before its barrier. Step s:
//   (c) S = Q K^T, dP = dO V^T (32 rows x 32 keys); P, dS (dS -> LDS)
//   (d) dV += P^T dO, dK += dS^T Q, with dO^T, Q^T read transposed from the stage
//   (a) store step s+1's rows into the ring, fetch step s+2's into registers
//   (e) barrier
//   (f) dQ^T (32 dims x 32 rows) = K^T dS^T over the block's 128 keys -> partials
// The LDS reads of each group of products are issued during the previous
// group's products. All MFMAs are 16x16x32.
// ---------------------------------------------------------------------------
constexpr int kBwdRows = 32;                                   // gathered rows per step
constexpr int kBwdRing = 4;                                    // row-major stages
constexpr int kBwdThreads = 256;                               // four waves, one per SIMD
constexpr int kBwdKeysPerWave = 32;                            // keys (and dQ dims) of one wave
constexpr int kBwdMaxItemEntries = kRowTilesPerItem * kBlock;  // entries of one item when G = 1

typedef __attribute__((address_space(3))) void* lds_ptr;
typedef __attribute__((address_space(3))) bf16x4* lds_bf16x4_ptr;

// Row-major tiles with 128-element rows: chunk ch
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

struct BwdRowStage {             // one step's gathered rows
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

// Scheduling: in the region that ends here, alternate M matrix instructions with one LDS
// read, N times, so the reads of the next group of operands issue while the current
// group's products run.
template <int N, int M>
__device__ __forceinline__ void interleave_mfma_ds_read() {
#pragma unroll
    for (int i = 0; i < N; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, M, 0);  // matrix instructions
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS reads
    }
    __builtin_amdgcn_sched_barrier(0);
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

// 16-bit LDS stores the compiler's wait insertion does not see. A plain LDS store
// made after global->LDS loads are issued makes the compiler wait for all of them (it
// cannot tell the destinations apart), which would drain the row prefetch every step.
// These stores go to a buffer no such load writes; the caller waits on lgkmcnt(0)
// before the barrier that publishes them. The _hi form stores the upper half of the
// register.
template <int OFF>
__device__ __forceinline__ void lds_store_lo16(uint32_t addr, uint32_t bits) {
    asm volatile("ds_write_b16 %0, %1 offset:%2" ::"v"(addr), "v"(bits), "i"(OFF) : "memory");
}
template <int OFF>
__device__ __forceinline__ void lds_store_hi16(uint32_t addr, uint32_t bits) {
    asm volatile("ds_write_b16_d16_hi %0, %1 offset:%2" ::"v"(addr), "v"(bits), "i"(OFF) : "memory");
}
// The 8 bf16 dS values of a lane, as the packed A operand holds them (element e of
// register pair j: e = 2j + half; element e is row 16 (e / 4) + e % 4 past the lane's 4 g4
// offset), into padded dS rows at byte address base + row * 2 * kDsRow.
__device__ __forceinline__ void store_ds8(uint32_t base, bf16x8 v) {
    const u32x4 w = __builtin_bit_cast(u32x4, v);
    lds_store_lo16<0 * 2 * kDsRow>(base, w.x);
    lds_store_hi16<1 * 2 * kDsRow>(base, w.x);
    lds_store_lo16<2 * 2 * kDsRow>(base, w.y);
    lds_store_hi16<3 * 2 * kDsRow>(base, w.y);
    lds_store_lo16<16 * 2 * kDsRow>(base, w.z);
    lds_store_hi16<17 * 2 * kDsRow>(base, w.z);
    lds_store_lo16<18 * 2 * kDsRow>(base, w.w);
    lds_store_hi16<19 * 2 * kDsRow>(base, w.w);
}

__global__ __launch_bounds__(256, 1) void k_bwd_main(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ d_o, const float* __restrict__ rowterm, long long rows,
    const int32_t* __restrict__ off, const int32_t* __restrict__ item_off, const int32_t* __restrict__ entries,
    __bf16* __restrict__ dq_part, __bf16* __restrict__ dq_sink, float* __restrict__ dkv_part, int N, int Hq,
    int Hkv, int gshift, int nblk, int top_k, int n_tiles, float scale, float scale_log2) {
    __shared__ __attribute__((aligned(16))) BwdRowStage ring[kBwdRing];         // also holds the K tile at item start
    __shared__ __attribute__((aligned(16))) __bf16 dsl[2][kBwdRows * kDsRow];  // dS [row][key], padded rows
    __shared__ int32_t ent_row[kBwdMaxItemEntries];  // per entry: (b*N + t)*Hq + g*G, the row of its first head
    __shared__ uint32_t ent_rec[kBwdMaxItemEntries];  // per entry: its dQ partial record times Hkv, plus g
    __shared__ int32_t ent_lim[kBwdMaxItemEntries];  // per entry: last key of the block its query attends
    static_assert(2 * sizeof(BwdRowStage) >= kBlock * kDim * sizeof(__bf16), "K tile must fit in two stages");

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in a scalar register
    const int l16 = lane & 15, g4 = lane >> 4;                   // MFMA lane in its 16-lane group, group
    const int G = 1 << gshift;
    const int P = kBlock >> gshift;
    const int kw0 = kBwdKeysPerWave * wave;  // this wave's first key (and first dQ dim)
    // within a (record, KV head) dQ partial: dims kw0 + 16 dt + 4 g4 .. +3 of head l16 % G (the
    // head's multiple of 16, for G > 16, is added per step)
    int dq_lane[2];
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) {
        const int dim = kw0 + 16 * dt + 4 * g4;
        dq_lane[dt] = (((dim >> 3) << gshift) + (l16 & ((1 << gshift) - 1))) * 8 + (dim & 7);
    }
    const int total_items = item_off[n_tiles];
    __bf16* ktile = ring[0].q;  // K [key][dim] during the item prologue

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
        for (int i = tid; i < ne; i += kBwdThreads) {
            const int en = entries[e0 + rt0 * P + i], t = en >> 8;
            ent_row[i] = (b * N + t) * Hq + g * G;
            ent_rec[i] = (uint32_t)((b * N + t) * top_k + (en & 255)) * (uint32_t)Hkv + (uint32_t)g;
            // the query's own position when it lies in this block (the causal diagonal), else 127
            ent_lim[i] = (t >> 7) == c ? t - c * kBlock : kBlock - 1;
        }
        // K tile -> LDS (row-major, swizzled through the source chunk): 8 x 4 rows per wave
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r0 = 32 * (i >> 1) + 8 * wave + 4 * (i & 1);
            const int row = r0 + (lane >> 4);
            const int ch = (lane & 15) ^ rsw(row);
            __builtin_amdgcn_global_load_lds((const void*)(k + tile_off + (size_t)row * kstride + ch * 8),
                                             (lds_ptr)(ktile + r0 * kDim), 16, 0, 0);
        }
        // own keys as B operands of S, dP: for key tile kt, lane holds K[kw0 + 16 kt + l16][32 kk + 8 g4 + e]
        bf16x8 kf[2][4], vf[2][4];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            const size_t krow = tile_off + (size_t)(kw0 + 16 * kt + l16) * kstride + 8 * g4;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                kf[kt][kk] = *(const bf16x8*)(k + krow + kk * 32);
                vf[kt][kk] = *(const bf16x8*)(v + krow + kk * 32);
            }
        }
        f32x4 dk[2][8], dv[2][8];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int nt = 0; nt < 8; ++nt)
#pragma unroll
                for (int i = 0; i < 4; ++i) dk[kt][nt][i] = dv[kt][nt][i] = 0.0f;
        MSA_WAIT_VMCNT(0);
        __syncthreads();  // ent, K tile
        // K^T fragments, A operands of dQ^T for dim tile dt: lane holds K[32 kk + 8 g4 + e][kw0 + 16 dt + l16]
        bf16x8 ktf[2][4];
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                ktf[dt][kk] = cat8(tr_rows4(ktile, 32 * kk + 8 * g4, kw0 + 16 * dt, l16),
                                   tr_rows4(ktile, 32 * kk + 8 * g4 + 4, kw0 + 16 * dt, l16));
        __syncthreads();  // the K tile is read; the ring may be refilled

        // Entry value (ent_row) of gathered row r, clamped to the item's last row: rows past
        // the end read a valid row (their P is 0 through the pad row term below).
        auto row_entry = [&](int r) -> int { return ent_row[min(r, nrows - 1) >> gshift]; };
        // Step j's rows: wave w fetches rows 8w .. 8w+7 of Q and of dO into registers, one
        // 16-byte chunk per lane, and wave 0 the rows' LSE * log2(e) and D (fetch_step); a
        // step later they are stored into ring[j % kBwdRing], the swizzle applied on the LDS
        // side (stash_step). Global->LDS loads are not used here: LDS reads issued after
        // them wait until they have written LDS. `ent` holds row_entry of the lane's rows
        // (h = 0, 1; then wave 0's row lane & 31), read beforehand.
        struct RowFetch {
            u32x4 q[2], d[2];
            float term;
        };
        auto fetch_step = [&](int j, const int (&ent)[3], RowFetch& f) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int rr = 8 * wave + 4 * h + (lane >> 4);
                const int r = min(j * kBwdRows + rr, nrows - 1);
                const int ri = ent[h] + (r & (G - 1));
                const size_t src = ((size_t)(uint32_t)ri << 7) + (lane & 15) * 8;
                f.q[h] = *(const u32x4*)(q + src);
                f.d[h] = *(const u32x4*)(d_o + src);
            }
            if (wave == 0) {
                const int r = j * kBwdRows + (lane & 31);
                const long long rt2 = r < nrows ? (long long)(ent[2] + (r & (G - 1))) : rows;  // padding: the pad row
                f.term = rowterm[(lane >> 5) * (rows + 1) + rt2];
            }
        };
        auto stash_step = [&](int j, const RowFetch& f) {
            BwdRowStage& R = ring[j % kBwdRing];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int rr = 8 * wave + 4 * h + (lane >> 4);
                const int o2 = ring_off(rr, lane & 15);
                *(u32x4*)(R.q + o2) = f.q[h];
                *(u32x4*)(R.d + o2) = f.d[h];
            }
            if (wave == 0) R.lse[lane] = f.term;  // lse[32] then dlt[32]
        };
        auto read_entries = [&](int j, int (&ent)[3]) {
#pragma unroll
            for (int h = 0; h < 2; ++h) ent[h] = row_entry(j * kBwdRows + 8 * wave + 4 * h + (lane >> 4));
            ent[2] = row_entry(j * kBwdRows + (lane & 31));  // used by wave 0
        };
        // The LDS reads of a step go in groups of at most eight operations, each issued one
        // group ahead of the products that use it (the compiler's wait before a use can only
        // leave 15 later LDS operations in flight).
        // Row operands of S (Q rows) and dP (dO rows) for row tile mt: rows 16 mt + l16,
        // dims 32 kk + 8 g4 + e
        auto load_rows = [&](const BwdRowStage& R, int mt, bf16x8 (&aq)[4], bf16x8 (&ad)[4]) {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int o2 = ring_off(16 * mt + l16, 4 * kk + g4);
                aq[kk] = *(const bf16x8*)(R.q + o2);
                ad[kk] = *(const bf16x8*)(R.d + o2);
            }
        };
        // The rows' LSE * log2(e), D and causal limits (rows 16 mt + 4 g4 .. +3) of step j;
        // padding rows take the last entry's limit (their P is 0 anyway)
        struct RowTerms {
            f32x4 l4[2], d4[2];
            int lim[2][4];
        };
        auto load_terms = [&](int j, RowTerms& rt) {
            const BwdRowStage& R = ring[j % kBwdRing];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                rt.l4[mt] = *(const f32x4*)(R.lse + 16 * mt + 4 * g4);
                rt.d4[mt] = *(const f32x4*)(R.dlt + 16 * mt + 4 * g4);
#pragma unroll
                for (int i = 0; i < 4; ++i) rt.lim[mt][i] = ent_lim[min(j * kBwdRows + 16 * mt + 4 * g4 + i, nrows - 1) >> gshift];
            }
        };
        // B operands of dV, dK for dim tiles n0, n0 + 1: the rows 4 g4 .. +3 and 16 + 4 g4 .. +3
        // of dO / Q at dim 16 n + l16, read transposed
        auto load_cols = [&](const BwdRowStage& R, int n0, bf16x8 (&bd)[2], bf16x8 (&bq)[2]) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int c0 = 16 * (n0 + u);
                bd[u] = cat8(tr_rows4(R.d, 4 * g4, c0, l16), tr_rows4(R.d, 16 + 4 * g4, c0, l16));
                bq[u] = cat8(tr_rows4(R.q, 4 * g4, c0, l16), tr_rows4(R.q, 16 + 4 * g4, c0, l16));
            }
        };

        // Step s + 1's rows are stored late in step s (before its barrier), from registers
        // fetched at the same point of step s - 1 (or in the prologue)
        int ent[3];
        RowFetch rf;
        read_entries(0, ent);
        fetch_step(0, ent, rf);
        stash_step(0, rf);
        if (nsteps > 1) {
            read_entries(1, ent);
            fetch_step(1, ent, rf);
        }
        __syncthreads();

        // step s's row terms, its first row tile's operands, the entries of step s + 2's rows
        // and of step s + 1's limits are read at the end of step s - 1
        RowTerms rtm;
        bf16x8 aq0[4], ad0[4], aq1[4], ad1[4];
        load_terms(0, rtm);
        read_entries(2, ent);
        load_rows(ring[0], 0, aq0, ad0);
        for (int s = 0; s < nsteps; ++s) {
            const BwdRowStage& R = ring[s % kBwdRing];
            __bf16* ds_s = dsl[s & 1];

            // (c) S = Q K^T, dP = dO V^T: 32 rows x this wave's 32 keys; for key tile kt,
            // register 4 mt + i holds row 16 mt + 4 g4 + i, column key kw0 + 16 kt + l16.
            // Row tile 0's operands were read at the end of the previous step; row tile 1's
            // are read during tile 0's products, the first dim tiles of (d) during tile 1's.
            f32x4 sa[2][2], pa[2][2];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) sa[mt][kt][i] = pa[mt][kt][i] = 0.0f;
            __builtin_amdgcn_sched_barrier(0);
            load_rows(R, 1, aq1, ad1);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                for (int kt = 0; kt < 2; ++kt) {
                    sa[0][kt] = mfma16(aq0[kk], kf[kt][kk], sa[0][kt]);
                    pa[0][kt] = mfma16(ad0[kk], vf[kt][kk], pa[0][kt]);
                }
            interleave_mfma_ds_read<8, 2>();
            bf16x8 bd0[2], bq0[2];
            load_cols(R, 0, bd0, bq0);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                for (int kt = 0; kt < 2; ++kt) {
                    sa[1][kt] = mfma16(aq1[kk], kf[kt][kk], sa[1][kt]);
                    pa[1][kt] = mfma16(ad1[kk], vf[kt][kk], pa[1][kt]);
                }
            interleave_mfma_ds_read<8, 2>();
            float pv[2][8];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        pv[kt][4 * mt + i] =
                            __builtin_amdgcn_exp2f(__builtin_fmaf(sa[mt][kt][i], scale_log2, -rtm.l4[mt][i]));
            // causal mask, only where some row of this wave's lanes lies on the diagonal
            bool diag = false;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) diag |= rtm.lim[mt][i] < kBlock - 1;
            if (__ballot(diag) != 0ull) {
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (kw0 + 16 * kt + l16 > rtm.lim[mt][i]) pv[kt][4 * mt + i] = 0.0f;
            }
            // P^T, dS^T as A operands of dV, dK: k index 8 g4 + e is row 4 g4 + e (e < 4)
            // and row 16 + 4 g4 + e - 4 (e >= 4), exactly the rows this lane holds
            bf16x8 pb[2], db[2];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        pb[kt][4 * mt + i] = (__bf16)pv[kt][4 * mt + i];
                        db[kt][4 * mt + i] = (__bf16)(pv[kt][4 * mt + i] * (pa[mt][kt][i] - rtm.d4[mt][i]));
                    }
            __builtin_amdgcn_sched_barrier(0);
            const uint32_t ds_base = (uint32_t)(uintptr_t)(lds_ptr)(ds_s + 4 * g4 * kDsRow + kw0 + l16);
            store_ds8(ds_base, db[0]);
            store_ds8(ds_base + 32, db[1]);
            __builtin_amdgcn_sched_barrier(0);
            // (d) dV += P^T dO, dK += dS^T Q: own 32 keys x 128 dims, two dim tiles per group,
            // each group's operands read during the previous group's products
            auto dkv_group = [&](int n0, const bf16x8 (&bd)[2], const bf16x8 (&bq)[2]) {
#pragma unroll
                for (int u = 0; u < 2; ++u)
#pragma unroll
                    for (int kt = 0; kt < 2; ++kt) {
                        dv[kt][n0 + u] = mfma16(pb[kt], bd[u], dv[kt][n0 + u]);
                        dk[kt][n0 + u] = mfma16(db[kt], bq[u], dk[kt][n0 + u]);
                    }
            };
            bf16x8 bd1[2], bq1[2];
            load_cols(R, 2, bd1, bq1);
            dkv_group(0, bd0, bq0);
            interleave_mfma_ds_read<8, 1>();
            load_cols(R, 4, bd0, bq0);
            dkv_group(2, bd1, bq1);
            interleave_mfma_ds_read<8, 1>();
            load_cols(R, 6, bd1, bq1);
            dkv_group(4, bd0, bq0);
            interleave_mfma_ds_read<8, 1>();
            dkv_group(6, bd1, bq1);
            __builtin_amdgcn_sched_barrier(0);
            // (a) step s + 1's rows (fetched a step ago) into LDS, then step s + 2's fetched: late
            // in the step, so the wait for the fetch also finds the previous step's dQ stores done
            if (s + 1 < nsteps) stash_step(s + 1, rf);
            if (s + 2 < nsteps) fetch_step(s + 2, ent, rf);
            // (e) the barrier makes all waves' LDS writes of this step (dS, step s + 1's rows)
            // visible
            MSA_WAIT_LGKM0();  // this lane's dS stores (not tracked by the compiler) are done
            lds_barrier();

            // (f) dQ^T (unscaled) = K^T dS^T for dims kw0 .. kw0 + 31 and the 32 rows; the next
            // step's row terms and first row tile (its rows landed before the barrier) are read
            // during the products
            bf16x8 bs[2][4];
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    bs[rt][kk] = *(const bf16x8*)(ds_s + (16 * rt + l16) * kDsRow + 32 * kk + 8 * g4);
            uint32_t rec[2];  // the dQ partial records (times Hkv, plus g) of this step's rows
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) rec[rt] = ent_rec[min(s * kBwdRows + 16 * rt + l16, nrows - 1) >> gshift];
            __builtin_amdgcn_sched_barrier(0);
            f32x4 qa[2][2];
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int dt = 0; dt < 2; ++dt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) qa[rt][dt][i] = 0.0f;
            // (read unconditionally, so the reads share the products' scheduling region; after the
            // last step they read stale LDS that is not used)
            load_rows(ring[(s + 1) % kBwdRing], 0, aq0, ad0);
            load_terms(s + 1, rtm);
            read_entries(s + 3, ent);  // fetched late in step s + 1
            // register i of qa[rt][dt] holds dim kw0 + 16 dt + 4 g4 + i of row 16 rt + l16
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                    for (int dt = 0; dt < 2; ++dt) qa[rt][dt] = mfma16(ktf[dt][kk], bs[rt][kk], qa[rt][dt]);
            interleave_mfma_ds_read<16, 1>();
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int dt = 0; dt < 2; ++dt) {
                    // partial record [(b*N + t)*top_k + slot][KV head][16 chunks][G heads][8 dims]: the
                    // four entries of a store each get two whole 128-byte lines (chunks 2i, 2i+1 of
                    // their group's heads). Rows past the end store to the sink. Below the (record,
                    // KV head) pair the offset is the lane's, plus the head's multiple of 16 (G > 16).
                    const int r = s * kBwdRows + 16 * rt + l16;
                    const int hx = (s * kBwdRows + 16 * rt) & (G - 1) & ~15;
                    __bf16* dst = r < nrows ? dq_part + ((size_t)rec[rt] << (7 + gshift)) + dq_lane[dt] + hx * 8
                                            : dq_sink;
                    bf16x4 w4;
#pragma unroll
                    for (int i = 0; i < 4; ++i) w4[i] = (__bf16)qa[rt][dt][i];
                    __builtin_nontemporal_store(w4, (bf16x4*)dst);  // read once, by k_bwd_dq_sum
                }
        }

        // item partials [item][dK, dV][key / 4][dim][key % 4], fp32; dK carries the softmax
        // scale. Tile (kt, nt) holds keys kw0 + 16 kt + 4 g4 .. +3 (its four registers) of dim
        // 16 nt + l16: one 16-byte store, and 16 lanes cover 256 contiguous bytes. Like the dQ
        // partials they are read once, by a later kernel: nontemporal stores.
        float* pk = dkv_part + (size_t)item * 2 * kBlock * kDim;
        float* pv2 = pk + (size_t)kBlock * kDim;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) {
                const int o = (((kw0 + 16 * kt + 4 * g4) >> 2) * kDim + 16 * nt + l16) * 4;
                __builtin_nontemporal_store(dk[kt][nt] * scale, (f32x4*)(pk + o));
                __builtin_nontemporal_store(dv[kt][nt], (f32x4*)(pv2 + o));
            }
    }
}

// ---------------------------------------------------------------------------
// dQ[b, t, h] = scale * sum over the valid slots of the partials; one workgroup per (b, t).
// Thread j takes the 8 dims at j * 8 of each record ([KV head][chunk][head in group][8]),
// so the reads of one slot's record are contiguous.
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
    const int G = 1 << gshift;
    for (int j = tid; j < Hq * 16; j += 256) {
        const int g = j >> (gshift + 4), chunk = (j >> gshift) & 15, head = g * G + (j & (G - 1));
        const int32_t* sg = sel + g * top_k;
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
    // a quarter of the block's values per workgroup (blockIdx.y), 4 elements per unit; the
    // partials are [key / 4][dim][key % 4], so unit e is the 16 bytes at e * 4
    const int e_end = (blockIdx.y + 1) * (kBlock * kDim / 16);
    for (int e = blockIdx.y * (kBlock * kDim / 16) + threadIdx.x; e < e_end; e += 256) {
        f32x4 ak = {0.0f, 0.0f, 0.0f, 0.0f}, av = {0.0f, 0.0f, 0.0f, 0.0f};
        int it = i0;
        // four items' partials requested at once, added in item order
        for (; it + 4 <= i1; it += 4) {
            f32x4 xk[4], xv[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                xk[u] = __builtin_nontemporal_load((const f32x4*)(dkv_part + (size_t)(it + u) * 2 * part + e * 4));
                xv[u] = __builtin_nontemporal_load((const f32x4*)(dkv_part + (size_t)(it + u) * 2 * part + part + e * 4));
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                ak += xk[u];
                av += xv[u];
            }
        }
        for (; it < i1; ++it) {
            ak += __builtin_nontemporal_load((const f32x4*)(dkv_part + (size_t)it * 2 * part + e * 4));
            av += __builtin_nontemporal_load((const f32x4*)(dkv_part + (size_t)it * 2 * part + part + e * 4));
        }
        // unit e holds keys 4 (e / 128) .. +3 of dim e % 128; consecutive threads write
        // consecutive dims of one key
        const int key0 = 4 * (e / kDim), dim = e % kDim;
        const size_t o = (((size_t)b * N + (size_t)c * kBlock + key0) * Hkv + g) * kDim + dim;
        const size_t key_stride = (size_t)Hkv * kDim;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            dk[o + u * key_stride] = (__bf16)ak[u];
            dv[o + u * key_stride] = (__bf16)av[u];
        }
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
    hipLaunchKernelGGL(k_bwd_main, dim3(grid), dim3(kBwdThreads), 0, stream, (const __bf16*)q, (const __bf16*)k,
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
