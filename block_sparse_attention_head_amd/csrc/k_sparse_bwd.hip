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
//                     (and the K^T slice for dims 32w .. 32w+31) as MFMA
//                     operands in registers. Per 32 gathered rows:
//                       S = Q K^T, dP = dO V^T    (rows x own keys, one lane per key)
//                       P, dS                      (bf16, dS also into LDS)
//                       dV += P^T dO, dK += dS^T Q (Q, dO staged transposed in LDS)
//                       dQ_rows = dS K             (all 128 keys, own 32 dims)
//                     dQ rows go to fp32 per-(t, slot, head) partials; dK, dV
//                     to one fp32 partial per work item.
//   k_bwd_dq_sum      dQ = scale * sum of the valid slots' partials, to bf16.
//   k_bwd_dkdv_reduce dK, dV of each key block = sum of its items' partials, to
//                     bf16 (zero for blocks no query selected).
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
// ---------------------------------------------------------------------------
constexpr int kBwdRows = 32;                                   // gathered rows per step
constexpr int kBwdMaxItemEntries = kRowTilesPerItem * kBlock;  // entries of one item when G = 1

// 64-byte lines of 32 bf16 (4 chunks); chunk ch of line r sits at ch ^ ((r >> 1) & 3).
__device__ __forceinline__ int tline_offset(int r, int ch) { return r * kBwdRows + ((ch ^ ((r >> 1) & 3)) << 3); }

struct BwdStage {
    __bf16 qr[kBwdRows * kDim];  // Q rows [row][dim] (swz_chunk_offset)
    __bf16 dr[kBwdRows * kDim];  // dO rows
    __bf16 qt[kDim * kBwdRows];  // Q^T [dim][tpos(row)] (tline_offset)
    __bf16 dt[kDim * kBwdRows];  // dO^T
    float lse2[kBwdRows];        // LSE * log2(e)
    float dlt[kBwdRows];         // D
    int lim[kBwdRows];           // last key offset of the block the row attends (127 off its own block, -1 padding)
    int rec[kBwdRows];           // (b*N + t)*top_k + slot of the row, -1 padding
};

// One step's rows held in registers between their global loads and their LDS stores.
struct BwdPrefetch {
    uint4 qv[2], dv[2];  // row-major chunks
    bf16x8 tr[4];        // 4 rows x 8 dims of Q or dO, for the transposed copy
    float lse2, dlt;
    int lim, rec;
};

__global__ __launch_bounds__(256, 1) void k_bwd_main(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ d_o, const float* __restrict__ lse, const float* __restrict__ delta,
    const int32_t* __restrict__ off, const int32_t* __restrict__ item_off, const int32_t* __restrict__ entries,
    float* __restrict__ dq_part, float* __restrict__ dkv_part, int N, int Hq, int Hkv, int gshift, int nblk,
    int top_k, int n_tiles, float scale, float scale_log2) {
    __shared__ __attribute__((aligned(16))) BwdStage st;
    __shared__ __attribute__((aligned(16))) __bf16 dsl[kBwdRows * kBlock];  // dS [row][key] (swz_chunk_offset)
    __shared__ __attribute__((aligned(16))) __bf16 kts[kDim * kBlock];       // K^T [dim][key] (swz_chunk_offset)
    __shared__ int32_t ent[kBwdMaxItemEntries];                              // this item's (t << 8 | slot)

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
    const int G = 1 << gshift;
    const int P = kBlock >> gshift;
    const int my_key = wave * 32 + l32;  // key of this lane inside the block
    const int total_items = item_off[n_tiles];
    const float log2e = 1.4426950408889634f;

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
        // K^T of the block: 4 keys x 8 dims per unit, 512 units
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int unit = tid + 256 * u, kg = unit >> 4, dc = unit & 15;
            bf16x8 rows[4];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
                rows[rr] = *(const bf16x8*)(k + tile_off + (size_t)(kg * 4 + rr) * kstride + dc * 8);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                bf16x4 w;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) w[rr] = rows[rr][e];
                *(bf16x4*)(kts + swz_chunk_offset(dc * 8 + e, kg >> 1) + ((kg & 1) << 2)) = w;
            }
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
        }
        f32x16 dk[4], dv[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int i = 0; i < 16; ++i) dk[nt][i] = dv[nt][i] = 0.0f;
        __syncthreads();  // ent, kts
        // K^T slice as the B operand of dQ: lane holds K[16 kk + 8 h + e][32 wave + l32]
        bf16x8 ktf[8];
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) ktf[kk] = *(const bf16x8*)(kts + swz_chunk_offset(32 * wave + l32, 2 * kk + h));

        // entry and head of gathered row r of this item
        auto row_src = [&](int r, bool& ok, int& t, int& slot, int& head) {
            ok = r < nrows;
            const int en = ent[ok ? (r >> gshift) : 0];
            t = en >> 8;
            slot = en & 255;
            head = g * G + (ok ? (r & (G - 1)) : 0);
        };
        auto load_step = [&](int s, BwdPrefetch& pf) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int idx = tid + 256 * u, rr = idx >> 4, ch = idx & 15;
                bool ok;
                int t, slot, head;
                row_src(s * kBwdRows + rr, ok, t, slot, head);
                const size_t a = (((size_t)b * N + t) * Hq + head) * kDim + ch * 8;
                pf.qv[u] = *(const uint4*)(q + a);
                pf.dv[u] = *(const uint4*)(d_o + a);
                if (!ok) pf.qv[u] = pf.dv[u] = make_uint4(0, 0, 0, 0);
            }
            {
                const int which = tid >> 7, u = tid & 127, rg = u >> 4, dc = u & 15;
                const __bf16* src = which ? d_o : q;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    bool ok;
                    int t, slot, head;
                    row_src(s * kBwdRows + rg * 4 + rr, ok, t, slot, head);
                    pf.tr[rr] = *(const bf16x8*)(src + (((size_t)b * N + t) * Hq + head) * kDim + dc * 8);
                    if (!ok)
#pragma unroll
                        for (int e = 0; e < 8; ++e) pf.tr[rr][e] = (__bf16)0.0f;
                }
            }
            if (tid < kBwdRows) {
                bool ok;
                int t, slot, head;
                row_src(s * kBwdRows + tid, ok, t, slot, head);
                pf.lse2 = ok ? lse[((size_t)b * Hq + head) * N + t] * log2e : 0.0f;
                pf.dlt = ok ? delta[((size_t)b * N + t) * Hq + head] : 0.0f;
                pf.lim = !ok ? -1 : ((t >> 7) == c ? t - c * kBlock : kBlock - 1);
                pf.rec = ok ? ((b * N + t) * top_k + slot) : -1;
            }
        };
        auto store_step = [&](const BwdPrefetch& pf) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int idx = tid + 256 * u, rr = idx >> 4, ch = idx & 15;
                *(uint4*)(st.qr + swz_chunk_offset(rr, ch)) = pf.qv[u];
                *(uint4*)(st.dr + swz_chunk_offset(rr, ch)) = pf.dv[u];
            }
            {
                const int which = tid >> 7, u = tid & 127, rg = u >> 4, dc = u & 15;
                __bf16* dstT = which ? st.dt : st.qt;
                const int p0 = tpos(rg * 4);  // rows 4rg .. 4rg+3 sit at p0 .. p0+3
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    bf16x4 w;
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) w[rr] = pf.tr[rr][e];
                    *(bf16x4*)(dstT + tline_offset(dc * 8 + e, p0 >> 3) + (p0 & 7)) = w;
                }
            }
            if (tid < kBwdRows) {
                st.lse2[tid] = pf.lse2;
                st.dlt[tid] = pf.dlt;
                st.lim[tid] = pf.lim;
                st.rec[tid] = pf.rec;
            }
        };

        BwdPrefetch pf;
        load_step(0, pf);
        store_step(pf);
        __syncthreads();

        for (int s = 0; s < nsteps; ++s) {
            if (s + 1 < nsteps) load_step(s + 1, pf);

            // S = Q K^T, dP = dO V^T: 32 rows x this wave's 32 keys; register i holds row mfma32_row(i, h)
            f32x16 sa, pa;
#pragma unroll
            for (int i = 0; i < 16; ++i) sa[i] = pa[i] = 0.0f;
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                const int o2 = swz_chunk_offset(l32, 2 * kk + h);
                sa = mfma32(*(const bf16x8*)(st.qr + o2), kf[kk], sa);
                pa = mfma32(*(const bf16x8*)(st.dr + o2), vf[kk], pa);
            }
            // P and dS; the rows this lane holds are 8j + 4h + u
            bf16x8 pb[2], db[2];
            int rec[16];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4 l4 = *(const f32x4*)(st.lse2 + 8 * j + 4 * h);
                const f32x4 d4 = *(const f32x4*)(st.dlt + 8 * j + 4 * h);
                const int4 m4 = *(const int4*)(st.lim + 8 * j + 4 * h);
                const int4 r4 = *(const int4*)(st.rec + 8 * j + 4 * h);
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int i = 4 * j + u;
                    const int lim = u == 0 ? m4.x : u == 1 ? m4.y : u == 2 ? m4.z : m4.w;
                    rec[i] = u == 0 ? r4.x : u == 1 ? r4.y : u == 2 ? r4.z : r4.w;
                    float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[i], scale_log2, -l4[u]));
                    if (my_key > lim) p = 0.0f;
                    const __bf16 dsv = (__bf16)(p * (pa[i] - d4[u]));
                    pb[i >> 3][i & 7] = (__bf16)p;
                    db[i >> 3][i & 7] = dsv;
                    dsl[swz_chunk_offset(mfma32_row(i, h), my_key >> 3) + (my_key & 7)] = dsv;
                }
            }
            // dV += P^T dO, dK += dS^T Q: own keys x 128 dims, k = the 32 rows (in tpos order)
#pragma unroll
            for (int hs = 0; hs < 2; ++hs)
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
                    const int o3 = tline_offset(nt * 32 + l32, 2 * hs + h);
                    dv[nt] = mfma32(pb[hs], *(const bf16x8*)(st.dt + o3), dv[nt]);
                    dk[nt] = mfma32(db[hs], *(const bf16x8*)(st.qt + o3), dk[nt]);
                }
            __syncthreads();  // dS of all keys is in LDS; this step's stage is no longer read
            if (s + 1 < nsteps) store_step(pf);

            // dQ rows (unscaled) for dims 32 wave .. 32 wave + 31: sum over the block's 128 keys
            f32x16 qa;
#pragma unroll
            for (int i = 0; i < 16; ++i) qa[i] = 0.0f;
#pragma unroll
            for (int kk = 0; kk < 8; ++kk)
                qa = mfma32(*(const bf16x8*)(dsl + swz_chunk_offset(l32, 2 * kk + h)), ktf[kk], qa);
            const int r0 = s * kBwdRows;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                if (rec[i] < 0) continue;
                const int head = g * G + ((r0 + mfma32_row(i, h)) & (G - 1));
                dq_part[((size_t)rec[i] * Hq + head) * kDim + 32 * wave + l32] = qa[i];
            }
            __syncthreads();  // next step's stage is in LDS; dS reads are done
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
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_bwd_dq_sum(const float* __restrict__ dq_part,
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
    const size_t slot_stride = (size_t)Hq * kDim;
    const float* base = dq_part + (size_t)bt * top_k * slot_stride;
    for (int u = tid; u < Hq * (kDim / 4); u += 256) {  // 4 dims per unit
        const int head = u / (kDim / 4), d4 = (u % (kDim / 4)) * 4;
        const int32_t* sg = sel + (head >> gshift) * top_k;
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int s = 0; s < top_k; ++s) {
            const int cc = sg[s];
            if (cc < 0 || cc > cl) continue;
            acc += *(const f32x4*)(base + s * slot_stride + (size_t)head * kDim + d4);
        }
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (__bf16)(acc[e] * scale);
        *(bf16x4*)(dq + ((size_t)bt * Hq + head) * kDim + d4) = w;
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
                       ws.plan.entries, ws.dq_part, ws.dkv_part, d.N, d.Hq, d.Hkv, d.gshift, d.nblk, d.top_k, n,
                       d.scale, d.scale * log2e);
    return hipGetLastError();
}

hipError_t launch_bwd_dq_sum(const int32_t* block_idx, void* dq, const BwdWs& ws, const Dims& d,
                             hipStream_t stream) {
    const size_t lds = (size_t)d.Hkv * d.top_k * sizeof(int32_t);
    hipLaunchKernelGGL(k_bwd_dq_sum, dim3((unsigned)(d.B * d.N)), dim3(256), lds, stream, ws.dq_part, block_idx,
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
