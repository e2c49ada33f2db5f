// Sparse main attention, phase 2: global softmax combine of the slot partials.
//
// [MSA summary] "GPU kernel co-design": two-phase forward, partial attention
// then a global softmax-combine kernel. Per (b, t, head), with the slot
// partials (O_s normalised, lse_s):
//   M = max_s lse_s,  w_s = exp(lse_s - M),  L = sum_s w_s,
//   O = sum_s w_s O_s / L,  LSE = M + ln L.
//
// The slot of the query's own (local) block is computed here rather than in the
// partial kernel (combine_folds_local: top_k <= 16): the block is the same for all
// 128 positions of a block, so its attention is a dense causal tile, and the
// (row, local block) pair then needs no gathered query, no record written and no
// record read back. k_combine_all merges records only (every slot from the partial
// kernel) for longer selections.
#include "msa_device.hpp"
#include "msa_internal.hpp"

namespace msa {

constexpr int kFoldSlots = 16;        // top_k the folded combine takes
constexpr int kFoldOob = 0x40000000;  // a buffer offset past every buffer the folded combine reads

bool combine_folds_local(const Dims& d) { return d.top_k <= kFoldSlots; }

// Partial O layout: [(b*Nc + t - p0)*top_k + slot][g][chunk c][G heads][8], where
// chunk c = hf*8 + dt*2 + i0/8 holds dims 32*dt + 8*(i/4) + 4*hf + i%4 for
// i = i0 .. i0+7 (the order the MFMA result registers are in).
//
// k_combine_all, one workgroup per (b, t):
//   0. the position's selection rows (H_kv x top_k) and slot LSEs (top_k x H_q,
//      contiguous) are loaded cooperatively into LDS;
//   1. one thread per head turns them into weights w_s / L and writes LSE;
//   2. each thread takes (group, chunk, head) pieces in record order, so every
//      load instruction reads a contiguous run; slots are loaded eight at a time
//      before any is used (top_k <= 16), accumulated in fp32 and put in an LDS
//      copy of the position's output row (8 slots in flight at a time keeps
//      the kernel small enough for 6 waves per SIMD);
//   3. the row (H_q x 128 bf16, contiguous in O) is written in 16-byte pieces.
// The slot records are read exactly once and O is not read again here, so both
// go through nontemporal loads and stores: each load instruction of a wave
// covers whole cache lines (64 lanes x 16 contiguous bytes), so no line is
// fetched twice (9% faster than plain accesses at 128K tokens).
constexpr int kCombineFastSlots = 16;

__global__ __launch_bounds__(256, 6) void k_combine_all(const __bf16* __restrict__ part_o, const float* __restrict__ part_lse,
                                                 const int32_t* __restrict__ block_idx, __bf16* __restrict__ o,
                                                 float* __restrict__ lse, int N, int p0, int Nc, int Hq, int Hkv,
                                                 int gshift, int top_k) {
    // dynamic LDS: orow [Hq][128] bf16 | wts [top_k][Hq] fp32 | inv_l [Hq] fp32 | sel [Hkv][top_k] int32
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    __bf16* orow = (__bf16*)smem;
    float* wts = (float*)(smem + (size_t)Hq * kDim * 2);
    float* inv_l = wts + (size_t)top_k * Hq;
    int32_t* sel = (int32_t*)(inv_l + Hq);
    const int tid = threadIdx.x;
    const int bt = blockIdx.x;  // (b, t - p0) inside the chunk
    const int b = bt / Nc, t = p0 + (bt - b * Nc);
    const int cl = t >> 7;
    const size_t rec0 = (size_t)bt * top_k;  // first record of this position

    // 0. selection rows and slot LSEs into LDS
    for (int i = tid; i < Hkv * top_k; i += 256) {
        const int g = i / top_k, s = i - g * top_k;
        sel[i] = block_idx[(((size_t)b * Hkv + g) * N + t) * top_k + s];
    }
    for (int i = tid; i < top_k * Hq; i += 256) wts[i] = part_lse[rec0 * Hq + i];
    __syncthreads();

    // 1. per head: M = max lse_s, w_s = exp(lse_s - M), L = sum w_s over valid slots
    for (int head = tid; head < Hq; head += 256) {
        const int32_t* sg = sel + (head >> gshift) * top_k;
        float M = -INFINITY;
        for (int s = 0; s < top_k; ++s) {
            const int c = sg[s];
            if (c >= 0 && c <= cl) M = fmaxf(M, wts[s * Hq + head]);
        }
        float L = 0.0f;
        for (int s = 0; s < top_k; ++s) {
            const int c = sg[s];
            const float w = (c >= 0 && c <= cl) ? expf(wts[s * Hq + head] - M) : 0.0f;
            L += w;
            wts[s * Hq + head] = w;
        }
        inv_l[head] = L > 0.0f ? 1.0f / L : 0.0f;
        lse[((size_t)b * Hq + head) * N + t] = M + logf(L);
    }
    __syncthreads();

    // 2. weighted sum of the slot records; j -> (group, chunk, head in the group), the
    //    record order, so that consecutive threads read consecutive 16-byte pieces
    const size_t slot_stride = (size_t)16 * Hq * 8;
    const int G = 1 << gshift;
    for (int j = tid; j < Hq * 16; j += 256) {
        const int ch = (j >> gshift) & 15, head = (j >> (gshift + 4)) * G + (j & (G - 1));
        const __bf16* src = part_o + rec0 * slot_stride + (size_t)j * 8;
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
        if (top_k <= kCombineFastSlots) {
#pragma unroll
            for (int s0 = 0; s0 < kCombineFastSlots; s0 += 8) {  // 8 slots in flight per batch
                bf16x8 x[8];
                float w[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    w[u] = s0 + u < top_k ? wts[(s0 + u) * Hq + head] : 0.0f;
                    if (w[u] != 0.0f) x[u] = __builtin_nontemporal_load((const bf16x8*)(src + (s0 + u) * slot_stride));
                }
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    if (w[u] != 0.0f)
#pragma unroll
                        for (int e = 0; e < 8; ++e) acc[e] += w[u] * (float)x[u][e];
            }
        } else {
            for (int s = 0; s < top_k; ++s) {
                const float w = wts[s * Hq + head];
                if (w != 0.0f) {
                    const bf16x8 x = *(const bf16x8*)(src + s * slot_stride);
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[e] += w * (float)x[e];
                }
            }
        }
        const float inv = inv_l[head];
        const int hf = ch >> 3, dt = (ch & 7) >> 1, i0 = (ch & 1) * 8;
        const int dim_a = 32 * dt + 2 * i0 + 4 * hf;  // elements 0..3 -> dim_a.., 4..7 -> dim_a+8..
        bf16x4 wa, wb;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            wa[e] = (__bf16)(acc[e] * inv);
            wb[e] = (__bf16)(acc[4 + e] * inv);
        }
        *(bf16x4*)(orow + head * kDim + dim_a) = wa;
        *(bf16x4*)(orow + head * kDim + dim_a + 8) = wb;
    }
    __syncthreads();

    // 3. the position's output row is contiguous in O: write it in 16-byte pieces
    uint4* dst = (uint4*)(o + ((size_t)b * N + t) * Hq * kDim);
    const uint4* srcl = (const uint4*)orow;
    for (int j = tid; j < Hq * 16; j += 256) __builtin_nontemporal_store(((const u32x4*)srcl)[j], (u32x4*)dst + j);
}

// The causal attention of a lane's row (lane half h of row l32) to the block staged in
// ks / vts, over the first NMT 32-key tiles (the later ones are masked for every row of
// the tile): the local O, normalised, goes to row l32 of `ow` in the record layout;
// returns l and sets mb (the row max times the scale, log2 units).
template <int NMT>
__device__ __forceinline__ float local_attn(const bf16x8 (&qa)[8], const __bf16* ks, const __bf16* vts, __bf16* ow,
                                            int l32, int h, int lim, float scale_log2, float& mb_out) {
    f32x16 sacc[NMT];
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[mt][i] = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) {
            const bf16x8 a = *(const bf16x8*)(ks + swz_chunk_offset(mt * 32 + l32, 2 * kk + h));
            sacc[mt] = mfma32(a, qa[kk], sacc[mt]);
        }
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if (mt * 32 + mfma32_row(i, 0) > lim) sacc[mt][i] = -INFINITY;
    float m = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) m = fmaxf(m, sacc[mt][i]);
    m = wave_max_xor32(m);
    const float mb = m * scale_log2;
    bf16x8 pf[2 * NMT];
    float l = 0.0f;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[mt][half * 8 + e], scale_log2, -mb));
                l += pv;
                pf[mt * 2 + half][e] = (__bf16)pv;
            }
    l = wave_sum_xor32(l);
    const float inv_l = 1.0f / l;
    // O^T = V^T P^T, 64 dims at a time
#pragma unroll
    for (int dh = 0; dh < 2; ++dh) {
        f32x16 oacc[2];
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[j][i] = 0.0f;
#pragma unroll
        for (int kk = 0; kk < 2 * NMT; ++kk)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const bf16x8 a = *(const bf16x8*)(vts + swz_chunk_offset((dh * 2 + j) * 32 + l32, 2 * kk + h));
                oacc[j] = mfma32(a, pf[kk], oacc[j]);
            }
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int i0 = 0; i0 < 16; i0 += 8) {
                bf16x8 w8;
#pragma unroll
                for (int e = 0; e < 8; ++e) w8[e] = (__bf16)(oacc[j][i0 + e] * inv_l);
                *(bf16x8*)(ow + swz_chunk_offset(l32, h * 8 + (dh * 2 + j) * 2 + i0 / 8)) = w8;
            }
    }
    mb_out = mb;
    return l;
}

// The combine with the local block folded in. One workgroup of eight waves per
// (b, g, local block c): K and V^T of block c are staged once, and each wave takes
// 32 rows (positions x G heads) of the block's row tiles in turn:
//   A. one lane per row and lane half, as in the partial kernel: the row's causal
//      attention to block c (local_attn) gives its local O and LSE; with the row's
//      slot LSEs that fixes M, the slot weights, 1/L and the output LSE. The local O
//      (normalised, bf16, in the record layout) and the weights go to the wave's
//      LDS area;
//   B. one lane per 16-byte record piece, a group's heads adjacent as the records
//      hold them: the weighted sum of the local piece and the row's other slot
//      records, in place in LDS, the next piece's record loads in flight meanwhile;
//   C. the rows, reordered to head-dim order, written to O in 16-byte pieces.
// A slot whose block is not an earlier visible block (padding, the local block
// itself, a block after the query's) has weight 0 and is not loaded; a repeated
// local block counts once per slot it fills, as a repeated record would.
constexpr int kFoldWts = 20;  // per row: 16 slot weights, the local weight, 1/L, the slots to load, a pad
__global__ __launch_bounds__(512) void k_combine(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ part_o, const float* __restrict__ part_lse, const int32_t* __restrict__ block_idx,
    __bf16* __restrict__ o, float* __restrict__ lse, int N, int p0, int Nc, int Hq, int Hkv, int gshift, int top_k,
    float scale_log2) {
    __shared__ __attribute__((aligned(16))) __bf16 ks[kBlock * kDim];
    __shared__ __attribute__((aligned(16))) __bf16 vts[kDim * kBlock];
    __shared__ __attribute__((aligned(16))) __bf16 orow[8][32 * kDim];
    __shared__ __attribute__((aligned(16))) float wts[8][32 * kFoldWts];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
    const int G = 1 << gshift;
    const int P = kBlock >> gshift;
    const int r = (wave & 3) * 32 + l32;
    const int pslot = r >> gshift, hh = r & (G - 1);
    const float ln2 = 0.69314718055994531f;
    const int nloc = Nc >> 7;
    const int cb = blockIdx.x % nloc, bg = blockIdx.x / nloc, g = bg % Hkv, b = bg / Hkv;
    const int c = (p0 >> 7) + cb;
    const size_t qhead = (size_t)g * G + hh;
    if (tid < 256) stage_kv_tile(k, v, ks, vts, b, g, c, N, Hkv, tid);
    __syncthreads();
    __bf16* ow = orow[wave];
    float* ww = wts[wave];
    const size_t rec_blk = ((size_t)b * Nc + (size_t)c * kBlock - p0) * top_k;
    const __amdgpu_buffer_rsrc_t r_o = uniform_rsrc(part_o + rec_blk * 16 * Hq * 8, kBlock * top_k * 16 * Hq * 16);
    const __amdgpu_buffer_rsrc_t r_l = uniform_rsrc(part_lse + rec_blk * Hq, kBlock * top_k * Hq * 4);
    const __amdgpu_buffer_rsrc_t r_s =
        uniform_rsrc(block_idx + (((size_t)b * Hkv + g) * N + (size_t)c * kBlock) * top_k, kBlock * top_k * 4);
    const int slot_bytes = 16 * Hq * 16;
    const int gw = gshift < 5 ? gshift : 5;

    for (int rt = wave >> 2; rt < G; rt += 2) {
        // ---- A: this lane's row
        const int t = c * kBlock + rt * P + pslot;
        const int tb = t - c * kBlock;
        bf16x8 qa[8];
        const __bf16* qrow = q + (((size_t)b * N + t) * Hq + qhead) * kDim + 8 * h;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) qa[kk] = *(const bf16x8*)(qrow + kk * 16);
        // the row's selection and slot LSEs; a lane that needs no value reads past the
        // buffer's end, which returns 0 and touches no memory
        int cs[kFoldSlots];
        float ls[kFoldSlots];
#pragma unroll
        for (int s = 0; s < kFoldSlots; ++s) {
            const int x = (int)__builtin_amdgcn_raw_buffer_load_b32(r_s, s < top_k ? (tb * top_k + s) * 4 : kFoldOob, 0, 0);
            cs[s] = s < top_k ? x : -1;
        }
        const int lbase = (tb * top_k * Hq + (int)qhead) * 4;
#pragma unroll
        for (int s = 0; s < kFoldSlots; ++s) {
            const bool ok = cs[s] >= 0 && cs[s] < c;
            const float x =
                __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r_l, ok ? lbase + s * Hq * 4 : kFoldOob, 0, 0));
            ls[s] = ok ? x : -INFINITY;
        }
        asm volatile("" ::: "memory");
        // key tiles past the row tile's last position are masked for every row: skipped
        const int nmt = ((rt + 1) * P - 1) / 32 + 1;
        const int lim = tb - 4 * h;
        float mb, l;
        if (nmt == 1) l = local_attn<1>(qa, ks, vts, ow, l32, h, lim, scale_log2, mb);
        else if (nmt == 2) l = local_attn<2>(qa, ks, vts, ow, l32, h, lim, scale_log2, mb);
        else if (nmt == 3) l = local_attn<3>(qa, ks, vts, ow, l32, h, lim, scale_log2, mb);
        else l = local_attn<4>(qa, ks, vts, ow, l32, h, lim, scale_log2, mb);
        const float lse_loc = (mb + __builtin_amdgcn_logf(l)) * ln2;
        // M over the valid slots (the local block's LSE once it occurs), the weights, 1/L
        float M = -INFINITY;
        int nl = 0;
#pragma unroll
        for (int s = 0; s < kFoldSlots; ++s) {
            nl += cs[s] == c;
            M = fmaxf(M, ls[s]);
        }
        if (nl) M = fmaxf(M, lse_loc);
        float wv[kFoldWts];
        float L = nl ? (float)nl * expf(lse_loc - M) : 0.0f;
        wv[16] = L;
#pragma unroll
        for (int s = 0; s < kFoldSlots; ++s) {
            wv[s] = ls[s] != -INFINITY ? expf(ls[s] - M) : 0.0f;
            L += wv[s];
        }
        wv[17] = L > 0.0f ? 1.0f / L : 0.0f;
        uint32_t lmask = 0;
#pragma unroll
        for (int s = 0; s < kFoldSlots; ++s) lmask |= (wv[s] != 0.0f ? 1u : 0u) << s;
        wv[18] = __builtin_bit_cast(float, lmask);
        wv[19] = 0.0f;
        // both lanes of a row hold the same values: lane half h writes half of them
#pragma unroll
        for (int e = 0; e < kFoldWts / 2; ++e) ww[l32 * kFoldWts + h * (kFoldWts / 2) + e] = wv[h * (kFoldWts / 2) + e];
        lse[((size_t)b * Hq + qhead) * N + t] = M + logf(L);  // both lanes of the row: the same value
        // LDS operations of one wave complete in order; the fences keep the compiler from
        // moving this wave's LDS accesses across the hand-over between lanes
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // ---- B: piece p = it * 64 + lane is (row, chunk). The wave's rows come in runs
        // of 2^gw heads of one position (all G heads, or 32 of them when G > 32), and p
        // takes a run's heads fastest, then the chunks, then the runs. The record loads of
        // piece it + 1 are issued before piece it is summed; a piece's weights are read
        // from LDS when it is summed.
        bf16x8 x[2][kFoldSlots];
        auto issue = [&](int it, bf16x8 (&xb)[kFoldSlots]) {
            const int pc = it * 64 + lane;
            const int row = (pc >> (gw + 4) << gw) + (pc & ((1 << gw) - 1)), ch = (pc >> gw) & 15;
            const int rr = (wave & 3) * 32 + row;     // row inside the tile
            const int tbp = rt * P + (rr >> gshift);  // its position inside the block
            const int vb = tbp * top_k * 16 * Hq * 16 + ((g * 16 + ch) * G + (rr & (G - 1))) * 16;
            const uint32_t lm = __builtin_bit_cast(uint32_t, ww[row * kFoldWts + 18]);
#pragma unroll
            for (int s = 0; s < kFoldSlots; ++s)
                xb[s] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                                       r_o, (lm >> s) & 1u ? vb + s * slot_bytes : kFoldOob, 0, 2));
        };
        issue(0, x[0]);
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            __builtin_amdgcn_sched_barrier(0);
            if (it + 1 < 8) issue(it + 1, x[(it + 1) & 1]);
            const int cur = it & 1;
            const int pc = it * 64 + lane;
            const int row = (pc >> (gw + 4) << gw) + (pc & ((1 << gw) - 1)), ch = (pc >> gw) & 15;
            const bf16x8 xlb = *(const bf16x8*)(ow + swz_chunk_offset(row, ch));  // the local piece
            const float* wr = ww + row * kFoldWts;
            float acc[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = wr[16] * (float)xlb[e];
#pragma unroll
            for (int s4 = 0; s4 < kFoldSlots; s4 += 4) {
                const f32x4 w4 = *(const f32x4*)(wr + s4);
#pragma unroll
                for (int u = 0; u < 4; ++u)
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[e] += w4[u] * (float)x[cur][s4 + u][e];
            }
            const float il = wr[17];
            bf16x8 ob;
#pragma unroll
            for (int e = 0; e < 8; ++e) ob[e] = (__bf16)(acc[e] * il);
            *(bf16x8*)(ow + swz_chunk_offset(row, ch)) = ob;  // in place, record order
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int piece = it * 64 + lane;
            const int row = piece >> 4, ch = piece & 15;
            // dims 8 ch .. 8 ch + 7 = 32 dt + 8 q + (0..7): record chunk dt * 2 + q / 2 holds
            // the first four, chunk 8 + dt * 2 + q / 2 the last four, at element 4 (q % 2)
            const int dt = ch >> 2, qq = ch & 3, ce = (qq & 1) * 4;
            const uint2 lo = *(const uint2*)(ow + swz_chunk_offset(row, dt * 2 + (qq >> 1)) + ce);
            const uint2 hi = *(const uint2*)(ow + swz_chunk_offset(row, 8 + dt * 2 + (qq >> 1)) + ce);
            const u32x4 val = {lo.x, lo.y, hi.x, hi.y};
            const int rr = (wave & 3) * 32 + row;
            const int tt = c * kBlock + rt * P + (rr >> gshift);
            const size_t head = (size_t)g * G + (rr & (G - 1));
            __builtin_nontemporal_store(val, (u32x4*)(o + (((size_t)b * N + tt) * Hq + head) * kDim) + ch);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

size_t combine_lds_bytes(const Dims& d) {
    return (size_t)d.Hq * kDim * 2 + ((size_t)d.top_k + 1) * d.Hq * 4 + (size_t)d.Hkv * d.top_k * 4;
}

hipError_t launch_sparse_combine(const void* q, const void* k, const void* v, const int32_t* block_idx, void* o,
                                 float* lse, const SparseWs& ws, const Dims& d, hipStream_t stream) {
    if (combine_folds_local(d)) {
        const float log2e = 1.4426950408889634f;
        hipLaunchKernelGGL(k_combine, dim3(d.B * d.Hkv * (d.Nc / kBlock)), dim3(512), 0, stream, (const __bf16*)q,
                           (const __bf16*)k, (const __bf16*)v, (const __bf16*)ws.part_o, ws.part_lse, block_idx,
                           (__bf16*)o, lse, d.N, d.p0, d.Nc, d.Hq, d.Hkv, d.gshift, d.top_k, d.scale * log2e);
    } else {
        hipLaunchKernelGGL(k_combine_all, dim3(d.B * d.Nc), dim3(256), combine_lds_bytes(d), stream,
                           (const __bf16*)ws.part_o, ws.part_lse, block_idx, (__bf16*)o, lse, d.N, d.p0, d.Nc, d.Hq,
                           d.Hkv, d.gshift, d.top_k);
    }
    return hipGetLastError();
}

}  // namespace msa
