// Index scores and causal block max-pool on bf16 MFMA.
//
// [MSA summary] "Architecture: two-stage block-sparse attention": the index
// query head of each group is scored against the one shared index key head
// over the visible keys and the scores are aggregated into 128-token blocks.
// [Flash-MSA] "About MSA" item 1 and "Proxy attention": the aggregation is a
// max, causal inside the query's own block.
//
// The index queries of all heads form one [N*H_idx, 128] matrix (their memory
// layout already is), because every head is scored against the same keys.
// A workgroup owns 256 of those rows (held in registers as the MFMA B operand)
// and streams kIdxChunk key blocks through a double-buffered LDS tile filled by
// buffer loads straight to LDS, the next block's issued during the current
// block's products. Each wave computes S^T = K_blk * Q^T for its 64
// rows, so a lane holds one query row and the block max is an in-lane max plus
// one exchange between the wave's halves. Each lane keeps its row's maxima for
// the chunk in registers and writes them as one 128-byte run.
//
// Fused with the selection (k_index_topk): [MSA summary] "GPU kernel
// co-design" selects on the raw pooled scores, and [Flash-MSA] "Proxy
// attention" keeps the query's own block plus the top_k - 1 best earlier ones.
// Since a lane already owns a row and key blocks arrive in ascending order, the
// lane keeps its row's best blocks in registers as they arrive; the pooled
// matrix never reaches memory and no selection pass follows.
#include "msa_device.hpp"
#include "msa_internal.hpp"

namespace msa {

constexpr int kIdxTileRows = 256;  // (position, index head) rows per workgroup
constexpr int kIdxChunk = 32;      // key blocks per workgroup: one 128-byte pooled run per row
constexpr int kStreamCap = 16;     // list length of the single-pass selection: top_k <= 17

typedef __attribute__((address_space(3))) void* lds_ptr;

// Buffer resource word 3 for raw 32-bit accesses on gfx9-family targets.
constexpr int kIdxRawBufferWord3 = 0x00020000;

// Staging of a key block into an LDS buffer with buffer loads straight to LDS,
// eight per wave. Instruction i of wave w fills 16-byte slots p = (4i + w) * 64 +
// lane, i.e. row p / 16 = 16i + 4w + lane / 16, stored chunk p % 16, which holds
// logical chunk (p % 16) ^ (row % 16); row % 16 does not depend on i, so one
// per-lane byte offset (computed once) serves every load, and the block and the
// instruction only move the scalar offset. `wave` is wave-uniform (a scalar
// register). The resource spans this batch's N index keys (N * 256 bytes < 2^31).
struct KeyStage {
    __amdgpu_buffer_rsrc_t rsrc;
    uint32_t lane_off;
    int wave;
    __device__ __forceinline__ KeyStage(const __bf16* kb, int N, int wave_, int lane) : wave(wave_) {
        rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)kb, (short)0, N * kDim * 2, kIdxRawBufferWord3);
        const int row0 = 4 * wave_ + (lane >> 4);
        lane_off = (uint32_t)(row0 * kDim + (((lane & 15) ^ (row0 & 15)) * 8)) * 2u;
    }
    // load i of key block `blk` into LDS buffer `dst`
    __device__ __forceinline__ void load(int blk, __bf16* dst, int i) const {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr)(dst + (i * 4 + wave) * 64 * 8), 16, lane_off,
                                                 (blk * kBlock + i * 16) * kDim * 2, 0, 0);
    }
    __device__ __forceinline__ void all(int blk, __bf16* dst) const {
#pragma unroll
        for (int i = 0; i < 8; ++i) load(blk, dst, i);
    }
};

// B operand (Q^T) of a wave: lane holds row (r0 + wave*64 + nt*32 + l32), dims kk*16 + 8h .. +7;
// rows past R are zero and get query position -1 (never the diagonal block).
__device__ __forceinline__ void load_q_rows(const __bf16* __restrict__ qb, int r0, int R, int H, int wave, int h,
                                            int l32, bf16x8 (&qf)[2][8], int (&trow)[2]) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        const int row = r0 + wave * 64 + nt * 32 + l32;
        trow[nt] = row < R ? row / H : -1;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            if (row < R) {
                qf[nt][kk] = *(const bf16x8*)(qb + (size_t)row * kDim + kk * 16 + 8 * h);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) qf[nt][kk][e] = (__bf16)0.0f;
            }
        }
    }
}

// Max score of this lane's row (row tile h of the wave) over the visible keys of key
// block c, staged in LDS at kt. DIAG: some row of the wave lies in block c (the causal
// diagonal), so keys past a row's own position are masked; lim0, lim1 are those
// positions minus 4h (key = mt*32 + 8*(i/4) + 4h + i%4 <= lim <=> mt*32 + 8*(i/4) + i%4
// <= lim - 4h, so every comparison is against a compile-time constant).
// The four 32-key M tiles are software-pipelined: tile mt's products are issued while
// tile mt - 1's accumulators are reduced (two accumulator sets). The common, unmasked
// path has no branch, so the reductions interleave with the matrix instructions.
// The next key block's staging loads (block `nblk_` into the idle buffer `ndst`) are issued
// from here: spread two per M tile on the common path, so a wave never stalls on a
// burst of eight loads queued behind the other waves' (all eight at the start on the
// diagonal path, after the first tile's products).
template <bool DIAG>
__device__ __forceinline__ float block_row_max_t(const __bf16* kt, const bf16x8 (&qf)[2][8], int lim0, int lim1,
                                                 int h, int l32, const KeyStage& st, int nblk_, __bf16* ndst) {
    float m0 = -INFINITY, m1 = -INFINITY;
    f32x16 acc[2][2];
    auto products = [&](int mt, f32x16 (&a)[2]) {
#pragma unroll
        for (int i = 0; i < 16; ++i) a[0][i] = a[1][i] = 0.0f;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            const bf16x8 k8 = *(const bf16x8*)(kt + swz_chunk_offset(mt * 32 + l32, 2 * kk + h));
            a[0] = mfma32(k8, qf[0][kk], a[0]);
            a[1] = mfma32(k8, qf[1][kk], a[1]);
        }
    };
    auto reduce = [&](int mt, const f32x16 (&a)[2]) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (DIAG) {
                const int key_h0 = mt * 32 + mfma32_row(i, 0);
                if (key_h0 <= lim0) m0 = fmaxf(m0, a[0][i]);
                if (key_h0 <= lim1) m1 = fmaxf(m1, a[1][i]);
            } else {
                m0 = fmaxf(m0, a[0][i]);
                m1 = fmaxf(m1, a[1][i]);
            }
        }
    };
    products(0, acc[0]);
    if (DIAG) {
        st.all(nblk_, ndst);
    } else {
        st.load(nblk_, ndst, 0);
        st.load(nblk_, ndst, 1);
    }
#pragma unroll
    for (int mt = 1; mt < 4; ++mt) {
        products(mt, acc[mt & 1]);
        reduce(mt - 1, acc[(mt - 1) & 1]);
        if (!DIAG) {
            st.load(nblk_, ndst, 2 * mt);
            st.load(nblk_, ndst, 2 * mt + 1);
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // an operand read
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // two products
                __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // two max steps
                if (kk == 3 || kk == 7) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // a staging load
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    reduce(3, acc[1]);
    m0 = wave_max_xor32(m0);
    m1 = wave_max_xor32(m1);
    return h ? m1 : m0;  // after the exchange lane-half h owns row tile h
}

__device__ __forceinline__ float block_row_max(const __bf16* kt, const bf16x8 (&qf)[2][8], const int (&trow)[2],
                                               int c, int h, int l32, const KeyStage& st, int nblk_, __bf16* ndst) {
    const bool diag0 = (trow[0] >> 7) == c, diag1 = (trow[1] >> 7) == c;
    const int lim0 = (diag0 ? trow[0] - c * kBlock : kBlock - 1) - 4 * h;
    const int lim1 = (diag1 ? trow[1] - c * kBlock : kBlock - 1) - 4 * h;
    return __any(diag0 || diag1) ? block_row_max_t<true>(kt, qf, lim0, lim1, h, l32, st, nblk_, ndst)
                                 : block_row_max_t<false>(kt, qf, lim0, lim1, h, l32, st, nblk_, ndst);
}

__global__ __launch_bounds__(256, 2) void k_index_pool(const __bf16* __restrict__ q_idx,
                                                       const __bf16* __restrict__ k_idx,
                                                       float* __restrict__ pooled, int N, int H, int nblk) {
    const int tile = blockIdx.x, chunk = blockIdx.y, b = blockIdx.z;
    const int R = N * H;
    const int r0 = tile * kIdxTileRows;
    const int r_end = min(r0 + kIdxTileRows, R);
    const int nkb = ((r_end - 1) / H) / kBlock + 1;  // key blocks seen by this tile's last query
    const int c0 = chunk * kIdxChunk;
    if (c0 >= nkb) return;
    const int c1 = min(c0 + kIdxChunk, nkb);

    __shared__ __attribute__((aligned(16))) __bf16 ks[2][kBlock * kDim];  // double-buffered key block

    const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const __bf16* qb = q_idx + (size_t)b * R * kDim;
    const __bf16* kb = k_idx + (size_t)b * N * kDim;

    const KeyStage st(kb, N, wave, lane);
    st.all(c0, ks[0]);
    bf16x8 qf[2][8];
    int trow[2];
    load_q_rows(qb, r0, R, H, wave, h, l32, qf, trow);

    // pv[j] ends up holding this lane's row max for key block c1 - kIdxChunk + j
    float pv[kIdxChunk];
#pragma unroll
    for (int j = 0; j < kIdxChunk; ++j) pv[j] = -INFINITY;

    for (int c = c0; c < c1; ++c) {
        const int buf = (c - c0) & 1;
        __builtin_amdgcn_s_waitcnt(0);  // this thread's loads of block c have landed
        __syncthreads();                // ... and everyone's; the other buffer is free again
        // the last block stages itself again into the idle buffer (no branch in the loop body)
        const int cn = c + 1 < c1 ? c + 1 : c;
        const float m = block_row_max(ks[buf], qf, trow, c, h, l32, st, cn, ks[buf ^ 1]);
#pragma unroll
        for (int j = 0; j + 1 < kIdxChunk; ++j) pv[j] = pv[j + 1];
        pv[kIdxChunk - 1] = m;
    }
    __builtin_amdgcn_s_waitcnt(0);  // the last block's repeated staging has landed before the LDS is released

    const int row = r0 + wave * 64 + h * 32 + l32;
    if (row < R) {
        const int t = row / H, g = row - t * H;
        const int cend = min(c1, (t >> 7) + 1);
        float* dst = pooled + (((size_t)b * H + g) * N + t) * nblk;
        if (c1 - c0 == kIdxChunk && cend == c1 && (nblk & 3) == 0) {
#pragma unroll
            for (int q4 = 0; q4 < kIdxChunk / 4; ++q4)
                *(f32x4*)(dst + c0 + 4 * q4) = (f32x4){pv[4 * q4], pv[4 * q4 + 1], pv[4 * q4 + 2], pv[4 * q4 + 3]};
        } else {
#pragma unroll
            for (int j = 0; j < kIdxChunk; ++j) {
                const int c = c1 - kIdxChunk + j;
                if (c >= c0 && c < cend) dst[c] = pv[j];
            }
        }
    }
}

// Index scores and selection in one pass, with no pooled matrix in memory. A
// workgroup owns a 256-row tile and walks every key block its rows can see, in
// ascending order; after each block the lane owning a row inserts that block's
// max into the row's running list of the kStreamCap best (score key, block)
// pairs among the blocks before the row's own. The list stays sorted by score
// key, descending; a block arriving later has a larger index than every listed
// one, so a strict comparison keeps equal scores in ascending block order, which
// is the order of the 64-bit keys used by the selection kernel: the chosen set is
// the same. Tiles run heaviest (latest) first so the long causal rows start early.
__global__ __launch_bounds__(256, 2) void k_index_topk(const __bf16* __restrict__ q_idx,
                                                       const __bf16* __restrict__ k_idx,
                                                       int32_t* __restrict__ block_idx, int N, int H, int top_k,
                                                       int tiles) {
    const int id = blockIdx.x, B = gridDim.x / tiles;
    const int tile = tiles - 1 - id / B, b = id - (id / B) * B;
    const int R = N * H;
    const int r0 = tile * kIdxTileRows;
    const int r_end = min(r0 + kIdxTileRows, R);
    const int nkb = ((r_end - 1) / H) / kBlock + 1;

    __shared__ __attribute__((aligned(16))) __bf16 ks[2][kBlock * kDim];

    const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const __bf16* qb = q_idx + (size_t)b * R * kDim;
    const __bf16* kb = k_idx + (size_t)b * N * kDim;

    const KeyStage st(kb, N, wave, lane);
    st.all(0, ks[0]);
    bf16x8 qf[2][8];
    int trow[2];
    load_q_rows(qb, r0, R, H, wave, h, l32, qf, trow);

    const int row = r0 + wave * 64 + h * 32 + l32;
    const int cl = row < R ? (row / H) >> 7 : -1;  // the row's own block; only blocks c < cl compete
    // score key 0 sits below every finite score's key, so empty slots are never chosen
    uint32_t ls[kStreamCap];
    int lb[kStreamCap];
#pragma unroll
    for (int i = 0; i < kStreamCap; ++i) {
        ls[i] = 0u;
        lb[i] = -1;
    }

    for (int c = 0; c < nkb; ++c) {
        const int buf = c & 1;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        const int cn = c + 1 < nkb ? c + 1 : c;  // the last block stages itself again into the idle buffer
        const float m = block_row_max(ks[buf], qf, trow, c, h, l32, st, cn, ks[buf ^ 1]);
        // insert before the first listed key it exceeds; everything after moves down one
        // slot (comparing the displaced entry instead would reorder equal scores)
        const uint32_t xs = c < cl ? order_key(m) : 0u;
        bool gt[kStreamCap];
#pragma unroll
        for (int i = 0; i < kStreamCap; ++i) gt[i] = xs > ls[i];
#pragma unroll
        for (int i = kStreamCap - 1; i > 0; --i) {
            ls[i] = gt[i] ? (gt[i - 1] ? ls[i - 1] : xs) : ls[i];
            lb[i] = gt[i] ? (gt[i - 1] ? lb[i - 1] : c) : lb[i];
        }
        ls[0] = gt[0] ? xs : ls[0];
        lb[0] = gt[0] ? c : lb[0];
    }
    __builtin_amdgcn_s_waitcnt(0);  // the last block's repeated staging has landed before the LDS is released
    if (row >= R) return;

    const int t = row / H, g = row - t * H;
    int32_t* dst = block_idx + (((size_t)b * H + g) * N + t) * top_k;
    if (cl + 1 <= top_k) {  // every visible block
        for (int s2 = 0; s2 < top_k; ++s2) dst[s2] = s2 <= cl ? s2 : -1;
        return;
    }
    // the need best, in ascending block order, then the row's own block
    const int need = top_k - 1;
#pragma unroll
    for (int i = 0; i < kStreamCap; ++i) {
        if (i < need) {
            int pos = 0;
#pragma unroll
            for (int j = 0; j < kStreamCap; ++j) pos += (j < need && lb[j] < lb[i]) ? 1 : 0;
            dst[pos] = lb[i];
        }
    }
    dst[need] = cl;
}

// pooled[b,g,t,c] = -inf for c > t/128 (the part no query can see).
__global__ __launch_bounds__(256) void k_pooled_fill_upper(float* __restrict__ pooled, int N, int nblk,
                                                           long long rows) {
    const long long row = (long long)blockIdx.x;
    if (row >= rows) return;
    const int t = (int)(row % N);
    float* dst = pooled + row * nblk;
    for (int c = (t >> 7) + 1 + threadIdx.x; c < nblk; c += 256) dst[c] = -INFINITY;
}

hipError_t launch_index_pool(const void* q_idx, const void* k_idx, float* pooled, const Dims& d, bool fill_upper,
                             hipStream_t stream) {
    const int H = d.Hkv;  // index heads == KV heads
    const long long R = (long long)d.N * H;
    const int tiles = (int)((R + kIdxTileRows - 1) / kIdxTileRows);
    const int chunks = (d.nblk + kIdxChunk - 1) / kIdxChunk;
    dim3 grid(tiles, chunks, d.B);
    hipLaunchKernelGGL(k_index_pool, grid, dim3(256), 0, stream, (const __bf16*)q_idx, (const __bf16*)k_idx, pooled,
                       d.N, H, d.nblk);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !fill_upper) return e;
    const long long rows = (long long)d.B * H * d.N;
    hipLaunchKernelGGL(k_pooled_fill_upper, dim3((unsigned)rows), dim3(256), 0, stream, pooled, d.N, d.nblk, rows);
    return hipGetLastError();
}

bool index_topk_fusable(const Dims& d) { return d.top_k - 1 <= kStreamCap; }

hipError_t launch_index_topk(const void* q_idx, const void* k_idx, int32_t* block_idx, const Dims& d,
                             hipStream_t stream) {
    const int H = d.Hkv;
    const long long R = (long long)d.N * H;
    const int tiles = (int)((R + kIdxTileRows - 1) / kIdxTileRows);
    hipLaunchKernelGGL(k_index_topk, dim3((unsigned)(tiles * d.B)), dim3(256), 0, stream, (const __bf16*)q_idx,
                       (const __bf16*)k_idx, block_idx, d.N, H, d.top_k, tiles);
    return hipGetLastError();
}

}  // namespace msa
