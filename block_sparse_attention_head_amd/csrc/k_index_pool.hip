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
// and streams kIdxChunk key blocks through LDS. Each wave computes
// S^T = K_blk * Q^T for its 64 rows, so one lane holds one query row and the
// block max is an in-lane max plus one exchange between the wave's halves.
// The per-block maxima are staged in LDS and written as contiguous runs.
#include "msa_device.hpp"
#include "msa_internal.hpp"

namespace msa {

constexpr int kIdxTileRows = 256;  // (position, index head) rows per workgroup
constexpr int kIdxChunk = 16;      // key blocks per workgroup

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

    __shared__ __attribute__((aligned(16))) __bf16 ks[kBlock * kDim];
    __shared__ float stage[kIdxChunk * kIdxTileRows];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
    const __bf16* qb = q_idx + (size_t)b * R * kDim;
    const __bf16* kb = k_idx + (size_t)b * N * kDim;

    // B operand (Q^T): lane holds row (wave*64 + nt*32 + l32), dims kk*16 + 8h .. +7.
    bf16x8 qf[2][8];
    int trow[2];
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

    for (int c = c0; c < c1; ++c) {
        __syncthreads();  // every wave is done reading the previous key block
        const __bf16* src = kb + (size_t)c * kBlock * kDim;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int idx = tid + i * 256, key = idx >> 4, ch = idx & 15;
            const uint4 val = *(const uint4*)(src + key * kDim + ch * 8);
            *(uint4*)(ks + swz_chunk_offset(key, ch)) = val;
        }
        __syncthreads();

        f32x16 acc[4][2];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[mt][nt][i] = 0.0f;

#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const bf16x8 a = *(const bf16x8*)(ks + swz_chunk_offset(mt * 32 + l32, 2 * kk + h));
                acc[mt][0] = mfma32(a, qf[0][kk], acc[mt][0]);
                acc[mt][1] = mfma32(a, qf[1][kk], acc[mt][1]);
            }
        }

#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const int t = trow[nt];
            const bool diag = (t >> 7) == c;  // the query's own block: keep keys j <= t only
            float m = -INFINITY;
            if (__any(diag)) {
                const int lim = diag ? t - c * kBlock : kBlock - 1;
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        if (mt * 32 + mfma32_row(i, h) <= lim) m = fmaxf(m, acc[mt][nt][i]);
            } else {
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int i = 0; i < 16; ++i) m = fmaxf(m, acc[mt][nt][i]);
            }
            m = wave_max_xor32(m);
            if (h == nt) stage[(c - c0) * kIdxTileRows + wave * 64 + nt * 32 + l32] = m;
        }
    }
    __syncthreads();

    const int row = r0 + tid;
    if (row < R) {
        const int t = row / H, g = row - t * H;
        const int cl = t >> 7;
        float* dst = pooled + (((size_t)b * H + g) * N + t) * nblk;
        const int cend = min(c1, cl + 1);
        for (int c = c0; c < cend; ++c) dst[c] = stage[(c - c0) * kIdxTileRows + tid];
    }
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
    hipLaunchKernelGGL(k_index_pool, grid, dim3(256), 0, stream, (const __bf16*)q_idx, (const __bf16*)k_idx,
                       pooled, d.N, H, d.nblk);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !fill_upper) return e;
    const long long rows = (long long)d.B * H * d.N;
    hipLaunchKernelGGL(k_pooled_fill_upper, dim3((unsigned)rows), dim3(256), 0, stream, pooled, d.N, d.nblk, rows);
    return hipGetLastError();
}

}  // namespace msa
