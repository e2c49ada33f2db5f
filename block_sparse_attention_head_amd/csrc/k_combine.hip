// Sparse main attention, phase 2: global softmax combine of the slot partials.
//
// [MSA summary] "GPU kernel co-design": two-phase forward, partial attention
// then a global softmax-combine kernel. Per (b, t, head), with the slot
// partials (O_s normalised, lse_s):
//   M = max_s lse_s,  w_s = exp(lse_s - M),  L = sum_s w_s,
//   O = sum_s w_s O_s / L,  LSE = M + ln L.
#include "msa_device.hpp"
#include "msa_internal.hpp"

namespace msa {

// Partial record layout: element q = hf*64 + dt*16 + i of a record holds
// dim 32*dt + 8*(i/4) + 4*hf + i%4 (the order the MFMA result registers are in).
__global__ __launch_bounds__(256) void k_combine(const __bf16* __restrict__ part_o, const float* __restrict__ part_lse,
                                                 const int32_t* __restrict__ block_idx, __bf16* __restrict__ o,
                                                 float* __restrict__ lse, int N, int Hq, int Hkv, int gshift,
                                                 int top_k) {
    const int bt = blockIdx.x;
    const int b = bt / N, t = bt - b * N;
    const int cl = t >> 7;
    for (int j = threadIdx.x; j < Hq * 16; j += 256) {
        const int head = j >> 4, ch = j & 15;
        const int g = head >> gshift;
        const int32_t* bi = block_idx + (((size_t)b * Hkv + g) * N + t) * top_k;
        const size_t rec0 = ((size_t)b * N + t) * top_k;
        float M = -INFINITY;
        for (int s = 0; s < top_k; ++s) {
            const int c = bi[s];
            if (c >= 0 && c <= cl) M = fmaxf(M, part_lse[(rec0 + s) * Hq + head]);
        }
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
        float L = 0.0f;
        if (M != -INFINITY) {
            for (int s = 0; s < top_k; ++s) {
                const int c = bi[s];
                if (c < 0 || c > cl) continue;
                const size_t rec = (rec0 + s) * Hq + head;
                const float w = expf(part_lse[rec] - M);
                L += w;
                const bf16x8 x = *(const bf16x8*)(part_o + rec * kDim + ch * 8);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] += w * (float)x[e];
            }
        }
        const float inv = L > 0.0f ? 1.0f / L : 0.0f;
        const int hf = ch >> 3, dt = (ch & 7) >> 1, i0 = (ch & 1) * 8;
        const int dim_a = 32 * dt + 2 * i0 + 4 * hf;  // elements 0..3 -> dim_a.., 4..7 -> dim_a+8..
        __bf16* orow = o + (((size_t)b * N + t) * Hq + head) * kDim;
        bf16x4 wa, wb;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            wa[e] = (__bf16)(acc[e] * inv);
            wb[e] = (__bf16)(acc[4 + e] * inv);
        }
        *(bf16x4*)(orow + dim_a) = wa;
        *(bf16x4*)(orow + dim_a + 8) = wb;
        if (ch == 0) lse[((size_t)b * Hq + head) * N + t] = M + logf(L);
    }
}

hipError_t launch_sparse_combine(const int32_t* block_idx, void* o, float* lse, const SparseWs& ws, const Dims& d,
                                 hipStream_t stream) {
    hipLaunchKernelGGL(k_combine, dim3(d.B * d.N), dim3(256), 0, stream, (const __bf16*)ws.part_o, ws.part_lse,
                       block_idx, (__bf16*)o, lse, d.N, d.Hq, d.Hkv, d.gshift, d.top_k);
    return hipGetLastError();
}

}  // namespace msa
