// Device-side helpers shared by the libmsa kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "msa_internal.hpp"

namespace msa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// v_mfma_f32_32x32x16_bf16. Operand layouts (checked on the device):
//   A (32 x 16): lane l holds A[l % 32][8 * (l / 32) + e], e = 0..7
//   B (16 x 32): lane l holds B[8 * (l / 32) + e][l % 32]
//   D (32 x 32): lane l, register i holds D[8 * (i / 4) + 4 * (l / 32) + i % 4][l % 32]
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// v_mfma_f32_16x16x32_bf16. Operand layouts (checked on the device):
//   A (16 x 32): lane l holds A[l % 16][8 * (l / 16) + e], e = 0..7
//   B (32 x 16): lane l holds B[8 * (l / 16) + e][l % 16]
//   D (16 x 16): lane l, register i holds D[4 * (l / 16) + i][l % 16]
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Row of the 32x32 MFMA result held by lane-half `h` in register `i`.
__device__ __forceinline__ int mfma32_row(int i, int h) { return 8 * (i >> 2) + 4 * h + (i & 3); }

// A 128 x 128 bf16 tile in LDS, row-major with 256-byte rows cut into sixteen
// 16-byte chunks. Chunk `ch` of row `r` is stored at chunk slot ch ^ (r & 15),
// so the 32 rows read by one MFMA operand load fall into distinct banks.
__device__ __forceinline__ int swz_chunk_offset(int row, int ch) {
    return row * kDim + ((ch ^ (row & 15)) << 3);  // in bf16 elements
}

// Total order on fp32 scores as unsigned integers (larger float -> larger key),
// with -0.0 folded onto +0.0 so that equal scores compare equal.
__device__ __forceinline__ uint32_t order_key(float x) {
    const uint32_t u = __float_as_uint(x + 0.0f);  // -0 + 0 = +0 under round-to-nearest
    return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);  // negative: all bits flip; else the sign bit
}
// The score whose key is k (the inverse of order_key on +0 and the non-NaN floats).
__device__ __forceinline__ float key_score(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// 64-bit selection key: score first, then the LOWER block index wins ties.
__device__ __forceinline__ uint64_t select_key(float score, int block) {
    return ((uint64_t)order_key(score) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)block);
}
__device__ __forceinline__ int key_block(uint64_t key) {
    return (int)(0xFFFFFFFFu - (uint32_t)(key & 0xFFFFFFFFu));
}

// max(x[l], x[l ^ 32]) in every lane l. v_permlane32_swap gives lane l the values of lanes
// l % 32 and l % 32 + 32 (checked on the device), so no LDS round trip is needed.
__device__ __forceinline__ float wave_max_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// x[l] + x[l ^ 32] in every lane l (the two addends in the same order in both lanes of a pair).
__device__ __forceinline__ float wave_sum_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Position p of a key inside a V^T row in LDS: bits 2 and 3 of the key index are
// swapped, so that the 8 keys a lane feeds to one PV MFMA step (the keys its S^T
// registers hold) sit in one 16-byte chunk. The map is its own inverse.
__device__ __forceinline__ int vt_pos(int key) {
    return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
}

// Stage key block c of KV head g of batch b in LDS for the 32x32 MFMA attention step:
// K row-major (ks[key][dim]) and V transposed (vts[dim][vt_pos(key)]), both with
// swz_chunk_offset. K and V are [B, N, H_kv, 128] bf16. Threads tid = 0..255 take part
// (each loads 8 K chunks and 8 V chunks); the caller synchronises before and after.
__device__ __forceinline__ void stage_kv_tile(const __bf16* __restrict__ k, const __bf16* __restrict__ v,
                                              __bf16* ks, __bf16* vts, int b, int g, int c, int N, int Hkv,
                                              int tid) {
    const size_t tile_off = (((size_t)b * N + (size_t)c * kBlock) * Hkv + g) * kDim;
    const __bf16* kbase = k + tile_off;
    const __bf16* vbase = v + tile_off;
    const int kstride = Hkv * kDim;
    const int key0 = tid >> 4, ch = tid & 15;
    const int koff = key0 * kstride + ch * 8;
    uint4 kv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) kv[i] = *(const uint4*)(kbase + koff + i * 16 * kstride);  // keys key0 + 16 i
    const int voff = key0 * 4 * kstride + ch * 8;  // 4 keys 4*key0 + 64 i .. +3, dims 8 ch .. +7
    const int vp = vt_pos(key0 * 4);               // < 64, a multiple of 4
    bf16x8 rows[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) rows[i][rr] = *(const bf16x8*)(vbase + voff + (64 * i + rr) * kstride);
#pragma unroll
    for (int i = 0; i < 8; ++i) *(uint4*)(ks + swz_chunk_offset(key0 + 16 * i, ch)) = kv[i];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            bf16x4 w;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) w[rr] = rows[i][rr][e];
            *(bf16x4*)(vts + swz_chunk_offset(ch * 8 + e, (vp >> 3) + 8 * i) + (vp & 7)) = w;
        }
}

// A raw buffer descriptor over `bytes` bytes at p (p and bytes the same in every lane;
// they are read from the first lane so that the descriptor sits in scalar registers).
// Loads at offsets past `bytes` return 0 without touching memory.
constexpr int kRawBufferFlags = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void* p, int bytes) {
    const uint64_t a = (uint64_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), (short)0,
                                             __builtin_amdgcn_readfirstlane(bytes), kRawBufferFlags);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t x, int m) {
    uint32_t lo = __shfl_xor((uint32_t)x, m, 64);
    uint32_t hi = __shfl_xor((uint32_t)(x >> 32), m, 64);
    return ((uint64_t)hi << 32) | lo;
}

}  // namespace msa
