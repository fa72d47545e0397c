// Device-side helpers shared by the paged KV cache kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// Cache layout: [num_blocks][num_kv_heads][block_size][head_dim]; the rows of one
// (block, kv head) are contiguous, so a decode workgroup for one kv head streams whole
// block_size x head_dim tiles.
__device__ __forceinline__ int64_t cache_row(int64_t block, int kvh, int off, int num_kv_heads,
                                             int block_size) {
    return (block * num_kv_heads + kvh) * block_size + off;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// bf16 pair (packed in one dword) -> two floats, exact.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32; NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    bf16x2_t r = {(__bf16)f, (__bf16)0.0f};
    return __builtin_bit_cast(uint32_t, r) & 0xffffu;
}

// two floats -> packed bf16 pair (lo = a, hi = b), round to nearest even, one instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    bf16x2_t r = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, r);
}

// (lo16(w0), lo16(w1)) and (hi16(w0), hi16(w1)): the same element of two bf16 pairs side by side.
__device__ __forceinline__ uint32_t pair_lo(uint32_t w0, uint32_t w1) { return __builtin_amdgcn_perm(w1, w0, 0x05040100u); }
__device__ __forceinline__ uint32_t pair_hi(uint32_t w0, uint32_t w1) { return __builtin_amdgcn_perm(w1, w0, 0x07060302u); }

// dot of two bf16 pairs accumulated in fp32: acc + a.x*b.x + a.y*b.y (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b),
                                           acc, false);
}

// DPP lane permutations inside a row of 16 lanes.
// quad_perm [1,0,3,2] swaps neighbours, quad_perm [2,3,0,1] swaps pairs, row_half_mirror
// reverses each 8-lane half, row_mirror reverses the 16-lane row. Applied in that order to a
// sum, each step folds in a disjoint set of lanes, so after log2(n) steps every lane of an
// aligned n-lane group holds the group total.
enum : int { DPP_XOR1 = 0xB1, DPP_XOR2 = 0x4E, DPP_HALF_MIRROR = 0x141, DPP_MIRROR = 0x140 };

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over an aligned group of N lanes (N in {1, 2, 4, 8, 16}); every lane of the group gets it.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (N >= 2) v += dpp<DPP_XOR1>(v);
    if constexpr (N >= 4) v += dpp<DPP_XOR2>(v);
    if constexpr (N >= 8) v += dpp<DPP_HALF_MIRROR>(v);
    if constexpr (N >= 16) v += dpp<DPP_MIRROR>(v);
    return v;
}

// group_sum over K independent values, step-major: each butterfly step is applied to all K values
// before the next, so a DPP never reads the result of the instruction right before it (no wait states).
template <int N, int K>
__device__ __forceinline__ void group_sum_all(float *v) {
    if constexpr (N >= 2) {
#pragma unroll
        for (int k = 0; k < K; ++k) v[k] += dpp<DPP_XOR1>(v[k]);
    }
    if constexpr (N >= 4) {
#pragma unroll
        for (int k = 0; k < K; ++k) v[k] += dpp<DPP_XOR2>(v[k]);
    }
    if constexpr (N >= 8) {
#pragma unroll
        for (int k = 0; k < K; ++k) v[k] += dpp<DPP_HALF_MIRROR>(v[k]);
    }
    if constexpr (N >= 16) {
#pragma unroll
        for (int k = 0; k < K; ++k) v[k] += dpp<DPP_MIRROR>(v[k]);
    }
}

// Max over an aligned group of N lanes (N in {1, 2, 4, 8, 16}), same butterfly as group_sum.
template <int N>
__device__ __forceinline__ float group_max(float v) {
    if constexpr (N >= 2) v = fmaxf(v, dpp<DPP_XOR1>(v));
    if constexpr (N >= 4) v = fmaxf(v, dpp<DPP_XOR2>(v));
    if constexpr (N >= 8) v = fmaxf(v, dpp<DPP_HALF_MIRROR>(v));
    if constexpr (N >= 16) v = fmaxf(v, dpp<DPP_MIRROR>(v));
    return v;
}

// Bytes 2k and 2k + 1 of w, as signed 8-bit integers, to a bf16 pair (exact: |code| <= 128).
__device__ __forceinline__ uint32_t i8pair_to_bf16x2(uint32_t w, int k) {
    return pack_bf16x2((float)(int8_t)(w >> (16 * k)), (float)(int8_t)(w >> (16 * k + 8)));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Max and sum over lanes l, l ^ 16, l ^ 32 and l ^ 48 (one column of an MFMA result block), on the VALU:
// with both operands the same register, v_permlane16_swap leaves lane l holding the values of lanes l & ~16
// and l | 16, and v_permlane32_swap those of lanes l & ~32 and l | 32. Every lane of the four gets the same
// value (max and + are commutative, and each step combines the same two values in every lane).
__device__ __forceinline__ float lane_blocks_max(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float lane_blocks_sum(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// D = A B + C on one 16x16x32 bf16 MFMA (fp32 accumulate). Lane l supplies A[l%16][8*(l/16) .. +8]
// and B[8*(l/16) .. +8][l%16] (8 bf16 each, element order = reduction order) and holds
// D[4*(l/16) + i][l%16], i = 0..3.
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
}

// One 16-byte piece of the store: thread gid moves piece gid % CHUNKS of row gid / CHUNKS (row = token *
// num_kv_heads + kv head) from the new rows to the slot's row of the cache; slots < 0 and slots outside the
// pool move nothing. Consecutive threads take consecutive pieces of a row.
template <int CHUNKS>
__device__ __forceinline__ void store_piece(int64_t gid, const u32x4 *__restrict__ key, const u32x4 *__restrict__ value,
                                            u32x4 *__restrict__ key_cache, u32x4 *__restrict__ value_cache,
                                            const int32_t *__restrict__ slot_mapping, int64_t num_rows,
                                            int num_kv_heads, int block_size, int num_blocks) {
    const int64_t row = gid / CHUNKS;
    if (row >= num_rows) return;
    const int chunk = (int)(gid % CHUNKS);
    const int64_t token = row / num_kv_heads;
    const int kvh = (int)(row % num_kv_heads);
    const int32_t slot = slot_mapping[token];
    if (slot < 0) return;                          // padding token: nothing to write
    if (slot / block_size >= num_blocks) return;   // outside the pool: precondition broken, skip
    const int64_t block = slot / block_size;
    const int off = slot % block_size;
    const int64_t dst = cache_row(block, kvh, off, num_kv_heads, block_size) * CHUNKS + chunk;
    const int64_t src = row * CHUNKS + chunk;
    const u32x4 k = __builtin_nontemporal_load(key + src);
    const u32x4 v = __builtin_nontemporal_load(value + src);
    key_cache[dst] = k;
    value_cache[dst] = v;
}

}  // namespace pkv
