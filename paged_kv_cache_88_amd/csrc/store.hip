// kv_cache_store: scatter each new token's K and V rows into the slot named by slot_mapping,
// and kv_cache_gather, its inverse for one block table (used to check the store bit-exactly).
//
// A slot is physical_block * block_size + offset (nano-vllm walkthrough, section 2 context,
// slot_mapping; Mini-SGLang 源码解析（二）, section 6.7: out_loc allocated per new token and written
// into the page table). The copy is a pure byte move, so the result is bit-exact.
//
// Work decomposition: one thread moves 16 bytes. A (token, kv head) row is head_dim * elem
// bytes = CHUNKS 16-byte pieces; consecutive threads take consecutive pieces of the same row, so
// each wave reads a contiguous run of the source and writes whole 128-byte lines of the cache.
#include <algorithm>

#include "device_common.h"
#include "launch.h"

namespace pkv {

template <int CHUNKS>
__global__ void __launch_bounds__(256) store_kernel(const u32x4 *__restrict__ key, const u32x4 *__restrict__ value,
                                                    u32x4 *__restrict__ key_cache, u32x4 *__restrict__ value_cache,
                                                    const int32_t *__restrict__ slot_mapping, int64_t num_rows,
                                                    int num_kv_heads, int block_size, int num_blocks) {
    store_piece<CHUNKS>((int64_t)blockIdx.x * blockDim.x + threadIdx.x, key, value, key_cache, value_cache,
                        slot_mapping, num_rows, num_kv_heads, block_size, num_blocks);
}

template <int CHUNKS>
__global__ void __launch_bounds__(256) gather_kernel(u32x4 *__restrict__ key_out, u32x4 *__restrict__ value_out,
                                                     const u32x4 *__restrict__ key_cache,
                                                     const u32x4 *__restrict__ value_cache,
                                                     const int32_t *__restrict__ block_table_row, int64_t num_rows,
                                                     int num_kv_heads, int block_size, int num_blocks) {
    int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    int64_t row = gid / CHUNKS;            // row = token * num_kv_heads + kv head
    if (row >= num_rows) return;
    int chunk = (int)(gid % CHUNKS);
    int64_t token = row / num_kv_heads;
    int kvh = (int)(row % num_kv_heads);
    int64_t block = block_table_row[token / block_size];
    if (block < 0 || block >= num_blocks) {      // outside the pool: precondition broken, zeros
        key_out[row * CHUNKS + chunk] = u32x4{0, 0, 0, 0};
        value_out[row * CHUNKS + chunk] = u32x4{0, 0, 0, 0};
        return;
    }
    int off = (int)(token % block_size);
    int64_t src = cache_row(block, kvh, off, num_kv_heads, block_size) * CHUNKS + chunk;
    key_out[row * CHUNKS + chunk] = key_cache[src];
    value_out[row * CHUNKS + chunk] = value_cache[src];
}

// Quantizing store ("LLM Infra 101 v0.2: KV Cache", inference-engine list, KV Quantization: K/V kept as
// int8 or int4 instead of bf16). Each (token, kv head) row of D elements gets one fp32 scale, all in fp32
// with IEEE division, so codes are reproducible bit for bit:
//   int8 (FMT 0): scale = max|x| / 127, code = round_half_even(x / scale) clamped to [-127, 127], one byte;
//   fp8 (FMT 1):  scale = max|x| / 448, code = OCP float8 E4M3 of x / scale, rounded to nearest with
//                 ties to even by v_cvt_pk_fp8_f32 (|x / scale| <= 448 up to one rounding: never NaN), one byte;
//   int4 (FMT 2): scale = max|x| / 7, q = round_half_even(x / scale) clamped to [-7, 7], stored as u = q + 8
//                 in four bits, element 2j in the low half of byte j (rows of D / 2 bytes);
// zero rows get scale 0 and q = 0. Codes land in the cache [num_blocks][num_kv_heads][block_size][row bytes]
// at the slot's row, the scale at the same (block, kv head, offset) of the [num_blocks][num_kv_heads][block_size]
// scale array.
// One row per aligned group of D / 8 lanes, 8 elements per lane; the row max is a DPP butterfly.
enum { STORE_INT8 = 0, STORE_FP8 = 1, STORE_INT4 = 2 };
template <bool BF16, int D, int FMT>
__global__ void __launch_bounds__(256) store_q8_kernel(const void *__restrict__ key, const void *__restrict__ value,
                                                       uint8_t *__restrict__ key_cache, uint8_t *__restrict__ value_cache,
                                                       float *__restrict__ key_scale, float *__restrict__ value_scale,
                                                       const int32_t *__restrict__ slot_mapping, int64_t num_rows,
                                                       int num_kv_heads, int block_size, int num_blocks) {
    constexpr int L = D / 8;               // lanes per row
    constexpr int RB = FMT == STORE_INT4 ? D / 2 : D;     // bytes per cache row
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t row = gid / L;           // row = token * num_kv_heads + kv head; uniform over the group
    if (row >= num_rows) return;
    const int part = (int)(gid % L);
    const int64_t token = row / num_kv_heads;
    const int kvh = (int)(row % num_kv_heads);
    const int32_t slot = slot_mapping[token];
    if (slot < 0 || slot / block_size >= num_blocks) return;   // padding, or outside the pool: skip
    const int64_t crow = cache_row(slot / block_size, kvh, slot % block_size, num_kv_heads, block_size);
#pragma unroll
    for (int kv = 0; kv < 2; ++kv) {
        const void *src = kv ? value : key;
        float x[8];
        if constexpr (BF16) {
            const u32x4 w = ((const u32x4 *)src)[row * (D / 8) + part];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                x[2 * j] = bf16_lo(w[j]);
                x[2 * j + 1] = bf16_hi(w[j]);
            }
        } else {
            const f32x4 a = ((const f32x4 *)src)[row * (D / 4) + 2 * part];
            const f32x4 b = ((const f32x4 *)src)[row * (D / 4) + 2 * part + 1];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                x[j] = a[j];
                x[4 + j] = b[j];
            }
        }
        float a = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) a = fmaxf(a, fabsf(x[j]));
        a = group_max<L>(a);
        const float scale = a / (FMT == STORE_FP8 ? 448.0f : FMT == STORE_INT4 ? 7.0f : 127.0f);
        uint8_t *dst = (kv ? value_cache : key_cache) + crow * RB;
        if constexpr (FMT == STORE_FP8) {
            float qv[8];
            uint32_t packed[2];
#pragma unroll
            for (int j = 0; j < 8; ++j) qv[j] = a > 0.f ? x[j] / scale : 0.f;
#pragma unroll
            for (int w = 0; w < 2; ++w) {
                int p = __builtin_amdgcn_cvt_pk_fp8_f32(qv[4 * w], qv[4 * w + 1], 0, false);      // bytes 0, 1
                p = __builtin_amdgcn_cvt_pk_fp8_f32(qv[4 * w + 2], qv[4 * w + 3], p, true);        // bytes 2, 3
                packed[w] = (uint32_t)p;
            }
            *(uint2 *)(dst + 8 * part) = make_uint2(packed[0], packed[1]);
        } else if constexpr (FMT == STORE_INT4) {
            uint32_t packed = 0u;                          // element 8 part + j in bits 4 j .. 4 j + 3
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                float q = 0.f;
                if (a > 0.f) q = fminf(fmaxf(__builtin_rintf(x[j] / scale), -7.f), 7.f);
                packed |= (uint32_t)((int)q + 8) << (4 * j);
            }
            *(uint32_t *)(dst + 4 * part) = packed;
        } else {
            uint32_t packed[2] = {0u, 0u};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                float c = 0.f;
                if (a > 0.f) c = fminf(fmaxf(__builtin_rintf(x[j] / scale), -127.f), 127.f);
                packed[j / 4] |= ((uint32_t)(int32_t)c & 0xffu) << (8 * (j % 4));
            }
            *(uint2 *)(dst + 8 * part) = make_uint2(packed[0], packed[1]);
        }
        if (part == 0) (kv ? value_scale : key_scale)[crow] = scale;
    }
}

hipError_t launch_store_q8(bool bf16, int format, int head_dim, const void *key, const void *value, void *key_cache,
                           void *value_cache, float *key_scale, float *value_scale, const int32_t *slot_mapping,
                           int64_t num_tokens, int num_kv_heads, int block_size, int num_blocks, hipStream_t stream) {
    const int64_t rows = num_tokens * num_kv_heads;
    const int64_t threads = rows * (head_dim / 8);
    if (threads == 0) return hipSuccess;
    if (format < STORE_INT8 || format > STORE_INT4) return hipErrorInvalidValue;
    dim3 grid((unsigned)((threads + 255) / 256)), block(256);
    auto kc = (uint8_t *)key_cache, vc = (uint8_t *)value_cache;
#define PKV_STORE_Q8(B, DD, F)                                                                                          \
    hipLaunchKernelGGL((store_q8_kernel<B, DD, F>), grid, block, 0, stream, key, value, kc, vc, key_scale, value_scale, \
                       slot_mapping, rows, num_kv_heads, block_size, num_blocks)
#define PKV_STORE_Q8_D(B, F)                  \
    if (head_dim == 128) PKV_STORE_Q8(B, 128, F); \
    else PKV_STORE_Q8(B, 64, F)
#define PKV_STORE_Q8_F(B)                                                \
    if (format == STORE_FP8) { PKV_STORE_Q8_D(B, STORE_FP8); }           \
    else if (format == STORE_INT4) { PKV_STORE_Q8_D(B, STORE_INT4); }    \
    else { PKV_STORE_Q8_D(B, STORE_INT8); }
    if (bf16) {
        PKV_STORE_Q8_F(true)
    } else {
        PKV_STORE_Q8_F(false)
    }
#undef PKV_STORE_Q8_F
#undef PKV_STORE_Q8_D
#undef PKV_STORE_Q8
    return hipGetLastError();
}

// Copy whole blocks (all kv heads): one thread moves 16 bytes; blockIdx.y is the pair.
__global__ void __launch_bounds__(256) copy_blocks_kernel(u32x4 *__restrict__ key_cache, u32x4 *__restrict__ value_cache,
                                                          const int32_t *__restrict__ pairs, int64_t block_vecs,
                                                          int num_blocks) {
    const int32_t src = pairs[2 * blockIdx.y], dst = pairs[2 * blockIdx.y + 1];
    if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < block_vecs; i += (int64_t)gridDim.x * blockDim.x) {
        key_cache[(int64_t)dst * block_vecs + i] = key_cache[(int64_t)src * block_vecs + i];
        value_cache[(int64_t)dst * block_vecs + i] = value_cache[(int64_t)src * block_vecs + i];
    }
}

hipError_t launch_copy_blocks(void *key_cache, void *value_cache, const int32_t *pairs, int num_pairs, int64_t block_bytes,
                              int num_blocks, hipStream_t stream) {
    if (num_pairs == 0) return hipSuccess;
    const int64_t vecs = block_bytes / 16;
    const unsigned gx = (unsigned)std::min<int64_t>((vecs + 255) / 256, 64);
    hipLaunchKernelGGL(copy_blocks_kernel, dim3(gx, num_pairs), dim3(256), 0, stream, (u32x4 *)key_cache,
                       (u32x4 *)value_cache, pairs, vecs, num_blocks);
    return hipGetLastError();
}

hipError_t launch_store(const void *key, const void *value, void *key_cache, void *value_cache,
                        const int32_t *slot_mapping, int64_t num_tokens, int num_kv_heads, int row_bytes,
                        int block_size, int num_blocks, hipStream_t stream) {
    int64_t rows = num_tokens * num_kv_heads;
    int chunks = row_bytes / 16;
    int64_t threads = rows * chunks;
    if (threads == 0) return hipSuccess;
    dim3 grid((unsigned)((threads + 255) / 256)), block(256);
    auto k = (const u32x4 *)key, v = (const u32x4 *)value;
    auto kc = (u32x4 *)key_cache, vc = (u32x4 *)value_cache;
    switch (chunks) {
        case 8: hipLaunchKernelGGL(store_kernel<8>, grid, block, 0, stream, k, v, kc, vc, slot_mapping, rows, num_kv_heads, block_size, num_blocks); break;
        case 16: hipLaunchKernelGGL(store_kernel<16>, grid, block, 0, stream, k, v, kc, vc, slot_mapping, rows, num_kv_heads, block_size, num_blocks); break;
        case 32: hipLaunchKernelGGL(store_kernel<32>, grid, block, 0, stream, k, v, kc, vc, slot_mapping, rows, num_kv_heads, block_size, num_blocks); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_gather(void *key_out, void *value_out, const void *key_cache, const void *value_cache,
                         const int32_t *block_table_row, int64_t len, int num_kv_heads, int row_bytes, int block_size,
                         int num_blocks, hipStream_t stream) {
    int64_t rows = len * num_kv_heads;
    int chunks = row_bytes / 16;
    int64_t threads = rows * chunks;
    if (threads == 0) return hipSuccess;
    dim3 grid((unsigned)((threads + 255) / 256)), block(256);
    auto ko = (u32x4 *)key_out, vo = (u32x4 *)value_out;
    auto kc = (const u32x4 *)key_cache, vc = (const u32x4 *)value_cache;
    switch (chunks) {
        case 8: hipLaunchKernelGGL(gather_kernel<8>, grid, block, 0, stream, ko, vo, kc, vc, block_table_row, rows, num_kv_heads, block_size, num_blocks); break;
        case 16: hipLaunchKernelGGL(gather_kernel<16>, grid, block, 0, stream, ko, vo, kc, vc, block_table_row, rows, num_kv_heads, block_size, num_blocks); break;
        case 32: hipLaunchKernelGGL(gather_kernel<32>, grid, block, 0, stream, ko, vo, kc, vc, block_table_row, rows, num_kv_heads, block_size, num_blocks); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace pkv
