// Internal launch interface between the C-ABI layer (api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// Store and gather guard the pool on the device: a slot or block id outside
// [0, num_blocks * block_size) / [0, num_blocks) moves nothing (gather writes zeros).
hipError_t launch_store(const void *key, const void *value, void *key_cache, void *value_cache,
                        const int32_t *slot_mapping, int64_t num_tokens, int num_kv_heads, int row_bytes,
                        int block_size, int num_blocks, hipStream_t stream);

hipError_t launch_gather(void *key_out, void *value_out, const void *key_cache, const void *value_cache,
                         const int32_t *block_table_row, int64_t len, int num_kv_heads, int row_bytes,
                         int block_size, int num_blocks, hipStream_t stream);

hipError_t launch_copy_blocks(void *key_cache, void *value_cache, const int32_t *pairs, int num_pairs, int64_t block_bytes,
                              int num_blocks, hipStream_t stream);

struct DecodeArgs {
    void *out;
    const void *query;
    const void *key_cache;
    const void *value_cache;
    const int32_t *block_tables;
    int bt_stride;
    const int32_t *context_lens;
    int num_seqs;
    int max_context_len;   // lengths are clamped to it on the device
    int num_kv_heads;
    int64_t num_blocks;    // tokens whose block id lies outside [0, num_blocks) are skipped
    int log2_bs;
    int part_tokens;       // tokens per partition, a multiple of the block size
    int num_parts;         // ceil(max_context_len / part_tokens), >= 1
    float scale_log2e;
    int4 *items;           // work list, [num_seqs * num_parts]
    int *ctrl;             // ctrl[0] = number of work items
    float *ws_m;           // [num_seqs][num_heads][num_parts]   (used when num_parts > 1)
    float *ws_l;           // [num_seqs][num_heads][num_parts]
    float *ws_o;           // [num_seqs][num_heads][num_parts][head_dim]
};

hipError_t launch_decode(const DecodeArgs &a, bool bf16, int head_dim, int group, hipStream_t stream);
int decode_max_part_blocks();

struct PrefillArgs {
    void *out;
    const void *query;
    const void *key_cache;
    const void *value_cache;
    const int32_t *block_tables;
    int bt_stride;
    const int32_t *cu_seqlens_q;
    const int32_t *cu_seqlens_k;
    int num_seqs;
    int max_seqlen_q;      // query tiles past it are not launched
    int max_seqlen_k;      // key counts are clamped to it on the device
    int num_kv_heads;
    int64_t num_blocks;
    int log2_bs;
    float scale_log2e;
    int causal;
};

hipError_t launch_prefill(const PrefillArgs &a, bool bf16, int head_dim, int group, hipStream_t stream);

}  // namespace pkv
