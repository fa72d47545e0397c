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

// Quantized caches, one fp32 scale per row: format 0 int8 codes, 1 OCP float8 E4M3 codes, 2 int4 codes
// (offset by 8, two per byte).
hipError_t launch_store_q8(bool bf16, int format, int head_dim, const void *key, const void *value, void *key_cache,
                           void *value_cache, float *key_scale, float *value_scale, const int32_t *slot_mapping,
                           int64_t num_tokens, int num_kv_heads, int block_size, int num_blocks, hipStream_t stream);

hipError_t launch_copy_blocks(void *key_cache, void *value_cache, const int32_t *pairs, int num_pairs, int64_t block_bytes,
                              int num_blocks, hipStream_t stream);

// What a decode plan was made for: the sizes that fix the workspace layout and the unit list (num_seqs,
// max_context_len, num_kv_heads, num_heads, head_dim, log2 block_size) and the cache it sizes parts for
// (cache kind | query dtype << 4), after a magic word. The plan kernel writes it into the workspace's control
// block; the decode and reduce kernels compare it with their own before touching anything else and, on a
// mismatch, set the control block's error word and exit.
struct PlanKey {
    int w[8];
};
constexpr int PLAN_KEY_MAGIC = 0x504b5650;
constexpr int CTRL_PARTS = 0;          // int32 words of the 256-byte control block
constexpr int CTRL_RED = 1;            // entries of the reduce list
constexpr int CTRL_KEY = 8;            // [8, 16): the plan's key
constexpr int CTRL_ERR = 16;           // 0 after a plan; 1 once a run found a key other than its own

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
    int workers;           // resident one-wave workgroups (8 per compute unit)
    int compute_units;     // compute units (the matrix-core decode runs one workgroup on each)
    int min_strata;        // the plan aims at min_strata * workers units (at most that many when every
                           // sequence fits one unit per worker)
    int max_part_tiles;    // longest part, in 32-token tiles (its table slice must fit 64 lanes)
    int min_part_tiles;    // shortest part a sequence is split into, in tiles
    int64_t max_items;     // bound on the number of parts (sizes the work list and partials)
    float scale_log2e;
    int4 *items;           // work list, [max_items]
    int4 *seq_info;        // [num_seqs]: first partial slot, parts, part length, length
    int *red_list;         // [num_seqs]: sequences the reduce kernel serves (split, or empty), ctrl[CTRL_RED] of them
    int *ctrl;             // ctrl[0] = number of parts
    float *ws_m;           // [max_items][num_heads]
    float *ws_l;           // [max_items][num_heads]
    float *ws_o;           // [max_items][num_heads][head_dim]
    const float *key_scale = nullptr;     // 8-bit caches only: [num_blocks][num_kv_heads][block_size]
    const float *value_scale = nullptr;
    bool fp8_codes = false;               // quantized caches: E4M3 codes instead of int8
    bool int4_codes = false;              // quantized caches: 4-bit codes (two per byte) instead of int8
    bool run_only = false;                // decode and reduce from a work list already in the workspace
    PlanKey key{};                        // written by the plan, checked by the run
    // A decode step with its store (pkv_paged_decode_step): the store's rows move in the plan's launch.
    const void *st_key = nullptr;         // new rows [st_tokens][num_kv_heads][row bytes]
    const void *st_value = nullptr;
    void *st_key_cache = nullptr;
    void *st_value_cache = nullptr;
    const int32_t *st_slots = nullptr;    // [st_tokens]
    int64_t st_tokens = 0;
    int st_chunks = 0;                    // 16-byte pieces per row (8, 16 or 32); 0: no store in this call
    int st_block_size = 0;
};

hipError_t launch_decode(const DecodeArgs &a, bool bf16, int head_dim, int group, hipStream_t stream);
// 8-bit caches (int8 or E4M3 codes + per-row scales), bf16 query and output, head_dim 128, block_size >= 16.
hipError_t launch_decode_q8(const DecodeArgs &a, int group, hipStream_t stream);
// The plan kernel alone (the work list a later run_only call decodes from), for the kernel that will run:
// the matrix-core one (decode_uses_mfma, or any 8-bit cache) or not, over an 8-bit cache or not.
hipError_t launch_decode_plan(const DecodeArgs &a, bool mfma, bool q8, hipStream_t stream);
bool decode_uses_mfma(bool bf16, int head_dim, int group, int log2_bs);
int decode_max_part_blocks();
int decode_tile_tokens();

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
    const float *key_scale = nullptr;     // 8-bit caches only: [num_blocks][num_kv_heads][block_size]
    const float *value_scale = nullptr;
    bool fp8_codes = false;               // quantized caches: E4M3 codes instead of int8
    bool int4_codes = false;              // quantized caches: 4-bit codes (two per byte) instead of int8
};

hipError_t launch_prefill(const PrefillArgs &a, bool bf16, int head_dim, int group, hipStream_t stream);
// 8-bit caches (int8 or E4M3 codes + per-row scales), bf16 query and output, head_dim 128.
hipError_t launch_prefill_q8(const PrefillArgs &a, int group, hipStream_t stream);

}  // namespace pkv
