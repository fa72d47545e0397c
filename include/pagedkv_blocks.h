/*
 * pagedkv_blocks.h -- host-side KV block manager of libpagedkv.so (C ABI, CPU only, not thread-safe:
 * one manager per scheduler thread).
 *
 * It owns the bookkeeping that feeds the kernels of pagedkv.h: which physical blocks a request holds
 * (its block table), the slot of each new token (slot_mapping), and how full the pool is.
 * Sources:
 *   - "LLM Infra 101 v0.5" (ifuryst.com), section KV Block Manager: FIFO free list; allocate takes
 *     ceil(tokens / block_size) blocks, append takes the blocks a request's new length needs, release
 *     returns them; a request allocated twice, an unknown request, a negative count or too few free
 *     blocks is an error; section 推理: the usage metrics and the contiguous fixed-slot baseline.
 *   - nano-vllm walkthrough (lpnh.cn), section 3: with prefix caching, full blocks are keyed by a chained
 *     hash of the token ids, reused on a hit whose token ids match (after the first miss every later
 *     block misses), reference counted, released last block first, their hash kept after release.
 *   - "推理运行时" (wineandchord.com), section Prefix cache 与 copy-on-write: a branch that writes into a
 *     shared block that is not full copies it first.
 * Ownership: the manager is created and destroyed by the caller; buffers passed in are the caller's.
 * Errors: PKV_EINVAL for bad arguments or unknown / duplicate requests, PKV_ENOMEM when the pool has too
 * few free blocks (nothing changes then); pkv_bm_last_error() gives the message.
 */
#ifndef PAGEDKV_BLOCKS_H
#define PAGEDKV_BLOCKS_H

#include <stdint.h>

#include "pagedkv.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pkv_block_manager pkv_block_manager;

typedef struct {
    int64_t num_requests;
    int64_t allocated_tokens;                /* tokens held by live requests */
    int64_t reserved_tokens;                 /* used_blocks * block_size */
    int64_t internal_fragmentation_tokens;   /* reserved - allocated */
    double block_utilization;                /* allocated / reserved */
    int64_t used_blocks;                     /* blocks with a reference (shared blocks count once) */
    int64_t free_blocks;
    int64_t max_request_tokens;
    int64_t contiguous_reserved_tokens;      /* baseline: every request reserves the longest one's length */
    int64_t contiguous_fragmentation_tokens;
    double contiguous_utilization;
} pkv_bm_usage_t;

/* A pool of total_blocks blocks of block_size tokens; prefix_caching != 0 enables hashed block reuse. */
pkv_status pkv_bm_create(int32_t total_blocks, int32_t block_size, int32_t prefix_caching, pkv_block_manager **out);
void pkv_bm_destroy(pkv_block_manager *bm);

/* Blocks for a new request of num_tokens tokens. token_ids (host, [num_tokens]) are required with prefix
 * caching and ignored otherwise; *num_cached_tokens (may be NULL) receives the tokens served by reused
 * blocks (a multiple of block_size). */
pkv_status pkv_bm_allocate(pkv_block_manager *bm, int64_t request_id, int32_t num_tokens, const int32_t *token_ids,
                           int32_t *num_cached_tokens);

/* Grow a request by num_tokens tokens (decode steps, later prefill chunks). If its last block is shared
 * and not full, the block is replaced by a fresh one and the pair (old, new) is queued for
 * pkv_kv_cache_copy_blocks (copy-on-write). */
pkv_status pkv_bm_append(pkv_block_manager *bm, int64_t request_id, int32_t num_tokens, const int32_t *token_ids);

/* A new request sharing every block of an existing one (parallel sampling, beam branches). */
pkv_status pkv_bm_fork(pkv_block_manager *bm, int64_t parent_id, int64_t child_id);

/* Return a request's blocks, last block first; a block goes back to the free list when unreferenced. */
pkv_status pkv_bm_release(pkv_block_manager *bm, int64_t request_id);

/* The request's block table into out[0..capacity) (entries past its blocks set to -1; out may be NULL to
 * query the sizes). */
pkv_status pkv_bm_block_table(const pkv_block_manager *bm, int64_t request_id, int32_t *out, int32_t capacity,
                              int32_t *num_blocks, int64_t *num_tokens);

/* Slots of positions [first_position, first_position + count) of a request:
 * slot = block_table[pos / block_size] * block_size + pos % block_size. */
pkv_status pkv_bm_slot_mapping(const pkv_block_manager *bm, int64_t request_id, int64_t first_position, int32_t count,
                               int32_t *slots);

/* Pending copy-on-write pairs as [src0, dst0, src1, dst1, ...]; pairs == NULL only reports the count, a
 * non-NULL buffer of capacity >= count pairs receives them and empties the queue. */
pkv_status pkv_bm_take_copies(pkv_block_manager *bm, int32_t *pairs, int32_t capacity, int32_t *num_pairs);

pkv_status pkv_bm_usage(const pkv_block_manager *bm, pkv_bm_usage_t *usage);

const char *pkv_bm_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_BLOCKS_H */
