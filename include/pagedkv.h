/*
 * pagedkv.h -- C ABI of the MI355X (gfx950) paged KV cache library, libpagedkv.so.
 *
 * The library implements the hot path of a block-table paged KV cache:
 *   pkv_kv_cache_store          scatter new K/V rows into their slots;
 *   pkv_paged_attention_decode  one query token per sequence attends over its cached tokens;
 *   pkv_paged_attention_prefill a varlen chunk of queries per sequence attends causally over its
 *                               cached prefix plus the chunk;
 *   pkv_kv_cache_gather         inverse of the store for one block table (test helper);
 *   pkv_kv_cache_copy_blocks    copy whole blocks (copy-on-write of shared blocks);
 *   pkv_kv_cache_store_int8, pkv_paged_attention_decode_int8, pkv_paged_attention_prefill_int8:
 *                               the same over an int8 cache;
 *   pkv_kv_cache_store_fp8, pkv_paged_attention_decode_fp8, pkv_paged_attention_prefill_fp8:
 *                               the same over an fp8 (E4M3) cache;
 *   pkv_kv_cache_store_int4, pkv_paged_attention_decode_int4:
 *                               store and decode over an int4 cache (two codes per byte);
 *   pkv_paged_attention_decode_plan and pkv_paged_attention_decode_run (_int8_run, _fp8_run, _int4_run):
 *                               a decode call in two halves, the work list built once per step
 *                               and reused by every layer's attention;
 *   pkv_paged_decode_step       store + decode of one step in one call (one launch fewer);
 *   pkv_paged_attention_decode_noalloc, pkv_paged_attention_decode_status: a decode without a workspace
 *                               argument; the run status of a workspace.
 *
 * Vocabulary (nano-vllm walkthrough, section 2 context: is_prefill, cu_seqlens_q/k, max_seqlen_q/k,
 * slot_mapping, context_lens, block_tables; "推理运行时", section 分页 KV: logical block j of a
 * request maps to physical block b_j through its block table):
 *   block_size     tokens per physical block (a power of two, 1..256);
 *   block_tables   int32 [num_seqs][block_table_stride]: entry j is the physical block that holds
 *                  the sequence's logical tokens [j*block_size, (j+1)*block_size); entries past
 *                  ceil(len / block_size) are never read (any value, e.g. -1);
 *   slot           physical_block * block_size + offset_in_block, a flat token-row index;
 *   context_lens   int32 [num_seqs]: tokens each decode query attends to, the token stored this
 *                  step included ("LLM Infra 101 v0.2: KV Cache", section 推理);
 *   cu_seqlens_q/k int32 [num_seqs + 1] prefix sums of the per-sequence query counts and key counts.
 *
 * Memory layout (all device memory, row-major, densely packed, 16-byte aligned):
 *   key_cache, value_cache  [num_blocks][num_kv_heads][block_size][head_dim] of the dtype;
 *   decode query / out      [num_seqs][num_heads][head_dim];
 *   prefill query / out     [total_q][num_heads][head_dim], total_q = cu_seqlens_q[num_seqs];
 *   new key / value rows    [num_tokens][num_kv_heads][head_dim].
 * Query head h reads kv head h / (num_heads / num_kv_heads).
 *
 * Ownership and ordering: the caller owns every buffer; the library never allocates, frees or
 * synchronises. Every call is enqueued on `stream` (0 = the null stream) and returns before the
 * GPU work ends; ordering between calls is the caller's stream order (store before attention).
 *
 * Errors: a call returns PKV_OK or an error status and never aborts. Arguments known on the host
 * are checked before any launch (PKV_EINVAL for null or misaligned pointers, negative or
 * inconsistent sizes; PKV_EUNSUPPORTED for a head_dim, block_size or head grouping without a
 * kernel; PKV_EWORKSPACE for a too-small workspace); nothing is launched on error. Launch failures
 * return PKV_EHIP. pkv_last_error() gives the message of the calling thread's last error.
 * Contents of device arrays (slot values, block ids, lengths) are preconditions, not checked:
 * non-negative slots must be unique and < num_blocks * block_size; block ids read must lie in
 * [0, num_blocks); 0 <= context_lens[i] <= max_context_len; cu_seqlens non-decreasing with
 * per-sequence query count <= key count <= max_seqlen_k.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { PKV_F32 = 0, PKV_BF16 = 1 } pkv_dtype;
/* The cache a decode plan is made for: elements of the query's dtype, int8 codes or E4M3 codes. */
typedef enum { PKV_CACHE_ELEMENTS = 0, PKV_CACHE_INT8 = 1, PKV_CACHE_FP8 = 2, PKV_CACHE_INT4 = 3 } pkv_cache_kind;

typedef enum {
    PKV_OK = 0,
    PKV_EINVAL = 1,
    PKV_EUNSUPPORTED = 2,
    PKV_EWORKSPACE = 3,
    PKV_EHIP = 4,
    PKV_ENOMEM = 5          /* host block manager: too few free blocks */
} pkv_status;

/*
 * kv_cache_store ("reshape_and_cache"). For each n in [0, num_tokens) with s = slot_mapping[n] >= 0,
 * writes key[n] and value[n] ([num_kv_heads][head_dim] each) to row (s / block_size, :, s % block_size)
 * of key_cache / value_cache; slots < 0 are padding and write nothing. A pure copy: bit-exact.
 * Source: nano-vllm walkthrough, section 2 context (slot_mapping); Mini-SGLang 源码解析（二）,
 * section 6.7 (out_loc, one allocated slot per new token, written into the page table) and
 * section 7.2 (a spare page absorbs padding writes -- here a negative slot does).
 * slot_mapping: device int32 [num_tokens]. num_blocks bounds the pool (used for validation of sizes).
 */
pkv_status pkv_kv_cache_store(pkv_dtype dtype, const void *key, const void *value, void *key_cache,
                              void *value_cache, const int32_t *slot_mapping, int64_t num_tokens,
                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                              hipStream_t stream);

/*
 * Bytes of device workspace pkv_paged_attention_decode needs for these sizes (0 only when num_seqs is
 * 0). The call cuts sequences into parts on the device, from the actual context_lens, so that the batch
 * spreads evenly over the GPU; the size is the bound for any lengths up to max_context_len: a work list
 * of 16 bytes per part, 16 bytes per sequence, and the partial softmax state of every part (fp32 max,
 * sum and head_dim accumulators per head) that a reduce pass merges.
 */
size_t pkv_paged_attention_decode_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                                 int32_t head_dim, int32_t block_size, int32_t max_context_len);

/*
 * paged_attention_decode. For sequence i and query head h (kv head h / G, G = num_heads / num_kv_heads):
 *   out[i][h] = sum_{t < context_lens[i]} softmax_t(scale * query[i][h] . K_i[t]) V_i[t],
 * with K_i[t] = key_cache[block_tables[i][t / block_size]][h / G][t % block_size] and likewise V.
 * A sequence with context_lens[i] == 0 gets zeros. fp32 data computes in fp32. bf16 data: q.k and
 * p.v take bf16 operands with fp32 accumulation (on MFMA for head_dim 128 and block_size >= 16, on
 * v_dot2_f32_bf16 otherwise), the softmax weights rounded to bf16 for p.v (the denominator sums the same
 * rounded weights); output rounded to bf16 (nearest even).
 * Source: "推理运行时", section 分页 KV (attention reads K/V through the block table);
 * "LLM Infra 101 v0.2: KV Cache", section 推理 (decode attends to the cache plus the new token).
 * block_tables: device int32 [num_seqs][block_table_stride]; context_lens: device int32 [num_seqs];
 * max_context_len: host bound on context_lens (sizes the grid and the workspace), must be
 * <= block_table_stride * block_size. workspace: device memory, 256-byte aligned, of at least
 * pkv_paged_attention_decode_workspace_size(...) bytes; it holds the work list the call builds on the
 * device (longest partitions first) and the split-K partials. A call overwrites it; calls that share a
 * workspace must be ordered on one stream.
 * head_dim in {64, 128}; num_heads / num_kv_heads in 1..8.
 */
pkv_status pkv_paged_attention_decode(pkv_dtype dtype, void *out, const void *query, const void *key_cache,
                                      const void *value_cache, const int32_t *block_tables,
                                      int32_t block_table_stride, const int32_t *context_lens, int32_t num_seqs,
                                      int32_t max_context_len, int32_t num_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t block_size, int64_t num_blocks, float scale,
                                      void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * paged_decode_step: one decode step of a layer in one call: pkv_kv_cache_store of each sequence's new token
 * (key, value [num_seqs][num_kv_heads][head_dim]; slot_mapping device int32 [num_seqs], slot < 0 writes
 * nothing) followed by pkv_paged_attention_decode over the same caches, with the same results (bit-identical
 * caches and outputs). The store's rows move in the same launch as the decode's work-list plan (the plan reads
 * only context_lens, the store writes only cache rows), which saves a launch per step. Arguments, layouts,
 * workspace and errors are those of the two calls; key and value must be 16-byte aligned.
 * Source: the store-then-attend order of a decode step (nano-vllm walkthrough, section 2 context: slot_mapping
 * names where each new token's K/V go before attention reads the cache; "LLM Infra 101 v0.2: KV Cache",
 * section 推理: the new token attends to the cache and itself).
 */
pkv_status pkv_paged_decode_step(pkv_dtype dtype, const void *key, const void *value, const int32_t *slot_mapping,
                                 void *out, const void *query, void *key_cache, void *value_cache,
                                 const int32_t *block_tables, int32_t block_table_stride, const int32_t *context_lens,
                                 int32_t num_seqs, int32_t max_context_len, int32_t num_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int64_t num_blocks, float scale,
                                 void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * paged_attention_prefill (varlen, chunked). Sequence i owns query rows [cu_seqlens_q[i], cu_seqlens_q[i+1])
 * (Lq rows) and has Lk = cu_seqlens_k[i+1] - cu_seqlens_k[i] tokens in the cache, the last Lq of
 * which are this chunk (already stored); P = Lk - Lq is its cached prefix. Query row j of the chunk
 * is position P + j; when causal it attends to logical tokens [0, P + j], else to [0, Lk).
 * Same softmax, GQA mapping, block-table addressing and precision as decode (bf16 only: the
 * products run on MFMA with bf16 operands and fp32 accumulation; the softmax weights are rounded
 * to bf16 for the second product).
 * Source: nano-vllm walkthrough, section 2 context (cu_seqlens_q/k, max_seqlen_q/k, block_tables);
 * Mini-SGLang 源码解析（二）, sections 6.6 and 6.9 (a chunk extends cached_len by extend_len);
 * "推理运行时", sections Chunked prefill and Prefill 与 decode 输入 (flattened tokens with
 * per-sequence query ranges; chunked prefill has a cached history).
 * cu_seqlens_q, cu_seqlens_k: device int32 [num_seqs + 1], starting at 0. max_seqlen_q and
 * max_seqlen_k: host bounds on Lq and Lk (size the grid); max_seqlen_k <= block_table_stride * block_size.
 * dtype must be PKV_BF16; head_dim 128; num_heads / num_kv_heads in 1..8.
 */
pkv_status pkv_paged_attention_prefill(pkv_dtype dtype, void *out, const void *query, const void *key_cache,
                                       const void *value_cache, const int32_t *block_tables,
                                       int32_t block_table_stride, const int32_t *cu_seqlens_q,
                                       const int32_t *cu_seqlens_k, int32_t num_seqs, int32_t max_seqlen_q,
                                       int32_t max_seqlen_k, int32_t num_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t block_size, int64_t num_blocks, float scale,
                                       int32_t causal, hipStream_t stream);

/*
 * kv_cache_gather: logical tokens [0, len) of one block table row into contiguous key_out /
 * value_out [len][num_kv_heads][head_dim]; the inverse of the store, used to check it bit-exactly.
 * Source: nano-vllm walkthrough, section 2 Sequence (token i of a sequence sits in block i / block_size).
 * block_table_row: device int32 [ceil(len / block_size)].
 */
pkv_status pkv_kv_cache_gather(pkv_dtype dtype, void *key_out, void *value_out, const void *key_cache,
                               const void *value_cache, const int32_t *block_table_row, int32_t len,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                               hipStream_t stream);

/*
 * kv_cache_copy_blocks: for each pair k, physical block pairs[2k+1] of both caches becomes a copy of
 * block pairs[2k] (all kv heads, all block_size rows). Used for copy-on-write of a shared block before a
 * branch writes into it ("推理运行时", section Prefix cache 与 copy-on-write). pairs: device int32
 * [2 * num_pairs]; destinations must be distinct and no destination may be a source of another pair;
 * ids outside [0, num_blocks) are skipped.
 */
pkv_status pkv_kv_cache_copy_blocks(pkv_dtype dtype, void *key_cache, void *value_cache, const int32_t *pairs,
                                    int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                    int64_t num_blocks, hipStream_t stream);

/*
 * int8 KV cache ("LLM Infra 101 v0.2: KV Cache", inference-engine list, KV Quantization: the cache keeps
 * K/V as int8 instead of bf16, trading some accuracy for half the bytes). The pages fix no scheme; this
 * library keeps one fp32 scale per (token, kv head) row:
 *   scale = max_d |x_d| / 127,  code_d = round_half_even(x_d / scale) clamped to [-127, 127]
 * computed in fp32 with IEEE division (a row of zeros: scale 0, codes 0), so codes are bit-exact with
 * any implementation of the same formula. Dequantized, x_d ~ code_d * scale with |error| <= scale / 2.
 *   key_cache, value_cache  int8 [num_blocks][num_kv_heads][block_size][head_dim];
 *   key_scale, value_scale  fp32 [num_blocks][num_kv_heads][block_size], one per cache row.
 */

/*
 * kv_cache_store_int8: like pkv_kv_cache_store, but each (token, kv head) row of key / value (dtype
 * PKV_F32 or PKV_BF16, [num_tokens][num_kv_heads][head_dim], head_dim 64 or 128) is quantized as above;
 * its codes land in the int8 caches at the slot's row and its scale at the same (block, kv head, offset)
 * of the scale arrays. Rows must be finite. Cache pointers 16-byte aligned, scales 4-byte aligned.
 */
pkv_status pkv_kv_cache_store_int8(pkv_dtype dtype, const void *key, const void *value, int8_t *key_cache,
                                   int8_t *value_cache, float *key_scale, float *value_scale,
                                   const int32_t *slot_mapping, int64_t num_tokens, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t block_size, int64_t num_blocks, hipStream_t stream);

/*
 * paged_attention_decode_int8: pkv_paged_attention_decode over an int8 cache: attention over the
 * dequantized K/V (code * scale). dtype (query and out) must be PKV_BF16, head_dim 128, block_size >= 16
 * (PKV_EUNSUPPORTED otherwise). q.k runs on MFMA with the codes as exact bf16 integers and fp32
 * accumulation, times the row's K scale; each softmax weight is multiplied by its row's V scale and
 * rounded to bf16 for p.v (the denominator sums the unrounded weights). Scale arrays 16-byte aligned.
 * Workspace: pkv_paged_attention_decode_workspace_size with the same sizes.
 */
pkv_status pkv_paged_attention_decode_int8(pkv_dtype dtype, void *out, const void *query, const int8_t *key_cache,
                                           const int8_t *value_cache, const float *key_scale,
                                           const float *value_scale, const int32_t *block_tables,
                                           int32_t block_table_stride, const int32_t *context_lens, int32_t num_seqs,
                                           int32_t max_context_len, int32_t num_heads, int32_t num_kv_heads,
                                           int32_t head_dim, int32_t block_size, int64_t num_blocks, float scale,
                                           void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * fp8 KV cache (same source: an 8-bit cache instead of bf16). The pages name no 8-bit float format; this
 * library uses OCP float8 E4M3, the element type of gfx950's fp8 conversions: 1 sign bit, 4 exponent bits
 * (bias 7), 3 mantissa bits, subnormals (m / 8) * 2^-6, no infinities, NaN only for S.1111.111, largest
 * finite magnitude 448. One fp32 scale per (token, kv head) row:
 *   scale = max_d |x_d| / 448,  code_d = E4M3(x_d / scale), rounded to nearest, ties to even,
 * in fp32 with IEEE division (a row of zeros: scale 0, codes 0); |x_d / scale| <= 448 up to one rounding,
 * so no code is NaN. Dequantized, x_d ~ value(code_d) * scale with |error| <= 2^-4 |x_d| where
 * |x_d / scale| >= 2^-6, else <= 2^-10 scale.
 *   key_cache, value_cache  uint8 codes [num_blocks][num_kv_heads][block_size][head_dim];
 *   key_scale, value_scale  fp32 [num_blocks][num_kv_heads][block_size], one per cache row.
 */

/* kv_cache_store_fp8: pkv_kv_cache_store_int8 with E4M3 codes as above (same arguments, alignment, errors). */
pkv_status pkv_kv_cache_store_fp8(pkv_dtype dtype, const void *key, const void *value, uint8_t *key_cache,
                                  uint8_t *value_cache, float *key_scale, float *value_scale,
                                  const int32_t *slot_mapping, int64_t num_tokens, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t block_size, int64_t num_blocks, hipStream_t stream);

/*
 * paged_attention_decode_fp8: pkv_paged_attention_decode_int8 over an fp8 cache: attention over the
 * dequantized K/V (value(code) * scale), with the same restrictions (bf16 query and out, head_dim 128,
 * block_size >= 16), precision and workspace. The codes become exact bf16 values on the GPU.
 */
pkv_status pkv_paged_attention_decode_fp8(pkv_dtype dtype, void *out, const void *query, const uint8_t *key_cache,
                                          const uint8_t *value_cache, const float *key_scale,
                                          const float *value_scale, const int32_t *block_tables,
                                          int32_t block_table_stride, const int32_t *context_lens, int32_t num_seqs,
                                          int32_t max_context_len, int32_t num_heads, int32_t num_kv_heads,
                                          int32_t head_dim, int32_t block_size, int64_t num_blocks, float scale,
                                          void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * paged_attention_prefill_int8 / paged_attention_prefill_fp8: pkv_paged_attention_prefill over an int8 or
 * an fp8 (E4M3) cache (layouts and quantization as for the 8-bit decode above): attention over the
 * dequantized K/V, code * scale (int8) or value(code) * scale (E4M3). The codes become exact bf16 values in
 * the workgroup's K/V tiles; q.k runs on MFMA with fp32 accumulation and is multiplied by each key row's
 * K scale; each softmax weight is multiplied by its row's V scale and rounded to bf16 for p.v (the
 * denominator sums the unscaled weights). The chunk's rows must be stored (kv_cache_store_int8 / _fp8)
 * before the call. Same arguments, restrictions (bf16 query and out, head_dim 128) and errors as
 * pkv_paged_attention_prefill, plus key_scale, value_scale: device fp32 [num_blocks][num_kv_heads]
 * [block_size], 4-byte aligned (null: PKV_EINVAL).
 * Source: as pkv_paged_attention_prefill; the 8-bit cache as for pkv_paged_attention_decode_int8.
 */
pkv_status pkv_paged_attention_prefill_int8(pkv_dtype dtype, void *out, const void *query, const int8_t *key_cache,
                                            const int8_t *value_cache, const float *key_scale,
                                            const float *value_scale, const int32_t *block_tables,
                                            int32_t block_table_stride, const int32_t *cu_seqlens_q,
                                            const int32_t *cu_seqlens_k, int32_t num_seqs, int32_t max_seqlen_q,
                                            int32_t max_seqlen_k, int32_t num_heads, int32_t num_kv_heads,
                                            int32_t head_dim, int32_t block_size, int64_t num_blocks, float scale,
                                            int32_t causal, hipStream_t stream);
pkv_status pkv_paged_attention_prefill_fp8(pkv_dtype dtype, void *out, const void *query, const uint8_t *key_cache,
                                           const uint8_t *value_cache, const float *key_scale,
                                           const float *value_scale, const int32_t *block_tables,
                                           int32_t block_table_stride, const int32_t *cu_seqlens_q,
                                           const int32_t *cu_seqlens_k, int32_t num_seqs, int32_t max_seqlen_q,
                                           int32_t max_seqlen_k, int32_t num_heads, int32_t num_kv_heads,
                                           int32_t head_dim, int32_t block_size, int64_t num_blocks, float scale,
                                           int32_t causal, hipStream_t stream);

/*
 * int4 KV cache (same passage, which names int4 beside int8). The pages fix no scheme; this library keeps
 * one fp32 scale per (token, kv head) row and two 4-bit codes per byte:
 *   scale = max_d |x_d| / 7,  q_d = round_half_even(x_d / scale) clamped to [-7, 7],  u_d = q_d + 8,
 * computed in fp32 with IEEE division (a row of zeros: scale 0, u = 8); element 2j in the low four bits of
 * byte j, element 2j + 1 in the high four bits. Dequantized, x_d ~ q_d * scale with |error| <= scale / 2.
 *   key_cache, value_cache  uint8 [num_blocks][num_kv_heads][block_size][head_dim / 2];
 *   key_scale, value_scale  fp32 [num_blocks][num_kv_heads][block_size], one per cache row.
 */

/*
 * kv_cache_store_int4: pkv_kv_cache_store_int8 with the int4 codes above (rows of head_dim / 2 bytes).
 * key / value PKV_F32 or PKV_BF16, head_dim 64 or 128; rows must be finite. Cache pointers 16-byte aligned,
 * scales 4-byte aligned.
 */
pkv_status pkv_kv_cache_store_int4(pkv_dtype dtype, const void *key, const void *value, uint8_t *key_cache,
                                   uint8_t *value_cache, float *key_scale, float *value_scale,
                                   const int32_t *slot_mapping, int64_t num_tokens, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t block_size, int64_t num_blocks, hipStream_t stream);

/*
 * paged_attention_decode_int4: pkv_paged_attention_decode over an int4 cache: attention over the
 * dequantized K/V ((u - 8) * scale). dtype (query and out) must be PKV_BF16, head_dim 128, block_size >= 16
 * (PKV_EUNSUPPORTED otherwise). The codes enter the MFMA products as the exact bf16 values 136 + q; the
 * scores subtract 136 times the head's query sum, the outputs 136 times the sum of the bf16 weights that
 * multiplied V (fp32). Otherwise as pkv_paged_attention_decode_int8: K scale times each score, V scale
 * times each weight before its bf16 rounding, denominator over the unrounded weights. Scale arrays 16-byte
 * aligned. Workspace: pkv_paged_attention_decode_workspace_size with the same sizes.
 */
pkv_status pkv_paged_attention_decode_int4(pkv_dtype dtype, void *out, const void *query, const uint8_t *key_cache,
                                           const uint8_t *value_cache, const float *key_scale,
                                           const float *value_scale, const int32_t *block_tables,
                                           int32_t block_table_stride, const int32_t *context_lens, int32_t num_seqs,
                                           int32_t max_context_len, int32_t num_heads, int32_t num_kv_heads,
                                           int32_t head_dim, int32_t block_size, int64_t num_blocks, float scale,
                                           void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * paged_attention_decode_plan / paged_attention_decode_run: one decode call in two halves. A model runs
 * the same attention metadata (context_lens, block_tables) through every layer of a step (nano-vllm
 * walkthrough, section 2 context: the context is set once per forward pass and read by each layer's
 * attention), so the work list that pkv_paged_attention_decode builds from context_lens on every call can
 * be built once: pkv_paged_attention_decode_plan writes it into `workspace`; each
 * pkv_paged_attention_decode_run (or _int8_run / _fp8_run / _int4_run over a quantized cache) then decodes from it and
 * writes out, exactly as the whole call would (bit-identical results).
 * plan: context_lens (device int32 [num_seqs]) and the sizes a run will use; cache_kind is the cache the runs
 *   read (PKV_CACHE_ELEMENTS: the query's dtype; PKV_CACHE_INT8 / _FP8 / _INT4: a quantized cache, which
 *   needs a bf16 query, head_dim 128 and block_size >= 16), which sizes the parts for that kernel. Errors as for
 *   pkv_paged_attention_decode (no cache or output pointers are taken).
 * run: the arguments of pkv_paged_attention_decode (or of its _int8 / _fp8 / _int4 form) without context_lens. It
 *   needs a workspace planned with the same num_seqs, max_context_len, num_heads, num_kv_heads, head_dim,
 *   block_size, cache kind and query dtype, and the same context_lens (the caller's contract for the lengths:
 *   the work list records token ranges; a run over a stale plan attends over the planned lengths), and reads
 *   the plan in stream order. A run whose sizes differ from its plan's is detected on the device: it writes
 *   nothing and raises the workspace's run status (pkv_paged_attention_decode_status). A whole decode call
 *   leaves the same plan in its workspace.
 * Source: the attention metadata of the pages above, built once per step; the work list as for
 * pkv_paged_attention_decode.
 */
pkv_status pkv_paged_attention_decode_plan(pkv_dtype dtype, int32_t cache_kind, const int32_t *context_lens,
                                           int32_t num_seqs, int32_t max_context_len, int32_t num_heads,
                                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                           void *workspace, size_t workspace_bytes, hipStream_t stream);
pkv_status pkv_paged_attention_decode_run(pkv_dtype dtype, void *out, const void *query, const void *key_cache,
                                          const void *value_cache, const int32_t *block_tables,
                                          int32_t block_table_stride, int32_t num_seqs, int32_t max_context_len,
                                          int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                          int32_t block_size, int64_t num_blocks, float scale, void *workspace,
                                          size_t workspace_bytes, hipStream_t stream);
pkv_status pkv_paged_attention_decode_int8_run(pkv_dtype dtype, void *out, const void *query,
                                               const int8_t *key_cache, const int8_t *value_cache,
                                               const float *key_scale, const float *value_scale,
                                               const int32_t *block_tables, int32_t block_table_stride,
                                               int32_t num_seqs, int32_t max_context_len, int32_t num_heads,
                                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                               int64_t num_blocks, float scale, void *workspace,
                                               size_t workspace_bytes, hipStream_t stream);
pkv_status pkv_paged_attention_decode_fp8_run(pkv_dtype dtype, void *out, const void *query,
                                              const uint8_t *key_cache, const uint8_t *value_cache,
                                              const float *key_scale, const float *value_scale,
                                              const int32_t *block_tables, int32_t block_table_stride,
                                              int32_t num_seqs, int32_t max_context_len, int32_t num_heads,
                                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                              int64_t num_blocks, float scale, void *workspace,
                                              size_t workspace_bytes, hipStream_t stream);
pkv_status pkv_paged_attention_decode_int4_run(pkv_dtype dtype, void *out, const void *query,
                                               const uint8_t *key_cache, const uint8_t *value_cache,
                                               const float *key_scale, const float *value_scale,
                                               const int32_t *block_tables, int32_t block_table_stride,
                                               int32_t num_seqs, int32_t max_context_len, int32_t num_heads,
                                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                               int64_t num_blocks, float scale, void *workspace,
                                               size_t workspace_bytes, hipStream_t stream);

/*
 * paged_attention_decode_status: enqueues on `stream` a copy of the workspace's run status into *status (device
 * memory or pinned host memory; 4 bytes): 0 when every run since the workspace's last plan matched that plan,
 * 1 when a run found the workspace planned for other sizes. A plan (or whole decode call) records in the
 * workspace what it was made for: num_seqs, max_context_len, num_heads, num_kv_heads, head_dim, block_size,
 * the cache kind and the query dtype. A run compares that record with its own arguments before it reads the
 * work list and, on any difference, writes nothing (out keeps its contents) and sets the status to 1; the next
 * plan resets it to 0. Read the status after the run in stream order.
 * Source: none on the pages; this guards the plan/run split above (a run over a plan for other sizes would
 * otherwise index the workspace with another layout).
 */
pkv_status pkv_paged_attention_decode_status(const void *workspace, int32_t *status, hipStream_t stream);

/*
 * paged_attention_decode_noalloc: pkv_paged_attention_decode with no workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the call allocates nothing and takes no workspace; it uses a library-owned scratch array of
 * PKV_NOALLOC_SCRATCH_BYTES per GPU, created when the library's code loads on that GPU and held until the
 * process ends. Sizes whose workspace bound (pkv_paged_attention_decode_workspace_size) exceeds it are refused
 * with PKV_EWORKSPACE before anything is launched; other arguments, errors and results are those of
 * pkv_paged_attention_decode (bit-identical outputs). Every call on one GPU uses the same array and leaves
 * its contents there: calls that may overlap on one GPU (different streams, or host threads without an
 * order between their calls) race; keep them on one stream. Nothing in it needs to start at zero: each
 * call's plan kernel writes the work list and control words its decode and reduce kernels read.
 */
#define PKV_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
pkv_status pkv_paged_attention_decode_noalloc(pkv_dtype dtype, void *out, const void *query, const void *key_cache,
                                              const void *value_cache, const int32_t *block_tables,
                                              int32_t block_table_stride, const int32_t *context_lens,
                                              int32_t num_seqs, int32_t max_context_len, int32_t num_heads,
                                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                              int64_t num_blocks, float scale, hipStream_t stream);

/* Message of the calling thread's last non-OK status ("" if none). Owned by the library. */
const char *pkv_last_error(void);

/* Library version string. */
const char *pkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
