// C ABI of libpagedkv.so: argument validation, launch planning and dispatch.
// The declarations, argument meanings and error rules are in include/pagedkv.h.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "../../include/pagedkv.h"
#include "launch.h"

#define PKV_VERSION "pagedkv 0.1.0 (gfx950)"

namespace {

thread_local char g_err[512] = "";

pkv_status fail(pkv_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

pkv_status ok() {
    g_err[0] = '\0';
    return PKV_OK;
}

pkv_status hip_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return ok();
    return fail(PKV_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int elem_bytes(pkv_dtype d) { return d == PKV_F32 ? 4 : 2; }

int log2_exact(int v) {
    if (v <= 0 || (v & (v - 1))) return -1;
    int l = 0;
    while ((1 << l) < v) ++l;
    return l;
}

#define REQUIRE(cond, st, ...)                      \
    do {                                            \
        if (!(cond)) return fail(st, __VA_ARGS__);  \
    } while (0)

pkv_status check_common(pkv_dtype dtype, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                        int64_t num_blocks) {
    REQUIRE(dtype == PKV_F32 || dtype == PKV_BF16, PKV_EINVAL, "dtype %d is neither PKV_F32 nor PKV_BF16", (int)dtype);
    REQUIRE(num_kv_heads > 0, PKV_EINVAL, "num_kv_heads must be positive (got %d)", num_kv_heads);
    REQUIRE(head_dim == 64 || head_dim == 128, PKV_EUNSUPPORTED, "head_dim %d unsupported (64 or 128)", head_dim);
    REQUIRE(log2_exact(block_size) >= 0 && block_size <= 256, PKV_EUNSUPPORTED,
            "block_size %d unsupported (a power of two, 1..256)", block_size);
    REQUIRE(num_blocks >= 0, PKV_EINVAL, "num_blocks must be non-negative (got %lld)", (long long)num_blocks);
    REQUIRE(num_blocks * (int64_t)block_size <= INT32_MAX, PKV_EINVAL,
            "pool of %lld slots exceeds the int32 slot range", (long long)(num_blocks * block_size));
    return ok();
}

pkv_status check_heads(int32_t num_heads, int32_t num_kv_heads) {
    REQUIRE(num_heads > 0, PKV_EINVAL, "num_heads must be positive (got %d)", num_heads);
    REQUIRE(num_heads % num_kv_heads == 0, PKV_EINVAL, "num_heads %d is not a multiple of num_kv_heads %d",
            num_heads, num_kv_heads);
    REQUIRE(num_heads / num_kv_heads <= 8, PKV_EUNSUPPORTED, "num_heads / num_kv_heads = %d unsupported (1..8)",
            num_heads / num_kv_heads);
    REQUIRE(num_kv_heads <= 65535, PKV_EINVAL, "num_kv_heads %d exceeds 65535", num_kv_heads);
    return ok();
}

// Decode partitioning: partitions of DECODE_PART tokens (a multiple of every supported block size)
// keep each workgroup's share of a long context bounded, so a batch with a long tail still spreads
// over all compute units; sequences that fit one partition skip the reduce.
#ifndef PKV_DECODE_PART
#define PKV_DECODE_PART 1024
#endif
constexpr int DECODE_PART = PKV_DECODE_PART;

struct DecodePlan {
    int part_tokens;
    int num_parts;
    size_t ws_bytes;
    size_t off_items, off_m, off_l, off_o;
};

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

DecodePlan plan_decode(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                       int32_t block_size, int32_t max_context_len) {
    DecodePlan p{};
    // a partition spans at most decode_max_part_blocks() blocks (its table slice lives in one register)
    p.part_tokens = DECODE_PART < block_size * pkv::decode_max_part_blocks() ? DECODE_PART
                                                                             : block_size * pkv::decode_max_part_blocks();
    p.num_parts = max_context_len <= 0 ? 1 : (max_context_len + p.part_tokens - 1) / p.part_tokens;
    // [ctrl: 256 B][work items: num_seqs * num_parts int4][partials when num_parts > 1]
    (void)num_kv_heads;
    p.off_items = 256;
    p.ws_bytes = p.off_items + align256((size_t)num_seqs * p.num_parts * 16);
    if (p.num_parts > 1) {
        size_t n = (size_t)num_seqs * num_heads * p.num_parts;
        p.off_m = p.ws_bytes;
        p.off_l = p.off_m + align256(n * sizeof(float));
        p.off_o = p.off_l + align256(n * sizeof(float));
        p.ws_bytes = p.off_o + n * head_dim * sizeof(float);
    }
    return p;
}

}  // namespace

extern "C" {

const char *pkv_last_error(void) { return g_err; }

const char *pkv_version(void) { return PKV_VERSION; }

pkv_status pkv_kv_cache_store(pkv_dtype dtype, const void *key, const void *value, void *key_cache,
                              void *value_cache, const int32_t *slot_mapping, int64_t num_tokens,
                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                              hipStream_t stream) {
    pkv_status st = check_common(dtype, num_kv_heads, head_dim, block_size, num_blocks);
    if (st != PKV_OK) return st;
    REQUIRE(num_tokens >= 0, PKV_EINVAL, "num_tokens must be non-negative (got %lld)", (long long)num_tokens);
    if (num_tokens == 0) return ok();
    REQUIRE(key && value && key_cache && value_cache && slot_mapping, PKV_EINVAL, "null pointer argument");
    REQUIRE(aligned16(key) && aligned16(value) && aligned16(key_cache) && aligned16(value_cache), PKV_EINVAL,
            "key, value and cache pointers must be 16-byte aligned");
    REQUIRE(num_tokens * num_kv_heads <= (int64_t)1 << 40, PKV_EINVAL, "num_tokens too large");
    return hip_status(pkv::launch_store(key, value, key_cache, value_cache, slot_mapping, num_tokens, num_kv_heads,
                                        head_dim * elem_bytes(dtype), block_size, (int)num_blocks, stream),
                      "kv_cache_store launch");
}

pkv_status pkv_kv_cache_gather(pkv_dtype dtype, void *key_out, void *value_out, const void *key_cache,
                               const void *value_cache, const int32_t *block_table_row, int32_t len,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                               hipStream_t stream) {
    pkv_status st = check_common(dtype, num_kv_heads, head_dim, block_size, num_blocks);
    if (st != PKV_OK) return st;
    REQUIRE(len >= 0, PKV_EINVAL, "len must be non-negative (got %d)", len);
    if (len == 0) return ok();
    REQUIRE(key_out && value_out && key_cache && value_cache && block_table_row, PKV_EINVAL, "null pointer argument");
    REQUIRE(aligned16(key_out) && aligned16(value_out) && aligned16(key_cache) && aligned16(value_cache), PKV_EINVAL,
            "output and cache pointers must be 16-byte aligned");
    return hip_status(pkv::launch_gather(key_out, value_out, key_cache, value_cache, block_table_row, len,
                                         num_kv_heads, head_dim * elem_bytes(dtype), block_size, (int)num_blocks,
                                         stream),
                      "kv_cache_gather launch");
}

pkv_status pkv_kv_cache_copy_blocks(pkv_dtype dtype, void *key_cache, void *value_cache, const int32_t *pairs,
                                    int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                    int64_t num_blocks, hipStream_t stream) {
    pkv_status st = check_common(dtype, num_kv_heads, head_dim, block_size, num_blocks);
    if (st != PKV_OK) return st;
    REQUIRE(num_pairs >= 0 && num_pairs <= 65535, PKV_EINVAL, "num_pairs %d outside [0, 65535]", num_pairs);
    if (num_pairs == 0) return ok();
    REQUIRE(key_cache && value_cache && pairs, PKV_EINVAL, "null pointer argument");
    REQUIRE(aligned16(key_cache) && aligned16(value_cache), PKV_EINVAL, "cache pointers must be 16-byte aligned");
    const int64_t block_bytes = (int64_t)num_kv_heads * block_size * head_dim * elem_bytes(dtype);
    return hip_status(pkv::launch_copy_blocks(key_cache, value_cache, pairs, num_pairs, block_bytes, (int)num_blocks,
                                              stream),
                      "kv_cache_copy_blocks launch");
}

size_t pkv_paged_attention_decode_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                                 int32_t head_dim, int32_t block_size, int32_t max_context_len) {
    if (num_seqs <= 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || log2_exact(block_size) < 0) return 0;
    return plan_decode(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_context_len).ws_bytes;
}

pkv_status pkv_paged_attention_decode(pkv_dtype dtype, void *out, const void *query, const void *key_cache,
                                      const void *value_cache, const int32_t *block_tables,
                                      int32_t block_table_stride, const int32_t *context_lens, int32_t num_seqs,
                                      int32_t max_context_len, int32_t num_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t block_size, int64_t num_blocks, float scale,
                                      void *workspace, size_t workspace_bytes, hipStream_t stream) {
    pkv_status st = check_common(dtype, num_kv_heads, head_dim, block_size, num_blocks);
    if (st != PKV_OK) return st;
    st = check_heads(num_heads, num_kv_heads);
    if (st != PKV_OK) return st;
    REQUIRE(num_seqs >= 0 && num_seqs <= 65535, PKV_EINVAL, "num_seqs %d outside [0, 65535]", num_seqs);
    REQUIRE(max_context_len >= 0, PKV_EINVAL, "max_context_len must be non-negative (got %d)", max_context_len);
    REQUIRE(block_table_stride >= 0, PKV_EINVAL, "block_table_stride must be non-negative");
    REQUIRE((int64_t)max_context_len <= (int64_t)block_table_stride * block_size, PKV_EINVAL,
            "max_context_len %d exceeds block_table_stride %d * block_size %d", max_context_len, block_table_stride,
            block_size);
    REQUIRE(isfinite(scale), PKV_EINVAL, "scale must be finite");
    REQUIRE(num_blocks > 0 || max_context_len == 0, PKV_EINVAL, "empty pool with a non-empty context");
    if (num_seqs == 0) return ok();
    REQUIRE(out && query && key_cache && value_cache && context_lens, PKV_EINVAL, "null pointer argument");
    REQUIRE(block_tables || max_context_len == 0, PKV_EINVAL, "null block_tables");
    REQUIRE(aligned16(out) && aligned16(query) && aligned16(key_cache) && aligned16(value_cache), PKV_EINVAL,
            "out, query and cache pointers must be 16-byte aligned");
    DecodePlan plan = plan_decode(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_context_len);
    REQUIRE(plan.part_tokens / block_size <= pkv::decode_max_part_blocks(), PKV_EUNSUPPORTED,
            "partition spans too many blocks");
    REQUIRE(plan.num_parts <= 32767, PKV_EINVAL, "max_context_len too large (at most 32767 partitions of %d tokens)",
            plan.part_tokens);
    REQUIRE((int64_t)num_seqs * plan.num_parts * num_kv_heads <= (int64_t)1 << 24, PKV_EINVAL,
            "decode grid too large (num_seqs * partitions * num_kv_heads above 2^24)");
    REQUIRE(workspace != nullptr && workspace_bytes >= plan.ws_bytes, PKV_EWORKSPACE,
            "decode needs %zu bytes of workspace (got %zu)", plan.ws_bytes, workspace_bytes);
    REQUIRE(((uintptr_t)workspace & 255u) == 0, PKV_EINVAL, "workspace must be 256-byte aligned");
    pkv::DecodeArgs a{};
    a.out = out;
    a.query = query;
    a.key_cache = key_cache;
    a.value_cache = value_cache;
    a.block_tables = block_tables;
    a.bt_stride = block_table_stride;
    a.context_lens = context_lens;
    a.num_seqs = num_seqs;
    a.max_context_len = max_context_len;
    a.num_kv_heads = num_kv_heads;
    a.num_blocks = num_blocks;
    a.log2_bs = log2_exact(block_size);
    a.part_tokens = plan.part_tokens;
    a.num_parts = plan.num_parts;
    a.scale_log2e = scale * 1.4426950408889634f;
    a.ctrl = (int *)workspace;
    a.items = (int4 *)((char *)workspace + plan.off_items);
    if (plan.num_parts > 1) {
        a.ws_m = (float *)((char *)workspace + plan.off_m);
        a.ws_l = (float *)((char *)workspace + plan.off_l);
        a.ws_o = (float *)((char *)workspace + plan.off_o);
    }
    return hip_status(pkv::launch_decode(a, dtype == PKV_BF16, head_dim, num_heads / num_kv_heads, stream),
                      "paged_attention_decode launch");
}

pkv_status pkv_paged_attention_prefill(pkv_dtype dtype, void *out, const void *query, const void *key_cache,
                                       const void *value_cache, const int32_t *block_tables,
                                       int32_t block_table_stride, const int32_t *cu_seqlens_q,
                                       const int32_t *cu_seqlens_k, int32_t num_seqs, int32_t max_seqlen_q,
                                       int32_t max_seqlen_k, int32_t num_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t block_size, int64_t num_blocks, float scale,
                                       int32_t causal, hipStream_t stream) {
    pkv_status st = check_common(dtype, num_kv_heads, head_dim, block_size, num_blocks);
    if (st != PKV_OK) return st;
    st = check_heads(num_heads, num_kv_heads);
    if (st != PKV_OK) return st;
    REQUIRE(dtype == PKV_BF16, PKV_EUNSUPPORTED, "prefill runs on bf16 MFMA; dtype must be PKV_BF16");
    REQUIRE(head_dim == 128, PKV_EUNSUPPORTED, "prefill supports head_dim 128 (got %d)", head_dim);
    REQUIRE(num_seqs >= 0 && num_seqs <= 65535, PKV_EINVAL, "num_seqs %d outside [0, 65535]", num_seqs);
    REQUIRE(max_seqlen_q >= 0 && max_seqlen_k >= 0, PKV_EINVAL, "max_seqlen_q/k must be non-negative");
    REQUIRE(max_seqlen_q <= max_seqlen_k, PKV_EINVAL, "max_seqlen_q %d exceeds max_seqlen_k %d", max_seqlen_q,
            max_seqlen_k);
    REQUIRE(block_table_stride >= 0, PKV_EINVAL, "block_table_stride must be non-negative");
    REQUIRE((int64_t)max_seqlen_k <= (int64_t)block_table_stride * block_size, PKV_EINVAL,
            "max_seqlen_k %d exceeds block_table_stride %d * block_size %d", max_seqlen_k, block_table_stride,
            block_size);
    REQUIRE(isfinite(scale), PKV_EINVAL, "scale must be finite");
    REQUIRE(num_blocks > 0 || max_seqlen_k == 0, PKV_EINVAL, "empty pool with a non-empty context");
    if (num_seqs == 0 || max_seqlen_q == 0) return ok();
    REQUIRE(out && query && key_cache && value_cache && block_tables && cu_seqlens_q && cu_seqlens_k, PKV_EINVAL,
            "null pointer argument");
    REQUIRE(aligned16(out) && aligned16(query) && aligned16(key_cache) && aligned16(value_cache), PKV_EINVAL,
            "out, query and cache pointers must be 16-byte aligned");
    REQUIRE((int64_t)num_seqs * num_kv_heads * ((max_seqlen_q + 15) / 16 + 8) <= ((int64_t)1 << 26), PKV_EINVAL,
            "prefill grid too large");
    pkv::PrefillArgs a{};
    a.out = out;
    a.query = query;
    a.key_cache = key_cache;
    a.value_cache = value_cache;
    a.block_tables = block_tables;
    a.bt_stride = block_table_stride;
    a.cu_seqlens_q = cu_seqlens_q;
    a.cu_seqlens_k = cu_seqlens_k;
    a.num_seqs = num_seqs;
    a.max_seqlen_q = max_seqlen_q;
    a.max_seqlen_k = max_seqlen_k;
    a.num_kv_heads = num_kv_heads;
    a.num_blocks = num_blocks;
    a.log2_bs = log2_exact(block_size);
    a.scale_log2e = scale * 1.4426950408889634f;
    a.causal = causal ? 1 : 0;
    return hip_status(pkv::launch_prefill(a, true, head_dim, num_heads / num_kv_heads, stream),
                      "paged_attention_prefill launch");
}

}  // extern "C"
