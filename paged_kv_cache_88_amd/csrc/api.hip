// C ABI of libpagedkv.so: argument validation, launch planning and dispatch.
// The declarations, argument meanings and error rules are in include/pagedkv.h.
#include <math.h>
#include <stdarg.h>

#include <atomic>
#include <mutex>
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

// Decode work sizing. The plan kernel cuts sequences into parts on the device (see decode.hip); the host
// fixes the bounds it works within:
//   workers: resident waves, 8 per compute unit (2 per SIMD at the decode kernels' register budget),
//     capped at DECODE_MAX_WORKERS (MI355X: 256 CUs); the matrix-core kernel runs 4 of them per compute
//     unit over bf16 caches and 8 over 8-bit caches. The plan aims at DECODE_MIN_STRATA units per
//     worker, so a longest-first schedule can even out the ends;
//   max part length: its block-table slice must fit the 64 lanes of a wave (64 blocks when parts start on
//     a block boundary, i.e. block_size <= 32; 63 otherwise), in whole 32-token tiles;
//   min part length: DECODE_MIN_PART_TILES tiles, so partials never dominate the traffic.
// The number of parts is at most 2 B + ceil(strata workers / Hkv) + ceil(B * ceil(max_context_len / 32) / max_tiles)
// (each sequence adds at most one part above its share of the target length and one above its share of
// the slice limit; when the plan lengthens parts to fit one unit per worker there are at most
// strata workers / Hkv), which sizes the work list and the partial buffers.
#ifndef PKV_DECODE_MIN_STRATA
#define PKV_DECODE_MIN_STRATA 1
#endif
#ifndef PKV_DECODE_WAVES_PER_CU
#define PKV_DECODE_WAVES_PER_CU 8
#endif
constexpr int DECODE_WAVES_PER_CU = PKV_DECODE_WAVES_PER_CU;
constexpr int DECODE_MAX_WORKERS = 256 * DECODE_WAVES_PER_CU;
constexpr int DECODE_MIN_STRATA = PKV_DECODE_MIN_STRATA;
constexpr int DECODE_MIN_PART_TILES = 4;

// Per-device cache of the worker count. Any host thread may call in: the entries are atomics, and two
// threads that both miss compute and store the same value.
int decode_workers() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return DECODE_MAX_WORKERS;
    if (dev < 64) {
        const int w = cached[dev].load(std::memory_order_relaxed);
        if (w > 0) return w;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    const int w = cus * DECODE_WAVES_PER_CU < DECODE_MAX_WORKERS ? cus * DECODE_WAVES_PER_CU : DECODE_MAX_WORKERS;
    if (dev < 64) cached[dev].store(w, std::memory_order_relaxed);
    return w;
}

struct DecodePlan {
    int max_part_tiles;
    int64_t max_items;
    size_t ws_bytes;
    size_t off_items, off_info, off_red, off_m, off_l, off_o;
};

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

DecodePlan plan_decode(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                       int32_t block_size, int32_t max_context_len) {
    DecodePlan p{};
    const int tile = pkv::decode_tile_tokens();
    const int slice_blocks = block_size <= tile ? pkv::decode_max_part_blocks() : pkv::decode_max_part_blocks() - 1;
    p.max_part_tiles = slice_blocks * block_size / tile;
    const int64_t max_tiles_per_seq = ((int64_t)(max_context_len > 0 ? max_context_len : 0) + tile - 1) / tile;
    p.max_items = 2 * (int64_t)num_seqs +
                  ((int64_t)DECODE_MAX_WORKERS * DECODE_MIN_STRATA + num_kv_heads - 1) / num_kv_heads +
                  ((int64_t)num_seqs * max_tiles_per_seq + p.max_part_tiles - 1) / p.max_part_tiles;
    // [ctrl: 256 B][work list][per-sequence info][reduce list][partials m, l, o]
    const size_t n = (size_t)p.max_items * num_heads;
    p.off_items = 256;
    p.off_info = p.off_items + align256((size_t)p.max_items * 16);
    p.off_red = p.off_info + align256((size_t)num_seqs * 16);
    p.off_m = p.off_red + align256((size_t)num_seqs * 4);
    p.off_l = p.off_m + align256(n * sizeof(float));
    p.off_o = p.off_l + align256(n * sizeof(float));
    p.ws_bytes = p.off_o + n * head_dim * sizeof(float);
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

}  // extern "C"

namespace {

// Validation and argument set-up shared by the decode entry points. A whole call (DECODE_CALL) needs every
// pointer; a plan (DECODE_PLAN_ONLY) only context_lens and the workspace; a run (DECODE_RUN_ONLY) everything
// but context_lens, which its plan already read.
enum DecodeMode { DECODE_CALL, DECODE_PLAN_ONLY, DECODE_RUN_ONLY };

pkv_status decode_args(pkv::DecodeArgs &a, pkv_dtype dtype, void *out, const void *query,
                       const void *key_cache, const void *value_cache, const int32_t *block_tables,
                       int32_t block_table_stride, const int32_t *context_lens, int32_t num_seqs,
                       int32_t max_context_len, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                       int32_t block_size, int64_t num_blocks, float scale, void *workspace, size_t workspace_bytes,
                       DecodeMode mode = DECODE_CALL, int cache_kind = PKV_CACHE_ELEMENTS) {
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
    REQUIRE(context_lens || mode == DECODE_RUN_ONLY, PKV_EINVAL, "null context_lens");
    if (mode != DECODE_PLAN_ONLY) {
        REQUIRE(out && query && key_cache && value_cache, PKV_EINVAL, "null pointer argument");
        REQUIRE(block_tables || max_context_len == 0, PKV_EINVAL, "null block_tables");
        REQUIRE(aligned16(out) && aligned16(query) && aligned16(key_cache) && aligned16(value_cache), PKV_EINVAL,
                "out, query and cache pointers must be 16-byte aligned");
    }
    DecodePlan plan = plan_decode(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_context_len);
    REQUIRE((int64_t)num_seqs * (((int64_t)max_context_len + 31) / 32) < ((int64_t)1 << 30), PKV_EINVAL,
            "num_seqs * max_context_len too large (at most 2^35 tokens)");
    REQUIRE(plan.max_items * num_kv_heads <= (int64_t)1 << 26, PKV_EINVAL,
            "decode work list too large (num_kv_heads * parts above 2^26)");
    REQUIRE(workspace != nullptr && workspace_bytes >= plan.ws_bytes, PKV_EWORKSPACE,
            "decode needs %zu bytes of workspace (got %zu)", plan.ws_bytes, workspace_bytes);
    REQUIRE(((uintptr_t)workspace & 255u) == 0, PKV_EINVAL, "workspace must be 256-byte aligned");
    a = pkv::DecodeArgs{};
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
    a.workers = decode_workers();
    a.compute_units = a.workers / DECODE_WAVES_PER_CU;
    a.min_strata = DECODE_MIN_STRATA;
    a.max_part_tiles = plan.max_part_tiles;
    a.min_part_tiles = DECODE_MIN_PART_TILES;
    a.max_items = plan.max_items;
    a.scale_log2e = scale * 1.4426950408889634f;
    a.ctrl = (int *)workspace;
    a.items = (int4 *)((char *)workspace + plan.off_items);
    a.seq_info = (int4 *)((char *)workspace + plan.off_info);
    a.red_list = (int *)((char *)workspace + plan.off_red);
    a.ws_m = (float *)((char *)workspace + plan.off_m);
    a.ws_l = (float *)((char *)workspace + plan.off_l);
    a.ws_o = (float *)((char *)workspace + plan.off_o);
    a.run_only = mode == DECODE_RUN_ONLY;
    a.key = pkv::PlanKey{{pkv::PLAN_KEY_MAGIC, num_seqs, max_context_len, num_kv_heads, num_heads, head_dim,
                          a.log2_bs, cache_kind | ((int)dtype << 4)}};
    return ok();
}

}  // namespace

extern "C" {

pkv_status pkv_paged_attention_decode(pkv_dtype dtype, void *out, const void *query, const void *key_cache,
                                      const void *value_cache, const int32_t *block_tables,
                                      int32_t block_table_stride, const int32_t *context_lens, int32_t num_seqs,
                                      int32_t max_context_len, int32_t num_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t block_size, int64_t num_blocks, float scale,
                                      void *workspace, size_t workspace_bytes, hipStream_t stream) {
    pkv::DecodeArgs a{};
    pkv_status st = decode_args(a, dtype, out, query, key_cache, value_cache, block_tables,
                                block_table_stride, context_lens, num_seqs, max_context_len, num_heads, num_kv_heads,
                                head_dim, block_size, num_blocks, scale, workspace, workspace_bytes);
    if (st != PKV_OK || num_seqs == 0) return st;
    return hip_status(pkv::launch_decode(a, dtype == PKV_BF16, head_dim, num_heads / num_kv_heads, stream),
                      "paged_attention_decode launch");
}

pkv_status pkv_paged_decode_step(pkv_dtype dtype, const void *key, const void *value, const int32_t *slot_mapping,
                                 void *out, const void *query, void *key_cache, void *value_cache,
                                 const int32_t *block_tables, int32_t block_table_stride, const int32_t *context_lens,
                                 int32_t num_seqs, int32_t max_context_len, int32_t num_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int64_t num_blocks, float scale,
                                 void *workspace, size_t workspace_bytes, hipStream_t stream) {
    pkv::DecodeArgs a{};
    pkv_status st = decode_args(a, dtype, out, query, key_cache, value_cache, block_tables, block_table_stride,
                                context_lens, num_seqs, max_context_len, num_heads, num_kv_heads, head_dim, block_size,
                                num_blocks, scale, workspace, workspace_bytes);
    if (st != PKV_OK || num_seqs == 0) return st;
    REQUIRE(key && value && slot_mapping, PKV_EINVAL, "null pointer argument");
    REQUIRE(aligned16(key) && aligned16(value), PKV_EINVAL, "key and value pointers must be 16-byte aligned");
    a.st_key = key;
    a.st_value = value;
    a.st_key_cache = key_cache;
    a.st_value_cache = value_cache;
    a.st_slots = slot_mapping;
    a.st_tokens = num_seqs;
    a.st_chunks = head_dim * elem_bytes(dtype) / 16;
    a.st_block_size = block_size;
    return hip_status(pkv::launch_decode(a, dtype == PKV_BF16, head_dim, num_heads / num_kv_heads, stream),
                      "paged_decode_step launch");
}

}  // extern "C"

namespace {

// Shared bodies of the int8, fp8 and int4 entry points (the same layouts up to the row bytes, checks and
// kernels; only the code type differs). format: 0 int8, 1 fp8, 2 int4.
enum { Q_INT8 = 0, Q_FP8 = 1, Q_INT4 = 2 };
pkv_status store_q8(int format, const char *what, pkv_dtype dtype, const void *key, const void *value,
                    void *key_cache, void *value_cache, float *key_scale, float *value_scale,
                    const int32_t *slot_mapping, int64_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                    int32_t block_size, int64_t num_blocks, hipStream_t stream) {
    pkv_status st = check_common(dtype, num_kv_heads, head_dim, block_size, num_blocks);
    if (st != PKV_OK) return st;
    REQUIRE(num_tokens >= 0, PKV_EINVAL, "num_tokens must be non-negative (got %lld)", (long long)num_tokens);
    if (num_tokens == 0) return ok();
    REQUIRE(key && value && key_cache && value_cache && key_scale && value_scale && slot_mapping, PKV_EINVAL,
            "null pointer argument");
    REQUIRE(aligned16(key) && aligned16(value) && aligned16(key_cache) && aligned16(value_cache) &&
                ((uintptr_t)key_scale & 3u) == 0 && ((uintptr_t)value_scale & 3u) == 0,
            PKV_EINVAL, "key, value and cache pointers must be 16-byte aligned, scales 4-byte aligned");
    REQUIRE(num_tokens * num_kv_heads <= (int64_t)1 << 40, PKV_EINVAL, "num_tokens too large");
    return hip_status(pkv::launch_store_q8(dtype == PKV_BF16, format, head_dim, key, value, key_cache, value_cache,
                                           key_scale, value_scale, slot_mapping, num_tokens, num_kv_heads, block_size,
                                           (int)num_blocks, stream),
                      what);
}

pkv_status decode_q8(int format, const char *what, pkv_dtype dtype, void *out, const void *query,
                     const void *key_cache, const void *value_cache, const float *key_scale,
                     const float *value_scale, const int32_t *block_tables, int32_t block_table_stride,
                     const int32_t *context_lens, int32_t num_seqs, int32_t max_context_len, int32_t num_heads,
                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks, float scale,
                     void *workspace, size_t workspace_bytes, hipStream_t stream, DecodeMode mode = DECODE_CALL) {
    REQUIRE(dtype == PKV_BF16, PKV_EUNSUPPORTED, "quantized-cache decode takes a bf16 query (got dtype %d)",
            (int)dtype);
    REQUIRE(head_dim == 128, PKV_EUNSUPPORTED, "quantized-cache decode supports head_dim 128 (got %d)", head_dim);
    REQUIRE(block_size >= 16, PKV_EUNSUPPORTED, "quantized-cache decode needs block_size >= 16 (got %d)",
            block_size);
    pkv::DecodeArgs a{};
    const int kind = format == Q_FP8 ? PKV_CACHE_FP8 : format == Q_INT4 ? PKV_CACHE_INT4 : PKV_CACHE_INT8;
    pkv_status st = decode_args(a, dtype, out, query, key_cache, value_cache, block_tables, block_table_stride,
                                context_lens, num_seqs, max_context_len, num_heads, num_kv_heads, head_dim, block_size,
                                num_blocks, scale, workspace, workspace_bytes, mode, kind);
    if (st != PKV_OK || num_seqs == 0) return st;
    REQUIRE(key_scale && value_scale, PKV_EINVAL, "null scale array");
    REQUIRE(((uintptr_t)key_scale & 15u) == 0 && ((uintptr_t)value_scale & 15u) == 0, PKV_EINVAL,
            "scale arrays must be 16-byte aligned");
    a.key_scale = key_scale;
    a.value_scale = value_scale;
    a.fp8_codes = format == Q_FP8;
    a.int4_codes = format == Q_INT4;
    return hip_status(pkv::launch_decode_q8(a, num_heads / num_kv_heads, stream), what);
}

}  // namespace

extern "C" {

pkv_status pkv_kv_cache_store_int8(pkv_dtype dtype, const void *key, const void *value, int8_t *key_cache,
                                   int8_t *value_cache, float *key_scale, float *value_scale,
                                   const int32_t *slot_mapping, int64_t num_tokens, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t block_size, int64_t num_blocks, hipStream_t stream) {
    return store_q8(Q_INT8, "kv_cache_store_int8 launch", dtype, key, value, key_cache, value_cache, key_scale,
                    value_scale, slot_mapping, num_tokens, num_kv_heads, head_dim, block_size, num_blocks, stream);
}

pkv_status pkv_paged_attention_decode_int8(pkv_dtype dtype, void *out, const void *query, const int8_t *key_cache,
                                           const int8_t *value_cache, const float *key_scale,
                                           const float *value_scale, const int32_t *block_tables,
                                           int32_t block_table_stride, const int32_t *context_lens, int32_t num_seqs,
                                           int32_t max_context_len, int32_t num_heads, int32_t num_kv_heads,
                                           int32_t head_dim, int32_t block_size, int64_t num_blocks, float scale,
                                           void *workspace, size_t workspace_bytes, hipStream_t stream) {
    return decode_q8(Q_INT8, "paged_attention_decode_int8 launch", dtype, out, query, key_cache, value_cache,
                     key_scale, value_scale, block_tables, block_table_stride, context_lens, num_seqs,
                     max_context_len, num_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, workspace,
                     workspace_bytes, stream);
}

pkv_status pkv_kv_cache_store_fp8(pkv_dtype dtype, const void *key, const void *value, uint8_t *key_cache,
                                  uint8_t *value_cache, float *key_scale, float *value_scale,
                                  const int32_t *slot_mapping, int64_t num_tokens, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t block_size, int64_t num_blocks, hipStream_t stream) {
    return store_q8(Q_FP8, "kv_cache_store_fp8 launch", dtype, key, value, key_cache, value_cache, key_scale,
                    value_scale, slot_mapping, num_tokens, num_kv_heads, head_dim, block_size, num_blocks, stream);
}

pkv_status pkv_paged_attention_decode_fp8(pkv_dtype dtype, void *out, const void *query, const uint8_t *key_cache,
                                          const uint8_t *value_cache, const float *key_scale,
                                          const float *value_scale, const int32_t *block_tables,
                                          int32_t block_table_stride, const int32_t *context_lens, int32_t num_seqs,
                                          int32_t max_context_len, int32_t num_heads, int32_t num_kv_heads,
                                          int32_t head_dim, int32_t block_size, int64_t num_blocks, float scale,
                                          void *workspace, size_t workspace_bytes, hipStream_t stream) {
    return decode_q8(Q_FP8, "paged_attention_decode_fp8 launch", dtype, out, query, key_cache, value_cache,
                     key_scale, value_scale, block_tables, block_table_stride, context_lens, num_seqs,
                     max_context_len, num_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, workspace,
                     workspace_bytes, stream);
}

pkv_status pkv_kv_cache_store_int4(pkv_dtype dtype, const void *key, const void *value, uint8_t *key_cache,
                                   uint8_t *value_cache, float *key_scale, float *value_scale,
                                   const int32_t *slot_mapping, int64_t num_tokens, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t block_size, int64_t num_blocks, hipStream_t stream) {
    return store_q8(Q_INT4, "kv_cache_store_int4 launch", dtype, key, value, key_cache, value_cache, key_scale,
                    value_scale, slot_mapping, num_tokens, num_kv_heads, head_dim, block_size, num_blocks, stream);
}

pkv_status pkv_paged_attention_decode_int4(pkv_dtype dtype, void *out, const void *query, const uint8_t *key_cache,
                                           const uint8_t *value_cache, const float *key_scale,
                                           const float *value_scale, const int32_t *block_tables,
                                           int32_t block_table_stride, const int32_t *context_lens, int32_t num_seqs,
                                           int32_t max_context_len, int32_t num_heads, int32_t num_kv_heads,
                                           int32_t head_dim, int32_t block_size, int64_t num_blocks, float scale,
                                           void *workspace, size_t workspace_bytes, hipStream_t stream) {
    return decode_q8(Q_INT4, "paged_attention_decode_int4 launch", dtype, out, query, key_cache, value_cache,
                     key_scale, value_scale, block_tables, block_table_stride, context_lens, num_seqs,
                     max_context_len, num_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, workspace,
                     workspace_bytes, stream);
}

pkv_status pkv_paged_attention_decode_plan(pkv_dtype dtype, int32_t cache_kind, const int32_t *context_lens,
                                           int32_t num_seqs, int32_t max_context_len, int32_t num_heads,
                                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                           void *workspace, size_t workspace_bytes, hipStream_t stream) {
    REQUIRE(cache_kind == PKV_CACHE_ELEMENTS || cache_kind == PKV_CACHE_INT8 || cache_kind == PKV_CACHE_FP8 ||
                cache_kind == PKV_CACHE_INT4,
            PKV_EINVAL, "cache_kind %d is not PKV_CACHE_ELEMENTS, _INT8, _FP8 or _INT4", cache_kind);
    const bool q8 = cache_kind != PKV_CACHE_ELEMENTS;
    if (q8) {
        REQUIRE(dtype == PKV_BF16, PKV_EUNSUPPORTED, "quantized-cache decode takes a bf16 query (got dtype %d)",
                (int)dtype);
        REQUIRE(head_dim == 128, PKV_EUNSUPPORTED, "quantized-cache decode supports head_dim 128 (got %d)",
                head_dim);
        REQUIRE(block_size >= 16, PKV_EUNSUPPORTED, "quantized-cache decode needs block_size >= 16 (got %d)",
                block_size);
    }
    pkv::DecodeArgs a{};
    const pkv_status st = decode_args(a, dtype, nullptr, nullptr, nullptr, nullptr, nullptr,
                                      (max_context_len + block_size - 1) / (block_size > 0 ? block_size : 1),
                                      context_lens, num_seqs, max_context_len, num_heads, num_kv_heads, head_dim,
                                      block_size, 1, 1.0f, workspace, workspace_bytes, DECODE_PLAN_ONLY, cache_kind);
    if (st != PKV_OK || num_seqs == 0) return st;
    const bool mfma = q8 || pkv::decode_uses_mfma(dtype == PKV_BF16, head_dim, num_heads / num_kv_heads, a.log2_bs);
    return hip_status(pkv::launch_decode_plan(a, mfma, q8, stream), "paged_attention_decode_plan launch");
}

pkv_status pkv_paged_attention_decode_run(pkv_dtype dtype, void *out, const void *query, const void *key_cache,
                                          const void *value_cache, const int32_t *block_tables,
                                          int32_t block_table_stride, int32_t num_seqs, int32_t max_context_len,
                                          int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                          int32_t block_size, int64_t num_blocks, float scale, void *workspace,
                                          size_t workspace_bytes, hipStream_t stream) {
    pkv::DecodeArgs a{};
    const pkv_status st = decode_args(a, dtype, out, query, key_cache, value_cache, block_tables, block_table_stride,
                                      nullptr, num_seqs, max_context_len, num_heads, num_kv_heads, head_dim, block_size,
                                      num_blocks, scale, workspace, workspace_bytes, DECODE_RUN_ONLY);
    if (st != PKV_OK || num_seqs == 0) return st;
    return hip_status(pkv::launch_decode(a, dtype == PKV_BF16, head_dim, num_heads / num_kv_heads, stream),
                      "paged_attention_decode_run launch");
}

pkv_status pkv_paged_attention_decode_int8_run(pkv_dtype dtype, void *out, const void *query,
                                               const int8_t *key_cache, const int8_t *value_cache,
                                               const float *key_scale, const float *value_scale,
                                               const int32_t *block_tables, int32_t block_table_stride,
                                               int32_t num_seqs, int32_t max_context_len, int32_t num_heads,
                                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                               int64_t num_blocks, float scale, void *workspace,
                                               size_t workspace_bytes, hipStream_t stream) {
    return decode_q8(Q_INT8, "paged_attention_decode_int8_run launch", dtype, out, query, key_cache, value_cache,
                     key_scale, value_scale, block_tables, block_table_stride, nullptr, num_seqs, max_context_len,
                     num_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, workspace, workspace_bytes,
                     stream, DECODE_RUN_ONLY);
}

pkv_status pkv_paged_attention_decode_fp8_run(pkv_dtype dtype, void *out, const void *query,
                                              const uint8_t *key_cache, const uint8_t *value_cache,
                                              const float *key_scale, const float *value_scale,
                                              const int32_t *block_tables, int32_t block_table_stride,
                                              int32_t num_seqs, int32_t max_context_len, int32_t num_heads,
                                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                              int64_t num_blocks, float scale, void *workspace,
                                              size_t workspace_bytes, hipStream_t stream) {
    return decode_q8(Q_FP8, "paged_attention_decode_fp8_run launch", dtype, out, query, key_cache, value_cache,
                     key_scale, value_scale, block_tables, block_table_stride, nullptr, num_seqs, max_context_len,
                     num_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, workspace, workspace_bytes,
                     stream, DECODE_RUN_ONLY);
}

pkv_status pkv_paged_attention_decode_int4_run(pkv_dtype dtype, void *out, const void *query,
                                               const uint8_t *key_cache, const uint8_t *value_cache,
                                               const float *key_scale, const float *value_scale,
                                               const int32_t *block_tables, int32_t block_table_stride,
                                               int32_t num_seqs, int32_t max_context_len, int32_t num_heads,
                                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                               int64_t num_blocks, float scale, void *workspace,
                                               size_t workspace_bytes, hipStream_t stream) {
    return decode_q8(Q_INT4, "paged_attention_decode_int4_run launch", dtype, out, query, key_cache, value_cache,
                     key_scale, value_scale, block_tables, block_table_stride, nullptr, num_seqs, max_context_len,
                     num_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, workspace, workspace_bytes,
                     stream, DECODE_RUN_ONLY);
}

}  // extern "C"

namespace {

// Scratch of the no-allocation decode: one array per GPU in the library's code object, held until the process
// ends. Host code reaches it only through the device address looked up below, once per device with that
// device current, never through the array's name (a host-side stand-in).
static __device__ __align__(256) unsigned char scratch[PKV_NOALLOC_SCRATCH_BYTES];

constexpr int SCRATCH_MAX_DEVICES = 64;
std::atomic<void *> g_scratch_ptr[SCRATCH_MAX_DEVICES];
std::mutex g_scratch_mu;

pkv_status scratch_on_current_device(void **ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "hipGetDevice");
    REQUIRE(dev >= 0 && dev < SCRATCH_MAX_DEVICES, PKV_EUNSUPPORTED, "device %d: the no-allocation decode serves "
            "devices 0..%d", dev, SCRATCH_MAX_DEVICES - 1);
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_acquire);
        if (p == nullptr) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
            REQUIRE(p != nullptr && ((uintptr_t)p & 255u) == 0, PKV_EHIP, "scratch address %p unusable", p);
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return ok();
}

}  // namespace

extern "C" {

pkv_status pkv_paged_attention_decode_noalloc(pkv_dtype dtype, void *out, const void *query, const void *key_cache,
                                              const void *value_cache, const int32_t *block_tables,
                                              int32_t block_table_stride, const int32_t *context_lens,
                                              int32_t num_seqs, int32_t max_context_len, int32_t num_heads,
                                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                              int64_t num_blocks, float scale, hipStream_t stream) {
    const size_t need = pkv_paged_attention_decode_workspace_size(num_seqs, num_heads, num_kv_heads, head_dim,
                                                                  block_size, max_context_len);
    REQUIRE(need <= PKV_NOALLOC_SCRATCH_BYTES, PKV_EWORKSPACE,
            "these sizes need %zu bytes of decode workspace; the no-allocation decode holds %zu (use "
            "pkv_paged_attention_decode with a caller workspace)", need, (size_t)PKV_NOALLOC_SCRATCH_BYTES);
    // every host-side check first, against a stand-in address that nothing dereferences
    pkv::DecodeArgs a{};
    pkv_status st = decode_args(a, dtype, out, query, key_cache, value_cache, block_tables, block_table_stride,
                                context_lens, num_seqs, max_context_len, num_heads, num_kv_heads, head_dim,
                                block_size, num_blocks, scale, (void *)(uintptr_t)256, PKV_NOALLOC_SCRATCH_BYTES);
    if (st != PKV_OK || num_seqs == 0) return st;
    void *ws = nullptr;
    st = scratch_on_current_device(&ws);
    if (st != PKV_OK) return st;
    st = decode_args(a, dtype, out, query, key_cache, value_cache, block_tables, block_table_stride, context_lens,
                     num_seqs, max_context_len, num_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, ws,
                     PKV_NOALLOC_SCRATCH_BYTES);
    if (st != PKV_OK) return st;
    return hip_status(pkv::launch_decode(a, dtype == PKV_BF16, head_dim, num_heads / num_kv_heads, stream),
                      "paged_attention_decode_noalloc launch");
}

pkv_status pkv_paged_attention_decode_status(const void *workspace, int32_t *status, hipStream_t stream) {
    REQUIRE(workspace && status, PKV_EINVAL, "null pointer argument");
    REQUIRE(((uintptr_t)workspace & 255u) == 0, PKV_EINVAL, "workspace must be 256-byte aligned");
    return hip_status(hipMemcpyAsync(status, (const int *)workspace + pkv::CTRL_ERR, sizeof(int32_t), hipMemcpyDefault,
                                     stream),
                      "paged_attention_decode_status copy");
}

}  // extern "C"

namespace {

// Checks of a prefill call and its launch arguments (shared by the bf16 and the 8-bit-cache entry points);
// PKV_OK with nothing to launch when num_seqs or max_seqlen_q is 0.
pkv_status prefill_args(pkv::PrefillArgs &a, pkv_dtype dtype, void *out, const void *query, const void *key_cache,
                        const void *value_cache, const int32_t *block_tables, int32_t block_table_stride,
                        const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k, int32_t num_seqs,
                        int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t num_heads, int32_t num_kv_heads,
                        int32_t head_dim, int32_t block_size, int64_t num_blocks, float scale, int32_t causal) {
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
    a = pkv::PrefillArgs{};
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
    return ok();
}

pkv_status prefill_q8(bool fp8, const char *what, pkv_dtype dtype, void *out, const void *query,
                      const void *key_cache, const void *value_cache, const float *key_scale,
                      const float *value_scale, const int32_t *block_tables, int32_t block_table_stride,
                      const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k, int32_t num_seqs,
                      int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t num_heads, int32_t num_kv_heads,
                      int32_t head_dim, int32_t block_size, int64_t num_blocks, float scale, int32_t causal,
                      hipStream_t stream) {
    pkv::PrefillArgs a{};
    const pkv_status st = prefill_args(a, dtype, out, query, key_cache, value_cache, block_tables, block_table_stride,
                                       cu_seqlens_q, cu_seqlens_k, num_seqs, max_seqlen_q, max_seqlen_k, num_heads,
                                       num_kv_heads, head_dim, block_size, num_blocks, scale, causal);
    if (st != PKV_OK || num_seqs == 0 || max_seqlen_q == 0) return st;
    REQUIRE(key_scale && value_scale, PKV_EINVAL, "null scale array");
    REQUIRE(((uintptr_t)key_scale & 3u) == 0 && ((uintptr_t)value_scale & 3u) == 0, PKV_EINVAL,
            "scale arrays must be 4-byte aligned");
    a.key_scale = key_scale;
    a.value_scale = value_scale;
    a.fp8_codes = fp8;
    return hip_status(pkv::launch_prefill_q8(a, num_heads / num_kv_heads, stream), what);
}

}  // namespace

extern "C" {

pkv_status pkv_paged_attention_prefill(pkv_dtype dtype, void *out, const void *query, const void *key_cache,
                                       const void *value_cache, const int32_t *block_tables,
                                       int32_t block_table_stride, const int32_t *cu_seqlens_q,
                                       const int32_t *cu_seqlens_k, int32_t num_seqs, int32_t max_seqlen_q,
                                       int32_t max_seqlen_k, int32_t num_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t block_size, int64_t num_blocks, float scale,
                                       int32_t causal, hipStream_t stream) {
    pkv::PrefillArgs a{};
    const pkv_status st = prefill_args(a, dtype, out, query, key_cache, value_cache, block_tables, block_table_stride,
                                       cu_seqlens_q, cu_seqlens_k, num_seqs, max_seqlen_q, max_seqlen_k, num_heads,
                                       num_kv_heads, head_dim, block_size, num_blocks, scale, causal);
    if (st != PKV_OK || num_seqs == 0 || max_seqlen_q == 0) return st;
    return hip_status(pkv::launch_prefill(a, true, head_dim, num_heads / num_kv_heads, stream),
                      "paged_attention_prefill launch");
}

pkv_status pkv_paged_attention_prefill_int8(pkv_dtype dtype, void *out, const void *query, const int8_t *key_cache,
                                            const int8_t *value_cache, const float *key_scale,
                                            const float *value_scale, const int32_t *block_tables,
                                            int32_t block_table_stride, const int32_t *cu_seqlens_q,
                                            const int32_t *cu_seqlens_k, int32_t num_seqs, int32_t max_seqlen_q,
                                            int32_t max_seqlen_k, int32_t num_heads, int32_t num_kv_heads,
                                            int32_t head_dim, int32_t block_size, int64_t num_blocks, float scale,
                                            int32_t causal, hipStream_t stream) {
    return prefill_q8(false, "paged_attention_prefill_int8 launch", dtype, out, query, key_cache, value_cache,
                      key_scale, value_scale, block_tables, block_table_stride, cu_seqlens_q, cu_seqlens_k, num_seqs,
                      max_seqlen_q, max_seqlen_k, num_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
                      causal, stream);
}

pkv_status pkv_paged_attention_prefill_fp8(pkv_dtype dtype, void *out, const void *query, const uint8_t *key_cache,
                                           const uint8_t *value_cache, const float *key_scale,
                                           const float *value_scale, const int32_t *block_tables,
                                           int32_t block_table_stride, const int32_t *cu_seqlens_q,
                                           const int32_t *cu_seqlens_k, int32_t num_seqs, int32_t max_seqlen_q,
                                           int32_t max_seqlen_k, int32_t num_heads, int32_t num_kv_heads,
                                           int32_t head_dim, int32_t block_size, int64_t num_blocks, float scale,
                                           int32_t causal, hipStream_t stream) {
    return prefill_q8(true, "paged_attention_prefill_fp8 launch", dtype, out, query, key_cache, value_cache,
                      key_scale, value_scale, block_tables, block_table_stride, cu_seqlens_q, cu_seqlens_k, num_seqs,
                      max_seqlen_q, max_seqlen_k, num_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
                      causal, stream);
}

}  // extern "C"
