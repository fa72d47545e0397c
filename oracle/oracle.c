/*
 * CPU oracle for the block-table paged KV cache -- TEST INFRASTRUCTURE ONLY.
 *
 * Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may load this library.
 * It shares no source with the HIP library: it is a plain, slow, obviously correct restatement of
 * what the paged cache computes, in float64, with no online softmax, no split and no tiling.
 *
 * Layout it reads (chosen by the library and restated here independently):
 *   key_cache / value_cache : [num_blocks][num_kv_heads][block_size][head_dim]
 *   slot s                   : physical block s / block_size, offset s % block_size
 *   element dtype 0 = float32, 1 = bfloat16 (16-bit patterns, upcast exactly), 3 = float64
 *   int8 cache (orc_store_int8): codes [num_blocks][num_kv_heads][block_size][head_dim] int8 and one
 *   float32 scale per row, [num_blocks][num_kv_heads][block_size]
 *   fp8 cache (orc_store_fp8): the same with one-byte E4M3 codes in place of int8
 *   int4 cache (orc_store_int4): codes [num_blocks][num_kv_heads][block_size][head_dim / 2] bytes, two 4-bit
 *   codes per byte, and the same float32 scales
 *
 * Sources (web pages on the paged KV cache):
 *   - logical block j of a request lives in physical block block_table[j]; the kernel reads K/V
 *     through that map ("推理运行时", section 分页 KV);
 *   - token i of a request belongs to logical block i / block_size at offset i % block_size
 *     (nano-vllm walkthrough, section 2 Sequence, block(i));
 *   - slot_mapping names the row each new token's K/V is written to (nano-vllm walkthrough,
 *     section 2 context; Mini-SGLang 源码解析（二）, section 6.7, out_loc into the page table);
 *   - the decoded token attends to the cached tokens plus itself
 *     ("LLM Infra 101 v0.2: KV Cache", section 推理);
 *   - chunked prefill: a chunk attends to its cached prefix and to itself
 *     (Mini-SGLang 源码解析（二）, sections 6.6 and 6.9; "推理运行时", section Prefill 与 decode 输入);
 *   - a quantized cache keeps K/V as int8 (or another 8-bit type) instead of bf16, at some loss of
 *     accuracy ("LLM Infra 101 v0.2: KV Cache", inference-engine list, KV Quantization, which names int8
 *     and int4). The pages fix no scheme; the ones restated here are symmetric, one scale per (token, kv
 *     head) row, with int8 codes, OCP float8 E4M3 codes, or 4-bit codes.
 * Attention itself is the textbook definition softmax(scale * q . k) weighted sum of v.
 */
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_OK 0
#define ORC_EINVAL (-1)

static char g_err[512];

static int fail(const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return ORC_EINVAL;
}

const char *orc_last_error(void) { return g_err; }

static size_t elem_bytes(int dtype) { return dtype == 0 ? 4 : dtype == 3 ? 8 : 2; }

/* Element idx of a dtype-typed array, as double (exact for every dtype). */
static double elem(int dtype, const void *base, int64_t idx) {
    if (dtype == 0) return (double)((const float *)base)[idx];
    if (dtype == 3) return ((const double *)base)[idx];
    uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, 4);
    return (double)f;
}

/* Flat element index of (block, kv head, offset, dim) in a cache. */
static int64_t cache_index(int64_t block, int64_t head, int64_t off, int64_t d,
                           int64_t hkv, int64_t bs, int64_t dim) {
    return ((block * hkv + head) * bs + off) * dim + d;
}

/* Store: for each new token n with slot s >= 0, row s of the cache receives key[n] and value[n]. */
int orc_store(int dtype, const void *key, const void *value, void *key_cache, void *value_cache,
              const int32_t *slot_mapping, int64_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
              int32_t block_size, int64_t num_blocks) {
    if (dtype != 0 && dtype != 1 && dtype != 3) return fail("bad dtype %d", dtype);
    if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks < 0)
        return fail("bad sizes (tokens %lld, blocks %lld)", (long long)num_tokens, (long long)num_blocks);
    int64_t nslots = num_blocks * block_size;
    unsigned char *seen = (unsigned char *)calloc((size_t)(nslots > 0 ? nslots : 1), 1);
    if (!seen) return fail("out of memory");
    for (int64_t n = 0; n < num_tokens; ++n) {
        int64_t s = slot_mapping[n];
        if (s < 0) continue;
        if (s >= nslots) { free(seen); return fail("slot %lld outside the pool of %lld slots", (long long)s, (long long)nslots); }
        if (seen[s]) { free(seen); return fail("slot %lld written twice (token %lld)", (long long)s, (long long)n); }
        seen[s] = 1;
    }
    free(seen);
    size_t eb = elem_bytes(dtype);
    for (int64_t n = 0; n < num_tokens; ++n) {
        int64_t s = slot_mapping[n];
        if (s < 0) continue;
        int64_t block = s / block_size, off = s % block_size;
        for (int64_t h = 0; h < num_kv_heads; ++h) {
            int64_t dst = cache_index(block, h, off, 0, num_kv_heads, block_size, head_dim);
            int64_t src = (n * num_kv_heads + h) * head_dim;
            memcpy((char *)key_cache + dst * eb, (const char *)key + src * eb, (size_t)head_dim * eb);
            memcpy((char *)value_cache + dst * eb, (const char *)value + src * eb, (size_t)head_dim * eb);
        }
    }
    return ORC_OK;
}

/*
 * int8 quantization of rows of `dim` elements, one scale per row, all arithmetic in float32:
 *   a = max_d |x_d|,  scale = a / 127,  code_d = round_half_even(x_d / scale) clamped to [-127, 127];
 * a row of zeros gets scale 0 and codes 0. Dequantized, x_d ~ code_d * scale, |error| <= scale / 2.
 * Rows must be finite.
 */
int orc_quantize_int8(int dtype, const void *rows, int64_t nrows, int32_t dim, int8_t *codes, float *scales) {
    if (dtype != 0 && dtype != 1) return fail("bad dtype %d", dtype);
    if (nrows < 0 || dim <= 0) return fail("bad sizes (rows %lld, dim %d)", (long long)nrows, dim);
    for (int64_t r = 0; r < nrows; ++r) {
        float a = 0.0f;
        for (int32_t d = 0; d < dim; ++d) {
            float x = (float)elem(dtype, rows, r * dim + d);
            if (!isfinite(x)) return fail("row %lld holds a non-finite value", (long long)r);
            if (fabsf(x) > a) a = fabsf(x);
        }
        float scale = a / 127.0f;
        scales[r] = scale;
        for (int32_t d = 0; d < dim; ++d) {
            float code = 0.0f;
            if (a > 0.0f) {
                float x = (float)elem(dtype, rows, r * dim + d);
                code = nearbyintf(x / scale);
                if (code > 127.0f) code = 127.0f;
                if (code < -127.0f) code = -127.0f;
            }
            codes[r * dim + d] = (int8_t)code;
        }
    }
    return ORC_OK;
}

/* Store into an int8 cache: row (n, h) of key/value is quantized (orc_quantize_int8) and lands at slot
 * slot_mapping[n] exactly as in orc_store, its scale at the same (block, kv head, offset) of the scale
 * arrays. Negative slots are skipped; out-of-pool or repeated slots fail before anything is written. */
int orc_store_int8(int dtype, const void *key, const void *value, int8_t *key_cache, int8_t *value_cache,
                   float *key_scale, float *value_scale, const int32_t *slot_mapping, int64_t num_tokens,
                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks) {
    if (dtype != 0 && dtype != 1) return fail("bad dtype %d", dtype);
    if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks < 0)
        return fail("bad sizes (tokens %lld, blocks %lld)", (long long)num_tokens, (long long)num_blocks);
    int64_t nslots = num_blocks * block_size;
    unsigned char *seen = (unsigned char *)calloc((size_t)(nslots > 0 ? nslots : 1), 1);
    if (!seen) return fail("out of memory");
    for (int64_t n = 0; n < num_tokens; ++n) {
        int64_t s = slot_mapping[n];
        if (s < 0) continue;
        if (s >= nslots) { free(seen); return fail("slot %lld outside the pool of %lld slots", (long long)s, (long long)nslots); }
        if (seen[s]) { free(seen); return fail("slot %lld written twice (token %lld)", (long long)s, (long long)n); }
        seen[s] = 1;
    }
    free(seen);
    size_t eb = elem_bytes(dtype);
    for (int64_t n = 0; n < num_tokens; ++n) {
        int64_t s = slot_mapping[n];
        if (s < 0) continue;
        int64_t block = s / block_size, off = s % block_size;
        for (int64_t h = 0; h < num_kv_heads; ++h) {
            int64_t row = (block * num_kv_heads + h) * block_size + off;
            int64_t src = (n * num_kv_heads + h) * head_dim;
            int rc = orc_quantize_int8(dtype, (const char *)key + src * eb, 1, head_dim, key_cache + row * head_dim,
                                       key_scale + row);
            if (!rc) rc = orc_quantize_int8(dtype, (const char *)value + src * eb, 1, head_dim,
                                            value_cache + row * head_dim, value_scale + row);
            if (rc) return rc;
        }
    }
    return ORC_OK;
}

/* Dequantize int8 rows: out[r][d] = codes[r][d] * scales[r] in float64 (exact). */
int orc_dequantize_int8(const int8_t *codes, const float *scales, int64_t nrows, int32_t dim, double *out) {
    if (nrows < 0 || dim <= 0) return fail("bad sizes (rows %lld, dim %d)", (long long)nrows, dim);
    for (int64_t r = 0; r < nrows; ++r)
        for (int32_t d = 0; d < dim; ++d) out[r * dim + d] = (double)codes[r * dim + d] * (double)scales[r];
    return ORC_OK;
}

/*
 * int4 quantization of rows of `dim` (even) elements, one scale per row, all arithmetic in float32:
 *   a = max_d |x_d|,  scale = a / 7,  q_d = round_half_even(x_d / scale) clamped to [-7, 7];
 * stored offset by 8, u_d = q_d + 8 in [1, 15], two codes per byte: element 2j in the low four bits of
 * byte j, element 2j + 1 in the high four bits. A row of zeros gets scale 0 and codes u = 8 (q = 0).
 * Dequantized, x_d ~ q_d * scale, |error| <= scale / 2. Rows must be finite.
 */
int orc_quantize_int4(int dtype, const void *rows, int64_t nrows, int32_t dim, uint8_t *codes, float *scales) {
    if (dtype != 0 && dtype != 1) return fail("bad dtype %d", dtype);
    if (nrows < 0 || dim <= 0 || dim % 2) return fail("bad sizes (rows %lld, dim %d)", (long long)nrows, dim);
    for (int64_t r = 0; r < nrows; ++r) {
        float amax = 0.0f;
        for (int32_t d = 0; d < dim; ++d) {
            float x = (float)elem(dtype, rows, r * dim + d);
            if (!isfinite(x)) return fail("row %lld holds a non-finite value", (long long)r);
            if (fabsf(x) > amax) amax = fabsf(x);
        }
        float step = amax / 7.0f;
        scales[r] = step;
        for (int32_t j = 0; j < dim / 2; ++j) {
            int u[2];
            for (int half = 0; half < 2; ++half) {
                float q = 0.0f;
                if (amax > 0.0f) {
                    q = nearbyintf((float)elem(dtype, rows, r * dim + 2 * j + half) / step);
                    q = fminf(fmaxf(q, -7.0f), 7.0f);
                }
                u[half] = (int)q + 8;
            }
            codes[r * (dim / 2) + j] = (uint8_t)(u[0] | (u[1] << 4));
        }
    }
    return ORC_OK;
}

/* Store into an int4 cache: as orc_store_int8, with rows of head_dim / 2 bytes of orc_quantize_int4 codes. */
int orc_store_int4(int dtype, const void *key, const void *value, uint8_t *key_cache, uint8_t *value_cache,
                   float *key_scale, float *value_scale, const int32_t *slot_mapping, int64_t num_tokens,
                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks) {
    if (dtype != 0 && dtype != 1) return fail("bad dtype %d", dtype);
    if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || head_dim % 2 || block_size <= 0 || num_blocks < 0)
        return fail("bad sizes (tokens %lld, blocks %lld, head_dim %d)", (long long)num_tokens, (long long)num_blocks,
                    head_dim);
    int64_t nslots = num_blocks * block_size;
    unsigned char *seen = (unsigned char *)calloc((size_t)(nslots > 0 ? nslots : 1), 1);
    if (!seen) return fail("out of memory");
    for (int64_t n = 0; n < num_tokens; ++n) {
        int64_t s = slot_mapping[n];
        if (s < 0) continue;
        if (s >= nslots) { free(seen); return fail("slot %lld outside the pool of %lld slots", (long long)s, (long long)nslots); }
        if (seen[s]) { free(seen); return fail("slot %lld written twice (token %lld)", (long long)s, (long long)n); }
        seen[s] = 1;
    }
    free(seen);
    size_t eb = elem_bytes(dtype);
    int64_t row_bytes = head_dim / 2;
    for (int64_t n = 0; n < num_tokens; ++n) {
        int64_t s = slot_mapping[n];
        if (s < 0) continue;
        int64_t blk = s / block_size, pos = s % block_size;
        for (int64_t h = 0; h < num_kv_heads; ++h) {
            int64_t crow = (blk * num_kv_heads + h) * block_size + pos;
            int64_t src = (n * num_kv_heads + h) * head_dim;
            int rc = orc_quantize_int4(dtype, (const char *)key + src * eb, 1, head_dim,
                                       key_cache + crow * row_bytes, key_scale + crow);
            if (!rc) rc = orc_quantize_int4(dtype, (const char *)value + src * eb, 1, head_dim,
                                            value_cache + crow * row_bytes, value_scale + crow);
            if (rc) return rc;
        }
    }
    return ORC_OK;
}

/* Dequantize int4 rows: out[r][d] = (u_d - 8) * scales[r] in float64 (exact), u_d the 4-bit code of element d. */
int orc_dequantize_int4(const uint8_t *codes, const float *scales, int64_t nrows, int32_t dim, double *out) {
    if (nrows < 0 || dim <= 0 || dim % 2) return fail("bad sizes (rows %lld, dim %d)", (long long)nrows, dim);
    for (int64_t r = 0; r < nrows; ++r)
        for (int32_t d = 0; d < dim; ++d) {
            int byte = codes[r * (dim / 2) + d / 2];
            int u = (d % 2) ? (byte >> 4) : (byte & 15);
            out[r * dim + d] = (double)(u - 8) * (double)scales[r];
        }
    return ORC_OK;
}

/*
 * float8 E4M3 of the OCP 8-bit floating point format: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa
 * bits; exponent field 0 holds the subnormals (m / 8) * 2^-6; the pattern with every exponent and mantissa
 * bit set is NaN and there are no infinities, so finite magnitudes end at 1.75 * 2^8 = 448.
 * orc_e4m3_value: the value of a code (NaN for the two NaN patterns).
 */
double orc_e4m3_value(int code) {
    int sign = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
    if (e == 15 && m == 7) return NAN;
    double mag = e == 0 ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, e - 7);
    return sign ? -mag : mag;
}

/*
 * orc_e4m3_encode: v rounded to the E4M3 grid, to nearest with a tie going to the even mantissa; past the
 * largest finite value the grid continues with 480 (where the NaN pattern sits), so |v| <= 464 rounds to at
 * most 448 and |v| > 464 gives NaN. The sign bit is v's (-0.0 and small negatives give 0x80). Codes
 * 0x00 .. 0x7e are the non-negative finite values in increasing order; the nearest is found by bisection.
 * v must not be NaN.
 */
int orc_e4m3_encode(float v) {
    double a = fabs((double)v);
    int sign = signbit(v) ? 0x80 : 0;
    if (a > 464.0) return sign | 0x7f;
    if (a >= orc_e4m3_value(0x7e)) return sign | 0x7e;
    int lo = 0, hi = 0x7e;                    /* value(lo) <= a < value(hi) */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (orc_e4m3_value(mid) <= a) lo = mid;
        else hi = mid;
    }
    double dl = a - orc_e4m3_value(lo), dh = orc_e4m3_value(hi) - a;
    int c = dl < dh ? lo : dh < dl ? hi : ((lo & 1) ? hi : lo);
    return sign | c;
}

/*
 * fp8 quantization of rows of `dim` elements, one scale per row, all arithmetic in float32:
 *   a = max_d |x_d|,  scale = a / 448,  code_d = orc_e4m3_encode(x_d / scale);
 * a row of zeros gets scale 0 and codes 0. |x_d / scale| <= 448 up to one rounding, so no code is NaN.
 * Dequantized, x_d ~ e4m3_value(code_d) * scale, |error| <= 2^-4 |x_d| (normal codes) or 2^-10 scale.
 * Rows must be finite.
 */
int orc_quantize_fp8(int dtype, const void *rows, int64_t nrows, int32_t dim, uint8_t *codes, float *scales) {
    if (dtype != 0 && dtype != 1) return fail("bad dtype %d", dtype);
    if (nrows < 0 || dim <= 0) return fail("bad sizes (rows %lld, dim %d)", (long long)nrows, dim);
    for (int64_t r = 0; r < nrows; ++r) {
        float a = 0.0f;
        for (int32_t d = 0; d < dim; ++d) {
            float x = (float)elem(dtype, rows, r * dim + d);
            if (!isfinite(x)) return fail("row %lld holds a non-finite value", (long long)r);
            if (fabsf(x) > a) a = fabsf(x);
        }
        float scale = a / 448.0f;
        scales[r] = scale;
        for (int32_t d = 0; d < dim; ++d) {
            int code = 0;
            if (a > 0.0f) {
                float x = (float)elem(dtype, rows, r * dim + d);
                code = orc_e4m3_encode(x / scale);
            }
            codes[r * dim + d] = (uint8_t)code;
        }
    }
    return ORC_OK;
}

/* Store into an fp8 cache, exactly as orc_store_int8 with orc_quantize_fp8 codes. */
int orc_store_fp8(int dtype, const void *key, const void *value, uint8_t *key_cache, uint8_t *value_cache,
                  float *key_scale, float *value_scale, const int32_t *slot_mapping, int64_t num_tokens,
                  int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks) {
    if (dtype != 0 && dtype != 1) return fail("bad dtype %d", dtype);
    if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks < 0)
        return fail("bad sizes (tokens %lld, blocks %lld)", (long long)num_tokens, (long long)num_blocks);
    int64_t nslots = num_blocks * block_size;
    unsigned char *seen = (unsigned char *)calloc((size_t)(nslots > 0 ? nslots : 1), 1);
    if (!seen) return fail("out of memory");
    for (int64_t n = 0; n < num_tokens; ++n) {
        int64_t s = slot_mapping[n];
        if (s < 0) continue;
        if (s >= nslots) { free(seen); return fail("slot %lld outside the pool of %lld slots", (long long)s, (long long)nslots); }
        if (seen[s]) { free(seen); return fail("slot %lld written twice (token %lld)", (long long)s, (long long)n); }
        seen[s] = 1;
    }
    free(seen);
    size_t eb = elem_bytes(dtype);
    for (int64_t n = 0; n < num_tokens; ++n) {
        int64_t s = slot_mapping[n];
        if (s < 0) continue;
        int64_t block = s / block_size, off = s % block_size;
        for (int64_t h = 0; h < num_kv_heads; ++h) {
            int64_t row = (block * num_kv_heads + h) * block_size + off;
            int64_t src = (n * num_kv_heads + h) * head_dim;
            int rc = orc_quantize_fp8(dtype, (const char *)key + src * eb, 1, head_dim, key_cache + row * head_dim,
                                      key_scale + row);
            if (!rc) rc = orc_quantize_fp8(dtype, (const char *)value + src * eb, 1, head_dim,
                                           value_cache + row * head_dim, value_scale + row);
            if (rc) return rc;
        }
    }
    return ORC_OK;
}

/* Dequantize fp8 rows: out[r][d] = e4m3_value(codes[r][d]) * scales[r] in float64 (exact). */
int orc_dequantize_fp8(const uint8_t *codes, const float *scales, int64_t nrows, int32_t dim, double *out) {
    if (nrows < 0 || dim <= 0) return fail("bad sizes (rows %lld, dim %d)", (long long)nrows, dim);
    for (int64_t r = 0; r < nrows; ++r)
        for (int32_t d = 0; d < dim; ++d) out[r * dim + d] = orc_e4m3_value(codes[r * dim + d]) * (double)scales[r];
    return ORC_OK;
}

/* Copy blocks: for each pair k, physical block pairs[2k+1] of both caches becomes a copy of block pairs[2k]
 * (copy-on-write of a shared block). Sources are read before any destination is written. */
int orc_copy_blocks(int dtype, void *key_cache, void *value_cache, const int32_t *pairs, int32_t num_pairs,
                    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks) {
    size_t block_bytes = (size_t)num_kv_heads * block_size * head_dim * elem_bytes(dtype);
    for (int32_t k = 0; k < 2 * num_pairs; ++k)
        if (pairs[k] < 0 || pairs[k] >= num_blocks) return fail("block id %d outside the pool of %lld", pairs[k], (long long)num_blocks);
    char *tmp = (char *)malloc(block_bytes * 2 * (size_t)(num_pairs > 0 ? num_pairs : 1));
    if (!tmp) return fail("out of memory");
    for (int32_t k = 0; k < num_pairs; ++k) {
        memcpy(tmp + (2 * (size_t)k) * block_bytes, (char *)key_cache + (size_t)pairs[2 * k] * block_bytes, block_bytes);
        memcpy(tmp + (2 * (size_t)k + 1) * block_bytes, (char *)value_cache + (size_t)pairs[2 * k] * block_bytes, block_bytes);
    }
    for (int32_t k = 0; k < num_pairs; ++k) {
        memcpy((char *)key_cache + (size_t)pairs[2 * k + 1] * block_bytes, tmp + (2 * (size_t)k) * block_bytes, block_bytes);
        memcpy((char *)value_cache + (size_t)pairs[2 * k + 1] * block_bytes, tmp + (2 * (size_t)k + 1) * block_bytes, block_bytes);
    }
    free(tmp);
    return ORC_OK;
}

/* Gather: logical tokens [0, len) of one block table into contiguous rows [len][num_kv_heads][head_dim]. */
int orc_gather(int dtype, void *key_out, void *value_out, const void *key_cache, const void *value_cache,
               const int32_t *block_table_row, int32_t len, int32_t num_kv_heads, int32_t head_dim,
               int32_t block_size, int64_t num_blocks) {
    if (len < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0)
        return fail("bad sizes (len %d, block %d)", len, block_size);
    size_t eb = elem_bytes(dtype);
    for (int64_t t = 0; t < len; ++t) {
        int64_t block = block_table_row[t / block_size];
        if (block < 0 || block >= num_blocks)
            return fail("block id %lld outside the pool (token %lld)", (long long)block, (long long)t);
        int64_t off = t % block_size;
        for (int64_t h = 0; h < num_kv_heads; ++h) {
            int64_t src = cache_index(block, h, off, 0, num_kv_heads, block_size, head_dim);
            int64_t dst = (t * num_kv_heads + h) * head_dim;
            memcpy((char *)key_out + dst * eb, (const char *)key_cache + src * eb, (size_t)head_dim * eb);
            memcpy((char *)value_out + dst * eb, (const char *)value_cache + src * eb, (size_t)head_dim * eb);
        }
    }
    return ORC_OK;
}

/*
 * One attention row: out[d] = sum_t w_t v_t[d] / sum_t w_t, w_t = exp(s_t - max s), s_t = scale * q.k_t,
 * over the logical tokens t in [0, nkeys) of one block table, for KV head kvh. nkeys == 0 gives zeros.
 */
static void attend(int dtype, double *out, const void *query, int64_t qoff, const void *key_cache,
                   const void *value_cache, const int32_t *bt_row, int64_t nkeys, int64_t kvh,
                   int64_t hkv, int64_t dim, int64_t bs, double scale, double *s) {
    for (int64_t d = 0; d < dim; ++d) out[d] = 0.0;
    if (nkeys == 0) return;
    double m = -INFINITY;
    for (int64_t t = 0; t < nkeys; ++t) {
        int64_t block = bt_row[t / bs], off = t % bs;
        int64_t base = cache_index(block, kvh, off, 0, hkv, bs, dim);
        double dot = 0.0;
        for (int64_t d = 0; d < dim; ++d)
            dot += elem(dtype, query, qoff + d) * elem(dtype, key_cache, base + d);
        s[t] = scale * dot;
        if (s[t] > m) m = s[t];
    }
    double l = 0.0;
    for (int64_t t = 0; t < nkeys; ++t) {
        s[t] = exp(s[t] - m);
        l += s[t];
    }
    for (int64_t t = 0; t < nkeys; ++t) {
        int64_t block = bt_row[t / bs], off = t % bs;
        int64_t base = cache_index(block, kvh, off, 0, hkv, bs, dim);
        for (int64_t d = 0; d < dim; ++d) out[d] += s[t] * elem(dtype, value_cache, base + d);
    }
    for (int64_t d = 0; d < dim; ++d) out[d] /= l;
}

static int check_heads(int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size) {
    if (num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0)
        return fail("bad head sizes (%d, %d)", num_heads, num_kv_heads);
    if (num_heads % num_kv_heads != 0)
        return fail("num_heads %d is not a multiple of num_kv_heads %d", num_heads, num_kv_heads);
    return ORC_OK;
}

static int check_table(const int32_t *bt_row, int64_t nkeys, int64_t stride, int64_t bs, int64_t nblocks) {
    int64_t nb = (nkeys + bs - 1) / bs;
    if (nb > stride) return fail("context of %lld tokens exceeds the block-table row (%lld blocks)", (long long)nkeys, (long long)stride);
    for (int64_t j = 0; j < nb; ++j)
        if (bt_row[j] < 0 || bt_row[j] >= nblocks) return fail("block id %d outside the pool of %lld", bt_row[j], (long long)nblocks);
    return ORC_OK;
}

/*
 * Decode: one query token per sequence, attending over context_lens[i] cached tokens (the newest,
 * just stored, included). Query head h reads KV head h / (num_heads / num_kv_heads).
 * out: [n][num_heads][head_dim] doubles, for the sequences listed in seq_subset (all if NULL).
 */
int orc_decode(int dtype, double *out, const void *query, const void *key_cache, const void *value_cache,
               const int32_t *block_tables, int32_t stride, const int32_t *context_lens, int32_t num_seqs,
               int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
               int64_t num_blocks, double scale, const int32_t *seq_subset, int32_t n_subset, int32_t nthreads) {
    int rc = check_heads(num_heads, num_kv_heads, head_dim, block_size);
    if (rc) return rc;
    int32_t n = seq_subset ? n_subset : num_seqs;
    int32_t group = num_heads / num_kv_heads;
    int32_t max_len = 0;
    for (int32_t k = 0; k < n; ++k) {
        int32_t i = seq_subset ? seq_subset[k] : k;
        if (i < 0 || i >= num_seqs) return fail("sequence %d outside [0, %d)", i, num_seqs);
        if (context_lens[i] < 0) return fail("negative context length %d (sequence %d)", context_lens[i], i);
        rc = check_table(block_tables + (int64_t)i * stride, context_lens[i], stride, block_size, num_blocks);
        if (rc) return rc;
        if (context_lens[i] > max_len) max_len = context_lens[i];
    }
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    int64_t units = (int64_t)n * num_heads;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(max_len > 0 ? max_len : 1));
#pragma omp for schedule(dynamic, 4)
        for (int64_t u = 0; u < units; ++u) {
            int64_t k = u / num_heads, h = u % num_heads;
            int64_t i = seq_subset ? seq_subset[k] : k;
            attend(dtype, out + u * head_dim, query, (i * num_heads + h) * head_dim, key_cache, value_cache,
                   block_tables + i * stride, context_lens[i], h / group, num_kv_heads, head_dim, block_size,
                   scale, s);
        }
        free(s);
    }
    return ORC_OK;
}

/*
 * Varlen prefill: sequence i owns query rows [cu_q[i], cu_q[i+1]) and has Lk = cu_k[i+1] - cu_k[i]
 * tokens in the cache, the last Lq = cu_q[i+1] - cu_q[i] of which are this chunk; P = Lk - Lq is the
 * cached prefix. Query row j of the chunk sits at position P + j and, when causal, attends to keys
 * [0, P + j]; otherwise to all Lk keys.
 * out: [n][num_heads][head_dim] doubles, for the query rows listed in row_subset (all if NULL).
 */
int orc_prefill(int dtype, double *out, const void *query, const void *key_cache, const void *value_cache,
                const int32_t *block_tables, int32_t stride, const int32_t *cu_seqlens_q,
                const int32_t *cu_seqlens_k, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                int32_t head_dim, int32_t block_size, int64_t num_blocks, double scale, int32_t causal,
                const int32_t *row_subset, int32_t n_rows, int32_t nthreads) {
    int rc = check_heads(num_heads, num_kv_heads, head_dim, block_size);
    if (rc) return rc;
    if (num_seqs < 0) return fail("negative num_seqs %d", num_seqs);
    if (cu_seqlens_q[0] != 0 || cu_seqlens_k[0] != 0) return fail("cu_seqlens must start at 0 (%d, %d)", cu_seqlens_q[0], cu_seqlens_k[0]);
    int32_t max_lk = 0;
    for (int32_t i = 0; i < num_seqs; ++i) {
        int32_t lq = cu_seqlens_q[i + 1] - cu_seqlens_q[i], lk = cu_seqlens_k[i + 1] - cu_seqlens_k[i];
        if (lq < 0 || lk < 0) return fail("cu_seqlens decrease at sequence %d", i);
        if (lq > lk) return fail("sequence %d has more queries (%d) than keys (%d)", i, lq, lk);
        rc = check_table(block_tables + (int64_t)i * stride, lk, stride, block_size, num_blocks);
        if (rc) return rc;
        if (lk > max_lk) max_lk = lk;
    }
    int32_t total_q = cu_seqlens_q[num_seqs];
    int32_t n = row_subset ? n_rows : total_q;
    for (int32_t k = 0; k < n; ++k) {
        int32_t r = row_subset ? row_subset[k] : k;
        if (r < 0 || r >= total_q) return fail("query row %d outside [0, %d)", r, total_q);
    }
    int32_t group = num_heads / num_kv_heads;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    int64_t units = (int64_t)n * num_heads;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(max_lk > 0 ? max_lk : 1));
#pragma omp for schedule(dynamic, 4)
        for (int64_t u = 0; u < units; ++u) {
            int64_t k = u / num_heads, h = u % num_heads;
            int64_t r = row_subset ? row_subset[k] : k;
            int64_t i = 0;
            while (cu_seqlens_q[i + 1] <= r) ++i;       /* sequence that owns row r */
            int64_t lq = cu_seqlens_q[i + 1] - cu_seqlens_q[i];
            int64_t lk = cu_seqlens_k[i + 1] - cu_seqlens_k[i];
            int64_t j = r - cu_seqlens_q[i];
            int64_t nkeys = causal ? (lk - lq) + j + 1 : lk;
            attend(dtype, out + u * head_dim, query, (r * num_heads + h) * head_dim, key_cache, value_cache,
                   block_tables + i * stride, nkeys, h / group, num_kv_heads, head_dim, block_size, scale, s);
        }
        free(s);
    }
    return ORC_OK;
}

int orc_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
