"""Planted mistakes in the oracle must be caught by its pins.

Each mutant is a copy of oracle/oracle.c with one plausible mistake (a dropped term, a wrong sign
or index, a transposed layout, an off-by-one causal bound), compiled to a temporary library. The
pins of tests/pins.py and the oracle checks of tests/test_golden_host.py run against it; at least
one must fail. The real oracle passes them all (tests/test_oracle_pins.py).
"""
import os
import subprocess
import sys

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))

# Runs in a child process: a mutant that indexes out of bounds may crash, which also counts as caught.
RUNNER = r"""
import sys
sys.path[:0] = [sys.argv[2], sys.argv[3]]
import oracle, pins, test_golden_host as gh
m = oracle.Oracle(sys.argv[1])
checks = pins.ALL_CHECKS + [gh.test_oracle_slot_flattening_matches_2d_index_example,
                            gh.test_oracle_gather_follows_block_split_example]
failed = []
for c in checks:
    try:
        c(m)
    except (AssertionError, ValueError, IndexError):
        failed.append(c.__name__)
print("FAILED:" + ",".join(failed))
"""

MUTANTS = {
    "block_index_uses_modulo": ("int64_t block = bt_row[t / bs], off = t % bs;\n        int64_t base",
                                "int64_t block = bt_row[t % bs], off = t % bs;\n        int64_t base"),
    "offset_uses_division": ("int64_t block = bt_row[t / bs], off = t % bs;\n        int64_t base",
                             "int64_t block = bt_row[t / bs], off = t / bs;\n        int64_t base"),
    "softmax_sign_flipped": ("s[t] = exp(s[t] - m);", "s[t] = exp(m - s[t]);"),
    "scale_dropped": ("s[t] = scale * dot;", "s[t] = dot;"),
    "no_normalisation": ("out[d] /= l;", "out[d] /= 1.0;"),
    "gqa_modulo_mapping": ("h / group, num_kv_heads, head_dim, block_size,\n                   scale, s);",
                           "h % group, num_kv_heads, head_dim, block_size,\n                   scale, s);"),
    "layout_token_major": ("return ((block * hkv + head) * bs + off) * dim + d;",
                           "return ((block * bs + off) * hkv + head) * dim + d;"),
    "query_dim_dropped": ("dot += elem(dtype, query, qoff + d) * elem(dtype, key_cache, base + d);",
                          "dot += elem(dtype, query, qoff) * elem(dtype, key_cache, base + d);"),
    "causal_off_by_one": ("(lk - lq) + j + 1 : lk;", "(lk - lq) + j : lk;"),
    "causal_top_left": ("(lk - lq) + j + 1 : lk;", "j + 1 : lk;"),
    "store_block_offset_swapped": ("int64_t block = s / block_size, off = s % block_size;",
                                   "int64_t block = s % block_size, off = s / block_size;"),
    "store_value_into_key": ("memcpy((char *)value_cache + dst * eb, (const char *)value + src * eb",
                             "memcpy((char *)value_cache + dst * eb, (const char *)key + src * eb"),
    "decode_drops_newest_token": ("block_tables + i * stride, context_lens[i], h / group",
                                  "block_tables + i * stride, context_lens[i] - 1, h / group"),
    "value_dim_dropped": ("out[d] += s[t] * elem(dtype, value_cache, base + d);",
                          "out[d] += s[t] * elem(dtype, value_cache, base);"),
    "gather_reads_wrong_head": ("int64_t src = cache_index(block, h, off, 0, num_kv_heads, block_size, head_dim);",
                                "int64_t src = cache_index(block, 0, off, 0, num_kv_heads, block_size, head_dim);"),
    "prefill_row_owner_off_by_one": ("while (cu_seqlens_q[i + 1] <= r) ++i;", "while (cu_seqlens_q[i + 1] < r) ++i;"),
    "int8_truncates": ("code = nearbyintf(x / scale);", "code = truncf(x / scale);"),
    "int8_scale_over_128": ("float scale = a / 127.0f;", "float scale = a / 128.0f;"),
    "int8_signed_max": ("if (fabsf(x) > a) a = fabsf(x);", "if (x > a) a = x;"),
    "int8_dequant_drops_scale": ("(double)codes[r * dim + d] * (double)scales[r];", "(double)codes[r * dim + d];"),
    "int8_store_scale_at_offset": ("key_cache + row * head_dim,\n                                       key_scale + row);",
                                   "key_cache + row * head_dim,\n                                       key_scale + off);"),
    "fp8_exponent_bias_8": ("ldexp(1.0 + m / 8.0, e - 7);", "ldexp(1.0 + m / 8.0, e - 8);"),
    "fp8_subnormal_exponent": ("ldexp(m / 8.0, -6)", "ldexp(m / 8.0, -7)"),
    "fp8_ties_go_up": ("((lo & 1) ? hi : lo);", "hi;"),
    "fp8_scale_over_240": ("float scale = a / 448.0f;", "float scale = a / 240.0f;"),
    "fp8_dequant_drops_scale": ("orc_e4m3_value(codes[r * dim + d]) * (double)scales[r];",
                                "orc_e4m3_value(codes[r * dim + d]);"),
    "int4_scale_over_8": ("float step = amax / 7.0f;", "float step = amax / 8.0f;"),
    "int4_truncates": ("q = nearbyintf((float)elem(dtype, rows, r * dim + 2 * j + half) / step);",
                       "q = truncf((float)elem(dtype, rows, r * dim + 2 * j + half) / step);"),
    "int4_nibbles_swapped": ("(uint8_t)(u[0] | (u[1] << 4));", "(uint8_t)(u[1] | (u[0] << 4));"),
    "int4_twos_complement_codes": ("u[half] = (int)q + 8;", "u[half] = (int)q & 15;"),
    "int4_dequant_nibble_order": ("int u = (d % 2) ? (byte >> 4) : (byte & 15);",
                                  "int u = (d % 2) ? (byte & 15) : (byte >> 4);"),
    "int4_dequant_no_offset": ("out[r * dim + d] = (double)(u - 8) * (double)scales[r];",
                               "out[r * dim + d] = (double)u * (double)scales[r];"),
    "copy_blocks_key_only": ("memcpy((char *)value_cache + (size_t)pairs[2 * k + 1] * block_bytes, tmp + (2 * (size_t)k + 1) * block_bytes, block_bytes);",
                             ";"),
    "copy_blocks_key_into_source": ("memcpy((char *)key_cache + (size_t)pairs[2 * k + 1] * block_bytes, tmp",
                                    "memcpy((char *)key_cache + (size_t)pairs[2 * k] * block_bytes, tmp"),
    "copy_blocks_one_kv_head": ("size_t block_bytes = (size_t)num_kv_heads * block_size * head_dim * elem_bytes(dtype);",
                                "size_t block_bytes = (size_t)block_size * head_dim * elem_bytes(dtype);"),
    "copy_blocks_no_snapshot": ("tmp + (2 * (size_t)k) * block_bytes, block_bytes);",
                                "(char *)key_cache + (size_t)pairs[2 * k] * block_bytes, block_bytes);"),
    "copy_blocks_four_byte_elements": ("size_t block_bytes = (size_t)num_kv_heads * block_size * head_dim * elem_bytes(dtype);",
                                       "size_t block_bytes = (size_t)num_kv_heads * block_size * head_dim * 4;"),
    "int4_store_scale_at_offset": ("value_cache + crow * row_bytes, value_scale + crow);",
                                   "value_cache + crow * row_bytes, value_scale + pos);"),
}


@pytest.fixture(scope="module")
def source():
    with open(oracle.SRC, encoding="utf-8") as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, source, tmp_path):
    old, new = MUTANTS[name]
    assert old in source, f"mutation site for {name} not found"
    src = tmp_path / f"{name}.c"
    src.write_text(source.replace(old, new, 1), encoding="utf-8")      # first site only
    lib = oracle.build(force=True, src=str(src), out=str(tmp_path / f"lib{name}.so"))
    r = subprocess.run([sys.executable, "-c", RUNNER, os.fspath(lib), HERE, os.path.dirname(HERE)],
                       capture_output=True, text=True, timeout=300)
    if r.returncode != 0:
        return                                   # crashed or raised: detected
    line = [x for x in r.stdout.splitlines() if x.startswith("FAILED:")][-1]
    assert line != "FAILED:", f"mutant {name} passed every pin"
