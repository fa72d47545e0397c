"""Host-side parts of bench.py: the algorithmic byte and flop counts behind its throughput figures, checked
against brute-force counting on small synthetic workloads, and its refusal of more than one GPU."""
import os
import subprocess
import sys

import numpy as np

import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _decode_bytes_brute(c, code_bytes=None):
    """Count what one decode call must move, token by token: every context token's K and V row of every kv
    head (elements of e bytes, or one-byte codes plus a 4-byte scale), the query and output rows, each
    block-table entry the sequence uses and its context length."""
    e = 4 if c.dtype == W.F32 else 2
    total = 0
    for i in range(c.num_seqs):
        L = int(c.context_lens[i])
        for _t in range(L):
            for _h in range(c.num_kv_heads):
                total += 2 * (c.head_dim * e if code_bytes is None else int(c.head_dim * code_bytes) + 4)
        total += 4 * len(range(0, L, c.block_size))           # block ids of blocks holding its tokens
        total += 4                                              # its context length
        total += 2 * c.num_heads * c.head_dim * (e if code_bytes is None else 2)   # query and output
    return total


def test_decode_bytes_match_brute_force():
    for dtype, lens, bs in [(W.F32, [300, 70, 200, 513], 16), (W.BF16, [1, 15, 16, 17, 256, 257], 16),
                            (W.BF16, [5, 300], 256), (W.BF16, [33], 1)]:
        nb = sum(W.blocks_for_tokens(n, bs) for n in lens) + 2
        c = W.make_decode_case("bytes", 3, dtype, lens, 8, 2, 64, bs, nb)
        assert bench.decode_bytes(c) == _decode_bytes_brute(c)
        if dtype == W.BF16:
            assert bench.decode_bytes_q8(c) == _decode_bytes_brute(c, code_bytes=1)
            assert bench.decode_bytes_q4(c) == _decode_bytes_brute(c, code_bytes=0.5)


def test_store_bytes_match_brute_force():
    c = W.make_decode_case("store", 4, W.BF16, [3, 9, 40], 8, 2, 128, 16, 16)
    n = len(c.slot_mapping)
    brute = sum(2 * 2 * c.num_kv_heads * c.head_dim * 2 + 4 for _ in range(n))   # K, V read and written; slot
    assert bench.store_bytes(c) == brute


def test_prefill_flops_match_brute_force():
    for causal in (True, False):
        c = W.make_prefill_case("flops", 5, W.BF16, [0, 7, 64], [5, 1, 33], 8, 2, 128, 16, 32, causal=causal)
        pairs = 0
        for i in range(c.num_seqs):
            p, q = int(c.prefix_lens[i]), int(c.chunk_lens[i])
            for j in range(q):                                   # query row j sits at position p + j
                pairs += sum(1 for t in range(p + q) if (t <= p + j or not causal))
        # a multiply-add is 2 flops; QK^T and PV each take head_dim of them per visible pair and head
        assert bench.prefill_flops(c) == 2 * 2 * c.head_dim * c.num_heads * pairs


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
