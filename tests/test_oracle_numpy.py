"""The NumPy statement of the decode (oracle/numpy_decode.py) against the C oracle, on the CPU.

Both compute in float64 from the same storage-form inputs, one with plain loops in C, the other with
gathered blocks and BLAS products, so they agree to rounding (a few ulps of float64): a wrong block lookup,
head mapping, scale or softmax in either shows up far above that."""
import numpy as np
import pytest

from oracle import numpy_decode
import workloads as W


def _stored_pool(orc, c):
    kc, vc = c.pool.dense()
    orc.store(c.dtype, c.key, c.value, kc, vc, c.slot_mapping)
    return kc, vc


def _agree(a, b):
    assert np.all(np.isfinite(a)) and np.all(np.isfinite(b))
    err = np.abs(a - b) / (1.0 + np.abs(b))
    assert err.max() <= 1e-12, f"max relative difference {err.max():.3g}"


def test_tiny_config_fp32(orc):
    c = W.make_config(1)
    kc, vc = _stored_pool(orc, c)
    ref = orc.decode(c.dtype, c.query, kc, vc, c.block_tables, c.context_lens, c.scale)
    _agree(numpy_decode.decode(c.dtype, c.query, kc, vc, c.block_tables, c.context_lens, c.scale), ref)


@pytest.mark.parametrize("hq,hkv,bs", [(8, 8, 16), (32, 8, 16), (16, 2, 64), (8, 1, 256)])
def test_bf16_groups_and_blocks(orc, hq, hkv, bs):
    lens = np.array([1, bs - 1, bs, bs + 1, 3 * bs + 5, 700], np.int32)
    nb = int(sum(W.blocks_for_tokens(int(n), bs) for n in lens)) + 3
    c = W.make_decode_case("np", 11, W.BF16, lens, hq, hkv, 128, bs, nb)
    kc, vc = _stored_pool(orc, c)
    ref = orc.decode(c.dtype, c.query, kc, vc, c.block_tables, c.context_lens, c.scale)
    _agree(numpy_decode.decode(c.dtype, c.query, kc, vc, c.block_tables, c.context_lens, c.scale), ref)


def test_subset_and_empty_context(orc):
    lens = np.array([40, 0, 17, 300], np.int32)
    nb = int(sum(W.blocks_for_tokens(int(n), 16) for n in lens)) + 2
    c = W.make_decode_case("np-empty", 12, W.BF16, lens, 32, 8, 128, 16, nb)
    kc, vc = _stored_pool(orc, c)
    seqs = np.array([3, 1, 0], np.int32)
    ref = orc.decode(c.dtype, c.query, kc, vc, c.block_tables, c.context_lens, c.scale, seqs=np.sort(seqs))
    got = numpy_decode.decode(c.dtype, c.query, kc, vc, c.block_tables, c.context_lens, c.scale, seqs=np.sort(seqs))
    _agree(got, ref)
    assert not np.any(got[1])                              # the empty context gives zeros
