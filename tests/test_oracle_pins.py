"""The oracle against closed forms, a library routine and invariants (tests/pins.py), plus its
argument checks and bf16 handling."""
import math

import numpy as np
import pytest

import pins
from workloads import BF16, F32, bf16_bits_to_f32, f32_to_bf16_bits, make_decode_case, make_prefill_case


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(orc, check):
    check(orc)


def test_decode_vs_sdpa_wider(orc):
    pins.check_decode_vs_sdpa(orc, hq=8, hkv=8, d=64, bs=16, lens=(1, 15, 16, 17, 33, 100), seed=5)
    pins.check_decode_vs_sdpa(orc, hq=32, hkv=8, d=128, bs=16, lens=(2, 40, 70), seed=6)


def test_prefill_non_causal_vs_sdpa(orc):
    pins.check_prefill_vs_sdpa(orc, causal=False)


def test_store_rejects_bad_slots(orc):
    kc = np.zeros((2, 1, 4, 2), np.float32)
    vc = np.zeros_like(kc)
    key = np.ones((2, 1, 2), np.float32)
    with pytest.raises(ValueError, match="outside the pool"):
        orc.store(F32, key, key, kc, vc, np.array([1, 8], np.int32))
    with pytest.raises(ValueError, match="written twice"):
        orc.store(F32, key, key, kc, vc, np.array([3, 3], np.int32))
    assert not kc.any() and not vc.any()      # nothing written on error


def test_decode_rejects_bad_metadata(orc):
    kc = np.zeros((4, 2, 4, 8), np.float32)
    q = np.zeros((1, 6, 8), np.float32)
    with pytest.raises(ValueError, match="multiple"):
        orc.decode(F32, np.zeros((1, 3, 8), np.float32), kc, kc, np.array([[0]], np.int32),
                   np.array([2], np.int32), 1.0)
    with pytest.raises(ValueError, match="outside the pool"):
        orc.decode(F32, q[:, :4], kc, kc, np.array([[4]], np.int32), np.array([2], np.int32), 1.0)
    with pytest.raises(ValueError, match="exceeds"):
        orc.decode(F32, q[:, :4], kc, kc, np.array([[0]], np.int32), np.array([5], np.int32), 1.0)


def test_prefill_rejects_more_queries_than_keys(orc):
    kc = np.zeros((4, 1, 4, 8), np.float32)
    q = np.zeros((3, 1, 8), np.float32)
    with pytest.raises(ValueError, match="more queries"):
        orc.prefill(F32, q, kc, kc, np.array([[0]], np.int32), np.array([0, 3], np.int32),
                    np.array([0, 2], np.int32), 1.0)


def test_empty_context_gives_zeros(orc):
    kc = np.full((2, 1, 4, 8), np.nan, np.float32)
    q = np.ones((2, 2, 8), np.float32)
    out = orc.decode(F32, q, kc, kc, np.array([[-1], [-1]], np.int32), np.array([0, 0], np.int32), 1.0)
    assert np.array_equal(out, np.zeros_like(out))


def test_nan_beyond_context_is_never_read(orc):
    """Generated pools hold NaN after each sequence's last valid token and in unowned blocks."""
    c = make_decode_case("t", 3, F32, [5, 16, 17, 1], 4, 2, 8, 4, 16)
    kc, vc = c.pool.dense()
    orc.store(F32, c.key, c.value, kc, vc, c.slot_mapping)
    out = orc.decode(F32, c.query, kc, vc, c.block_tables, c.context_lens, c.scale)
    assert np.isfinite(out).all()
    # one token fewer than stored: the new token's row is NaN only if the store missed it
    p = make_prefill_case("p", 3, F32, [0, 5, 8], [3, 4, 1], 4, 2, 8, 4, 16)
    kc, vc = p.pool.dense()
    orc.store(F32, p.key, p.value, kc, vc, p.slot_mapping)
    out = orc.prefill(F32, p.query, kc, vc, p.block_tables, p.cu_seqlens_q, p.cu_seqlens_k, p.scale)
    assert np.isfinite(out).all()


def test_store_then_decode_reads_new_token(orc):
    """The slot the generator picks for the new token is logical position L - 1 of its table."""
    c = make_decode_case("t", 4, F32, [9, 4, 1], 2, 1, 4, 4, 12)
    kc, vc = c.pool.dense()
    orc.store(F32, c.key, c.value, kc, vc, c.slot_mapping)
    for i, n in enumerate(c.context_lens):
        ko, vo = orc.gather(F32, kc, vc, c.block_tables[i], int(n))
        assert np.array_equal(ko[-1], c.key[i]) and np.array_equal(vo[-1], c.value[i])
        assert np.isfinite(ko).all() and np.isfinite(vo).all()


def test_bf16_is_upcast_exactly(orc):
    """bf16 inputs equal their exact float32 upcasts run through the fp32 path."""
    c = make_decode_case("b", 7, BF16, [7, 20], 4, 2, 16, 8, 8)
    kc, vc = c.pool.dense()
    orc.store(BF16, c.key, c.value, kc, vc, c.slot_mapping)
    a = orc.decode(BF16, c.query, kc, vc, c.block_tables, c.context_lens, c.scale)
    b = orc.decode(F32, bf16_bits_to_f32(c.query), bf16_bits_to_f32(kc), bf16_bits_to_f32(vc), c.block_tables,
                   c.context_lens, c.scale)
    assert np.array_equal(a, b)


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.0e38, 1e-40, 1.0 + 2 ** -8 + 2 ** -20],
                 np.float32)
    got = bf16_bits_to_f32(f32_to_bf16_bits(x))
    want = [1.0, 1.0, 1.0 + 4 * 2 ** -8, -2.5, float(np.float32(3.0e38)), None, 1.0 + 2 ** -7]
    assert got[0] == want[0] and got[1] == want[1] and got[2] == want[2] and got[3] == want[3]
    assert got[6] == want[6]
    assert math.isclose(got[4], 3.0e38, rel_tol=2 ** -8)
    assert np.isnan(bf16_bits_to_f32(f32_to_bf16_bits(np.array([np.nan], np.float32))))[0]
