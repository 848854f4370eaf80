"""Pins of the packing oracle (CPU only): hand-packed words and round trips."""

import numpy as np
import pytest

from oracle import pack_ref, unpack_ref


def test_hand_vectors_4bit_and_2bit():
    assert pack_ref([[1, 2, 3, 4, 5, 6, 7, 8]], 4)[0, 0] == 0x87654321
    assert pack_ref([[3, 2, 1, 0] * 4], 2)[0, 0] == 0x1B1B1B1B
    assert pack_ref([[0xAB, 0x01, 0xFF, 0x10]], 8)[0, 0] == 0x10FF01AB


def test_hand_vector_3bit():
    codes = list(range(8)) * 4  # 32 codes, 96 bits
    # The stream is the octal digits 7,6,...,0 repeated, least significant first:
    # value = sum_i codes[i] * 8**i.  Per group of 8 codes that is octal 76543210 = 0xFAC688.
    value = 0
    for rep in range(4):
        value |= 0xFAC688 << (24 * rep)
    words = [(value >> (32 * w)) & 0xFFFFFFFF for w in range(3)]
    np.testing.assert_array_equal(pack_ref([codes], 3)[0], words)
    assert words == [0x88FAC688, 0xC688FAC6, 0xFAC688FA]


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_round_trip(bits):
    rng = np.random.default_rng(bits)
    codes = rng.integers(0, 2 ** bits, size=(5, 96))
    p = pack_ref(codes, bits)
    assert p.shape == (5, 96 * bits // 32) and p.dtype == np.uint32
    np.testing.assert_array_equal(unpack_ref(p, 96, bits), codes)


def test_rejects_bad_shapes():
    with pytest.raises(ValueError):
        pack_ref(np.zeros((1, 10), dtype=int), 3)
    with pytest.raises(ValueError):
        pack_ref(np.full((1, 8), 16), 4)
