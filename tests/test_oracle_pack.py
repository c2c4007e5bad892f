"""Pins of the oracle's 2-bit packing: literal bytes worked out by hand from
the layout rule, a bit-by-bit pure-Python packer, and round trips."""
import json
import os

import numpy as np

from oracle.pack import pack_k_codes, pack_v_codes, unpack_k_codes, unpack_v_codes

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pack_bytes.json")


def test_literal_bytes():
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        row = np.zeros((1, 128), np.uint8)
        row[0, :4] = c["codes"]
        assert pack_k_codes(row)[0, 0] == int(c["byte"], 16), c


def _bitwise_pack_row(codes):
    out = bytearray(len(codes) // 4)
    for idx, c in enumerate(codes):
        for bit in range(2):
            if (int(c) >> bit) & 1:
                pos = 2 * idx + bit
                out[pos // 8] |= 1 << (pos % 8)
    return np.frombuffer(bytes(out), np.uint8)


def test_k_layout_bitwise():
    rng = np.random.default_rng(5)
    c = rng.integers(0, 4, (6, 128)).astype(np.uint8)
    p = pack_k_codes(c)
    assert p.shape == (6, 32)
    for t in range(6):
        np.testing.assert_array_equal(p[t], _bitwise_pack_row(c[t]))
    np.testing.assert_array_equal(unpack_k_codes(p), c)


def test_v_layout_bitwise_and_position():
    rng = np.random.default_rng(6)
    c = rng.integers(0, 4, (256, 128)).astype(np.uint8)
    p = pack_v_codes(c)
    assert p.shape == (2, 128, 32)
    for g in range(2):
        for d in (0, 1, 63, 127):
            np.testing.assert_array_equal(p[g, d], _bitwise_pack_row(c[g * 128:(g + 1) * 128, d]))
    np.testing.assert_array_equal(unpack_v_codes(p), c)
    one = np.zeros((128, 128), np.uint8)
    one[5, 7] = 3          # token 5 = byte 1, bits 2..3 of channel 7's row
    p1 = pack_v_codes(one)
    assert p1[0, 7, 1] == 0x0C and p1.sum() == 0x0C
