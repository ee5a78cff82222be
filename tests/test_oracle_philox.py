"""Pins for the oracle's Philox4x64-10 against numpy's library generator."""

import numpy as np
import pytest

from oracle import philox4x64_10, row_uniforms
from oracle.philox import words_to_unit, words_to_unit53

M64 = (1 << 64) - 1


def numpy_block(counter, key):
    """numpy.random.Philox advances its 256-bit counter by one before each
    block, so a generator started at c - 1 yields the block of counter c."""
    c = sum(int(w) << (64 * j) for j, w in enumerate(counter))
    c = (c - 1) % (1 << 256)
    start = [(c >> (64 * j)) & M64 for j in range(4)]
    bg = np.random.Philox(counter=np.array(start, dtype=np.uint64),
                          key=np.array([int(key[0]), int(key[1])], dtype=np.uint64))
    return tuple(int(x) for x in bg.random_raw(4))


CASES = [
    ((0, 0, 0, 0), (0, 0)),
    ((1, 0, 0, 0), (0, 0)),
    ((4, 0, 0, 0), (7, 0)),
    ((3, 17, 0, 0), (123456789, 0)),
    ((5, 31, 1, 0), (2 ** 63 + 11, 0)),
    ((M64, M64, M64, M64), (M64, M64)),
    ((0x243F6A8885A308D3, 0x13198A2E03707344, 0xA4093822299F31D0, 0x082EFA98EC4E6C89),
     (0x452821E638D01377, 0xBE5466CF34E90C6C)),
]


@pytest.mark.parametrize("counter,key", CASES)
def test_matches_numpy_philox(counter, key):
    assert philox4x64_10(counter, key) == numpy_block(counter, key)


def test_matches_numpy_random_grid():
    rng = np.random.default_rng(5)
    for _ in range(50):
        ctr = tuple(int(x) for x in rng.integers(0, 2 ** 63, 4, dtype=np.int64))
        key = tuple(int(x) for x in rng.integers(0, 2 ** 63, 2, dtype=np.int64))
        assert philox4x64_10(ctr, key) == numpy_block(ctr, key)


def test_unit_mapping_ranges_and_exactness():
    """r: top 24 bits, exact in float32; u: top 53 bits, exact in float64."""
    assert words_to_unit(0) == 0.0
    assert words_to_unit(M64) == 1.0 - 2.0 ** -24
    assert words_to_unit(1 << 40) == 2.0 ** -24
    assert words_to_unit((1 << 40) - 1) == 0.0
    assert words_to_unit53(0) == 0.0
    assert words_to_unit53(M64) == 1.0 - 2.0 ** -53
    assert words_to_unit53(1 << 11) == 2.0 ** -53
    assert words_to_unit53((1 << 11) - 1) == 0.0
    fine = 0
    for seed in range(5):
        for i in range(4):
            r, u = row_uniforms(seed, 3, i)
            for x in (r, u):
                assert 0.0 <= x < 1.0
            assert float(np.float32(r)) == r                  # exact in float32
            assert (r * 2 ** 24) == int(r * 2 ** 24)
            assert (u * 2 ** 53) == int(u * 2 ** 53)
            fine += (u * 2 ** 24) != int(u * 2 ** 24)       # bits below 2^-24 are used
    assert fine >= 18


def test_streams_are_distinct():
    seen = set()
    for seed in (0, 1):
        for b in range(3):
            for i in range(5):
                for purpose in (0, 1):
                    seen.add(row_uniforms(seed, b, i, purpose))
    assert len(seen) == 2 * 3 * 5 * 2


def test_uniforms_roughly_uniform():
    r = np.array([row_uniforms(11, b, i)[0] for b in range(200) for i in range(10)])
    assert abs(r.mean() - 0.5) < 0.03
    assert abs(r.var() - 1 / 12) < 0.01
