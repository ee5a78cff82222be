"""Philox4x64-10 counter-based generator and the uniforms of one verify row.

Why: reproducible generation needs the acceptance coin flips and the
correction samples to come from a deterministic generator seeded from the
request ([SSD] "Quality, Evaluation, and Guardrails", item 3: sampling seed
propagation).  A counter-based generator lets a CPU and a GPU draw the very
same numbers without sharing state.

Philox4x64-10 (Salmon et al., SC'11): a 256-bit counter (c0..c3) and a
128-bit key (k0, k1).  One round multiplies c0 and c2 by two fixed 64-bit
constants, keeps both halves of each 128-bit product, and mixes:

    (hi0, lo0) = M0 * c0          (hi1, lo1) = M1 * c2
    c' = (hi1 ^ c1 ^ k0,  lo1,  hi0 ^ c3 ^ k1,  lo0)

and the key is bumped by two Weyl constants between rounds.  Ten rounds.

Pinned by: numpy.random.Philox (a library implementation of the same
generator; numpy advances its counter by one before it produces a block).

Uniform layout (a convention shared with the HIP library, fixed here):
    key     = (seed, 0)
    counter = (i, b, purpose, 0)        i = position, b = batch row
    r_{b,i} = (word0 >> 40) * 2**-24    acceptance draw (exact in float32,
                                        where the ratio test runs)
    u_{b,i} = (word1 >> 11) * 2**-53    inverse-CDF draw at row i (exact in
                                        float64, where u * R is formed, so
                                        the sampled law is not rounded to
                                        steps of 2**-24)
Both lie in [0, 1).  purpose 0 is the
verify step; purpose 1 is reserved for a harness that draws draft tokens, so
the two never share numbers.  The layout itself is pinned only by GPU/CPU
agreement (parity), since it is a convention rather than a fact of the pages.
"""

MASK64 = (1 << 64) - 1
PHILOX_M0 = 0xD2E7470EE14C6C93
PHILOX_M1 = 0xCA5A826395121157
PHILOX_W0 = 0x9E3779B97F4A7C15   # golden ratio
PHILOX_W1 = 0xBB67AE8584CAA73B   # sqrt(3) - 1

PURPOSE_VERIFY = 0
PURPOSE_DRAFT = 1


def _round(c, k):
    p0 = PHILOX_M0 * c[0]
    p1 = PHILOX_M1 * c[2]
    hi0, lo0 = p0 >> 64, p0 & MASK64
    hi1, lo1 = p1 >> 64, p1 & MASK64
    return (hi1 ^ c[1] ^ k[0], lo1, hi0 ^ c[3] ^ k[1], lo0)


def philox4x64_10(counter, key):
    """Return the four 64-bit output words for one counter/key pair."""
    c = tuple(int(x) & MASK64 for x in counter)
    k = [int(key[0]) & MASK64, int(key[1]) & MASK64]
    assert len(c) == 4 and len(k) == 2
    for rnd in range(10):
        if rnd:
            k[0] = (k[0] + PHILOX_W0) & MASK64
            k[1] = (k[1] + PHILOX_W1) & MASK64
        c = _round(c, k)
    return c


def words_to_unit(word):
    """Top 24 bits of a 64-bit word as a float in [0, 1)."""
    return (int(word) >> 40) * (2.0 ** -24)


def words_to_unit53(word):
    """Top 53 bits of a 64-bit word as a float in [0, 1)."""
    return (int(word) >> 11) * (2.0 ** -53)


def row_uniforms(seed, b, i, purpose=PURPOSE_VERIFY):
    """(r, u) for batch row b, position i: acceptance draw and resample draw."""
    w = philox4x64_10((i, b, purpose, 0), (seed, 0))
    return words_to_unit(w[0]), words_to_unit53(w[1])
