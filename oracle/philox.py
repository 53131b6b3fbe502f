"""Philox4x64-10 and the uniforms the accept rule draws.  Test infrastructure.

The accept rule needs one uniform per acceptance test and one per resampling
draw ([SD-EAGLE] "The Exactness Rule": r ~ Uniform(0, 1); [SD-review] §2,
algorithm step 3).  They come from a counter-based generator so that any call
replays bit-exactly from (seed, offset).  This module writes the generator out
from its published definition:

  Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3",
  SC'11, section 3 (the Philox S-box): per round, two 64x64->128 products of
  the even counter words with the multipliers M0, M1; the high halves are
  XORed with the odd words and the round key; the low halves pass through; the
  key is bumped by the Weyl constants W0, W1 between rounds; 10 rounds.

Counter layout used by both sides of the parity tests:
  key     = (seed, 0)
  counter = (v, b, offset, 0)      v = node index, b = sequence index
  word 0  -> u_acc(b, v): the acceptance uniform of candidate node v
  word 1  -> u_res(b, v): the resampling uniform if the walk ends at node v
  words 2, 3 unused.
A 64-bit word w maps to u = (2 * (w >> 12) + 1) * 2**-53, an odd multiple of
2**-53 in (0, 1), exactly representable in float64.
"""

MASK64 = (1 << 64) - 1
# Multipliers and Weyl key increments of Philox4x64 (SC'11, table 2 and
# section 3.3; W0 is the golden ratio, W1 is sqrt(3) - 1, as 64-bit fractions).
M0 = 0xD2E7470EE14C6C93
M1 = 0xCA5A826395121157
W0 = 0x9E3779B97F4A7C15
W1 = 0xBB67AE8584CAA73B
ROUNDS = 10


def philox4x64_10(counter, key):
    """Return the four 64-bit output words for a 4-word counter and 2-word key."""
    x0, x1, x2, x3 = (int(c) & MASK64 for c in counter)
    k0, k1 = (int(k) & MASK64 for k in key)
    for r in range(ROUNDS):
        if r > 0:
            k0 = (k0 + W0) & MASK64
            k1 = (k1 + W1) & MASK64
        prod0 = M0 * x0
        prod1 = M1 * x2
        hi0, lo0 = prod0 >> 64, prod0 & MASK64
        hi1, lo1 = prod1 >> 64, prod1 & MASK64
        x0, x1, x2, x3 = hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0
    return x0, x1, x2, x3


def word_to_uniform(w):
    """Map a 64-bit word to an odd multiple of 2**-53 in (0, 1) (exact in float64)."""
    return float(2 * ((int(w) & MASK64) >> 12) + 1) * 2.0 ** -53


def node_uniforms(seed, offset, b, v):
    """(u_acc, u_res) for sequence b, node v."""
    w = philox4x64_10((v, b, offset, 0), (seed, 0))
    return word_to_uniform(w[0]), word_to_uniform(w[1])


def uniforms(seed, offset, B, N1):
    """Arrays u_acc[B][N1], u_res[B][N1] (lists of lists of float64)."""
    u_acc = [[0.0] * N1 for _ in range(B)]
    u_res = [[0.0] * N1 for _ in range(B)]
    for b in range(B):
        for v in range(N1):
            u_acc[b][v], u_res[b][v] = node_uniforms(seed, offset, b, v)
    return u_acc, u_res
