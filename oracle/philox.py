"""Philox4x32-10 counter-based generator (oracle, test infrastructure).

Written from its published definition: J. K. Salmon, M. A. Moraes, R. O. Dror and
D. E. Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11. A 128-bit counter
(c0, c1, c2, c3) and a 64-bit key (k0, k1) go through ten rounds; each round forms the two
32x32 -> 64-bit products M0*c0 and M1*c2 and rewires the words as
(hi(M1*c2) ^ c1 ^ k0, lo(M1*c2), hi(M0*c0) ^ c3 ^ k1, lo(M0*c0)); between rounds the key is
bumped by the Weyl constants (W0, W1). The multipliers and Weyl constants are the paper's.

MagicDec (Section 3.1) samples with the speculative-decoding rule it cites (Leviathan et
al.), which needs uniform random numbers; the paper says nothing about their source. The
reading taken here fixes a counter layout so that a decision can be replayed exactly:

  key     = (seed & 0xffffffff, seed >> 32)
  counter = (word block j, (stream << 16) | position, sequence b, offset & 0xffffffff)

Stream 0 feeds the acceptance test of draft position i (word 0 of block 0); stream 1 feeds
the exponential race at the emitting position (token x takes word x % 4 of block x // 4);
stream 2 feeds the race that samples the draft token of draft step i (same word layout).
A 32-bit output x maps to the uniform u = (floor(x / 2^9) + 1/2) * 2^-23, which lies in
(0, 1) and is exactly representable in binary32 and binary64 alike.
"""

import numpy as np

M0 = 0xD2511F53
M1 = 0xCD9E8D57
W0 = 0x9E3779B9
W1 = 0xBB67AE85
MASK32 = 0xFFFFFFFF

STREAM_ACCEPT = 0
STREAM_RACE = 1
STREAM_DRAFT = 2


def philox4x32_10(counter, key):
    """Philox4x32-10 on arrays. counter: 4 arrays (or ints) of uint32 words; key: 2 words.

    Returns a tuple of 4 uint64 arrays holding the 32-bit output words.
    """
    c = [np.asarray(x, dtype=np.uint64) & MASK32 for x in counter]
    k0 = np.asarray(key[0], dtype=np.uint64) & MASK32
    k1 = np.asarray(key[1], dtype=np.uint64) & MASK32
    for rnd in range(10):
        if rnd > 0:
            k0 = (k0 + np.uint64(W0)) & MASK32
            k1 = (k1 + np.uint64(W1)) & MASK32
        p0 = np.uint64(M0) * c[0]
        p1 = np.uint64(M1) * c[2]
        hi0, lo0 = p0 >> np.uint64(32), p0 & MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & MASK32
        c = [hi1 ^ c[1] ^ k0, lo1, hi0 ^ c[3] ^ k1, lo0]
    return tuple(c)


def to_uniform(x):
    """Map 32-bit words to u in (0, 1): (x >> 9) * 2^-23 + 2^-24 (exact in float32)."""
    x = np.asarray(x, dtype=np.uint64)
    return (x >> np.uint64(9)).astype(np.float64) * 2.0 ** -23 + 2.0 ** -24


def _key(seed):
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    return (seed & MASK32, seed >> 32)


def accept_uniform(seed, offset, b, position):
    """The acceptance uniform u of draft position `position` of sequence b."""
    words = philox4x32_10((0, (STREAM_ACCEPT << 16) | int(position), int(b), int(offset) & MASK32),
                          _key(seed))
    return float(to_uniform(words[0]))


def _race_words(stream, seed, offset, b, position, vocab):
    nblk = (int(vocab) + 3) // 4
    j = np.arange(nblk, dtype=np.uint64)
    ones = np.ones(nblk, dtype=np.uint64)
    words = philox4x32_10((j, ones * ((int(stream) << 16) | int(position)), ones * int(b),
                           ones * (int(offset) & MASK32)), _key(seed))
    u = np.stack([to_uniform(wd) for wd in words], axis=1).reshape(-1)
    return u[: int(vocab)]


def race_uniforms(seed, offset, b, position, vocab):
    """Uniforms u'_x, x in [0, vocab), of the exponential race at `position` of sequence b."""
    return _race_words(STREAM_RACE, seed, offset, b, position, vocab)


def draft_uniforms(seed, offset, b, step, vocab):
    """Uniforms of the race that samples sequence b's draft token at draft step `step`."""
    return _race_words(STREAM_DRAFT, seed, offset, b, step, vocab)
