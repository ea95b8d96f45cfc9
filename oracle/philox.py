"""Philox4x32-10, the counter-based generator behind attention dropout.

[RPA] (appendix "Masks, packing, and dropout") draws the dropout mask from a
counter-based random number generator inside the kernels, so the backward
regenerates the forward's mask instead of storing it; the pages do not name
the generator.  The reading here: Philox4x32 with 10 rounds, as published by
Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3"
(SC 2011).  One round maps the counter (c0, c1, c2, c3) under the key
(k0, k1) to

    (hi(M1 c2) ^ c1 ^ k0,  lo(M1 c2),  hi(M0 c0) ^ c3 ^ k1,  lo(M0 c0))

with M0 = 0xD2511F53, M1 = 0xCD9E8D57 and hi / lo the upper / lower 32 bits
of the 64-bit product; the key is bumped by the Weyl constants (0x9E3779B9,
0xBB67AE85) after every round.

Dropout mask of pair (i, j) of slice (b, h) with probability p8 / 256
(p8 in 0..255): Philox of counter (j >> 2, i >> 2, b H + h, 0) under the key
(seed mod 2^32, seed >> 32) gives four words; byte (j & 3) of word (i & 3) is
the pair's uniform byte, and the pair is kept iff that byte >= p8.  Kept
probabilities are scaled by 256 / (256 - p8).  One call covers a 4 x 4 block
of pairs, so a lane holding four consecutive keys of one query, or four
consecutive queries of one key, needs one call.
"""

import numpy as np

M0, M1 = 0xD2511F53, 0xCD9E8D57
W0, W1 = 0x9E3779B9, 0xBB67AE85
MASK32 = 0xFFFFFFFF


def philox4x32(c0, c1, c2, c3, k0, k1, rounds=10):
    """Philox4x32 on arrays (broadcast) of uint32 counters and a key; returns
    the four output words as uint64 arrays holding 32-bit values."""
    c0, c1, c2, c3 = (np.asarray(x, dtype=np.uint64) & MASK32 for x in (c0, c1, c2, c3))
    k0 = np.uint64(int(k0) & MASK32)
    k1 = np.uint64(int(k1) & MASK32)
    m0, m1 = np.uint64(M0), np.uint64(M1)
    s32 = np.uint64(32)
    mask = np.uint64(MASK32)
    for _ in range(rounds):
        p0 = m0 * c0  # < 2^64: both factors below 2^32
        p1 = m1 * c2
        c0, c1, c2, c3 = ((p1 >> s32) ^ c1 ^ k0, p1 & mask, (p0 >> s32) ^ c3 ^ k1, p0 & mask)
        k0 = np.uint64((int(k0) + W0) & MASK32)
        k1 = np.uint64((int(k1) + W1) & MASK32)
    return c0, c1, c2, c3


def keep_mask(N, bh, p8, seed):
    """Boolean [N, N] dropout keep-mask of slice index bh = b H + h."""
    i = np.arange(N, dtype=np.uint64)[:, None]
    j = np.arange(N, dtype=np.uint64)[None, :]
    words = philox4x32(j >> np.uint64(2), i >> np.uint64(2), np.uint64(bh), np.uint64(0),
                       int(seed) & MASK32, int(seed) >> 32)
    sel = (i & np.uint64(3)).astype(np.int64)
    w = np.choose(np.broadcast_to(sel, (N, N)), [np.broadcast_to(x, (N, N)) for x in words])
    byte = (w >> ((j & np.uint64(3)) * np.uint64(8))) & np.uint64(0xFF)
    return byte >= np.uint64(p8)


def keep_scale(p8):
    """Factor of a kept probability: 1 / (1 - p8 / 256)."""
    return 256.0 / (256.0 - p8)
