"""Dropout on the attention probabilities, for the float64 oracle.

Test infrastructure only, like the rest of this package.

The pages list dropout among the attention operations fused into one kernel
(chipfoundryservices.com glossary "flash attention algorithm", "Kernel
Fusion"); they do not define it. The reading used here is the
usual one for attention: after the row softmax, each probability p_ij is kept
with probability 1 - rate and then divided by 1 - rate, or zeroed; the saved
log-sum-exp is that of the scores before dropout, so the backward pass can
rebuild p_ij and the same keep decisions.

Keep decisions come from a counter-based generator so that the forward pass,
the backward pass and this oracle draw the same bits without storing a mask:
Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As
Easy as 1, 2, 3", SC'11). One call maps a 128-bit counter and a 64-bit key to
128 bits; its round is
    (c0, c1, c2, c3) -> (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0))
with M0 = 0xD2511F53, M1 = 0xCD9E8D57, and the key advances by
(0x9E3779B9, 0xBB67AE85) between the ten rounds.

Element (query i, key j) of query head bh = b * H + h (batch included) uses
counter (i >> 2, j >> 2, bh, 0) and key (seed mod 2^32, seed >> 32); of the
four output words it takes word i & 3 and of that word byte j & 3 (bits
8 (j & 3) .. 8 (j & 3) + 7). So one call decides a 4 x 4 block of elements,
and a row of four consecutive keys or a column of four consecutive queries
both come from one call. The element is kept iff its byte >= t, where the
rate is quantised to t / 256 with t = round(256 rate) (at most 255); the keep
probability is then exactly (256 - t) / 256 and kept values are scaled by
256 / (256 - t).
"""

import numpy as np

PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
MASK32 = 0xFFFFFFFF


def philox4x32(counter, key, rounds=10):
    """Philox4x32 of counters [..., 4] (uint32) under key (k0, k1); returns [..., 4] uint32."""
    c = np.asarray(counter, dtype=np.uint64) & MASK32
    c0, c1, c2, c3 = (c[..., i].copy() for i in range(4))
    k0, k1 = int(key[0]) & MASK32, int(key[1]) & MASK32
    for r in range(rounds):
        if r:
            k0 = (k0 + PHILOX_W0) & MASK32
            k1 = (k1 + PHILOX_W1) & MASK32
        p0 = c0 * np.uint64(PHILOX_M0)  # exact: both factors < 2^32
        p1 = c2 * np.uint64(PHILOX_M1)
        hi0, lo0 = p0 >> np.uint64(32), p0 & np.uint64(MASK32)
        hi1, lo1 = p1 >> np.uint64(32), p1 & np.uint64(MASK32)
        c0, c1, c2, c3 = hi1 ^ c1 ^ np.uint64(k0), lo1, hi0 ^ c3 ^ np.uint64(k1), lo0
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)


def threshold(rate):
    """Byte threshold t (keep iff byte >= t) for a dropout rate in [0, 1)."""
    if not (0.0 <= rate < 1.0):
        raise ValueError("dropout rate must be in [0, 1)")
    return min(255, int(np.floor(rate * 256.0 + 0.5)))


def keep_scale(rate):
    """Factor applied to kept probabilities: 256 / (256 - t)."""
    return 256.0 / (256.0 - threshold(rate))


def random_bytes(seed, bh, rows, keys):
    """The generator's byte for every (rows[r], keys[c]) of query head bh: uint8 [R, C]."""
    rows = np.asarray(rows, dtype=np.int64)
    keys = np.asarray(keys, dtype=np.int64)
    seed = int(seed)
    key = (seed & MASK32, (seed >> 32) & MASK32)
    ctr = np.zeros((rows.size, keys.size, 4), dtype=np.uint64)
    ctr[..., 0] = (rows >> 2)[:, None]
    ctr[..., 1] = (keys >> 2)[None, :]
    ctr[..., 2] = bh
    words = philox4x32(ctr, key)
    word = np.take_along_axis(words, (rows & 3)[:, None, None].repeat(keys.size, axis=1), axis=2)[..., 0]
    shift = (8 * (keys & 3)).astype(np.uint32)[None, :]
    return ((word >> shift) & np.uint32(0xFF)).astype(np.uint8)


def keep_mask(seed, bh, rows, keys, rate):
    """Boolean keep decisions for every (rows[r], keys[c]) of query head bh."""
    return random_bytes(seed, bh, rows, keys) >= threshold(rate)
