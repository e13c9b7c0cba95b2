"""Shared-seed dropout for the oracle (test infrastructure only).

MLM-review, "key terms" and "approach" sections: dropout is synchronised, i.e.
every device applies the same dropout mask.  The pages do not say how the mask
is drawn.  Reading taken here: the mask is a pure function of
``(seed, offset, element index)`` built on the counter-based generator
Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as
1, 2, 3", SC'11), so that every shard, and every rank, that applies dropout to
the same replicated tensor draws the same mask without any communication.

Element ``j`` (flat row-major index into the full replicated tensor) takes
word ``j mod 4`` of ``Philox4x32-10(counter=(j // 4, offset), key=seed)``,
where the 64-bit ``j // 4`` fills counter words 0-1 (low word first) and the
64-bit ``offset`` fills words 2-3.  The element is kept iff that word is
``>= floor(p * 2**32)`` with ``p`` taken as the float32 value that crosses the
library boundary; kept values are scaled by ``1 / (1 - p)``.
"""

import numpy as np

_MASK32 = np.uint64(0xFFFFFFFF)
# Philox4x32 multipliers, from the SC'11 paper.
_M0 = np.uint64(0xD2511F53)
_M1 = np.uint64(0xCD9E8D57)
# Weyl key increments: 2**32 times the fractional part of the golden ratio and
# of sqrt(3) - 1 (the paper's choice); pinned by their closed form in the tests.
_W0 = np.uint64(0x9E3779B9)
_W1 = np.uint64(0xBB67AE85)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Ten-round Philox4x32 block function.

    Arguments are arrays (or scalars) of 32-bit counter words ``c0..c3`` and
    key words ``k0, k1``; returns the four 32-bit output words as uint64
    arrays holding values < 2**32.

    One round: multiply counter word 0 by M0 and word 2 by M1 as full 64-bit
    products, then the new state is
    (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2), hi(M0*c0) ^ c3 ^ k1, lo(M0*c0)).
    Between rounds the key is bumped by (W0, W1) modulo 2**32.
    """
    c0, c1, c2, c3, k0, k1 = (np.asarray(v, dtype=np.uint64) & _MASK32
                              for v in (c0, c1, c2, c3, k0, k1))
    for rnd in range(10):
        if rnd > 0:
            k0 = (k0 + _W0) & _MASK32
            k1 = (k1 + _W1) & _MASK32
        p0 = _M0 * c0          # < 2**64: exact in uint64
        p1 = _M1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def dropout_threshold(p):
    """Integer keep threshold ``floor(p * 2**32)`` for the float32 value of p."""
    p32 = float(np.float32(p))
    if not (0.0 <= p32 < 1.0):
        raise ValueError("dropout probability must lie in [0, 1)")
    return int(np.floor(p32 * 4294967296.0))


def dropout_random_words(start, count, seed, offset):
    """The 32-bit random word of elements ``start .. start+count-1``."""
    j = np.arange(start, start + count, dtype=np.uint64)
    blk = j >> np.uint64(2)
    lane = (j & np.uint64(3)).astype(np.int64)
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    offset = int(offset) & 0xFFFFFFFFFFFFFFFF
    w = philox4x32_10(blk & _MASK32, blk >> np.uint64(32),
                      offset & 0xFFFFFFFF, offset >> 32,
                      seed & 0xFFFFFFFF, seed >> 32)
    words = np.stack(w, axis=0)
    return words[lane, np.arange(count)]


def dropout_keep_mask(n, p, seed, offset, start=0):
    """Boolean keep mask of ``n`` elements starting at flat index ``start``."""
    thr = dropout_threshold(p)
    if n == 0:
        return np.zeros(0, dtype=bool)
    return dropout_random_words(start, n, seed, offset) >= np.uint64(thr)


def dropout(x, p, seed, offset, start=0):
    """Apply the shared-seed dropout to ``x`` (any shape, row-major flat index).

    Returns ``(y, keep)`` with ``y = x / (1 - p)`` where kept and 0 elsewhere,
    in float64.  The same call applied to an upstream gradient is the backward.
    """
    x = np.asarray(x, dtype=np.float64)
    keep = dropout_keep_mask(x.size, p, seed, offset, start).reshape(x.shape)
    scale = 1.0 / (1.0 - float(np.float32(p)))
    return np.where(keep, x * scale, 0.0), keep
