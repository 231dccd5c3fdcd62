"""Rows whose RMSNorm mean square sits on or next to an fp32 rounding
boundary (test data, built with exact integer arithmetic).

tie_row: fp16 values on a 2^-7 grid in [-4, 4) whose squares (multiples of
2^-14) add up exactly, in fp64 and in any order, to K times an fp32 midpoint:
every evaluation order gives the same mean square, the midpoint itself, which
rounds to the even neighbour.

straddle_row: the tie row with `n_tiny` entries (zeros of the tie row)
replaced by 2^-24, the smallest fp16 subnormal.  Its exact mean square lies
just above the midpoint, by less than the fp64 rounding of the whole sum: a
correctly rounded sum (math.fsum) keeps the tiny squares and rounds up, while
an order that adds each tiny square to a partial sum of ordinary size drops
it and lands on the midpoint, which rounds to even (down, by construction).
"""

import numpy as np

K = 4096
TINY = 2.0 ** -24


def _grid_row(rng):
    return rng.integers(-512, 512, K).astype(np.int64)          # x = a / 128


def tie_row(seed=0, zero_start=0, zeros=1024, big_from=None):
    """(x float64 [K], midpoint): sum of (128 x)^2 = S_int with
    S_int / 2^14 / K an fp32 midpoint between two floats of [4, 8) whose lower
    neighbour has an even significand.  Entries zero_start .. zero_start +
    zeros - 1 are exactly 0 (room for the straddle row's tiny values); with
    big_from, the `zeros` entries from that index on have |x| >= 3."""
    rng = np.random.default_rng(seed)
    a = _grid_row(rng)
    a = np.where(a == 0, 1, a)
    if big_from is not None:
        b = a[big_from:big_from + zeros]
        a[big_from:big_from + zeros] = np.sign(b) * (384 + np.abs(b) % 128)
    a[zero_start:zero_start + zeros] = 0
    free = [j for j in range(K) if not (zero_start <= j < zero_start + zeros)
            and not (big_from is not None and big_from <= j < big_from + zeros)]
    # ms = S_int * 2^-26; fp32 midpoints in [4, 8) are (2p + 1) * 2^-22, i.e.
    # S_int = (2p + 1) * 16; the lower neighbour 2p * 2^-22 has an even
    # significand when p is even: S_int = 16 (mod 64)
    for j in free:
        for b in range(-383, 384):
            if b == 0:
                continue
            S = int((a * a).sum()) - int(a[j]) ** 2 + b * b
            if S % 64 == 16 and 4 * 2 ** 26 <= S < 8 * 2 ** 26:
                a[j] = b
                return a.astype(np.float64) / 128.0, S * 2.0 ** -26
    raise RuntimeError("no adjustment found")


def straddle_row(seed=0, n_tiny=768, tiny_start=0, big_from=None):
    """(x float64 [K], midpoint): the tie row with n_tiny of its zeros (from
    tiny_start on) set to 2^-24; their squares add n_tiny * 2^-48 to the exact
    sum, 0.75 of an fp64 step at the sum for n_tiny = 768."""
    x, mid = tie_row(seed, zero_start=tiny_start, big_from=big_from)
    x = x.copy()
    x[tiny_start:tiny_start + n_tiny] = TINY
    return x, mid
