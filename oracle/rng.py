"""ORACLE (test infrastructure only): counter-based Rademacher signs.

The rotation of the residual is a seeded randomized Hadamard (JL) transform and
FlashJoLT sketches with a random test matrix (paper landing page, abstract;
vendor page: Johnson-Lindenstrauss rotation).  The pages do not fix a
generator, so both draw from one counter-based stream built on the SplitMix64
output function (Steele, Lea & Flood, "Fast splittable pseudorandom number
generators", OOPSLA 2014):

    mix64(z) = z ^= z >> 30; z *= 0xBF58476D1CE4E5B9;
               z ^= z >> 27; z *= 0x94D049BB133111EB; z ^= z >> 31   (mod 2^64)

    key      = mix64(mix64(seed) + item_id)
    word     = mix64(key + (stream << 56) + index)
    sign     = -1 if bit 63 of word is set else +1

Stream 0 gives the rotation signs (index = feature), stream 1 the sketch
matrix Omega (index = row * k + column, rows in token-unfolding column order).
"""
from __future__ import annotations

import numpy as np

MASK = (1 << 64) - 1
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def mix64_int(z: int) -> int:
    z &= MASK
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK
    return z ^ (z >> 31)


def mix64_array(z: np.ndarray) -> np.ndarray:
    z = z.astype(np.uint64, copy=True)
    with np.errstate(over="ignore"):
        z ^= z >> np.uint64(30)
        z *= _M1
        z ^= z >> np.uint64(27)
        z *= _M2
        z ^= z >> np.uint64(31)
    return z


def item_key(seed: int, item_id: int) -> int:
    return mix64_int((mix64_int(seed) + item_id) & MASK)


def rademacher(seed: int, item_id: int, stream: int, index: np.ndarray) -> np.ndarray:
    """+-1.0 (fp64) for each counter value in ``index``."""
    key = item_key(seed, item_id)
    base = np.uint64((key + (stream << 56)) & MASK)
    idx = np.asarray(index, dtype=np.uint64)
    with np.errstate(over="ignore"):
        w = mix64_array(idx + base)
    return np.where((w >> np.uint64(63)) != 0, -1.0, 1.0)


def rotation_signs(seed: int, item_id: int, d: int) -> np.ndarray:
    return rademacher(seed, item_id, 0, np.arange(d, dtype=np.uint64))


def sketch_matrix(seed: int, item_id: int, n: int, k: int) -> np.ndarray:
    """Omega (n x k), entry (row, col) from counter row * k + col."""
    idx = np.arange(n * k, dtype=np.uint64)
    return rademacher(seed, item_id, 1, idx).reshape(n, k)
