"""ORACLE (test infrastructure only): the randomized Hadamard (JL) rotation, fp64.

Pages: the truncation residual is rotated by a Johnson-Lindenstrauss rotation
before low-bit quantization (vendor page; author page abstract; landing page
abstract: "a rotated low-bit quantizer captures the truncation residual").
Reading: one rotation per (layer, head, token) row along the feature axis,

    r' = (1/sqrt(d)) * H_d * (s o r),      r = s o ((1/sqrt(d)) * H_d * r'),

with H_d the Sylvester-ordered Hadamard matrix, H[i][j] = (-1)^popcount(i & j),
and s a seeded +-1 vector per item (the fast JL transform of Ailon & Chazelle).
H_d is symmetric with H_d H_d = d I, so the scaled transform is its own inverse.
"""
from __future__ import annotations

import numpy as np


def fwht(x: np.ndarray) -> np.ndarray:
    """Unnormalised Walsh-Hadamard transform along the last axis (Sylvester order).

    Butterfly with stride h = 1, 2, 4, ...: (a, b) -> (a + b, a - b).
    """
    y = np.array(x, dtype=np.float64, copy=True)
    d = y.shape[-1]
    if d & (d - 1):
        raise ValueError("length must be a power of two")
    lead = y.shape[:-1]
    h = 1
    while h < d:
        y = y.reshape(lead + (d // (2 * h), 2, h))
        a = y[..., 0, :].copy()
        b = y[..., 1, :].copy()
        y[..., 0, :] = a + b
        y[..., 1, :] = a - b
        y = y.reshape(lead + (d,))
        h *= 2
    return y


def rotate(r: np.ndarray, signs: np.ndarray) -> np.ndarray:
    d = r.shape[-1]
    return fwht(r * signs) / np.sqrt(d)


def unrotate(rp: np.ndarray, signs: np.ndarray) -> np.ndarray:
    d = rp.shape[-1]
    return signs * (fwht(rp) / np.sqrt(d))
