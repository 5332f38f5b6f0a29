"""ORACLE (test infrastructure only): decode attention over a compressed cache.

Pages: a fused decode kernel evaluates attention directly over the stored
factors, without materializing the dense K and V tensors (paper landing page,
abstract).  What such a kernel computes is plain softmax attention over the
cache the stored factors represent; the oracle therefore decodes K and V from
the payloads (the reconstruction of codec.decode, kept in fp64 without the
final rounding to the cache dtype, since attention over the factors never
forms that rounded tensor) and applies the textbook definition.

Readings (the pages give no formula):
  * one query vector per query head and decode step; grouped-query attention
    maps query head j of a layer to KV head j // G, G = query heads / KV heads;
  * scores s_t = scale * (q . k_t), weights p = softmax(s) over the cached
    tokens, output o = sum_t p_t v_t; the log-sum-exp of the scores is returned
    too, so that attention over tokens kept outside the compressed cache can be
    merged with this part (the flash-decoding rule).
"""
from __future__ import annotations

import numpy as np

from . import codec


def softmax_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """q (G, d), K (T, d), V (T, d) -> o (G, d), lse (G,), in fp64."""
    q = np.asarray(q, dtype=np.float64)
    s = scale * (q @ np.asarray(K, dtype=np.float64).T)            # (G, T)
    m = np.max(s, axis=1, keepdims=True)
    w = np.exp(s - m)
    den = np.sum(w, axis=1, keepdims=True)
    o = (w @ np.asarray(V, dtype=np.float64)) / den
    return o, (m + np.log(den))[:, 0]


def decoded(enc: codec.Encoded, shape, seed: int, item_id: int, dtype: str) -> np.ndarray:
    """The cache an item's payload represents, in fp64 (no final rounding)."""
    L, H, T, d = shape
    return codec.decode(enc, L, H, T, d, seed, item_id, dtype, out_round=False)


def decode_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """q (L, Hq, d) against a layer group's K, V (L, H, T, d): grouped-query
    attention, query head j of layer l on KV head j // (Hq / H).
    Returns o (L, Hq, d) and lse (L, Hq)."""
    L, Hq, d = q.shape
    H = K.shape[1]
    G = Hq // H
    o = np.zeros((L, Hq, d))
    lse = np.zeros((L, Hq))
    for l in range(L):
        for h in range(H):
            oo, ll = softmax_attention(q[l, h * G:(h + 1) * G], K[l, h], V[l, h], scale)
            o[l, h * G:(h + 1) * G] = oo
            lse[l, h * G:(h + 1) * G] = ll
    return o, lse
