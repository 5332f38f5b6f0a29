"""ORACLE (test infrastructure only): stored parameters, residual codec, decode.

Pages: the truncation residual is captured by a rotated low-bit quantizer
(landing page abstract); the rotation is a Johnson-Lindenstrauss rotation,
and the quantized, rotated residual gives back energy that the truncation
dropped (vendor page; author page abstract).  Errors are reported on the
reconstructed cache (relative Frobenius error, author page abstract).

Readings:
  * stored Tucker parameters are the leading blocks U_t[:, :r_t], U_f[:, :r_f],
    C[:, :, :r_t, :r_f], rounded (RNE) to the parameter dtype (bf16; fp32 for
    fp32 caches);
  * the low-rank part is the Tucker product of the stored parameters,
    X^_lh = U_t (C_lh U_f^T), formed here in fp64 with no intermediate
    rounding (the pages fix no intermediate precision; a decoder that holds
    C_lh U_f^T to a finite precision differs from this by that precision);
  * the residual is closed-loop: R = X - X^ with X^ the reconstruction from the
    stored, rounded parameters;
  * output is rounded (RNE) to the cache dtype.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from . import quant, wht
from .rng import rotation_signs


def param_round(dtype: str):
    return quant.round_f32 if dtype == "f32" else quant.round_bf16


@dataclass
class StoredParams:
    Ut: np.ndarray     # T x r_t  (values of the stored dtype, as fp64)
    Uf: np.ndarray     # d x r_f
    C: np.ndarray      # L x H x r_t x r_f


@dataclass
class Encoded:
    rt: int
    rf: int
    bits: int
    params: StoredParams
    words: Optional[np.ndarray]       # (G, bits) uint64, G = N / 64
    scale_bits: Optional[np.ndarray]  # (G,) uint16 bf16 patterns
    rotated: Optional[np.ndarray]     # fp32 rotated residual, (G, 64)


def stored_params(U_t, U_f, C_full, rt: int, rf: int, dtype: str) -> StoredParams:
    if rt == 0 or rf == 0:
        rt = rf = 0
    rnd = param_round(dtype)
    L, H = C_full.shape[:2]
    return StoredParams(Ut=rnd(U_t[:, :rt]), Uf=rnd(U_f[:, :rf]),
                        C=rnd(C_full[:, :, :rt, :rf]).reshape(L, H, rt, rf))


def low_rank(p: StoredParams, L: int, H: int, T: int, d: int, dtype: str) -> np.ndarray:
    """X^_lh = U_t (C_lh U_f^T) from the stored parameters, in fp64."""
    rt = p.Ut.shape[1]
    if rt == 0:
        return np.zeros((L, H, T, d))
    W = np.matmul(p.C, p.Uf.T[None, None])               # L x H x rt x d
    return np.matmul(p.Ut[None, None], W)


def encode(X: np.ndarray, p: StoredParams, bits: int, seed: int, item_id: int,
           dtype: str) -> Encoded:
    L, H, T, d = X.shape
    Xhat = low_rank(p, L, H, T, d, dtype)
    rt, rf = p.Ut.shape[1], p.Uf.shape[1]
    if bits == 0:
        return Encoded(rt, rf, 0, p, None, None, None)
    R = X - Xhat
    s = rotation_signs(seed, item_id, d)
    rp = wht.rotate(R, s)
    x32 = rp.astype(np.float32).reshape(-1, quant.GROUP)
    q, sbits = quant.quantize_groups(x32, bits)
    words = quant.pack_codes(quant.codes_from_q(q, bits), bits)
    return Encoded(rt, rf, bits, p, words, sbits, x32)


def decode(enc: Encoded, L: int, H: int, T: int, d: int, seed: int, item_id: int,
           dtype: str, out_round: bool = True) -> np.ndarray:
    Xhat = low_rank(enc.params, L, H, T, d, dtype)
    Xt = Xhat
    if enc.bits > 0:
        u = quant.unpack_codes(enc.words, enc.bits)
        q = quant.q_from_codes(u, enc.bits)
        rtil_rot = quant.dequantize_groups(q, enc.scale_bits).reshape(L, H, T, d)
        s = rotation_signs(seed, item_id, d)
        Xt = Xhat + wht.unrotate(rtil_rot, s)
    return param_round(dtype)(Xt) if out_round else Xt
