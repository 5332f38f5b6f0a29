"""ORACLE (test infrastructure only): b-bit residual quantizer and bit-plane packing.

Pages: "a rotated low-bit quantizer captures the truncation residual" (landing
page abstract); the residual bit-width b is allocated per group together with
the Tucker ranks.  The pages fix neither the quantizer nor the layout, so this
follows the plainest symmetric per-group scheme, defined in fp32 so that codes
are reproducible bit for bit:

  x      = fp32(r')                                (rotated residual)
  amax   = max |x| over a group of 64 consecutive features
  qmax   = 2^(b-1) - 1                             (b = 2 is ternary)
  s32    = fl32(amax / qmax);  scale = bf16_RNE(s32);  inv = fl32(1 / scale)
  q      = clamp(rint_half_even(fl32(x * inv)), -qmax, qmax);  q = 0 if scale = 0
  u      = q + 2^(b-1)                             (code, in [1, 2^b - 1])
  decode = q * scale

Packing: per group and bit-plane p < b, one little-endian uint64 whose bit j
is bit p of u_j; the words of group g sit at byte 8 * (g * b + p).  Groups run
over (layer, head, token, feature / 64) in row-major order; the bf16 scales form
an array in the same order.
"""
from __future__ import annotations

import numpy as np

GROUP = 64


def f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16 bit pattern (finite inputs)."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp64 -> fp32 (RNE) -> bf16 (RNE), returned as fp64 values."""
    return bf16_bits_to_f32(f32_to_bf16_bits(np.asarray(x, dtype=np.float32))).astype(np.float64)


def round_f32(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def qmax_for(bits: int) -> int:
    return (1 << (bits - 1)) - 1


def quantize_groups(x32: np.ndarray, bits: int):
    """Quantize fp32 values grouped along the last axis (length 64).

    Returns (q, scale_bits): integer codes q in [-qmax, qmax] (int32, same
    shape as x32) and the bf16 scale bit patterns (one per group).
    """
    x32 = np.asarray(x32, dtype=np.float32)
    if x32.shape[-1] != GROUP:
        raise ValueError("groups must have 64 elements")
    qm = qmax_for(bits)
    amax = np.max(np.abs(x32), axis=-1)
    s32 = (amax / np.float32(qm)).astype(np.float32)
    sbits = f32_to_bf16_bits(s32)
    scale = bf16_bits_to_f32(sbits)
    zero = scale == 0
    with np.errstate(divide="ignore"):
        inv = (np.float32(1.0) / np.where(zero, np.float32(1.0), scale)).astype(np.float32)
    y = (x32 * inv[..., None]).astype(np.float32)
    q = np.rint(y)
    q = np.clip(q, -qm, qm).astype(np.int32)
    q[zero] = 0
    return q, sbits


def dequantize_groups(q: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    """q * scale in fp64 (exact: q is a small integer and scale a bf16 value)."""
    return q.astype(np.float64) * bf16_bits_to_f32(scale_bits).astype(np.float64)[..., None]


def codes_from_q(q: np.ndarray, bits: int) -> np.ndarray:
    return (q + (1 << (bits - 1))).astype(np.uint64)


def q_from_codes(u: np.ndarray, bits: int) -> np.ndarray:
    return u.astype(np.int64) - (1 << (bits - 1))


def pack_bitplanes(u: np.ndarray, bits: int) -> np.ndarray:
    """u: (G, 64) codes -> (G, bits) uint64 words, word p bit j = bit p of u[j]."""
    u = np.asarray(u, dtype=np.uint64)
    G = u.shape[0]
    words = np.zeros((G, bits), dtype=np.uint64)
    shifts = np.arange(GROUP, dtype=np.uint64)
    for p in range(bits):
        plane = (u >> np.uint64(p)) & np.uint64(1)
        words[:, p] = np.bitwise_or.reduce(plane << shifts[None, :], axis=1)
    return words


def unpack_bitplanes(words: np.ndarray, bits: int) -> np.ndarray:
    words = np.asarray(words, dtype=np.uint64)
    G = words.shape[0]
    u = np.zeros((G, GROUP), dtype=np.uint64)
    shifts = np.arange(GROUP, dtype=np.uint64)
    for p in range(bits):
        plane = (words[:, p:p + 1] >> shifts[None, :]) & np.uint64(1)
        u |= plane << np.uint64(p)
    return u


def words_to_bytes(words: np.ndarray) -> bytes:
    return np.ascontiguousarray(words, dtype="<u8").tobytes()
