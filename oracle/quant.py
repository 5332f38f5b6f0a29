"""ORACLE (test infrastructure only): b-bit residual quantizer and group bit-stream packing.

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

Packing (the pages fix no layout): each group is one little-endian bit stream
of 64 b bits = 8 b bytes, element j's code in stream bits [b j, b j + b), bit k
of the stream being bit (k mod 8) of byte k / 8.  Group g starts at byte 8 b g.
Groups run over (layer, head, token, feature / 64) in row-major order; the bf16
scales form an array in the same order.  The same bytes read as b
little-endian uint64 words per group are the "codes" array.
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


def pack_codes(u: np.ndarray, bits: int) -> np.ndarray:
    """u: (G, 64) codes -> (G, bits) uint64 words of the group bit stream."""
    u = np.asarray(u, dtype=np.uint64)
    G = u.shape[0]
    planes = ((u[:, :, None] >> np.arange(bits, dtype=np.uint64)[None, None, :]) & np.uint64(1))
    stream = planes.reshape(G, GROUP * bits).astype(np.uint8)       # stream bit k = element k // b, bit k % b
    by = np.packbits(stream, axis=1, bitorder="little")              # (G, 8 b) bytes
    return by.view("<u8").reshape(G, bits).astype(np.uint64)


def unpack_codes(words: np.ndarray, bits: int) -> np.ndarray:
    words = np.ascontiguousarray(np.asarray(words, dtype=np.uint64)).astype("<u8")
    G = words.shape[0]
    by = words.view(np.uint8).reshape(G, 8 * bits)
    stream = np.unpackbits(by, axis=1, bitorder="little").reshape(G, GROUP, bits).astype(np.uint64)
    return np.sum(stream << np.arange(bits, dtype=np.uint64)[None, None, :], axis=2).astype(np.uint64)


def words_to_bytes(words: np.ndarray) -> bytes:
    return np.ascontiguousarray(words, dtype="<u8").tobytes()
