"""Pins for the oracle's quantizer, packing and the distortion constants."""
import json
import os

import numpy as np
import pytest
from scipy import special

from oracle import quant
from oracle.calibrate import measure


def test_worked_examples(golden_dir):
    doc = json.load(open(os.path.join(golden_dir, "quant_examples.json")))
    for ex in doc["examples"]:
        b = ex["bits"]
        x = np.array(ex["x"], dtype=np.float32)[None, :]
        q, s = quant.quantize_groups(x, b)
        assert q[0].tolist() == ex["q"], ex["note"]
        assert int(s[0]) == int(ex["scale_bf16"], 16), ex["note"]
        w = quant.pack_codes(quant.codes_from_q(q, b), b)
        assert ["0x%016x" % int(v) for v in w[0]] == ex["words"], ex["note"]
        # bytes: word p of the group at byte offset 8 p, little endian
        raw = quant.words_to_bytes(w)
        for p, hw in enumerate(ex["words"]):
            assert raw[8 * p:8 * p + 8] == int(hw, 16).to_bytes(8, "little")
        # element j's code sits in stream bits [b j, b j + b)
        stream = int.from_bytes(raw, "little")
        for j, qj in enumerate(ex["q"]):
            assert (stream >> (b * j)) & ((1 << b) - 1) == qj + (1 << (b - 1))


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 8])
def test_error_bound_range_symmetry(bits):
    rg = np.random.default_rng(bits)
    x = (rg.standard_normal((4096, 64)) * np.exp(rg.uniform(-20, 20, (4096, 1)))).astype(np.float32)
    x[0] = 0.0                                           # all-zero group
    q, s = quant.quantize_groups(x, bits)
    sc = quant.bf16_bits_to_f32(s).astype(np.float64)
    qm = quant.qmax_for(bits)
    assert q.min() >= -qm and q.max() <= qm
    assert np.all(q[0] == 0) and sc[0] == 0
    err = np.abs(x.astype(np.float64) - quant.dequantize_groups(q, s))
    assert np.all(err <= sc[:, None] / 2 * (1 + 2.0 ** -20))
    q2, s2 = quant.quantize_groups(-x, bits)
    assert np.array_equal(q2, -q) and np.array_equal(s2, s)
    u = quant.codes_from_q(q, bits)
    assert u.min() >= 1 and u.max() <= (1 << bits) - 1
    assert np.array_equal(quant.unpack_codes(quant.pack_codes(u, bits), bits), u)


def test_bf16_rounding_half_even():
    f = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -7 + 2 ** -9], dtype=np.float32)
    b = quant.f32_to_bf16_bits(f)
    # 1 + 2^-8 is a tie -> even (1.0); 1 + 3*2^-8 is a tie -> even (1 + 2^-6)
    assert [hex(int(v)) for v in b] == ["0x3f80", "0x3f80", "0x3f82", "0x3f81"]


def test_delta_b_constants(golden_dir):
    doc = json.load(open(os.path.join(golden_dir, "delta_b.json")))
    delta = doc["delta"]
    assert delta[0] == 1.0
    # an independent Monte-Carlo draw agrees to 1 %
    fresh = measure(n_groups=1 << 15, seed=12345, bits=(2, 3, 4))
    for b in (2, 3, 4):
        assert abs(fresh[b] / delta[b] - 1) < 0.01
    # decreasing in b, roughly 4x per extra bit at high resolution
    for b in range(3, 9):
        assert delta[b] < delta[b - 1]
    assert 3.0 < delta[7] / delta[8] < 5.0


def _half_normal_moment(a, b, c):
    """Integral over [a, b] (0 <= a <= b) of (x - c)^2 times the half-normal
    density 2 phi(x), from the Gaussian partial moments:
    int phi = Phi(b) - Phi(a), int x phi = phi(a) - phi(b),
    int x^2 phi = Phi(b) - Phi(a) + a phi(a) - b phi(b)."""
    Phi = lambda x: 0.5 * (1.0 + special.erf(x / np.sqrt(2.0)))
    phi = lambda x: np.exp(-0.5 * x * x) / np.sqrt(2.0 * np.pi)
    m0 = Phi(b) - Phi(a)
    m1 = phi(a) - phi(b)
    m2 = m0 + a * phi(a) - b * phi(b)
    return 2.0 * (m2 - 2.0 * c * m1 + c * c * m0)


def _delta_exact(bits, n=200001, hi=9.0):
    """Expected relative squared error of the b-bit group quantizer on iid N(0,1)
    groups of 64, by quadrature over the group's absmax M (order statistics),
    not by sampling.  Given M, the scale is s = bf16(M / qmax); the other 63
    magnitudes are iid half-normal conditioned below M and each is rounded to
    the nearest multiple k s (k <= qmax, larger values clamped to qmax s); the
    absmax element itself is rounded the same way.  The per-element energy is 1,
    so delta_b = E[group squared error] / 64."""
    qm = (1 << (bits - 1)) - 1
    M = np.linspace(1e-3, hi, n)
    s = quant.bf16_bits_to_f32(quant.f32_to_bf16_bits((M / qm).astype(np.float32))).astype(np.float64)
    F = special.erf(M / np.sqrt(2.0))                      # P(|x| < M)
    k = np.arange(qm + 1)[:, None]
    a = np.clip((k - 0.5) * s, 0.0, M)
    b = np.clip((k + 0.5) * s, 0.0, M)
    b[-1] = M                                              # everything above (qmax - 1/2) s -> qmax s
    inner = _half_normal_moment(a, b, k * s).sum(axis=0) / F
    top = M - np.minimum(np.rint(M / s), qm) * s
    dens = 64.0 * F ** 63 * 2.0 * np.exp(-0.5 * M * M) / np.sqrt(2.0 * np.pi)     # density of M
    g = 63.0 * inner + top * top
    return float(np.trapezoid(g * dens, M) / 64.0), float(np.trapezoid(dens, M))


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
def test_delta_b_matches_exact_quadrature(golden_dir, bits):
    """The frozen delta_b (a 2^20-group Monte-Carlo run of the oracle's
    quantizer) against its expectation computed independently in closed form:
    Monte-Carlo error at 2^20 groups is about 3e-4 relative, so 1e-3 pins the
    definition (relative MSE against the input energy), the scale rule and the
    rounding; the high-resolution limit (63/64) E[M^2] / (12 qmax^2) is the
    b -> infinity check of the same expression."""
    delta = json.load(open(os.path.join(golden_dir, "delta_b.json")))["delta"]
    exact, mass = _delta_exact(bits)
    assert abs(mass - 1.0) < 1e-9
    assert abs(delta[bits] / exact - 1.0) < 1e-3, (bits, delta[bits], exact)
    if bits >= 6:
        f = lambda m: m * m * 64 * special.erf(m / np.sqrt(2)) ** 63 * 2 * np.exp(-m * m / 2) / np.sqrt(2 * np.pi)
        em2 = float(np.trapezoid(f(np.linspace(0, 12, 400001)), np.linspace(0, 12, 400001)))
        qm = (1 << (bits - 1)) - 1
        assert abs(exact / ((63 / 64) * em2 / (12 * qm * qm)) - 1) < 0.02
