"""Pins for the oracle's quantizer, packing and the distortion constants."""
import json
import os

import numpy as np
import pytest

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
