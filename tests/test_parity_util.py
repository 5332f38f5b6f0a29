"""CPU checks of the boundary-case comparison used by the GPU codec tests: a
residual perturbed within the bound passes; a planted wrong code or scale fails."""
import numpy as np
import pytest

import synth
from oracle import codec as ocodec, quant as oquant, tucker
from tests.parity_util import check_codes, row_tolerance


def _case(bits):
    cfg = synth.config("mistral7b_gqa_1k", T=128, L=2, H=2)
    it = synth.make_item(cfg, synth.item_specs(cfg)[1])
    X = it.x
    U_t = tucker.token_factor_exact(X, 8)[1]
    U_f = tucker.feature_factor(X)[1]
    sp = ocodec.stored_params(U_t, U_f, tucker.core_full(X, U_t, U_f), 8, 8, "bf16")
    enc = ocodec.encode(X, sp, bits, it.seed, it.item_id, "bf16")
    R = X - ocodec.low_rank(sp, 2, 2, 128, 128, "bf16")
    return X, sp, enc, R, it


@pytest.mark.parametrize("bits", [3, 8])
def test_perturbed_residual_passes(bits):
    X, sp, enc, R, it = _case(bits)
    tol = row_tolerance(sp.Ut, sp.Uf, sp.C, R)
    # move X^ by a quarter of the bound's per-element share, as the GPU's
    # hi + lo product and fp32 accumulation may
    Wa = np.matmul(np.abs(sp.C), np.abs(sp.Uf).T[None, None])
    A = np.matmul(np.abs(sp.Ut)[None, None], Wa)
    noise = np.random.default_rng(0).uniform(-1, 1, X.shape) * 2.0 ** -16 * A
    enc2 = ocodec.encode(X + noise, sp, bits, it.seed, it.item_id, "bf16")
    u1, u2 = oquant.unpack_codes(enc.words, bits), oquant.unpack_codes(enc2.words, bits)
    nc, ns = check_codes(u2, u1, enc2.scale_bits, enc.scale_bits, enc.rotated, tol, bits, 128)
    assert nc + ns > 0 or bits == 3          # at 8 bits some codes do move


def test_planted_wrong_code_fails():
    X, sp, enc, R, it = _case(4)
    tol = row_tolerance(sp.Ut, sp.Uf, sp.C, R)
    u = oquant.unpack_codes(enc.words, 4)
    y = np.abs(enc.rotated / oquant.bf16_bits_to_f32(enc.scale_bits)[:, None])
    g, e = np.unravel_index(np.argmin(np.abs((y % 1) - 0.0)), y.shape)     # farthest from a boundary
    bad = u.copy()
    bad[g, e] = bad[g, e] + 1 if bad[g, e] < 15 else bad[g, e] - 1
    with pytest.raises(AssertionError):
        check_codes(bad, u, enc.scale_bits, enc.scale_bits, enc.rotated, tol, 4, 128)
    sc = enc.scale_bits.copy()
    sc[5] += 1
    with pytest.raises(AssertionError):
        check_codes(u, u, sc, enc.scale_bits, enc.rotated, tol, 4, 128)
