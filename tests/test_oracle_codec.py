"""Pins for the oracle's residual codec and end-to-end compress / decompress.

Closed-loop identities: the decoded error equals the rotated quantization
error exactly (the rotation is orthogonal), each rotated coordinate is within
half a scale step, no residual (b = 0) reproduces the stored low-rank part, and
no Tucker part (r = 0) reduces to plain rotated quantization of X.
"""
import json
import os

import numpy as np
import pytest

import synth
from oracle import codec, pipeline, quant, rng, tucker, wht


@pytest.fixture(scope="module")
def item():
    cfg = synth.config("mistral7b_gqa_1k", T=128, L=2, H=2)
    return cfg, synth.make_item(cfg, synth.item_specs(cfg)[0])


def _factors(X, rt):
    lam_t, U_t = tucker.token_factor_exact(X, rt)
    lam_f, U_f = tucker.feature_factor(X)
    return U_t, U_f, tucker.core_full(X, U_t, U_f)


@pytest.mark.parametrize("rt,rf,b", [(16, 24, 4), (8, 8, 2), (32, 128, 3), (0, 0, 4), (24, 16, 0)])
def test_closed_loop_identities(item, rt, rf, b):
    cfg, it = item
    X = it.x
    L, H, T, d = X.shape
    U_t, U_f, C = _factors(X, 32)
    sp = codec.stored_params(U_t, U_f, C, rt, rf, "bf16")
    enc = codec.encode(X, sp, b, it.seed, it.item_id, "bf16")
    Xt = codec.decode(enc, L, H, T, d, it.seed, it.item_id, "bf16", out_round=False)
    Xhat = codec.low_rank(sp, L, H, T, d, "bf16")
    if b == 0:
        assert np.array_equal(Xt, Xhat)
        return
    s = rng.rotation_signs(it.seed, it.item_id, d)
    r_rot = wht.rotate(X - Xhat, s).reshape(-1, 64)
    scale = quant.bf16_bits_to_f32(enc.scale_bits).astype(np.float64)
    deq = quant.dequantize_groups(quant.q_from_codes(quant.unpack_codes(enc.words, b), b),
                                  enc.scale_bits)
    # per rotated coordinate: |r' - q s| <= s / 2 (+ the fp32 rounding of r')
    assert np.all(np.abs(r_rot - deq) <= scale[:, None] / 2 + 2.0 ** -23 * np.abs(r_rot))
    # orthogonality: ||X~ - X|| = ||dequant - r'||
    e1 = np.linalg.norm(Xt - X)
    e2 = np.linalg.norm(deq - r_rot)
    assert abs(e1 - e2) <= 1e-10 * np.linalg.norm(X)
    if rt == 0:
        assert not np.any(Xhat)


def test_stored_params_are_leading_blocks(item):
    cfg, it = item
    U_t, U_f, C = _factors(it.x, 32)
    sp = codec.stored_params(U_t, U_f, C, 16, 24, "bf16")
    assert sp.Ut.shape == (it.T, 16) and sp.Uf.shape == (it.d, 24) and sp.C.shape == (it.L, it.H, 16, 24)
    assert np.array_equal(sp.Ut, quant.round_bf16(U_t[:, :16]))
    # bf16 values: zero low 16 bits of the fp32 pattern
    assert not np.any(sp.C.astype(np.float32).view(np.uint32) & 0xFFFF)


def test_pipeline_budget_and_error(item, golden_dir):
    cfg, it = item
    delta = json.load(open(os.path.join(golden_dir, "delta_b.json")))["delta"]
    specs = synth.item_specs(cfg)[:2]
    items = [synth.make_item(cfg, s) for s in specs]
    budget = synth.budget_for_ratio(cfg, 2.0, n_items=2)
    p = pipeline.Params(mode="randomized", rt_max=32, budget=budget, delta=delta)
    pl = pipeline.plan([i.x for i in items], [i.seed for i in items], [i.item_id for i in items],
                       "bf16", p)
    assert pl.feasible
    tot = sum(int(t["B"][[tuple(r) for r in t["cand"].tolist()].index(a)]) for t, a in zip(pl.tables, pl.alloc))
    assert tot <= budget
    for i, a, f in zip(items, pl.alloc, pl.factors):
        enc = pipeline.compress_item(i.x, f, a, i.seed, i.item_id, "bf16")
        Xt = pipeline.decompress_item(enc, i.x.shape, i.seed, i.item_id, "bf16")
        err = pipeline.rel_fro(Xt, i.x)
        # the modelled distortion predicts the realised error within a factor
        t = pl.tables[items.index(i)]
        Dm = float(t["D"][[tuple(r) for r in t["cand"].tolist()].index(a)])
        assert 0.5 < err ** 2 * np.sum(i.x ** 2) / Dm < 2.0
        assert err < 0.2
