"""Pins for the oracle's partial Tucker factors, core and energy table.

Against closed forms and invariants: exact reconstruction at full rank,
orthonormal factors, the HOSVD error bound (De Lathauwer, De Moor & Vandewalle
2000) with equality for single-mode truncation (Eckart-Young), Pythagoras for
the truncation energy, and exact recovery of a planted noise-free Tucker
tensor by both the exact and the randomized token factor (Halko, Martinsson &
Tropp 2011: with k >= rank and no noise the range finder is exact).
"""
import numpy as np
import pytest

import synth
from oracle import tucker
from oracle.linalg import orth


def _lowrank(U_t, U_f, C, rt, rf):
    return np.matmul(np.matmul(U_t[:, :rt][None, None], C[:, :, :rt, :rf]), U_f[:, :rf].T[None, None])


def _sin_subspace(A, B):
    """Largest principal-angle sine between span(A) and span(B) (orthonormal columns)."""
    Qa, Qb = orth(A), orth(B)
    s = np.linalg.svd(Qa - Qb @ (Qb.T @ Qa), compute_uv=False)
    return float(s.max()) if s.size else 0.0


@pytest.fixture(scope="module")
def small_item():
    cfg = synth.config("tiny_exact_f32", T=64, L=2, H=3, d=64)
    return synth.make_item(cfg, synth.item_specs(cfg)[0])


def test_full_rank_is_exact(small_item):
    X = small_item.x
    T, d = X.shape[2], X.shape[3]
    lam_t, U_t = tucker.token_factor_exact(X, T)
    lam_f, U_f = tucker.feature_factor(X)
    C = tucker.core_full(X, U_t, U_f)
    Xh = _lowrank(U_t, U_f, C, T, d)
    assert np.linalg.norm(X - Xh) / np.linalg.norm(X) <= 1e-12
    assert np.max(np.abs(U_t.T @ U_t - np.eye(T))) <= 1e-12
    assert np.max(np.abs(U_f.T @ U_f - np.eye(d))) <= 1e-12
    # eigenvalues of the Grams are the energies along each mode
    assert abs(lam_t.sum() / np.sum(X * X) - 1) <= 1e-12
    assert abs(lam_f.sum() / np.sum(X * X) - 1) <= 1e-12


def test_hosvd_bound_and_single_mode_equality(small_item):
    X = small_item.x
    T, d = X.shape[2], X.shape[3]
    lam_t, U_t = tucker.token_factor_exact(X, T)
    lam_f, U_f = tucker.feature_factor(X)
    C = tucker.core_full(X, U_t, U_f)
    E = tucker.energy_table(C)
    nx2 = float(np.sum(X * X))
    for rt, rf in [(4, 8), (16, 12), (30, 40), (64, 5), (1, 64), (64, 64)]:
        err2 = float(np.sum((X - _lowrank(U_t, U_f, C, rt, rf)) ** 2))
        bound = float(lam_t[rt:].sum() + lam_f[rf:].sum())
        assert err2 <= bound * (1 + 1e-10) + 1e-12 * nx2
        # Pythagoras: the discarded energy equals ||X||^2 - S(r_t, r_f)
        assert abs(err2 - (nx2 - tucker.captured_energy(E, rt, rf))) <= 1e-11 * nx2
    for rt in (3, 17, 40):
        err2 = float(np.sum((X - _lowrank(U_t, U_f, C, rt, d)) ** 2))
        assert abs(err2 - lam_t[rt:].sum()) <= 1e-11 * nx2
    for rf in (5, 33):
        err2 = float(np.sum((X - _lowrank(U_t, U_f, C, T, rf)) ** 2))
        assert abs(err2 - lam_f[rf:].sum()) <= 1e-11 * nx2


@pytest.mark.parametrize("mode", ["exact", "randomized"])
def test_planted_noise_free_recovery(mode):
    cfg = synth.config("tiny_exact_f32", T=128, L=2, H=4, d=64, dtype="f32")
    spec = synth.item_specs(cfg)[0]
    it = synth.make_item(cfg, spec, sigma=0.0, keep_planted=True)
    # fp32 storage of the planted tensor limits what "exact" can mean; use the
    # unrounded planted tensor itself for the pin
    U, V, Cp = it.planted["U"], it.planted["V"], it.planted["C"]
    X = np.matmul(np.matmul(U[None, None], Cp), V.T[None, None])
    rt, rf = spec.rank_t, spec.rank_f
    lam_f, U_f = tucker.feature_factor(X)
    if mode == "exact":
        lam_t, U_t = tucker.token_factor_exact(X, 2 * rt)
    else:
        lam_t, U_t = tucker.token_factor_randomized(X, 2 * rt, 10, 1, 5, 1)
    assert lam_t[rt] / lam_t[0] <= 1e-13
    assert lam_f[rf] / lam_f[0] <= 1e-13
    assert _sin_subspace(U_t[:, :rt], U) <= 1e-10
    assert _sin_subspace(U_f[:, :rf], V) <= 1e-10
    C = tucker.core_full(X, U_t, U_f)
    Xh = _lowrank(U_t, U_f, C, rt, rf)
    assert np.linalg.norm(X - Xh) / np.linalg.norm(X) <= 1e-10


def test_randomized_tracks_exact_with_noise():
    cfg = synth.config("mistral7b_gqa_1k", T=256, L=2, H=2)
    it = synth.make_item(cfg, synth.item_specs(cfg)[1])
    X = it.x
    lam_e, U_e = tucker.token_factor_exact(X, 64)
    lam_r, U_r = tucker.token_factor_randomized(X, 64, 10, 1, 0, 1)
    # Ritz values never exceed the true eigenvalues (Cauchy interlacing) and
    # the leading, well-separated ones are close
    assert np.all(lam_r <= lam_e * (1 + 1e-12))
    assert np.all(lam_r[:8] >= 0.9 * lam_e[:8])
    A = tucker.unfold_token(X)
    cap_e = np.sum((U_e.T @ A) ** 2)
    cap_r = np.sum((U_r.T @ A) ** 2)
    assert cap_r <= cap_e * (1 + 1e-12) and cap_r >= 0.97 * cap_e
