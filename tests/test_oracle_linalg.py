"""Pins for the oracle's eigensolver, QR, RNG and Hadamard transform.

Each is checked against something other than itself: LAPACK (scipy) for the
eigen-decomposition and QR, SplitMix64's published output sequence for the
counter hash, and the explicit Sylvester Hadamard matrix for the transform.
"""
import numpy as np
import pytest
import scipy.linalg as sla

from oracle import linalg, rng, wht


def _spd(n, m, seed):
    G = np.random.default_rng(seed).standard_normal((n, m))
    return G @ G.T


@pytest.mark.parametrize("n", [1, 2, 7, 64, 65, 138])
def test_jacobi_matches_lapack(n):
    G = _spd(n, n + 40, n)
    lam, V = linalg.eigh_desc(G)
    w, Vl = sla.eigh(G)
    w, Vl = w[::-1], Vl[:, ::-1]
    nrm = np.linalg.norm(G)
    assert np.max(np.abs(lam - w)) <= 1e-12 * nrm
    assert np.linalg.norm(G @ V - V * lam) <= 1e-12 * nrm
    assert np.max(np.abs(V.T @ V - np.eye(n))) <= 1e-13
    # eigenvectors agree with LAPACK's where the gap is not tiny
    for i in range(n):
        gap = min([abs(w[i] - w[j]) for j in range(n) if j != i] or [np.inf])
        if gap >= 1e-6 * w[0]:
            v, u = V[:, i], Vl[:, i]
            sin = np.linalg.norm(v - (v @ u) * u)
            assert sin <= 1e-10


def test_jacobi_indefinite_and_degenerate():
    # an indefinite matrix with a repeated eigenvalue: eigenvalues still exact,
    # and the repeated pair spans the right 2-dimensional space
    Q = linalg.orth(np.random.default_rng(3).standard_normal((6, 6)))
    w = np.array([5.0, 2.0, 2.0, -1.0, -3.0, 0.0])
    G = Q @ np.diag(w) @ Q.T
    lam, V = linalg.eigh_desc(G)
    assert np.allclose(lam, np.sort(w)[::-1], atol=1e-13)
    P = V[:, 1:3] @ V[:, 1:3].T
    Pref = Q[:, 1:3] @ Q[:, 1:3].T
    assert np.max(np.abs(P - Pref)) <= 1e-12


def test_sign_normalization_rule():
    V = np.array([[0.6, -0.8], [-0.8, 0.6]])
    S = linalg.sign_normalize(V)
    assert np.array_equal(S, np.array([[-0.6, 0.8], [0.8, -0.6]]))
    T = linalg.sign_normalize(np.array([[-0.5], [0.5]]))   # tie -> lowest index positive
    assert T[0, 0] == 0.5 and T[1, 0] == -0.5


@pytest.mark.parametrize("m,k", [(5, 5), (40, 7), (300, 33)])
def test_householder_qr(m, k):
    Y = np.random.default_rng(m * k).standard_normal((m, k))
    Q, R = linalg.householder_qr(Y)
    assert np.max(np.abs(Q @ R - Y)) <= 1e-13 * np.max(np.abs(Y)) * k
    assert np.max(np.abs(Q.T @ Q - np.eye(k))) <= 1e-13
    assert np.allclose(np.tril(R, -1), 0.0)
    assert np.all(np.diag(R) >= 0)
    # LAPACK's QR, made unique by the same sign rule, is the same factorisation
    Ql, Rl = np.linalg.qr(Y)
    s = np.sign(np.diag(Rl))
    assert np.max(np.abs(Q - Ql * s)) <= 1e-12
    assert np.max(np.abs(R - Rl * s[:, None])) <= 1e-12 * np.max(np.abs(Y)) * k


def test_splitmix64_published_sequence():
    # SplitMix64 seeded with 0 returns mix64(gamma * i), i = 1, 2, 3, ...
    # (Steele, Lea & Flood 2014; gamma = 0x9E3779B97F4A7C15)
    g = 0x9E3779B97F4A7C15
    got = [rng.mix64_int((i * g) & rng.MASK) for i in (1, 2, 3)]
    assert got == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    arr = rng.mix64_array(np.array([g, 2 * g % (1 << 64)], dtype=np.uint64))
    assert [int(v) for v in arr] == got[:2]


def test_rademacher_streams():
    s0 = rng.rademacher(7, 3, 0, np.arange(1 << 16, dtype=np.uint64))
    s1 = rng.rademacher(7, 3, 1, np.arange(1 << 16, dtype=np.uint64))
    s2 = rng.rademacher(7, 4, 0, np.arange(1 << 16, dtype=np.uint64))
    assert set(np.unique(s0)) == {-1.0, 1.0}
    assert abs(s0.mean()) < 0.02 and abs(s1.mean()) < 0.02
    assert abs(np.mean(s0 * s1)) < 0.02 and abs(np.mean(s0 * s2)) < 0.02
    # the sign is bit 63 of the hashed counter
    key = rng.item_key(7, 3)
    w = rng.mix64_int((key + 5) & rng.MASK)
    assert s0[5] == (-1.0 if w >> 63 else 1.0)
    om = rng.sketch_matrix(7, 3, 4, 3)
    w = rng.mix64_int((key + (1 << 56) + 2 * 3 + 1) & rng.MASK)
    assert om[2, 1] == (-1.0 if w >> 63 else 1.0)


@pytest.mark.parametrize("d", [1, 2, 8, 64, 128])
def test_fwht_is_sylvester_hadamard(d):
    x = np.random.default_rng(d).standard_normal((5, d))
    H = sla.hadamard(d)
    assert np.max(np.abs(wht.fwht(x) - x @ H.T)) <= 1e-12 * d


@pytest.mark.parametrize("d", [64, 128])
def test_rotation_norm_and_inverse(d):
    x = np.random.default_rng(d).standard_normal((100, d))
    s = rng.rotation_signs(11, 2, d)
    y = wht.rotate(x, s)
    assert np.max(np.abs(np.linalg.norm(y, axis=1) / np.linalg.norm(x, axis=1) - 1)) <= 1e-14
    assert np.max(np.abs(wht.unrotate(y, s) - x)) <= 1e-14 * np.max(np.abs(x)) * 8
