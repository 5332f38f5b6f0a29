"""GPU parity of the plan's symmetric eigensolver (jolt_eigh hook) with the
oracle's fp64 Jacobi eigensolver.

Both solvers the library carries are covered: the Householder-tridiagonal one
(bisection + twisted-factorization vectors + Newton-Schulz steps), for
n <= 140 with the matrix in LDS and for 140 < n <= 272 with it in registers,
and the two-sided Jacobi one (forced, up to n = 142, and as the hand-back for
numerically repeated eigenvalues at n <= 140).  Matrices: the token Gram W = B B^T of the
FlashJoLT sketch and the feature Gram of Mistral-7B-shaped synthetic items,
random symmetric, rank-deficient, clustered and degenerate ones.

Tolerances (fp32 arithmetic on matrices with ||A||_2 = s):
  eigenvalues      |lam - lam_ref| <= 2e-5 s   (a few hundred fp32 ulps of s)
  residual         ||A v - lam v|| <= 2e-5 s per column
  orthonormality   max |V^T V - I| <= 1e-4
  subspace         sin angle <= 1e-2 between leading subspaces wherever the
                   eigengap exceeds 1e-3 lam_1
"""
import numpy as np
import pytest

import synth
from oracle import linalg as olin
from oracle import tucker as otuck
from tests.gpu_util import jolt_binding, torch_cuda

pytestmark = pytest.mark.gpu


def _run(mats, force_jacobi=False):
    torch = torch_cuda()
    jb = jolt_binding()
    n = mats[0].shape[0]
    count = len(mats)
    a = torch.from_numpy(np.stack(mats).astype(np.float32)).cuda()
    vec = torch.empty((count, n, n), dtype=torch.float32, device="cuda")
    lam = torch.empty((count, n), dtype=torch.float32, device="cuda")
    info = torch.full((count,), 99, dtype=torch.int32, device="cuda")
    wsb = jb.jolt_eigh_workspace_size(n, count, force_jacobi)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
    h = jb.jolt_create()
    try:
        jb.jolt_eigh(h, n, count, a.data_ptr(), n, n * n, vec.data_ptr(), lam.data_ptr(), info.data_ptr(),
                     force_jacobi, ws.data_ptr(), wsb, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
    finally:
        jb.jolt_destroy(h)
    return vec.cpu().numpy().astype(np.float64), lam.cpu().numpy().astype(np.float64), info.cpu().numpy()


def _check(M, V, lam, tag):
    M = np.asarray(M, dtype=np.float32).astype(np.float64)      # what the device received
    M = 0.5 * (M + M.T)
    ref_lam, ref_V = olin.eigh_desc(M)
    s = max(abs(ref_lam[0]), abs(ref_lam[-1]), 1e-30)
    n = M.shape[0]
    assert np.all(np.diff(lam) <= 0), tag + ": eigenvalues not descending"
    assert np.max(np.abs(lam - ref_lam)) <= 2e-5 * s, (tag, np.max(np.abs(lam - ref_lam)) / s)
    res = np.linalg.norm(M @ V - V * lam, axis=0)
    assert res.max() <= 2e-5 * s, (tag, res.max() / s)
    assert np.max(np.abs(V.T @ V - np.eye(n))) <= 1e-4, tag
    for r in range(1, n):
        if ref_lam[r - 1] - ref_lam[r] > 1e-3 * abs(ref_lam[0]):
            sine = np.linalg.norm(ref_V[:, r:].T @ V[:, :r], 2)
            assert sine <= 1e-2, (tag, r, sine)
    # sign convention: largest-magnitude entry (first such row) positive
    best = np.argmax(np.abs(V), axis=0)
    assert np.all(V[best, np.arange(n)] > 0), tag


def _sketch_grams(cfg, count):
    """Token Gram B B^T of the q = 1 randomized range finder and the feature
    Gram, built in fp64 by the oracle, for `count` synthetic items."""
    out_w, out_g = [], []
    for it in synth.make_items(cfg, count):
        A = otuck.unfold_token(it.x)
        k = cfg.rt_max + cfg.oversample
        rng = np.random.default_rng(it.seed)
        Y = A @ rng.standard_normal((A.shape[1], k))
        Q = np.linalg.qr(Y)[0]
        Q = np.linalg.qr(A @ np.linalg.qr(A.T @ Q)[0])[0]
        B = Q.T @ A
        out_w.append(B @ B.T)
        out_g.append(otuck.feature_gram(it.x))
    return out_w, out_g


@pytest.mark.parametrize("force_jacobi", [False, True])
def test_sketch_and_feature_grams(force_jacobi):
    cfg = synth.config("mistral7b_gqa_1k", L=2, H=4, T=512)
    W, G = _sketch_grams(cfg, 3)
    for mats, tag in ((W, "token W"), (G, "feature G")):
        V, lam, info = _run(mats, force_jacobi)
        if force_jacobi:
            assert np.all(info > 0), info
        else:
            assert np.all(info == 0), info          # the tridiagonal solver kept them
        for i, M in enumerate(mats):
            _check(M, V[i], lam[i], "%s %d jacobi=%d" % (tag, i, force_jacobi))


@pytest.mark.parametrize("n", [1, 2, 3, 31, 64, 97, 128, 140])
def test_random_symmetric_sizes(n):
    rng = np.random.default_rng(1000 + n)
    mats = []
    for _ in range(3):
        B = rng.standard_normal((n, n))
        mats.append(0.5 * (B + B.T))
    V, lam, info = _run(mats)
    for i, M in enumerate(mats):
        _check(M, V[i], lam[i], "random n=%d #%d" % (n, i))


@pytest.mark.parametrize("n", [141, 142])
def test_jacobi_sizes(n):
    """The largest orders the Jacobi solver takes (forced), and the wide
    tridiagonal solver on the same matrices."""
    rng = np.random.default_rng(n)
    B = rng.standard_normal((n, 2 * n))
    M = B @ B.T
    V, lam, info = _run([M], force_jacobi=True)
    assert info[0] > 0
    _check(M, V[0], lam[0], "jacobi n=%d" % n)
    V, lam, info = _run([M])
    assert info[0] == 0
    _check(M, V[0], lam[0], "wide n=%d" % n)


def test_rank_deficient_and_graded():
    rng = np.random.default_rng(7)
    mats = []
    G = rng.standard_normal((138, 5))
    mats.append(G @ G.T)                                          # rank 5
    U = np.linalg.qr(rng.standard_normal((138, 138)))[0]
    mats.append(U @ np.diag(0.8 ** np.arange(138)) @ U.T)        # graded spectrum
    mats.append(U @ np.diag(np.r_[np.linspace(100, 10, 20), 1 + 1e-3 * rng.standard_normal(118)]) @ U.T)
    V, lam, info = _run(mats)
    for i, M in enumerate(mats):
        _check(M, V[i], lam[i], "structured %d" % i)


def test_repeated_eigenvalues_fall_back_to_jacobi():
    rng = np.random.default_rng(3)
    U = np.linalg.qr(rng.standard_normal((60, 60)))[0]
    ev = np.r_[[10.0] * 5, [1.0] * 10, np.linspace(0.5, 0.1, 45)]
    mats = [U @ np.diag(ev) @ U.T, np.eye(60), np.zeros((60, 60)), np.diag(np.r_[[3.0] * 30, [1.0] * 30])]
    V, lam, info = _run(mats)
    assert np.all(info != -1), info
    for i, M in enumerate(mats):
        _check(M, V[i], lam[i], "repeated %d" % i)


# ---------------------------------------------------------------- the wide solver (140 < n <= 272)
@pytest.mark.parametrize("n", [143, 160, 200, 266, 272])
def test_wide_random_sizes(n):
    rng = np.random.default_rng(2000 + n)
    mats = []
    for _ in range(3):
        B = rng.standard_normal((n, n))
        mats.append(0.5 * (B + B.T))
    V, lam, info = _run(mats)
    assert np.all(info == 0), info
    for i, M in enumerate(mats):
        _check(M, V[i], lam[i], "wide random n=%d #%d" % (n, i))


def test_wide_sketch_gram_k266():
    """Token Gram W = B B^T of a k = 266 sketch (rank limit 256 + 10)."""
    cfg = synth.config("moe_gqa_batch16_8k", L=2, H=4, T=1024, rank_t=150)
    W, G = _sketch_grams(cfg, 2)
    assert W[0].shape == (266, 266)
    V, lam, info = _run(W)
    assert np.all(info == 0), info
    for i, M in enumerate(W):
        _check(M, V[i], lam[i], "wide token W %d" % i)


def test_wide_structured():
    rng = np.random.default_rng(17)
    n = 266
    mats = []
    G = rng.standard_normal((n, 5))
    mats.append(G @ G.T)                                          # rank 5
    U = np.linalg.qr(rng.standard_normal((n, n)))[0]
    mats.append(U @ np.diag(0.9 ** np.arange(n)) @ U.T)          # graded spectrum
    mats.append(U @ np.diag(np.r_[np.linspace(100, 10, 40), 1 + 1e-3 * rng.standard_normal(n - 40)]) @ U.T)
    V, lam, info = _run(mats)
    # the rank-deficient matrix (261 zero eigenvalues) and the tight cluster are
    # flagged (jolt_plan re-plans such items with block Jacobi); the rest pass
    assert info[1] == 0 and np.all((info == 0) | (info == -3)), info
    for i, M in enumerate(mats):
        if info[i] == 0:
            _check(M, V[i], lam[i], "wide structured %d" % i)


def test_wide_repeated_eigenvalues_flagged_or_exact():
    """Exactly repeated eigenvalues: the wide solver has no Jacobi hand-back, so
    each matrix is either solved to the usual tolerances (info 0) or reported
    with info -3."""
    rng = np.random.default_rng(5)
    n = 200
    U = np.linalg.qr(rng.standard_normal((n, n)))[0]
    ev = np.r_[[10.0] * 5, [1.0] * 10, np.linspace(0.5, 0.1, n - 15)]
    mats = [U @ np.diag(ev) @ U.T, np.eye(n), np.diag(np.r_[[3.0] * 100, [1.0] * 100])]
    V, lam, info = _run(mats)
    assert np.all((info == 0) | (info == -3)), info
    for i, M in enumerate(mats):
        if info[i] == 0:
            _check(M, V[i], lam[i], "wide repeated %d" % i)
