"""ORACLE (test infrastructure only): eigensolver wrapper and Householder QR, fp64.

Sources: the paper landing page ("A JoLT for the KV cache", abstract) fixes a
partial Tucker decomposition along the token and feature modes with an exact
token-mode SVD, and a randomized approximation of it (FlashJoLT).  Both factor
computations reduce to symmetric eigenproblems and thin QR factorisations:
  * the left singular vectors of the token unfolding A are the eigenvectors of
    A A^T, ranked by lambda = sigma^2;
  * the randomized range finder needs an orthonormal basis of a tall sketch.
"""
from __future__ import annotations

import numpy as np

from ._native import jacobi_raw


def sign_normalize(V: np.ndarray) -> np.ndarray:
    """Flip each column so its largest-magnitude entry is positive.

    Ties in magnitude go to the lowest row index (np.argmax returns the first).
    """
    V = np.array(V, dtype=np.float64, copy=True)
    if V.size == 0:
        return V
    idx = np.argmax(np.abs(V), axis=0)
    sgn = np.sign(V[idx, np.arange(V.shape[1])])
    sgn[sgn == 0] = 1.0
    return V * sgn[None, :]


def eigh_desc(G: np.ndarray, max_sweeps: int = 60, tol: float = 1e-15):
    """Eigen-decomposition of symmetric G by cyclic Jacobi.

    Returns (lam, V): eigenvalues in descending order and the matching
    orthonormal eigenvectors as columns, each column sign-normalised.
    """
    G = np.asarray(G, dtype=np.float64)
    G = 0.5 * (G + G.T)
    w, V, sweeps = jacobi_raw(G, max_sweeps=max_sweeps, tol=tol)
    if sweeps < 0:
        raise RuntimeError("oracle Jacobi did not converge in %d sweeps" % max_sweeps)
    order = np.argsort(-w, kind="stable")
    return w[order], sign_normalize(V[:, order])


def householder_qr(Y: np.ndarray):
    """Thin QR of a tall matrix by Householder reflections, R_ii >= 0.

    For j = 0..k-1 the reflector H_j = I - 2 v v^T maps column j of the
    current trailing block onto a multiple of e_j; Q = H_0 H_1 ... H_{k-1}
    restricted to the first k columns.  Finally the signs of R's diagonal are
    made non-negative (columns of Q flipped to match).
    """
    Y = np.asarray(Y, dtype=np.float64)
    m, k = Y.shape
    if m < k:
        raise ValueError("householder_qr needs a tall matrix")
    R = Y.copy()
    vs = []
    for j in range(k):
        x = R[j:, j]
        nx = np.linalg.norm(x)
        if nx == 0.0:
            vs.append(None)
            continue
        alpha = -nx if x[0] >= 0 else nx
        v = x.copy()
        v[0] -= alpha
        nv = np.linalg.norm(v)
        if nv == 0.0:
            vs.append(None)
            continue
        v /= nv
        R[j:, j:] -= 2.0 * np.outer(v, v @ R[j:, j:])
        vs.append(v)
    Q = np.zeros((m, k))
    Q[np.arange(k), np.arange(k)] = 1.0
    for j in range(k - 1, -1, -1):
        v = vs[j]
        if v is None:
            continue
        Q[j:, :] -= 2.0 * np.outer(v, v @ Q[j:, :])
    R = np.triu(R[:k, :])
    d = np.sign(np.diag(R))
    d[d == 0] = 1.0
    return Q * d[None, :], R * d[:, None]


def orth(Y: np.ndarray) -> np.ndarray:
    """Orthonormal basis of range(Y): the Q factor of Householder QR."""
    return householder_qr(Y)[0]
