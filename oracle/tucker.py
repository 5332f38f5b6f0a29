"""ORACLE (test infrastructure only): partial Tucker factors, core and energies.

Pages (paper landing page, abstract; author page abstract; vendor page): a
grouped prefill cache is a fourth-order tensor X[layer][head][token][feature];
JoLT applies a partial Tucker decomposition along the token and feature modes
only, leaving the head and layer modes intact.  FlashJoLT replaces the exact
token-mode SVD with a randomized approximation.

Readings (where the pages are silent):
  * truncated HOSVD: both factors come from X itself (no HOOI iterations);
  * the token factor is shared by all layers and heads of the group, and so
    is the feature factor; the core is per (layer, head);
  * factors are sorted by eigenvalue, so the core for ranks (r_t, r_f) is the
    leading block of the full core, and the truncation energy is exact.
"""
from __future__ import annotations

import numpy as np

from .linalg import eigh_desc, orth, sign_normalize
from .rng import sketch_matrix


def unfold_token(X: np.ndarray) -> np.ndarray:
    """A = unfold_t(X): T x (L*H*d), column index (l*H + h)*d + f."""
    L, H, T, d = X.shape
    return X.transpose(2, 0, 1, 3).reshape(T, L * H * d)


def feature_gram(X: np.ndarray) -> np.ndarray:
    """G_f = sum over (layer, head, token) of x x^T  (d x d)."""
    d = X.shape[-1]
    F = X.reshape(-1, d)
    return F.T @ F


def feature_factor(X: np.ndarray):
    """(lambda_f, U_f): all d eigenpairs of G_f, descending."""
    return eigh_desc(feature_gram(X))


def token_factor_exact(X: np.ndarray, rt_max: int):
    """Exact token factor: leading eigenvectors of G_t = A A^T (T x T).

    The left singular vectors of A are the eigenvectors of A A^T, ranked by
    lambda = sigma^2.
    """
    A = unfold_token(X)
    lam, U = eigh_desc(A @ A.T)
    return lam[:rt_max], U[:, :rt_max]


def token_factor_randomized(X: np.ndarray, rt_max: int, oversample: int,
                            power_iters: int, seed: int, item_id: int):
    """FlashJoLT token factor: randomized range finder + small SVD.

    Halko, Martinsson & Tropp (SIAM Review 2011), Alg. 4.4 (randomized
    subspace iteration) followed by Alg. 5.1 (direct SVD of B = Q^T A):
      k = rt_max + oversample;  Omega: seeded Rademacher n x k
      Y = A Omega;  Q = orth(Y)
      repeat power_iters times:  Q = orth(A orth(A^T Q))
      B = Q^T A;  W = B B^T = U~ Lambda U~^T;  U_t = Q U~[:, :rt_max]
    """
    A = unfold_token(X)
    T, n = A.shape
    k = rt_max + oversample
    Omega = sketch_matrix(seed, item_id, n, k)
    Q = orth(A @ Omega)
    for _ in range(power_iters):
        Z = orth(A.T @ Q)
        Q = orth(A @ Z)
    B = Q.T @ A
    lam, Ut = eigh_desc(B @ B.T)
    U = Q @ Ut[:, :rt_max]
    return lam[:rt_max], sign_normalize(U)


def core_full(X: np.ndarray, U_t: np.ndarray, U_f: np.ndarray) -> np.ndarray:
    """C_full[l, h] = U_t^T X[l, h] U_f   (rt_max x rf_max per (layer, head))."""
    return np.matmul(np.matmul(U_t.T[None, None], X), U_f[None, None])


def energy_table(C: np.ndarray) -> np.ndarray:
    """E[i, j] = sum over (layer, head) of C[l, h, i, j]^2."""
    return np.sum(C * C, axis=(0, 1))


def captured_energy(E: np.ndarray, rt: int, rf: int) -> float:
    """S(r_t, r_f) = sum of E over the leading r_t x r_f block."""
    if rt == 0 or rf == 0:
        return 0.0
    return float(np.sum(E[:rt, :rf]))
