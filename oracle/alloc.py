"""ORACLE (test infrastructure only): byte accounting, distortion model and the
single-Lagrangian-dual allocation of (token rank, feature rank, residual bits).

Pages: a single Lagrangian dual allocates the Tucker ranks and the residual
bit-widths together, per layer group and separately for keys and values, under
one byte budget (author page abstract; landing page abstract: "a single
Lagrangian dual allocates per-group Tucker ranks and residual bit-widths under a
global byte constraint"; podcast, "The Core Mechanism": no pre-split K/V
budgets, bits move between the K and V sides).

Readings:
  * items are (sequence, layer group, K|V); all items share one lambda;
  * candidates: r_t in {0, step, .., rt_max}, r_f in {0, step, .., rf_max},
    b in the allowed set; r_t = 0 or r_f = 0 means no Tucker part (both 0);
  * bytes(r_t, r_f, b) = e (T r_t + d r_f + L H r_t r_f) + [b > 0] (N b / 8 + 2 N / 64)
    with e the parameter element size (2 for bf16, 4 for fp32) and N = L H T d;
  * distortion D = delta_b * max(0, ||X||^2 - S(r_t, r_f)), delta_0 = 1, where
    delta_b is the relative MSE of the b-bit quantizer on Gaussian groups (the
    JL rotation makes the residual close to Gaussian);
  * A(lambda) = per item argmin of D + lambda * bytes, ties to fewer bytes, then
    smaller r_t, r_f, b; lambda* = the least lambda >= 0 with total bytes of
    A(lambda) <= budget.  Evaluated here in exact rational arithmetic on the
    fp64 / int64 table entries.
"""
from __future__ import annotations

import itertools
from fractions import Fraction
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np


def candidate_grid(rt_max: int, rf_max: int, step: int, bits: Sequence[int]) -> np.ndarray:
    """Distinct candidates (r_t, r_f, b), sorted; (0, 0, b) stands for 'no Tucker part'."""
    out = set()
    for b in bits:
        out.add((0, 0, int(b)))
        for rt in range(step, rt_max + 1, step):
            for rf in range(step, rf_max + 1, step):
                out.add((rt, rf, int(b)))
    return np.array(sorted(out), dtype=np.int64).reshape(-1, 3)


def item_bytes(L: int, H: int, T: int, d: int, e: int, rt: int, rf: int, b: int) -> int:
    if rt == 0 or rf == 0:
        rt = rf = 0
    N = L * H * T * d
    params = e * (T * rt + d * rf + L * H * rt * rf)
    resid = (N * b // 8 + 2 * N // 64) if b > 0 else 0
    return int(params + resid)


def bytes_table(L, H, T, d, e, cand: np.ndarray) -> np.ndarray:
    return np.array([item_bytes(L, H, T, d, e, int(rt), int(rf), int(b)) for rt, rf, b in cand],
                    dtype=np.int64)


def distortion_table(E: np.ndarray, normX2: float, delta: Sequence[float],
                     cand: np.ndarray) -> np.ndarray:
    """D(r_t, r_f, b) = delta_b * max(0, ||X||^2 - S(r_t, r_f)) in fp64."""
    P = np.cumsum(np.cumsum(np.asarray(E, dtype=np.float64), axis=0), axis=1)
    out = np.empty(len(cand), dtype=np.float64)
    for i, (rt, rf, b) in enumerate(cand):
        S = 0.0 if (rt == 0 or rf == 0) else float(P[rt - 1, rf - 1])
        out[i] = float(delta[b]) * max(0.0, normX2 - S)
    return out


# --------------------------------------------------------------------------
# exact Lagrangian allocation
# --------------------------------------------------------------------------
def _key(D: Fraction, lam: Fraction, B: int, c) -> tuple:
    return (D + lam * B, B, int(c[0]), int(c[1]), int(c[2]))


def argmin_at(lam: Fraction, cand: np.ndarray, D: np.ndarray, B: np.ndarray) -> int:
    """Index of A(lambda) for one item, exact, with the stated tie-breaks."""
    Df = [Fraction(float(x)) for x in D]
    best = None
    bi = -1
    for i in range(len(cand)):
        k = _key(Df[i], lam, int(B[i]), cand[i])
        if best is None or k < best:
            best, bi = k, i
    return bi


def lower_hull(cand: np.ndarray, D: np.ndarray, B: np.ndarray) -> List[int]:
    """Candidates that A(lambda) can return for some lambda >= 0, by bytes ascending.

    Keep, for each byte count, the best (D, r_t, r_f, b); keep only points whose
    D strictly decreases as bytes grow; then the lower convex hull with
    collinear middle points removed (at a tie the fewer-bytes end wins).
    """
    Df = [Fraction(float(x)) for x in D]
    order = sorted(range(len(cand)),
                   key=lambda i: (int(B[i]), Df[i], int(cand[i][0]), int(cand[i][1]), int(cand[i][2])))
    stair: List[int] = []
    for i in order:
        if stair and int(B[stair[-1]]) == int(B[i]):
            continue
        if stair and not (Df[i] < Df[stair[-1]]):
            continue
        stair.append(i)
    hull: List[int] = []
    for i in stair:
        while len(hull) >= 2:
            o, a = hull[-2], hull[-1]
            cross = (int(B[a]) - int(B[o])) * (Df[i] - Df[o]) - (Df[a] - Df[o]) * (int(B[i]) - int(B[o]))
            if cross <= 0:
                hull.pop()
            else:
                break
        hull.append(i)
    return hull


def _breakpoints(hull: List[int], D: np.ndarray, B: np.ndarray) -> List[Fraction]:
    """s_j = (D_j - D_{j+1}) / (B_{j+1} - B_j) between consecutive hull vertices."""
    out = []
    for j in range(len(hull) - 1):
        a, b = hull[j], hull[j + 1]
        out.append((Fraction(float(D[a])) - Fraction(float(D[b]))) / (int(B[b]) - int(B[a])))
    return out


def _vertex_at(hull: List[int], bps: List[Fraction], lam: Fraction) -> int:
    """Hull vertex chosen at lambda: v_J with J = #{j : s_j > lambda}."""
    J = sum(1 for s in bps if s > lam)
    return hull[J]


def lagrangian_allocate(tables: List[Dict], budget: int):
    """Single dual over all items.

    tables[i] = {"cand": (C,3) int, "D": (C,) fp64, "B": (C,) int64}.
    Returns (choice indices, lambda* as Fraction or None if infeasible,
    feasible flag).  When infeasible the minimum-byte choices are returned.
    """
    hulls, bps = [], []
    for t in tables:
        h = lower_hull(t["cand"], t["D"], t["B"])
        hulls.append(h)
        bps.append(_breakpoints(h, t["D"], t["B"]))

    def total(lam: Fraction) -> int:
        return sum(int(t["B"][_vertex_at(h, s, lam)]) for t, h, s in zip(tables, hulls, bps))

    min_total = sum(int(t["B"][h[0]]) for t, h in zip(tables, hulls))
    if min_total > budget:
        return [h[0] for h in hulls], None, False
    lam = Fraction(0)
    if total(lam) > budget:
        slopes = sorted(set(s for ss in bps for s in ss))
        lo, hi = 0, len(slopes) - 1          # total(slopes[-1]) == min_total <= budget
        while lo < hi:
            mid = (lo + hi) // 2
            if total(slopes[mid]) <= budget:
                hi = mid
            else:
                lo = mid + 1
        lam = slopes[lo]
    choice = [_vertex_at(h, s, lam) for h, s in zip(hulls, bps)]
    return choice, lam, True


def exhaustive_allocate(tables: List[Dict], budget: int):
    """Constrained optimum by enumeration (tiny grids only).

    Minimises total D subject to total bytes <= budget; ties to fewer total
    bytes.  Returns (choice indices, total D) or (None, None) if infeasible.
    """
    best = None
    best_choice = None
    for combo in itertools.product(*[range(len(t["cand"])) for t in tables]):
        Bt = sum(int(t["B"][c]) for t, c in zip(tables, combo))
        if Bt > budget:
            continue
        Dt = sum(Fraction(float(t["D"][c])) for t, c in zip(tables, combo))
        key = (Dt, Bt)
        if best is None or key < best:
            best, best_choice = key, combo
    if best is None:
        return None, None
    return list(best_choice), best[0]
