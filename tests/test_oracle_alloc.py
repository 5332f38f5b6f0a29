"""Pins for the oracle's byte accounting and single-dual allocation.

The Lagrangian allocation is checked against brute force: the per-lambda
argmin over every candidate, and the exhaustive constrained optimum over tiny
grids.  At budgets equal to the bytes of some A(lambda) (hull vertices) the
Lagrangian solution is optimal, so the two distortions agree exactly; at other
budgets it is feasible and no better than the optimum.
"""
import itertools
from fractions import Fraction

import numpy as np
import pytest

from oracle import alloc


def _rand_tables(n_items, n_cand, seed):
    rg = np.random.default_rng(seed)
    tabs = []
    for i in range(n_items):
        cand = np.array([(k, 0, 0) for k in range(n_cand)], dtype=np.int64)
        B = rg.integers(10, 200, n_cand).astype(np.int64)
        D = rg.uniform(0, 100, n_cand)
        tabs.append({"cand": cand, "B": B, "D": D})
    return tabs


def _totals(tabs, choice):
    return (sum(int(t["B"][c]) for t, c in zip(tabs, choice)),
            sum(Fraction(float(t["D"][c])) for t, c in zip(tabs, choice)))


def test_candidate_grid_counts():
    assert len(alloc.candidate_grid(128, 128, 8, (0, 2, 3, 4))) == 1028
    assert len(alloc.candidate_grid(256, 128, 8, (0, 2, 3, 4))) == 2052
    g = alloc.candidate_grid(16, 16, 8, (0, 4))
    assert [tuple(r) for r in g] == [(0, 0, 0), (0, 0, 4), (8, 8, 0), (8, 8, 4), (8, 16, 0),
                                     (8, 16, 4), (16, 8, 0), (16, 8, 4), (16, 16, 0), (16, 16, 4)]


def test_bytes_formula_by_counting():
    # count stored elements explicitly: U_t (T x rt), U_f (d x rf), core (L H rt rf),
    # residual codes (b bits per element) and one bf16 scale per 64 elements
    L, H, T, d = 2, 3, 40, 64
    N = L * H * T * d
    for e in (2, 4):
        for rt, rf, b in [(0, 0, 0), (0, 0, 4), (8, 16, 0), (16, 8, 2), (24, 64, 3), (0, 16, 4)]:
            ut = np.zeros((T, rt if rf else 0)); uf = np.zeros((d, rf if rt else 0))
            core = np.zeros((L, H, ut.shape[1], uf.shape[1]))
            n_codes_bits = N * b if b else 0
            n_scales = N // 64 if b else 0
            expect = e * (ut.size + uf.size + core.size) + n_codes_bits // 8 + 2 * n_scales
            assert alloc.item_bytes(L, H, T, d, e, rt, rf, b) == expect


@pytest.mark.parametrize("seed", range(6))
def test_per_lambda_argmin_is_brute_force(seed):
    tabs = _rand_tables(3, 12, seed)
    for t in tabs:
        hull = alloc.lower_hull(t["cand"], t["D"], t["B"])
        bps = alloc._breakpoints(hull, t["D"], t["B"])
        lams = [Fraction(0)] + bps + [b + Fraction(1, 7) for b in bps] + [b - Fraction(1, 1000) for b in bps]
        for lam in lams:
            if lam < 0:
                continue
            assert alloc._vertex_at(hull, bps, lam) == alloc.argmin_at(lam, t["cand"], t["D"], t["B"])


@pytest.mark.parametrize("seed", range(8))
def test_lagrangian_vs_exhaustive(seed):
    tabs = _rand_tables(3, 5, 100 + seed)
    min_b = sum(int(t["B"].min()) for t in tabs)
    max_b = sum(int(t["B"].max()) for t in tabs)
    # hull-vertex budgets: the bytes of A(lambda) at every breakpoint
    vertex_budgets = set()
    for t in tabs:
        h = alloc.lower_hull(t["cand"], t["D"], t["B"])
        for lam in [Fraction(0)] + alloc._breakpoints(h, t["D"], t["B"]):
            ch = [alloc.argmin_at(lam, u["cand"], u["D"], u["B"]) for u in tabs]
            vertex_budgets.add(_totals(tabs, ch)[0])
    prev_D = None
    for budget in sorted(set(range(min_b - 5, max_b + 5, 7)) | vertex_budgets):
        choice, lam, ok = alloc.lagrangian_allocate(tabs, budget)
        opt, Dopt = alloc.exhaustive_allocate(tabs, budget)
        if budget < min_b:
            assert not ok and opt is None
            continue
        assert ok
        Bt, Dt = _totals(tabs, choice)
        assert Bt <= budget
        assert Dt >= Dopt
        if budget in vertex_budgets:
            assert Dt == Dopt
        # the returned choice is the direct argmin at lambda*
        assert choice == [alloc.argmin_at(lam, t["cand"], t["D"], t["B"]) for t in tabs]
        # lambda* is the least feasible lambda: just below it the budget is exceeded
        if lam > 0:
            below = lam - Fraction(1, 10 ** 12)
            ch = [alloc.argmin_at(below, t["cand"], t["D"], t["B"]) for t in tabs]
            assert _totals(tabs, ch)[0] > budget
        if budget >= min_b and prev_D is not None:
            pass
    # distortion is non-increasing in the budget
    Ds = []
    for budget in range(min_b, max_b + 1, 3):
        choice, lam, ok = alloc.lagrangian_allocate(tabs, budget)
        Ds.append(_totals(tabs, choice)[1])
    assert all(a >= b for a, b in zip(Ds, Ds[1:]))


def test_joint_dual_beats_pre_split():
    # K-like item: rank is cheap and valuable; V-like: bits are.  At hull budgets
    # the single dual is at least as good as any split of the budget.
    cand = np.array(list(itertools.product([0, 8, 16], [0], [0, 2, 4])), dtype=np.int64)
    rg = np.random.default_rng(9)
    tabs = []
    for _ in range(2):
        B = np.array([1 + 50 * r + 30 * b for r, _, b in cand], dtype=np.int64)
        D = np.array([100.0 / (1 + r) / (1 + b * b) for r, _, b in cand]) * rg.uniform(0.5, 2.0)
        tabs.append({"cand": cand, "B": B, "D": D})
    for t in tabs:
        h = alloc.lower_hull(t["cand"], t["D"], t["B"])
    budgets = set()
    for lam in [Fraction(x, 10) for x in range(0, 200)]:
        ch = [alloc.argmin_at(lam, t["cand"], t["D"], t["B"]) for t in tabs]
        budgets.add(_totals(tabs, ch)[0])
    for budget in budgets:
        choice, lam, ok = alloc.lagrangian_allocate(tabs, budget)
        Dj = _totals(tabs, choice)[1]
        for split in range(0, budget + 1):
            best = []
            for t, cap in zip(tabs, (split, budget - split)):
                feas = [i for i in range(len(cand)) if int(t["B"][i]) <= cap]
                if not feas:
                    break
                best.append(min(Fraction(float(t["D"][i])) for i in feas))
            if len(best) == 2:
                assert Dj <= best[0] + best[1]


def test_infeasible_returns_min_bytes():
    tabs = _rand_tables(2, 6, 5)
    min_b = sum(int(t["B"].min()) for t in tabs)
    choice, lam, ok = alloc.lagrangian_allocate(tabs, min_b - 1)
    assert not ok and lam is None
    assert [int(t["B"][c]) for t, c in zip(tabs, choice)] == [int(t["B"].min()) for t in tabs]


def test_distortion_table_definition():
    E = np.arange(1, 13, dtype=np.float64).reshape(3, 4)
    cand = np.array([(0, 0, 0), (0, 0, 4), (1, 1, 0), (2, 3, 2), (3, 4, 4)], dtype=np.int64)
    delta = [1.0, None, 0.5, 0.1, 0.01]
    D = alloc.distortion_table(E, 100.0, delta, cand)
    assert D.tolist() == [100.0, 1.0, 99.0, 0.5 * (100 - (1 + 2 + 3 + 5 + 6 + 7)), 0.01 * max(0, 100 - 78)]
