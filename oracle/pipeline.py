"""ORACLE (test infrastructure only): the whole compress / decompress path per item.

Step order follows the landing page abstract: partial Tucker factors (exact
token-mode eigensolve, or the FlashJoLT randomized approximation) -> core ->
single-dual allocation of (r_t, r_f, b) under one byte budget -> stored
parameters -> rotated low-bit residual -> reconstruction.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

from . import alloc as _alloc
from . import codec, tucker


@dataclass
class Params:
    mode: str = "randomized"          # "exact" | "randomized"
    rt_max: int = 128
    rf_max: int = 0                   # 0 -> d
    rank_step: int = 8
    bits: Tuple[int, ...] = (0, 2, 3, 4)
    oversample: int = 10
    power_iters: int = 1
    budget: Optional[int] = None      # None -> fixed ranks
    fixed: Optional[Tuple[int, int, int]] = None
    delta: Optional[Sequence[float]] = None   # delta_b for b = 0..8


@dataclass
class ItemFactors:
    lam_t: np.ndarray
    U_t: np.ndarray
    lam_f: np.ndarray
    U_f: np.ndarray
    C_full: np.ndarray
    E: np.ndarray
    normX2: float


@dataclass
class Plan:
    factors: List[ItemFactors]
    tables: List[Dict]
    alloc: List[Tuple[int, int, int]]
    lam: Optional[object]
    feasible: bool = True


def factor_item(X: np.ndarray, p: Params, seed: int, item_id: int) -> ItemFactors:
    d = X.shape[-1]
    rf_max = p.rf_max or d
    lam_f, U_f = tucker.feature_factor(X)
    if p.mode == "exact":
        lam_t, U_t = tucker.token_factor_exact(X, p.rt_max)
    else:
        lam_t, U_t = tucker.token_factor_randomized(X, p.rt_max, p.oversample,
                                                    p.power_iters, seed, item_id)
    U_f = U_f[:, :rf_max]
    lam_f = lam_f[:rf_max]
    C = tucker.core_full(X, U_t, U_f)
    return ItemFactors(lam_t, U_t, lam_f, U_f, C, tucker.energy_table(C),
                       float(np.sum(X * X)))


def item_tables(f: ItemFactors, shape, e: int, p: Params) -> Dict:
    L, H, T, d = shape
    cand = _alloc.candidate_grid(p.rt_max, p.rf_max or d, p.rank_step, p.bits)
    return {"cand": cand,
            "B": _alloc.bytes_table(L, H, T, d, e, cand),
            "D": _alloc.distortion_table(f.E, f.normX2, p.delta, cand)}


def plan(Xs: Sequence[np.ndarray], seeds: Sequence[int], item_ids: Sequence[int],
         dtype: str, p: Params) -> Plan:
    e = 4 if dtype == "f32" else 2
    factors = [factor_item(X, p, s, i) for X, s, i in zip(Xs, seeds, item_ids)]
    if p.budget is None:
        rt, rf, b = p.fixed
        return Plan(factors, [], [(rt, rf, b)] * len(Xs), None)
    tables = [item_tables(f, X.shape, e, p) for f, X in zip(factors, Xs)]
    choice, lam, ok = _alloc.lagrangian_allocate(tables, p.budget)
    al = [tuple(int(v) for v in t["cand"][c]) for t, c in zip(tables, choice)]
    return Plan(factors, tables, al, lam, ok)


def compress_item(X, f: ItemFactors, a, seed: int, item_id: int, dtype: str) -> codec.Encoded:
    rt, rf, b = a
    sp = codec.stored_params(f.U_t, f.U_f, f.C_full, rt, rf, dtype)
    return codec.encode(X, sp, b, seed, item_id, dtype)


def decompress_item(enc: codec.Encoded, shape, seed: int, item_id: int, dtype: str,
                    out_round: bool = True) -> np.ndarray:
    L, H, T, d = shape
    return codec.decode(enc, L, H, T, d, seed, item_id, dtype, out_round=out_round)


def rel_fro(Xt: np.ndarray, X: np.ndarray) -> float:
    return float(np.linalg.norm((Xt - X).ravel()) / np.linalg.norm(X.ravel()))
