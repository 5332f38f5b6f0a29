"""Comparators and allocator variants on synthetic caches, run through libjolt.

Comparators (the author page abstract reports JoLT's error roughly an order
of magnitude below cross-layer SVD and 4-bit quantization):
  * 4-bit: every item stored as its rotated residual only, (r_t, r_f, b) =
    (0, 0, 4) -- the codec with no Tucker part;
  * cross-layer SVD: a truncated SVD of the layer group's token unfolding (the
    group's layers and heads side by side as feature blocks), i.e. fixed
    (r, d, 0) in exact token mode with the largest r on the rank grid that fits
    the budget (the feature factor is then a full orthonormal basis and the
    reconstruction is the rank-r projection of the unfolding);
  * JoLT: the single dual over (r_t, r_f, b) under the same budget.
Allocator variants (K and V are allocated under one budget rather than a split
fixed in advance: podcast, "The Core Mechanism"; author page abstract):
  * pre-split: the K items and the V items each get a fixed share of the
    budget and their own dual, for a range of shares, against the joint dual;
  * distortion model: the residual quantizer's relative error measured per item
    and bit width, against the Gaussian-group constants delta_b the dual uses.
Everything here calls the C ABI; only arithmetic on the results (sums of
errors and bytes) happens in Python.
"""
from __future__ import annotations

import numpy as np

from . import binding as jb


def _errors(torch, xs, outs):
    """Per item (squared error, energy) of a reconstruction, in fp64 on the GPU."""
    res = []
    for x, o in zip(xs, outs):
        xf = (x.to(torch.int32) << 16).view(torch.float32).double() if x.dtype == torch.int16 else x.double()
        of = (o.to(torch.int32) << 16).view(torch.float32).double() if o.dtype == torch.int16 else o.double()
        res.append((float(torch.sum((of - xf) ** 2)), float(torch.sum(xf * xf))))
    return res


def _aggregate(errs, kv):
    """Relative Frobenius error over the K items (kv 0) and over the V items."""
    out = {}
    for name, want in (("K", 0), ("V", 1)):
        e = sum(a for (a, _), k in zip(errs, kv) if k == want)
        s = sum(b for (_, b), k in zip(errs, kv) if k == want)
        out[name] = float(np.sqrt(e / s)) if s > 0 else None
    return out


def _run(torch, cfg_c, jitems, xs, allocs=None):
    J = jb.Jolt(cfg_c, jitems)
    if allocs is None:
        allocs, lam = J.plan(xs)
    else:
        J.plan(xs)
        lam = None
    pays = J.alloc_payloads(allocs)
    J.compress(xs, pays, allocs)
    outs = [torch.empty_like(x) for x in xs]
    J.decompress(pays, outs, allocs)
    torch.cuda.synchronize()
    errs = _errors(torch, xs, outs)
    J.close()
    return allocs, lam, errs


def comparators(torch, cfg, jitems, xs, kv, delta, ratio):
    """JoLT, 4-bit and cross-layer SVD at one budget ratio (versus bf16)."""
    dense = sum(2 * it.L * it.H * it.T * it.d for it in jitems)
    budget = int(dense // ratio)
    out = {"ratio": ratio, "budget_bytes": budget}
    jc = jb.make_config("randomized", rt_max=cfg.rt_max, oversample=cfg.oversample, power_iters=cfg.power_iters,
                        rank_step=cfg.rank_step, bits=cfg.bits, budget=budget, delta=delta)
    allocs, lam, errs = _run(torch, jc, jitems, xs)
    out["jolt"] = {"error": _aggregate(errs, kv), "bytes": int(sum(a.bytes for a in allocs)), "lambda": lam,
                   "allocation": sorted(set((a.rt, a.rf, a.bits) for a in allocs))}
    # 4-bit: residual only (its bytes are fixed by b = 4)
    q4 = jb.make_config("randomized", rt_max=cfg.rt_max, oversample=cfg.oversample, bits=(0, 4), budget=-1,
                        fixed=(0, 0, 4), delta=delta)
    a4, _, e4 = _run(torch, q4, jitems, xs)
    b4 = int(sum(a.bytes for a in a4))
    out["quant4"] = {"error": _aggregate(e4, kv), "bytes": b4, "ratio": dense / b4}
    # cross-layer SVD: exact token mode, the largest grid rank that fits
    T, d = jitems[0].T, jitems[0].d
    rmax = min(256, T)
    r = 0
    for cand in range(cfg.rank_step, rmax + 1, cfg.rank_step):
        if sum(jb.jolt_item_bytes(it, cand, d, 0) for it in jitems) <= budget:
            r = cand
    if r > 0 and T <= 2048:
        sv = jb.make_config("exact", rt_max=r, bits=(0,), budget=-1, fixed=(r, d, 0), delta=delta)
        asv, _, esv = _run(torch, sv, jitems, xs)
        out["cross_layer_svd"] = {"error": _aggregate(esv, kv), "bytes": int(sum(a.bytes for a in asv)), "rank": r}
    return out


def presplit(torch, cfg, jitems, xs, kv, delta, ratio, shares=(0.3, 0.4, 0.5, 0.6, 0.7)):
    """The joint dual against duals with the budget split between K and V in
    advance, on the GPU's energy tables: modelled distortion (the dual's
    objective) of each."""
    dense = sum(2 * it.L * it.H * it.T * it.d for it in jitems)
    budget = int(dense // ratio)
    jc = jb.make_config("randomized", rt_max=cfg.rt_max, oversample=cfg.oversample, power_iters=cfg.power_iters,
                        rank_step=cfg.rank_step, bits=cfg.bits, budget=budget, delta=delta)
    J = jb.Jolt(jc, jitems)
    allocs, lam = J.plan(xs)
    torch.cuda.synchronize()
    tables = []
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    bits = [b for b in range(9) if (int(jc.bits_mask) >> b) & 1]
    for i, it in enumerate(jitems):
        v = J.factors(i)
        E = np.empty(v.rt_max * it.d, dtype=np.float32)
        nx = np.empty(1, dtype=np.float64)
        assert hip.hipMemcpy(E.ctypes.data_as(ctypes.c_void_p), ctypes.c_void_p(v.energy), E.nbytes, 2) == 0
        assert hip.hipMemcpy(nx.ctypes.data_as(ctypes.c_void_p), ctypes.c_void_p(v.normx2), 8, 2) == 0
        E = E.reshape(v.rt_max, it.d).astype(np.float64)
        cand, D, B = [], [], []
        for rt in range(0, v.rt_max + 1, cfg.rank_step):
            for rf in range(0, v.rf_max + 1, cfg.rank_step):
                if (rt == 0) != (rf == 0):
                    continue
                S = E[:rt, :rf].sum() if rt else 0.0
                for b in bits:
                    cand.append((rt, rf, b))
                    D.append(delta[b] * max(0.0, float(nx[0]) - S))
                    B.append(jb.jolt_item_bytes(it, rt, rf, b))
        tables.append((np.array(cand, dtype=np.int32), np.array(D), np.array(B, dtype=np.int64)))
    J.close()
    total = lambda alloc: float(sum(a.distortion for a in alloc))
    st, joint, lam_j = jb.jolt_plan_from_tables([t[0] for t in tables], [t[1] for t in tables],
                                                [t[2] for t in tables], budget)
    out = {"ratio": ratio, "joint": {"distortion": total(joint), "lambda": lam_j,
                                     "K_bytes": int(sum(a.bytes for a, k in zip(joint, kv) if k == 0)),
                                     "V_bytes": int(sum(a.bytes for a, k in zip(joint, kv) if k == 1))}}
    rows = []
    for sh in shares:
        dist = 0.0
        ok = True
        for want, part in ((0, int(budget * sh)), (1, budget - int(budget * sh))):
            idx = [i for i, k in enumerate(kv) if k == want]
            st, al, _ = jb.jolt_plan_from_tables([tables[i][0] for i in idx], [tables[i][1] for i in idx],
                                                 [tables[i][2] for i in idx], part)
            ok &= st == jb.JOLT_OK
            dist += total(al)
        rows.append({"K_share": sh, "distortion": dist, "feasible": bool(ok)})
    out["presplit"] = rows
    return out


def measured_delta(torch, cfg, jitems, xs, delta, rt, rf, bits=(2, 3, 4)):
    """The residual quantizer's relative error measured per item at fixed ranks
    (r_t, r_f): ||X - X~||^2 / ||X - X^||^2 with X^ the Tucker part (the same
    payload decoded with no residual), against the model constant delta_b."""
    rows = []
    for b in bits:
        jc = jb.make_config("randomized", rt_max=cfg.rt_max, oversample=cfg.oversample,
                            power_iters=cfg.power_iters, bits=(0, b), budget=-1, fixed=(rt, rf, b), delta=delta)
        J = jb.Jolt(jc, jitems)
        allocs, _ = J.plan(xs)
        pays = J.alloc_payloads(allocs)
        J.compress(xs, pays, allocs)
        full = [torch.empty_like(x) for x in xs]
        tuck = [torch.empty_like(x) for x in xs]
        J.decompress(pays, full, allocs)
        a0 = [jb.jolt_alloc(a.rt, a.rf, 0, 0, 0, 0.0) for a in allocs]
        J.decompress(pays, tuck, a0)
        torch.cuda.synchronize()
        e_full = _errors(torch, xs, full)
        e_tuck = _errors(torch, xs, tuck)
        ratios = [ef / et for (ef, _), (et, _) in zip(e_full, e_tuck) if et > 0]
        rows.append({"bits": b, "model": delta[b], "measured_mean": float(np.mean(ratios)),
                     "measured_min": float(np.min(ratios)), "measured_max": float(np.max(ratios))})
        J.close()
    return {"ranks": [rt, rf], "rows": rows}
