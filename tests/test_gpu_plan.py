"""GPU parity of jolt_plan / jolt_compress / jolt_decompress against the oracle.

Free-running comparison (each side computes its own factors and allocation):
  * factor subspaces: largest principal-angle sine <= 1e-2 for every leading
    block whose eigengap exceeds 1e-3 of the top eigenvalue;
  * ||X||^2 and the energy table agree to fp32 accuracy: a row of the table
    belongs to one token eigenvector, and inside a cluster of eigenvalues whose
    gaps are below that same 1e-3 threshold only the cluster's span is
    determined (any rounding difference rotates the vectors within it and
    moves energy between their rows), so such rows are compared through the
    cluster's sum; a row with gaps above the threshold on both sides is
    compared on its own;
  * the chosen allocation fits the budget;
  * the GPU reconstruction error <= 1.05 x the oracle's error + 1e-4.
"""
import ctypes
import json
import os

import numpy as np
import pytest

import synth
from oracle import pipeline as opipe
from tests.gpu_util import jolt_binding, out_values, rel, to_device, torch_cuda

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DELTA = json.load(open(os.path.join(ROOT, "tests", "golden", "delta_b.json")))["delta"]


def _sine(A, B):
    Qa = np.linalg.qr(A)[0]
    Qb = np.linalg.qr(B)[0]
    s = np.linalg.svd(Qa - Qb @ (Qb.T @ Qa), compute_uv=False)
    return float(s.max()) if s.size else 0.0


def _gap_blocks(lam, tol=1e-3):
    """Leading block sizes r with lam[r-1] - lam[r] > tol * lam[0]."""
    return [r for r in range(1, len(lam)) if lam[r - 1] - lam[r] > tol * lam[0]]


def _fetch(torch, ptr, count, dtype=np.float32):
    """Copy `count` values from a device pointer into a host numpy array."""
    torch.cuda.synchronize()
    out = np.empty(count, dtype=dtype)
    hip = _hip()
    rc = hip.hipMemcpy(out.ctypes.data_as(ctypes.c_void_p), ctypes.c_void_p(ptr), out.nbytes, 2)
    assert rc == 0
    return out


_HIP = None


def _hip():
    global _HIP
    if _HIP is None:
        _HIP = ctypes.CDLL("libamdhip64.so")
        _HIP.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
        _HIP.hipMemcpy.restype = ctypes.c_int
    return _HIP


def _plan_parity(cfg, n_items, mode, rt_max, ratio=None, fixed=None, oversample=10, sub_tol=1e-2,
                 item_offset=0, codec=True):
    torch = torch_cuda()
    jb = jolt_binding()
    specs = synth.item_specs(cfg)[item_offset:item_offset + n_items]
    items = [synth.make_item(cfg, sp) for sp in specs]
    L, H, T, d = cfg.L, cfg.H, cfg.T, cfg.d
    budget = synth.budget_for_ratio(cfg, ratio, n_items=n_items) if ratio else None
    p = opipe.Params(mode=mode, rt_max=rt_max, oversample=oversample, budget=budget, fixed=fixed, delta=DELTA,
                     bits=cfg.bits)
    print("oracle plan", cfg.name, (cfg.L, cfg.H, cfg.T, cfg.d), mode, n_items, "items", flush=True)
    ref = opipe.plan([i.x for i in items], [i.seed for i in items], [i.item_id for i in items], cfg.dtype, p)
    jitems = [jb.make_item(L, H, T, d, cfg.dtype, i.item_id, i.seed) for i in items]
    jcfg = jb.make_config(mode, rt_max=rt_max, oversample=oversample, bits=cfg.bits,
                          budget=budget if budget is not None else -1, fixed=fixed or (0, 0, 0), delta=DELTA)
    J = jb.Jolt(jcfg, jitems)
    xs = [to_device(i, torch) for i in items]
    print("plan", cfg.name, (L, H, T, d), mode, rt_max, flush=True)
    allocs, lam = J.plan(xs)
    torch.cuda.synchronize()
    assert J.status == jb.JOLT_OK, J.status
    if budget is not None:
        assert sum(a.bytes for a in allocs) <= budget
    for i, (it, f) in enumerate(zip(items, ref.factors)):
        v = J.factors(i)
        Ut = _fetch(torch, v.ut, rt_max * T).reshape(rt_max, T).T
        Uf = _fetch(torch, v.uf, d * d).reshape(d, d)
        lam_t = _fetch(torch, v.lam_t, rt_max)
        lam_f = _fetch(torch, v.lam_f, d)
        nx2 = _fetch(torch, v.normx2, 1, np.float64)[0]
        E = _fetch(torch, v.energy, rt_max * d).reshape(rt_max, d)
        assert abs(nx2 / f.normX2 - 1) < 1e-5
        assert np.max(np.abs(lam_f - f.lam_f)) <= 1e-4 * f.lam_f[0]
        assert np.max(np.abs(lam_t - f.lam_t)) <= 1e-3 * f.lam_t[0]
        assert np.max(np.abs(Ut.T @ Ut - np.eye(rt_max))) < 1e-3
        assert np.max(np.abs(Uf.T @ Uf - np.eye(d))) < 1e-4
        for r in _gap_blocks(f.lam_f):
            assert _sine(Uf[:, :r], f.U_f[:, :r]) <= sub_tol, ("feature", r)
        for r in _gap_blocks(f.lam_t):
            assert _sine(Ut[:, :r], f.U_t[:, :r]) <= sub_tol, ("token", r)
        bounds = [0] + _gap_blocks(f.lam_t[:rt_max]) + [rt_max]
        for lo, hi in zip(bounds[:-1], bounds[1:]):
            assert np.max(np.abs(E[lo:hi].sum(0) - f.E[lo:hi].sum(0))) <= 1e-3 * f.E.max(), ("energy rows", lo, hi)
    if not codec:
        J.close()
        return allocs, ref
    pays = J.alloc_payloads(allocs)
    J.compress(xs, pays, allocs)
    outs = [torch.empty_like(x) for x in xs]
    J.decompress(pays, outs, allocs)
    torch.cuda.synchronize()
    for k, (it, a, f, o, oa) in enumerate(zip(items, allocs, ref.factors, outs, ref.alloc)):
        enc = opipe.compress_item(it.x, f, oa, it.seed, it.item_id, cfg.dtype)
        xr = opipe.decompress_item(enc, it.x.shape, it.seed, it.item_id, cfg.dtype)
        e_ref = rel(xr, it.x)
        e_gpu = rel(out_values(o, cfg.dtype), it.x)
        print("item", it.item_id, "gpu", (a.rt, a.rf, a.bits), e_gpu, "oracle", oa, e_ref, flush=True)
        assert e_gpu <= 1.05 * e_ref + 1e-4
        hdr = pays[k][:64].cpu().numpy().tobytes()
        assert jb.jolt_payload_validate(hdr, jitems[k], a) == jb.JOLT_OK
    J.close()
    return allocs, ref


@pytest.mark.parametrize("shape", [(2, 4, 512, 128, 64), (4, 8, 1024, 128, 128)], ids=["small", "c2shape"])
def test_randomized_plan_parity(shape):
    L, H, T, d, rt_max = shape
    cfg = synth.config("mistral7b_gqa_1k", L=L, H=H, T=T, d=d)
    _plan_parity(cfg, 4 if T < 1024 else 2, "randomized", rt_max, ratio=2.0)


def test_tiny_exact_f32_full_config():
    """The whole fp32 exact configuration: 2 x 4 x 256 x 64, fixed (16, 12, 4)."""
    cfg = synth.config("tiny_exact_f32")
    allocs, ref = _plan_parity(cfg, 2, "exact", 16, fixed=(16, 12, 4))
    assert all((a.rt, a.rf, a.bits) == (16, 12, 4) for a in allocs)


def test_exact_bf16_block_jacobi():
    cfg = synth.config("mistral7b_gqa_1k", L=2, H=4, T=512)
    _plan_parity(cfg, 2, "exact", 64, ratio=2.0)


def test_randomized_wide_sketch():
    """k = 256 + 10 > 142: the small SVD goes through block Jacobi."""
    cfg = synth.config("llama2_13b_mha_4k", L=2, H=4, T=1024)
    _plan_parity(cfg, 2, "randomized", 256, ratio=3.0)


# ---------------------------------------------------------------- full item sizes, free running
@pytest.mark.timeout(900)
def test_fullsize_free_running_llama2_13b_item():
    """One whole 4 x 40 x 4096 x 128 item (k = 266), each side with its own
    factors: eigenvalues, energy table, subspaces where the gap allows, and the
    reconstruction error."""
    _plan_parity(synth.config("llama2_13b_mha_4k"), 1, "randomized", 256, ratio=3.0)


@pytest.mark.timeout(900)
def test_fullsize_free_running_mistral_exact_items():
    """Two whole 4 x 8 x 1024 x 128 items in exact token mode (1024 x 1024 token
    Gram): the oracle's fp64 Jacobi against the GPU's block Jacobi."""
    _plan_parity(synth.config("mistral7b_gqa_1k"), 2, "exact", 128, ratio=2.0)


@pytest.mark.timeout(900)
def test_fullsize_free_running_llama31_8b_item():
    """One whole 4 x 8 x 65536 x 128 item (537 MB): factors, eigenvalues and the
    energy table against the oracle's own (the codec on this shape is covered
    by the full-size sampled-block tests)."""
    _plan_parity(synth.config("llama31_8b_gqa_64k"), 1, "randomized", 256, ratio=2.0, codec=False)
