"""The comparators and allocator variants (kv_cache_compression_jolt_amd/studies.py)
run through libjolt on a reduced Mistral-7B-shaped cache.

The cross-layer SVD comparator is the rank-r projection of the token
unfolding, so its squared error is the Eckart-Young value: the sum of the
token Gram's eigenvalues past r (the oracle's exact ones), up to bf16
rounding of the stored parameters and of the output (about 2^-8 relative per
element, added in quadrature to a residual of at least 30% here)."""
import json
import os

import numpy as np
import pytest

import synth
from oracle import tucker
from tests.gpu_util import jolt_binding, to_device, torch_cuda

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DELTA = json.load(open(os.path.join(ROOT, "tests", "golden", "delta_b.json")))["delta"]


def test_comparators_and_allocator_variants():
    torch = torch_cuda()
    jb = jolt_binding()
    from kv_cache_compression_jolt_amd import studies
    cfg = synth.config("mistral7b_gqa_1k", L=2, H=4, T=512, rt_max=64)
    items = synth.make_items(cfg, 4)
    xs = [to_device(i, torch) for i in items]
    jitems = [jb.make_item(i.L, i.H, i.T, i.d, "bf16", i.item_id, i.seed) for i in items]
    kv = [i.kv for i in items]
    res = studies.comparators(torch, cfg, jitems, xs, kv, DELTA, 2.0)
    print(res, flush=True)
    r = res["cross_layer_svd"]["rank"]
    num = den = {0: 0.0, 1: 0.0}
    num, den = {0: 0.0, 1: 0.0}, {0: 0.0, 1: 0.0}
    for it in items:
        lam, _ = tucker.token_factor_exact(it.x, min(it.T, it.L * it.H * it.d))
        x2 = float(np.sum(it.x ** 2))
        num[it.kv] += x2 - float(np.sum(lam[:r]))
        den[it.kv] += x2
    for k, name in ((0, "K"), (1, "V")):
        ey = np.sqrt(num[k] / den[k])
        got = res["cross_layer_svd"]["error"][name]
        assert abs(got - ey) <= 0.01 * ey + 2e-3, (name, got, ey)
    # the 4-bit comparator uses exactly its accounted bytes: (b/8 + 2/64) per element
    n = sum(it.L * it.H * it.T * it.d for it in items)
    assert res["quant4"]["bytes"] == n // 2 + n // 32
    assert res["jolt"]["bytes"] <= res["budget_bytes"]
    ps = studies.presplit(torch, cfg, jitems, xs, kv, DELTA, 3.0)
    assert ps["joint"]["distortion"] > 0 and all(row["distortion"] > 0 for row in ps["presplit"] if row["feasible"])
    md = studies.measured_delta(torch, cfg, jitems, xs, DELTA, 32, 32, bits=(4,))
    print(ps, md, flush=True)
    row = md["rows"][0]
    # the rotated residual is close to Gaussian: the measured relative error of
    # the 4-bit quantizer is the model's within a wide margin
    assert 0.5 * row["model"] <= row["measured_mean"] <= 2.0 * row["model"]
