"""jolt_decompress_noalloc (the entry point that allocates nothing: its W~
workspace is the library's fixed device scratch) against jolt_decompress on
the same payloads: identical outputs on two calls in a row, the second with
a smaller input, and a call that would need more than the fixed scratch is
refused before any launch."""
import json
import os

import numpy as np
import pytest

import synth
from tests.gpu_util import jolt_binding, to_device, torch_cuda

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DELTA = json.load(open(os.path.join(ROOT, "tests", "golden", "delta_b.json")))["delta"]


def _compressed(torch, jb, cfg, n, rt_max, ratio):
    items = synth.make_items(cfg, n)
    jitems = [jb.make_item(i.L, i.H, i.T, i.d, cfg.dtype, i.item_id, i.seed) for i in items]
    budget = synth.budget_for_ratio(cfg, ratio, n_items=n)
    J = jb.Jolt(jb.make_config("randomized", rt_max=rt_max, budget=budget, delta=DELTA), jitems)
    xs = [to_device(i, torch) for i in items]
    allocs, _ = J.plan(xs)
    assert J.status == jb.JOLT_OK
    pays = J.alloc_payloads(allocs)
    J.compress(xs, pays, allocs)
    return J, allocs, pays, xs


def test_noalloc_decompress_matches_twice():
    torch = torch_cuda()
    jb = jolt_binding()
    cases = [(synth.config("mistral7b_gqa_1k"), 6, 128, 2.0),                       # 6 x 2 MiB of scratch
             (synth.config("mistral7b_gqa_1k", L=2, H=4, T=512), 2, 64, 3.0)]        # then a smaller call
    for cfg, n, rt_max, ratio in cases:
        J, allocs, pays, xs = _compressed(torch, jb, cfg, n, rt_max, ratio)
        ref = [torch.full_like(x, 7) for x in xs]
        J.decompress(pays, ref, allocs)
        got = [torch.full_like(x, -7) for x in xs]
        print("noalloc", cfg.name, (cfg.L, cfg.H, cfg.T), n, sorted(set((a.rt, a.rf, a.bits) for a in allocs)),
              flush=True)
        jb.jolt_decompress_noalloc(J.h, J.items, allocs, [p.data_ptr() for p in pays], [o.data_ptr() for o in got],
                                   torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        for a, b in zip(ref, got):
            assert torch.equal(a, b)
        J.close()


def test_noalloc_rejects_beyond_fixed_scratch():
    jb = jolt_binding()
    torch_cuda()
    h = jb.jolt_create(0)
    try:
        items = [jb.make_item(4, 8, 1024, 128, "bf16", i, 0) for i in range(17)]     # 17 x 4 MiB > 64 MiB
        allocs = [jb.jolt_alloc(256, 128, 4, 0, 0, 0.0) for _ in items]
        with pytest.raises(jb.JoltError) as e:
            jb.jolt_decompress_noalloc(h, items, allocs, [1] * 17, [1] * 17, 0)
        assert e.value.status == jb.JOLT_E_WORKSPACE
    finally:
        jb.jolt_destroy(h)
