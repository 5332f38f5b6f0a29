"""Benchmark: JoLT compress + decompress of a Mistral-7B-v0.3-shaped GQA prefill cache.

Workload (one step): 32 layers in 8 groups of 4, 8 KV heads, d = 128, 1024 tokens,
bf16, K and V of every group as separate items (16 items, 134 MB); FlashJoLT
token factor (oversampling 10, one power iteration), one global 2x budget.
A step is jolt_plan (factors + dual) + jolt_compress + jolt_decompress of all
16 items, inputs resident in HBM.  Inputs are seeded synthetic planted-Tucker
caches (see synth/), standing in for real Mistral-7B-v0.3 caches.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Prints one JSON line.  The metric is KV tokens compressed per second, counted
per layer group (groups x tokens / compress time); decompress GB/s and the
roofline of the dominant kernel ride along.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="mistral7b_gqa_1k")
    ap.add_argument("--ratio", type=float, default=2.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-items", type=int, default=2, help="items in the oracle's timed sample")
    ap.add_argument("--profile", action="store_true", help="few steps, no CPU baseline (for rocprofv3)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path (items shard across GPUs "
              "with one table all-gather; not built)", file=sys.stderr)
        return 2
    if args.profile:
        args.steps, args.warmup, args.no_cpu_baseline = min(args.steps, 3), 1, True

    import numpy as np
    import torch
    import synth
    from kv_cache_compression_jolt_amd import binding as jb

    jb.lib()
    dev = torch.device("cuda", 0)
    cfg = synth.config(args.config)
    delta = json.load(open(os.path.join(ROOT, "tests", "golden", "delta_b.json")))["delta"]
    t0 = time.time()
    items = synth.make_items(cfg)
    gen_s = time.time() - t0
    xs = []
    for it in items:
        raw = it.raw.view(np.int16) if it.raw.dtype == np.uint16 else it.raw
        xs.append(torch.from_numpy(raw.copy()).to(dev))
    budget = synth.budget_for_ratio(cfg, args.ratio)
    jitems = [jb.make_item(it.L, it.H, it.T, it.d, it.dtype, it.item_id, it.seed) for it in items]
    jcfg = jb.make_config("randomized", rt_max=cfg.rt_max, oversample=cfg.oversample,
                          power_iters=cfg.power_iters, rank_step=cfg.rank_step, bits=cfg.bits,
                          budget=budget, delta=delta)
    J = jb.Jolt(jcfg, jitems)
    allocs, lam = J.plan(xs)
    pays = J.alloc_payloads(allocs)
    outs = [torch.empty_like(x) for x in xs]
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev: ev[0].record(stream)
        J.plan(xs)
        if ev: ev[1].record(stream)
        J.compress(xs, pays, allocs)
        if ev: ev[2].record(stream)
        J.decompress(pays, outs, allocs)
        if ev: ev[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    plan_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    comp_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    dec_ms = sum(e[2].elapsed_time(e[3]) for e in evs) / args.steps
    step_ms = wall * 1e3 / args.steps

    # dominant streaming kernel: the fused decoder, timed alone (HIP events on its stream)
    reps = 20
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        J.decompress(pays, outs, allocs)
    e1.record(stream)
    torch.cuda.synchronize()
    dec_only_ms = e0.elapsed_time(e1) / reps

    N = cfg.elems_per_item
    dense_bytes = sum(2 * N for _ in items)
    read_bytes = 0
    for it, a in zip(jitems, allocs):
        rt = a.rt if a.rf else 0
        params = 2 * (it.T * rt + it.d * a.rf + it.L * it.H * rt * a.rf)
        resid = (N * a.bits // 8 + 2 * N // 64) if a.bits else 0
        read_bytes += params + resid
    alg_bytes = read_bytes + dense_bytes          # decoder: payload in, dense cache out
    achieved = alg_bytes / (dec_only_ms * 1e-3) / 1e9

    layer_group_tokens = cfg.groups * cfg.sequences * cfg.T
    compress_ms = plan_ms + comp_ms
    value = layer_group_tokens / (compress_ms * 1e-3)
    total_bytes = sum(a.bytes for a in allocs)

    out = {
        "metric": "KV tokens compressed/sec per layer group (+ decompress GB/s; % MFMA/HBM peak)",
        "value": round(value, 1),
        "unit": "layer-group tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "items": cfg.n_items, "item_shape": [cfg.L, cfg.H, cfg.T, cfg.d],
                   "token_mode": "randomized", "oversample": cfg.oversample, "power_iters": cfg.power_iters,
                   "budget_ratio": args.ratio, "budget_bytes": budget},
        "stage_ms": {"plan": round(plan_ms, 4), "compress": round(comp_ms, 4), "decompress": round(dec_ms, 4)},
        "decompress_GBps": round(dense_bytes / (dec_ms * 1e-3) / 1e9, 1),
        "compressed_bytes": int(total_bytes),
        "compression_ratio": round(dense_bytes / total_bytes, 4),
        "allocation": sorted(set((a.rt, a.rf, a.bits) for a in allocs)),
        "roofline": {"kernel": "fused decode (unpack, dequant, inverse rotation, + U_t W~ via MFMA)",
                     "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "launch_ms": round(dec_only_ms, 5), "algorithmic_bytes_per_launch": int(alg_bytes)},
        "input_gen_s": round(gen_s, 2),
    }

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, items, budget, delta, args.cpu_items, layer_group_tokens)

    print(json.dumps(out))
    J.close()
    return 0


def cpu_baseline(cfg, items, budget, delta, m, layer_group_tokens):
    """The oracle (fp64 numpy + C Jacobi) on a sample of m items, same pipeline."""
    import numpy as np
    from oracle import pipeline as opipe
    sample = items[:m]
    # the sample's share of the global budget keeps the allocation comparable
    sb = budget * m // len(items)
    p = opipe.Params(mode="randomized", rt_max=cfg.rt_max, rank_step=cfg.rank_step, bits=cfg.bits,
                     oversample=cfg.oversample, power_iters=cfg.power_iters, budget=sb, delta=delta)
    t0 = time.perf_counter()
    pl = opipe.plan([i.x for i in sample], [i.seed for i in sample], [i.item_id for i in sample], cfg.dtype, p)
    encs = [opipe.compress_item(i.x, f, a, i.seed, i.item_id, cfg.dtype)
            for i, f, a in zip(sample, pl.factors, pl.alloc)]
    t1 = time.perf_counter()
    for i, e in zip(sample, encs):
        opipe.decompress_item(e, i.x.shape, i.seed, i.item_id, cfg.dtype)
    t2 = time.perf_counter()
    tokens = layer_group_tokens * m / len(items)
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        threads = max([d.get("num_threads", 1) for d in info] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    return {"value": round(tokens / (t1 - t0), 2), "unit": "layer-group tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": "%d of %d items (plan + compress timed: %.2f s; decompress %.2f s)"
                      % (m, len(items), t1 - t0, t2 - t1)}


if __name__ == "__main__":
    sys.exit(main())
