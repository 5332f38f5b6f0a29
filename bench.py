"""Benchmark: JoLT compress + decompress of a Mistral-7B-v0.3-shaped GQA prefill cache.

Workload (one step): 32 layers in 8 groups of 4, 8 KV heads, d = 128, 1024 tokens,
bf16, K and V of every group as separate items (16 items, 134 MB); FlashJoLT
token factor (oversampling 10, one power iteration), one global 2x budget.
A step is jolt_plan (factors + dual) + jolt_compress + jolt_decompress of all
16 items, inputs resident in HBM.  Inputs are seeded synthetic planted-Tucker
caches (see synth/), standing in for real Mistral-7B-v0.3 caches.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Prints one JSON line.  The metric is KV tokens compressed per second, counted
per layer group (groups x tokens / (plan + compress time)); decompress GB/s,
per-kernel times and the roofline of the dominant kernel ride along.

Roofline: during the warmup steps every kernel timer of the library is on
(jolt_kernel_timer: a HIP event pair around each launch, on the launch
stream); the kernel with the most device time per step is the dominant one.
In the timed steps only its timer is on, and its average launch duration is
what the roofline divides the kernel's algorithmic work per launch by.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
FP32_VECTOR_PEAK_TFLOPS = 157.3
BF16_MFMA_PEAK_TFLOPS = 2500.0

KERNELS = ["k_eig_tridiag", "k_eig_trivec", "k_eig_backtr", "k_eig_polish", "k_chol_inv", "k_apply_linv", "k_sym_gram", "k_gemm", "k_reduce", "k_xm", "k_xtq",
           "k_gram_rows", "k_build_wt", "k_encode", "k_decode", "k_jacobi_lds"]
KERNEL_SOURCE = {"k_eig_tridiag": "k_eig.hip", "k_eig_trivec": "k_eig.hip", "k_eig_backtr": "k_eig.hip", "k_eig_polish": "k_eig.hip", "k_chol_inv": "k_orth.hip", "k_apply_linv": "k_orth.hip",
                 "k_gemm": "k_gemm.hip", "k_sym_gram": "k_gemm.hip", "k_xm": "k_plan.hip", "k_xtq": "k_plan.hip", "k_gram_rows": "k_plan.hip",
                 "k_encode": "k_codec.hip", "k_decode": "k_codec.hip", "k_build_wt": "k_codec.hip"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="mistral7b_gqa_1k")
    ap.add_argument("--ratio", type=float, default=2.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-items", type=int, default=16, help="items in the oracle's timed sample")
    ap.add_argument("--profile", action="store_true", help="few steps, no CPU baseline (for rocprofv3)")
    return ap.parse_args()


def work_per_step(cfg, jitems, allocs):
    """Algorithmic work of each kernel over one step: (kind, amount), kind 'bytes'
    (HBM bytes read + written once) or 'flops'."""
    k = cfg.rt_max + cfg.oversample
    q = cfg.power_iters
    out = {}
    xb = sum(2 * cfg.elems_per_item for _ in jitems)             # one read of every cache tensor
    n_lhd = [it.L * it.H * it.d for it in jitems]
    # passes over X: A M (1 + q launches), Q^T A (q + 1 launches, the last with hi + lo Q), feature Gram
    out["k_xm"] = ("bytes", (1 + q) * xb + sum((1 + q) * (2 * n * k + 4 * it.T * k) for n, it in zip(n_lhd, jitems)))
    out["k_xtq"] = ("bytes", (q + 1) * xb + sum(2 * it.T * k * (q + 2) + (q + 1) * 4 * k * n
                                                for n, it in zip(n_lhd, jitems)))
    out["k_gram_rows"] = ("bytes", xb + sum(4 * it.d * it.d for it in jitems))
    # dense symmetric eigendecompositions (token k x k and feature d x d per item):
    # Householder tridiagonalization 4/3 n^3; back-transform Q Z 2 n^3; polish:
    # the check V^T V on its upper tiles n^3 and one update V E 2 n^3 (the
    # tridiagonal eigenpairs in between are O(n^2) per multisection round)
    out["k_eig_tridiag"] = ("flops", sum(4.0 / 3 * (k ** 3 + it.d ** 3) for it in jitems))
    out["k_eig_backtr"] = ("flops", sum(2.0 * (k ** 3 + it.d ** 3) for it in jitems))
    out["k_eig_polish"] = ("flops", sum(3.0 * (k ** 3 + it.d ** 3) for it in jitems))
    # CholeskyQR inverse factor: n^3 / 3 (factor) + n^3 / 3 (inverse), 2 q + 2 factorizations
    out["k_chol_inv"] = ("flops", sum((2 * q + 2) * (2.0 / 3) * k ** 3 for _ in jitems))
    # CholeskyQR Grams and B B^T (symmetric: k (k + 1) len flops each) and the L^-1
    # applies (triangular: k (k + 1) len): T-long panels 1 + 2 q times (the last
    # twice), n-long panels q times, plus B B^T over n
    passes_t = q + 2
    out["k_sym_gram"] = ("flops", sum(k * (k + 1) * (passes_t * it.T + (q + 1) * n) for n, it in zip(n_lhd, jitems)))
    out["k_apply_linv"] = ("flops", sum(k * (k + 1) * (passes_t * it.T + q * n) for n, it in zip(n_lhd, jitems)))
    # U_t = Q U~ and P = U~^T B
    out["k_gemm"] = ("flops", sum(2 * cfg.rt_max * k * (it.T + n) for n, it in zip(n_lhd, jitems)))
    # decode: payload in, dense out; encode: dense in, codes + scales out (+ stored params)
    dec = enc = 0
    for it, a in zip(jitems, allocs):
        N = it.L * it.H * it.T * it.d
        rt = a.rt if a.rf else 0
        params = 2 * (it.T * rt + it.d * a.rf + it.L * it.H * rt * a.rf)
        resid = (N * a.bits // 8 + 2 * N // 64) if a.bits else 0
        dec += params + resid + 2 * N
        enc += 2 * N + params + resid
    out["k_decode"] = ("bytes", dec)
    out["k_encode"] = ("bytes", enc)
    return out


def source_hash(kernel):
    """Hash of the kernel's source and of plan.cpp (which sizes and groups its
    launches), as recorded with the counters in profiles/."""
    f = KERNEL_SOURCE.get(kernel)
    if not f:
        return None
    h = hashlib.sha256()
    for name in (f, "plan.cpp"):
        with open(os.path.join(ROOT, "kv_cache_compression_jolt_amd", "csrc", name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def pmc_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary of this
    kernel and workload, or None if there is none or the kernel source changed
    since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "%s_%s_pmc.txt" % (kernel, workload))
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m = re.search(r"source sha256\[:16\]: (\w+)", txt)
    b = re.search(r"hbm bytes per launch: ([0-9.eE+]+)", txt)
    if not m or not b or m.group(1) != source_hash(kernel):
        return None
    return float(b.group(1))


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path (items shard across GPUs "
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

    step()                       # first launches of every kernel (code objects load here)
    torch.cuda.synchronize()
    # warmup with every kernel timer on: per-kernel device time per step
    for kname in KERNELS:
        jb.jolt_kernel_timer(J.h, kname, True)
    for _ in range(max(args.warmup, 1)):
        step()
    torch.cuda.synchronize()
    per_step = {}
    for kname in KERNELS:
        ms, n = jb.jolt_kernel_time(J.h, kname)
        jb.jolt_kernel_timer(J.h, kname, False)
        if n:
            per_step[kname] = (ms / max(args.warmup, 1), n / max(args.warmup, 1))
    dominant = max(per_step, key=lambda kname: per_step[kname][0])
    jb.jolt_kernel_timer(J.h, dominant, True)

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for kk in range(args.steps):
        step(evs[kk])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    dom_ms, dom_launches = jb.jolt_kernel_time(J.h, dominant)
    jb.jolt_kernel_timer(J.h, dominant, False)
    plan_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    comp_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    dec_ms = sum(e[2].elapsed_time(e[3]) for e in evs) / args.steps
    step_ms = wall * 1e3 / args.steps

    work = work_per_step(cfg, jitems, allocs)
    launch_ms = dom_ms / max(dom_launches, 1)
    launches_per_step = dom_launches / args.steps
    if dominant in work:
        dom_kind, amount = work[dominant]
        per_launch = amount / max(launches_per_step, 1e-9)
        if dom_kind == "bytes":
            achieved = per_launch / (launch_ms * 1e-3) / 1e9
            peak, unit, bound = HBM_PEAK_GBS, "GB/s", "hbm"
        else:
            achieved = per_launch / (launch_ms * 1e-3) / 1e12
            peak, unit, bound = FP32_VECTOR_PEAK_TFLOPS, "TFLOP/s", "alu"
    else:
        dom_kind, per_launch, achieved, peak, unit, bound = "unknown", None, None, None, None, "unknown"
    traffic = pmc_traffic(dominant, cfg.name)

    N = cfg.elems_per_item
    dense_bytes = sum(2 * N for _ in items)
    layer_group_tokens = cfg.groups * cfg.sequences * cfg.T
    value = layer_group_tokens / ((plan_ms + comp_ms) * 1e-3)
    total_bytes = sum(a.bytes for a in allocs)

    kernel_table = {}
    for kname, (ms, n) in sorted(per_step.items(), key=lambda kv: -kv[1][0]):
        row = {"ms_per_step": round(ms, 4), "launches_per_step": round(n, 2)}
        if kname in work:
            kind, amount = work[kname]
            if kind == "bytes":
                row["GBps"] = round(amount / (ms * 1e-3) / 1e9, 1)
                row["hbm_frac"] = round(amount / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
            else:
                row["TFLOPs"] = round(amount / (ms * 1e-3) / 1e12, 3)
        kernel_table[kname] = row

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
        "roofline": {"kernel": dominant, "bound": bound,
                     "achieved": None if achieved is None else round(achieved, 3),
                     "peak": peak, "unit": unit,
                     "frac": None if achieved is None else round(achieved / peak, 5),
                     "traffic": traffic,
                     "launch_ms": round(launch_ms, 5), "launches_per_step": round(launches_per_step, 2),
                     "algorithmic_per_launch": per_launch, "algorithmic_kind": dom_kind},
        "kernels": kernel_table,
        "input_gen_s": round(gen_s, 2),
    }

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, items, budget, delta, args.cpu_items, layer_group_tokens)

    print(json.dumps(out))
    J.close()
    return 0


def cpu_baseline(cfg, items, budget, delta, m, layer_group_tokens):
    """The oracle (fp64 numpy + C Jacobi) on a sample of m items, same pipeline."""
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
