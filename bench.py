"""Benchmark: JoLT compress + decompress of an MoE-style GQA batch of prefill caches.

Default workload (the largest single-GPU configuration): 16 independent
sequences of 8192 tokens, each 32 layers in 8 groups of 4, 8 KV heads, d = 128,
bf16, K and V of every group as separate items (256 items of 67 MB, 17.2 GB);
FlashJoLT token factor (oversampling 10, one power iteration, rank limit 256),
one Lagrangian dual over all 256 items under a shared 2.5x budget.  A step is
jolt_plan (factors + dual) + jolt_compress + jolt_decompress of every item,
inputs resident in HBM.  Inputs are seeded synthetic planted-Tucker caches
(synth/), standing in for real prefill caches of the same shapes.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]

Prints one JSON line.  The metric is KV tokens compressed per second, counted
per layer group (sequences x groups x tokens / (plan + compress time));
decompress GB/s, per-kernel rates and the roofline of the dominant kernel ride
along, and (unless --no-mode-ratio) the exact / randomized plan + compress time
ratio on the Mistral-7B-shaped 1024-token cache, the counterpart of the pages'
FlashJoLT speedup.

Roofline: during the warmup steps every kernel timer of the library is on
(jolt_kernel_timer: a HIP event pair around each launch, on the launch
stream); the kernel with the most device time per step is the dominant one.
In the timed steps only its timer is on, and its average launch duration is
what the roofline divides the kernel's algorithmic work per launch by.  Each
kernel's work is both bytes (HBM, read + written once) and flops (on its own
unit); its bound is whichever of the two takes longer at the chip's peaks.
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
# dense MFMA bf16; fp32 (MFMA and vector); "bf16x3": fp32-accurate products formed
# from three bf16 MFMA products of hi/lo-split operands (hi hi + hi lo + lo hi),
# whose fp32-equivalent roof is a third of the bf16 peak
PEAK_TFLOPS = {"bf16": 2500.0, "fp32": 157.3, "bf16x3": 2500.0 / 3}

KERNELS = ["k_eig_tridiag", "k_eig_trivec", "k_eig_backtr", "k_eig_polish", "k_chol_inv", "k_apply_linv",
           "k_sym_gram", "k_gemm", "k_reduce", "k_xm", "k_xtq", "k_gram_rows", "k_build_wt", "k_encode",
           "k_decode", "k_jacobi_lds"]
KERNEL_SOURCE = {"k_eig_tridiag": "k_eig.hip", "k_eig_trivec": "k_eig.hip", "k_eig_backtr": "k_eig.hip",
                 "k_eig_polish": "k_eig.hip", "k_chol_inv": "k_orth.hip", "k_apply_linv": "k_orth.hip",
                 "k_gemm": "k_gemm.hip", "k_sym_gram": "k_gemm.hip", "k_xm": "k_plan.hip", "k_xtq": "k_plan.hip",
                 "k_gram_rows": "k_plan.hip", "k_encode": "k_codec.hip", "k_decode": "k_codec.hip",
                 "k_build_wt": "k_codec.hip"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="moe_gqa_batch16_8k")
    ap.add_argument("--ratio", type=float, default=0.0, help="budget ratio (0: the workload's first)")
    ap.add_argument("--items", type=int, default=0, help="use only the first N items (0: all)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-items", type=int, default=1, help="items in the oracle's timed sample")
    ap.add_argument("--no-mode-ratio", action="store_true")
    ap.add_argument("--no-studies", action="store_true", help="skip the comparators and allocator variants")
    ap.add_argument("--profile", action="store_true", help="few steps, no extras (for rocprofv3)")
    return ap.parse_args()


def work_per_step(cfg, jitems, allocs, mode="randomized"):
    """Algorithmic work of each kernel over one step: {kernel: (bytes, flops,
    flop unit)}; bytes are HBM bytes read + written once, flops those of the
    kernel's arithmetic unit ("bf16" MFMA, "bf16x3" for fp32-accurate products
    of split operands on the bf16 MFMA, or "fp32")."""
    k = cfg.rt_max + cfg.oversample
    q = cfg.power_iters
    out = {}
    X = [2 * it.L * it.H * it.T * it.d for it in jitems]           # bytes of one read of each item
    N = [it.L * it.H * it.T * it.d for it in jitems]
    n_lhd = [it.L * it.H * it.d for it in jitems]
    if mode == "randomized":
        # passes over X: A M (1 + q launches), Q^T A (q + 1 launches, the last with hi + lo Q)
        out["k_xm"] = (sum((1 + q) * (x + 2 * n * k + 4 * it.T * k) for x, n, it in zip(X, n_lhd, jitems)),
                       sum((1 + q) * 2.0 * nn * k for nn in N), "bf16")
        out["k_xtq"] = (sum((q + 1) * x + 2 * it.T * k * (q + 2) + (q + 1) * 4 * k * n
                            for x, n, it in zip(X, n_lhd, jitems)),
                        sum((q + 2) * 2.0 * nn * k for nn in N), "bf16")
        # CholeskyQR Grams and B B^T (symmetric: k (k + 1) len flops each) and the
        # L^-1 applies: T-long panels q + 2 times, n-long panels q (+1 for B B^T)
        out["k_sym_gram"] = (0, sum(k * (k + 1) * ((q + 2) * it.T + (q + 1) * n) for n, it in zip(n_lhd, jitems)),
                             "bf16x3")
        out["k_apply_linv"] = (sum(4 * k * ((q + 2) * it.T + q * n) * 2 for n, it in zip(n_lhd, jitems)),
                               sum(k * (k + 1) * ((q + 2) * it.T + q * n) for n, it in zip(n_lhd, jitems)), "fp32")
        out["k_chol_inv"] = (0, sum((2 * q + 2) * (2.0 / 3) * k ** 3 for _ in jitems), "fp32")
        out["k_gemm"] = (0, sum(2.0 * cfg.rt_max * k * (it.T + n) + 2.0 * cfg.rt_max * n * it.d
                                for n, it in zip(n_lhd, jitems)), "bf16x3")
        ne = k
    else:
        ne = jitems[0].T
    out["k_gram_rows"] = (sum(X), sum(2.0 * nn * it.d for nn, it in zip(N, jitems)), "bf16")
    # dense symmetric eigendecompositions (token and feature per item): Householder
    # tridiagonalization 4/3 n^3; back-transform Q Z 2 n^3; polish: the check
    # V^T V n^3 and one update 2 n^3
    out["k_eig_tridiag"] = (0, sum(4.0 / 3 * (ne ** 3 + it.d ** 3) for it in jitems), "fp32")
    out["k_eig_backtr"] = (0, sum(2.0 * (ne ** 3 + it.d ** 3) for it in jitems), "fp32")
    out["k_eig_polish"] = (0, sum(3.0 * (ne ** 3 + it.d ** 3) for it in jitems), "fp32")
    # codec: dense in / out, stored parameters, scales and codes; X^ = U~_t W~ as two
    # bf16 MFMA products (hi and lo planes of W~)
    dec = enc = 0
    fl = 0.0
    for it, a in zip(jitems, allocs):
        n_ = it.L * it.H * it.T * it.d
        rt = a.rt if a.rf else 0
        params = 2 * (it.T * rt + it.d * a.rf + it.L * it.H * rt * a.rf)
        resid = (n_ * a.bits // 8 + 2 * n_ // 64) if a.bits else 0
        dec += params + resid + 2 * n_
        enc += 2 * n_ + params + resid
        fl += 2.0 * 2 * n_ * ((rt + 15) // 16 * 16)
    out["k_decode"] = (dec, fl, "bf16")
    out["k_encode"] = (enc, fl, "bf16")
    return out


def roof(bytes_, flops, unit, ms):
    """Roofline of one kernel over `ms`: the binding peak and the fraction of it."""
    t_hbm = bytes_ / (HBM_PEAK_GBS * 1e9)
    t_fl = flops / (PEAK_TFLOPS[unit] * 1e12)
    s = ms * 1e-3
    if t_hbm >= t_fl:
        return {"bound": "hbm", "achieved": bytes_ / s / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": t_hbm / s}
    bound = "mfma" if unit in ("bf16", "bf16x3") else "alu"
    return {"bound": bound, "achieved": flops / s / 1e12, "peak": PEAK_TFLOPS[unit], "unit": "TFLOP/s",
            "precision": unit, "frac": t_fl / s}


def source_hash(kernel):
    """Hash of the kernel's source, of the shared device helpers and of
    plan.cpp and api.cpp (which size and group its launches), as recorded with
    the counters in profiles/."""
    f = KERNEL_SOURCE.get(kernel)
    if not f:
        return None
    h = hashlib.sha256()
    for name in (f, "dev_common.h", "plan.cpp", "api.cpp"):
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


def generate(cfg, n_items):
    """Stored bits of the first n_items items, generated in parallel (before the
    GPU is touched); yields (index, spec, bits)."""
    import synth
    specs = synth.item_specs(cfg, n_items)
    for i, raw in synth.iter_raw_parallel(cfg, specs):
        yield i, specs[i], raw


def upload(torch, raw, dev):
    import numpy as np
    a = raw.view(np.int16) if raw.dtype == np.uint16 else raw
    return torch.from_numpy(a).to(dev)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path (items would shard across "
              "GPUs with one energy-table all-gather; not built)", file=sys.stderr)
        return 2
    if args.profile:
        args.steps, args.warmup, args.no_cpu_baseline, args.no_mode_ratio = min(args.steps, 2), 1, True, True
        args.no_studies = True

    import synth
    cfg = synth.config(args.config)
    n_items = args.items or cfg.n_items
    ratio = args.ratio or (cfg.ratios[0] if cfg.ratios else 2.0)
    t0 = time.time()
    gen = generate(cfg, n_items)
    first = next(gen)                          # the worker pool is forked before the GPU is touched

    import numpy as np
    import torch
    from kv_cache_compression_jolt_amd import binding as jb

    jb.lib()
    dev = torch.device("cuda", 0)
    delta = json.load(open(os.path.join(ROOT, "tests", "golden", "delta_b.json")))["delta"]
    specs, xs, sample_raw = [], [], {}
    import itertools
    for i, spec, raw in itertools.chain([first], gen):
        specs.append(spec)
        xs.append(upload(torch, raw, dev))
        if i < args.cpu_items:
            sample_raw[i] = raw
        if (i + 1) % 32 == 0:
            print("bench: %d items uploaded" % (i + 1), file=sys.stderr, flush=True)
    gen_s = time.time() - t0
    print("bench: %d items generated and uploaded in %.1f s" % (len(xs), gen_s), file=sys.stderr, flush=True)
    budget = synth.budget_for_ratio(cfg, ratio, n_items=n_items)
    jitems = [jb.make_item(s.L, s.H, s.T, s.d, s.dtype, s.item_id, s.seed) for s in specs]
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
    print("bench: first step done", file=sys.stderr, flush=True)
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
    print("bench: warmup done, dominant kernel %s" % dominant, file=sys.stderr, flush=True)

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
    print("bench: timed steps done (%.2f ms per step)" % step_ms, file=sys.stderr, flush=True)

    work = work_per_step(cfg, jitems, allocs)
    launch_ms = dom_ms / max(dom_launches, 1)
    launches_per_step = dom_launches / args.steps
    if dominant in work:
        wb, wf, unit = work[dominant]
        per = 1.0 / max(launches_per_step, 1e-9)
        rl = roof(wb * per, wf * per, unit, launch_ms)
        rl["algorithmic_bytes_per_launch"] = wb * per
        rl["algorithmic_flops_per_launch"] = wf * per
    else:
        rl = {"bound": "unknown", "achieved": None, "peak": None, "unit": None, "frac": None}
    rl.update({"kernel": dominant, "traffic": pmc_traffic(dominant, cfg.name), "launch_ms": round(launch_ms, 5),
               "launches_per_step": round(launches_per_step, 2)})
    for key in ("achieved", "frac"):
        if rl.get(key) is not None:
            rl[key] = round(rl[key], 5)

    Nel = cfg.elems_per_item
    dense_bytes = 2 * Nel * n_items
    layer_group_tokens = n_items // 2 * cfg.T
    value = layer_group_tokens / ((plan_ms + comp_ms) * 1e-3)
    total_bytes = sum(a.bytes for a in allocs)

    kernel_table = {}
    for kname, (ms, n) in sorted(per_step.items(), key=lambda kv: -kv[1][0]):
        row = {"ms_per_step": round(ms, 4), "launches_per_step": round(n, 2)}
        if kname in work:
            wb, wf, unit = work[kname]
            r = roof(wb, wf, unit, ms)
            row.update({"bound": r["bound"], "frac": round(r["frac"], 4)})
            if wb:
                row["GBps"] = round(wb / (ms * 1e-3) / 1e9, 1)
            if wf:
                row["TFLOPs"] = round(wf / (ms * 1e-3) / 1e12, 2)
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
        "config": {"workload": cfg.name, "items": n_items, "item_shape": [cfg.L, cfg.H, cfg.T, cfg.d],
                   "sequences": cfg.sequences, "groups": cfg.groups,
                   "token_mode": "randomized", "oversample": cfg.oversample, "power_iters": cfg.power_iters,
                   "rt_max": cfg.rt_max, "budget_ratio": ratio, "budget_bytes": budget},
        "stage_ms": {"plan": round(plan_ms, 4), "compress": round(comp_ms, 4), "decompress": round(dec_ms, 4)},
        "decompress_GBps": round(dense_bytes / (dec_ms * 1e-3) / 1e9, 1),
        "compressed_bytes": int(total_bytes),
        "compression_ratio": round(dense_bytes / total_bytes, 4),
        "lambda": lam,
        "allocation": sorted(set((a.rt, a.rf, a.bits) for a in allocs)),
        "roofline": rl,
        "kernels": kernel_table,
        "input_gen_s": round(gen_s, 2),
    }
    J.close()
    del xs, outs, pays
    torch.cuda.empty_cache()

    if not args.no_mode_ratio:
        out["exact_vs_randomized"] = mode_ratio(torch, jb, dev, delta)
    if not args.no_studies:
        out["studies"] = run_studies(torch, jb, dev, delta)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, specs, sample_raw, budget, n_items, delta, layer_group_tokens)

    print(json.dumps(out))
    return 0


def mode_ratio(torch, jb, dev, delta, steps=3):
    """Plan + compress time of the exact and the randomized token modes on the
    Mistral-7B-shaped 1024-token cache (16 items, 2x budget)."""
    import numpy as np
    import synth
    cfg = synth.config("mistral7b_gqa_1k")
    specs = synth.item_specs(cfg)
    xs = [upload(torch, synth.make_item(cfg, s, keep_x=False).raw, dev) for s in specs]
    budget = synth.budget_for_ratio(cfg, 2.0)
    jitems = [jb.make_item(s.L, s.H, s.T, s.d, s.dtype, s.item_id, s.seed) for s in specs]
    stream = torch.cuda.current_stream()
    res = {}
    for mode in ("randomized", "exact"):
        jcfg = jb.make_config(mode, rt_max=cfg.rt_max, oversample=cfg.oversample, power_iters=cfg.power_iters,
                              rank_step=cfg.rank_step, bits=cfg.bits, budget=budget, delta=delta)
        J = jb.Jolt(jcfg, jitems)
        allocs, _ = J.plan(xs)
        pays = J.alloc_payloads(allocs)
        J.compress(xs, pays, allocs)
        torch.cuda.synchronize()
        ts = []
        for _ in range(steps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            allocs, _ = J.plan(xs)
            J.compress(xs, pays, allocs)
            b.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        res[mode + "_ms"] = round(float(np.median(ts)), 4)
        J.close()
    res["ratio"] = round(res["exact_ms"] / res["randomized_ms"], 3)
    res["workload"] = "mistral7b_gqa_1k (16 items of 4x8x1024x128 bf16, 2x budget), plan + compress"
    return res


def run_studies(torch, jb, dev, delta):
    """Comparators (4-bit, cross-layer SVD) and allocator variants (budget split
    between K and V in advance; measured residual distortion) on the
    Mistral-7B-shaped 1024-token cache."""
    import synth
    from kv_cache_compression_jolt_amd import studies
    cfg = synth.config("mistral7b_gqa_1k")
    specs = synth.item_specs(cfg)
    xs = [upload(torch, synth.make_item(cfg, s, keep_x=False).raw, dev) for s in specs]
    jitems = [jb.make_item(s.L, s.H, s.T, s.d, s.dtype, s.item_id, s.seed) for s in specs]
    kv = [s.kv for s in specs]
    res = {"workload": "mistral7b_gqa_1k (16 items of 4x8x1024x128 bf16)"}
    res["comparators"] = [studies.comparators(torch, cfg, jitems, xs, kv, delta, r) for r in (2.0, 3.76)]
    res["allocator_presplit"] = [studies.presplit(torch, cfg, jitems, xs, kv, delta, r) for r in (3.0, 4.0)]
    res["distortion_model"] = studies.measured_delta(torch, cfg, jitems, xs, delta, cfg.rt_max, cfg.d)
    print("bench: studies done", file=sys.stderr, flush=True)
    return res


def cpu_baseline(cfg, specs, sample_raw, budget, n_items, delta, layer_group_tokens):
    """The oracle (fp64 numpy + C Jacobi) on a sample of the workload's items:
    the same plan (with the sample's share of the budget), compress and
    decompress, wall-clock timed on this host."""
    import numpy as np
    import synth
    from oracle import pipeline as opipe
    idx = sorted(sample_raw)
    m = len(idx)
    xs = [synth.bf16_bits_to_f64(sample_raw[i]) if sample_raw[i].dtype == np.uint16
          else sample_raw[i].astype(np.float64) for i in idx]
    sp = [specs[i] for i in idx]
    sb = budget * m // n_items
    p = opipe.Params(mode="randomized", rt_max=cfg.rt_max, rank_step=cfg.rank_step, bits=cfg.bits,
                     oversample=cfg.oversample, power_iters=cfg.power_iters, budget=sb, delta=delta)
    t0 = time.perf_counter()
    pl = opipe.plan(xs, [s.seed for s in sp], [s.item_id for s in sp], cfg.dtype, p)
    encs = [opipe.compress_item(x, f, a, s.seed, s.item_id, cfg.dtype)
            for x, s, f, a in zip(xs, sp, pl.factors, pl.alloc)]
    t1 = time.perf_counter()
    for x, s, e in zip(xs, sp, encs):
        opipe.decompress_item(e, x.shape, s.seed, s.item_id, cfg.dtype)
    t2 = time.perf_counter()
    tokens = layer_group_tokens * m / n_items
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        threads = max([d.get("num_threads", 1) for d in info] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    return {"value": round(tokens / (t1 - t0), 2), "unit": "layer-group tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": "%d of %d items (plan + compress timed: %.2f s; decompress %.2f s)"
                      % (m, n_items, t1 - t0, t2 - t1)}


if __name__ == "__main__":
    sys.exit(main())
