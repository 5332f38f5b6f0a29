"""rocprofv3 summaries for profiles/: kernel-time tables and HBM traffic of one
kernel from hardware counters, scaled by a plain device copy of known size.

Counter runs (one counter per run; the program follows `--` directly):

  rocprofv3 --pmc FETCH_SIZE --output-format csv -d D/copy_fetch -- python3 -m kv_cache_compression_jolt_amd.pmc copy
  rocprofv3 --pmc WRITE_SIZE --output-format csv -d D/copy_write -- python3 -m kv_cache_compression_jolt_amd.pmc copy
  rocprofv3 --pmc FETCH_SIZE --output-format csv -d D/fetch -- python3 bench.py --profile
  rocprofv3 --pmc WRITE_SIZE --output-format csv -d D/write -- python3 bench.py --profile
  python3 -m kv_cache_compression_jolt_amd.pmc summarize D KERNEL WORKLOAD "COMMANDS"

FETCH_SIZE and WRITE_SIZE are read in KiB per dispatch.  The copy moves
COPY_BYTES in and COPY_BYTES out, so bytes = counter KiB x 1024 x (COPY_BYTES /
copy counter bytes); the summary records both factors.

Kernel-time table from a `rocprofv3 --kernel-trace --stats --output-format csv`
run:

  python3 -m kv_cache_compression_jolt_amd.pmc trace-summary D OUT "TITLE" "COMMAND"

Per-kernel means per dispatch of every counter in the counter runs under D
(one subfolder per pass; derived metrics such as MfmaUtil, LdsUtil,
LdsBankConflict and OccupancyPercent are computed by rocprofv3 itself):

  python3 -m kv_cache_compression_jolt_amd.pmc counters D OUT "TITLE" "COMMANDS" KERNEL [KERNEL ...]
"""
from __future__ import annotations

import csv
import glob
import hashlib
import os
import sys

COPY_BYTES = 512 * 1024 * 1024
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCES = {"k_eig_tridiag": "k_eig.hip", "k_eig_trivec": "k_eig.hip", "k_eig_backtr": "k_eig.hip", "k_eig_polish": "k_eig.hip",
           "k_eig_tridiag_w": "k_eig.hip", "k_eig_backtr_w": "k_eig.hip", "k_eig_polish_w": "k_eig.hip", "k_chol_inv": "k_orth.hip", "k_apply_linv": "k_orth.hip",
           "k_gemm": "k_gemm.hip", "k_gemm128": "k_gemm.hip", "k_gemm128_bx3": "k_gemm.hip", "k_sym_gram": "k_gemm.hip", "k_xm": "k_plan.hip", "k_xtq": "k_plan.hip", "k_gram_rows": "k_plan.hip",
           "k_encode": "k_codec.hip", "k_decode": "k_codec.hip", "k_build_wt": "k_codec.hip"}


def copy_kernel():
    import torch
    n = COPY_BYTES // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print("copied %d bytes x 3" % COPY_BYTES)


def _newest(d, suffix):
    """Most recent rocprofv3 output file of one kind under d (an output
    folder reused by several runs holds one file per run)."""
    files = glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True)
    if not files:
        raise SystemExit("no %s under %s" % (suffix, d))
    return max(files, key=os.path.getmtime)


def _rows(d):
    out = []
    with open(_newest(d, "counter_collection.csv"), newline="") as fh:
        out.extend(csv.DictReader(fh))
    return out


def _per_dispatch(d, counter, match):
    vals = {}
    for r in _rows(d):
        if r.get("Counter_Name", "").strip() != counter:
            continue
        if match(r.get("Kernel_Name", "")):
            key = r.get("Dispatch_Id") or r.get("Correlation_Id")
            vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
    return list(vals.values())


def source_hash(kernel):
    """Hash of the kernel's source, of the shared device helpers and of the
    host code that sizes and groups its launches (plan.cpp, api.cpp): counters
    taken before a change to any of them no longer describe a launch.  The
    same files as bench.py's source_hash."""
    h = hashlib.sha256()
    for f in (SOURCES[kernel], "dev_common.h", "plan.cpp", "api.cpp"):
        with open(os.path.join(ROOT, "kv_cache_compression_jolt_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def summarize(d, kernel, workload, commands):
    is_copy = lambda name: "copy" in name.lower() or "Copy" in name
    cf = max(_per_dispatch(os.path.join(d, "copy_fetch"), "FETCH_SIZE", is_copy))
    cw = max(_per_dispatch(os.path.join(d, "copy_write"), "WRITE_SIZE", is_copy))
    f_fetch = COPY_BYTES / (cf * 1024.0)
    f_write = COPY_BYTES / (cw * 1024.0)
    is_k = lambda name: ("::%s(" % kernel) in name or ("::%s<" % kernel) in name or name.startswith(kernel + "(")
    kf = _per_dispatch(os.path.join(d, "fetch"), "FETCH_SIZE", is_k)
    kw = _per_dispatch(os.path.join(d, "write"), "WRITE_SIZE", is_k)
    if not kf or not kw:
        raise SystemExit("no dispatches of %s in the counter runs" % kernel)
    fetch = sum(kf) / len(kf) * 1024.0 * f_fetch
    write = sum(kw) / len(kw) * 1024.0 * f_write
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    path = os.path.join(ROOT, "profiles", "%s_%s_pmc.txt" % (kernel, workload))
    with open(path, "w") as fh:
        fh.write("HBM traffic of %s, workload %s, from rocprofv3 hardware counters\n" % (kernel, workload))
        fh.write("commands:\n%s\n" % commands)
        fh.write("copy calibration: %d bytes each way; FETCH_SIZE read %.1f KiB (factor %.4f), "
                 "WRITE_SIZE read %.1f KiB (factor %.4f)\n" % (COPY_BYTES, cf, f_fetch, cw, f_write))
        fh.write("%s dispatches: FETCH_SIZE %d, WRITE_SIZE %d\n" % (kernel, len(kf), len(kw)))
        fh.write("fetch bytes per launch (scaled): %.6g\n" % fetch)
        fh.write("write bytes per launch (scaled): %.6g\n" % write)
        fh.write("hbm bytes per launch: %.6g\n" % (fetch + write))
        fh.write("source sha256[:16]: %s (%s + dev_common.h + plan.cpp + api.cpp)\n" % (source_hash(kernel), SOURCES[kernel]))
    print("wrote", path)


def trace_summary(d, out, title, command):
    rows = []
    with open(_newest(d, "kernel_stats.csv"), newline="") as fh:
        for r in csv.DictReader(fh):
            rows.append((r["Name"], int(r["Calls"]), float(r["TotalDurationNs"]) / 1e3,
                         float(r["AverageNs"]) / 1e3, float(r["Percentage"])))
    rows.sort(key=lambda t: -t[2])
    with open(out, "w") as fh:
        fh.write("%s\ncommand: %s\n\n" % (title, command))
        fh.write("%-72s %6s %12s %10s %7s\n" % ("kernel", "calls", "total_us", "avg_us", "pct"))
        for name, calls, tot, avg, pct in rows:
            fh.write("%-72s %6d %12.1f %10.2f %7.2f\n" % (name[:72], calls, tot, avg, pct))
    print("wrote", out)


def _all_rows(d):
    out = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                r["_file"] = f
                out.append(r)
    return out


def counters(d, out, title, commands, kernels):
    rows = _all_rows(d)
    table = {}
    for k in kernels:
        is_k = lambda name, k=k: ("::%s(" % k) in name or ("::%s<" % k) in name or name.startswith(k)
        per = {}
        for r in rows:
            if not is_k(r.get("Kernel_Name", "")):
                continue
            key = (r["_file"], r.get("Dispatch_Id") or r.get("Correlation_Id"))
            name = r.get("Counter_Name", "").strip()
            per.setdefault(name, {}).setdefault(key, 0.0)
            per[name][key] += float(r["Counter_Value"])
        table[k] = {n: (sum(v.values()) / len(v), len(v)) for n, v in per.items()}
    names = sorted({n for t in table.values() for n in t})
    with open(out, "w") as fh:
        fh.write("%s\ncommands:\n%s\n\n" % (title, commands))
        fh.write("mean per dispatch (dispatches in brackets)\n")
        for k in kernels:
            fh.write("\n%s\n" % k)
            for n in names:
                if n in table[k]:
                    v, c = table[k][n]
                    fh.write("  %-28s %16.6g  [%d]\n" % (n, v, c))
        fh.write("\nsource sha256[:16]: %s\n" % ", ".join(
            "%s %s" % (k, source_hash(k)) for k in kernels if k in SOURCES))
    print("wrote", out)


if __name__ == "__main__":
    cmd = sys.argv[1] if len(sys.argv) > 1 else ""
    if cmd == "copy":
        copy_kernel()
    elif cmd == "summarize":
        summarize(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5])
    elif cmd == "trace-summary":
        trace_summary(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5])
    elif cmd == "counters":
        counters(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5], sys.argv[6:])
    else:
        raise SystemExit(__doc__)
