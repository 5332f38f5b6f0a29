"""Build libjolt.so (HIP, gfx950) in-tree.

    python -m kv_cache_compression_jolt_amd.build          # incremental
    python -m kv_cache_compression_jolt_amd.build --force  # rebuild everything
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libjolt.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["api.cpp", "plan.cpp", "planner.cpp", "payload.cpp", "ktimer.cpp", "k_codec.hip", "k_plan.hip", "k_eig.hip", "k_orth.hip", "k_gemm.hip",
           "k_attn.hip"]
HEADERS = ["bf16_split.h", "dev_common.h", "jolt_internal.h", "plan_kernels.h", "planner.h", "payload.h", "api_internal.h", "attn.h"]

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    "-ffp-contract=off",                       # no silent FMA formation: quantizer rounding is specified
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I" + os.path.join(ROOT, "include"),
]


def _newest_header() -> float:
    paths = [os.path.join(CSRC, h) for h in HEADERS] + [os.path.join(ROOT, "include", "libjolt.h")]
    return max(os.path.getmtime(p) for p in paths)


def _compile(src: str, force: bool) -> str:
    out = os.path.join(OBJ, os.path.basename(src) + ".o")
    path = os.path.join(CSRC, src)
    if not force and os.path.exists(out) and os.path.getmtime(out) >= max(os.path.getmtime(path), _newest_header()):
        return out
    cmd = [HIPCC] + FLAGS + (["-x", "hip"] if src.endswith(".cpp") else []) + ["-c", path, "-o", out + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    os.replace(out + ".tmp", out)
    return out


def build(force: bool = False, jobs: int = 6) -> str:
    os.makedirs(OBJ, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, force), SOURCES))
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < max(os.path.getmtime(o) for o in objs):
        cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", LIB + ".tmp"] + objs
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed: %s\n%s" % (r.stdout, r.stderr))
        os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(force="--force" in sys.argv))
