"""ORACLE (test infrastructure only): the distortion-model constants delta_b.

delta_b is the relative mean squared error of the b-bit group quantizer on iid
N(0, 1) groups of 64 values -- the model the allocator uses for a JL-rotated
residual, which the rotation makes close to Gaussian.  delta_0 = 1 (no residual
keeps the whole truncation energy as error).

Running this module writes tests/golden/delta_b.json:
    python -m oracle.calibrate
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np

from . import quant

N_GROUPS = 1 << 20
CHUNK = 1 << 16
SEED = 0
BITS = (2, 3, 4, 5, 6, 7, 8)


def measure(n_groups: int = N_GROUPS, seed: int = SEED, bits=BITS):
    rng = np.random.default_rng(seed)
    err = {b: 0.0 for b in bits}
    energy = 0.0
    done = 0
    while done < n_groups:
        m = min(CHUNK, n_groups - done)
        x = rng.standard_normal((m, quant.GROUP)).astype(np.float32)
        x64 = x.astype(np.float64)
        energy += float(np.sum(x64 * x64))
        for b in bits:
            q, s = quant.quantize_groups(x, b)
            xr = quant.dequantize_groups(q, s)
            err[b] += float(np.sum((x64 - xr) ** 2))
        done += m
    delta = [1.0, float("nan")] + [0.0] * 7
    for b in bits:
        delta[b] = err[b] / energy
    return delta


def main(argv=None):
    delta = measure()
    here = os.path.dirname(os.path.abspath(__file__))
    out = os.path.join(here, os.pardir, "tests", "golden", "delta_b.json")
    doc = {
        "what": "relative MSE of the b-bit symmetric per-64-group quantizer "
                "(bf16 absmax scale, half-even rounding) on iid N(0,1) groups; "
                "index = bits; delta_0 = 1; b = 1 is not a valid width",
        "written_by": "python -m oracle.calibrate",
        "n_groups": N_GROUPS, "seed": SEED,
        "delta": [None if np.isnan(v) else v for v in delta],
    }
    with open(out, "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")
    print(json.dumps(doc["delta"]))
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
