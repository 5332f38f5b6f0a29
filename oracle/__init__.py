"""CPU ORACLE for the JoLT compressor -- TEST INFRASTRUCTURE ONLY.

A plain, slow, fp64 numpy (plus one small C Jacobi) implementation of what the
compressor computes, written from the pages about "A JoLT for the KV cache"
(Krishnan & Schulz): partial Tucker factors along the token and feature modes
(exact eigensolve or FlashJoLT randomized range finder), core and energy table,
single-Lagrangian-dual allocation of (r_t, r_f, b), rotated low-bit residual
codec, and reconstruction.

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import
this package.  It shares no code with the HIP library; the only common module
is the seeded input generator in ``synth``.

Parity unpinned (no passage or closed form to check against): the distortion
model's fidelity on real residuals (delta_b is pinned on Gaussian groups only),
and the pages' own quality numbers (0.009 / 0.006 relative error at 2x), which
need trained weights.
"""
from . import alloc, attention, codec, linalg, pipeline, quant, rng, tucker, wht  # noqa: F401
