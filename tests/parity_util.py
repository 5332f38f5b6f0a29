"""Test-side bounds for comparing the fused encoder's integer output with the
oracle's when both quantize residuals formed at different precisions.

The oracle forms the residual r = x - X^ in fp64.  The GPU forms X^ = U_t W~
with W~ = C U_f^T held as a bf16 hi + lo pair (|W - hi - lo| <= 2^-16 |W|,
after an fp32 product of bf16 factors, <= rf 2^-24 relative to its terms) and
accumulates U_t W~ in fp32 over 2 r_t terms (<= 2 r_t 2^-24 <= 2^-15 relative
to its terms for r_t <= 256).  So per element |dX^| <= 2^-14 a with
a[t, f] = sum_k |U_t[t, k]| sum_j |C[k, j]| |U_f[f, j]|.  The rotation is an
orthogonal map applied in fp32 (log2 d = 7 butterfly stages), so each rotated
value moves by at most ||dr_row||_2 <= 2^-14 ||a_row||_2 plus 2^-20 ||r_row||_2
of rounding.  A code may therefore differ from the oracle's only where the
oracle's scaled value y = r' / scale lies within that distance (times 1/scale)
of the midpoint between the two codes, and a scale only where the oracle's
absmax / qmax lies that close to a bf16 rounding midpoint.  A mismatch away from
every boundary is an error."""
import numpy as np

from oracle import quant as oquant


def row_tolerance(Ut, Uf, C, R):
    """Per-row bound (L, H, T) on the movement of a rotated residual value:
    2^-14 ||a_row||_2 + 2^-20 ||r_row||_2 (see the module docstring).
    Ut (T x rt), Uf (d x rf), C (L x H x rt x rf) are the stored parameters,
    R (L x H x T x d) the oracle's residual."""
    L, H, T, d = R.shape
    rt = Ut.shape[1]
    if rt == 0:
        a2 = np.zeros((L, H, T))
    else:
        Wa = np.matmul(np.abs(C), np.abs(Uf).T[None, None])          # L H rt d
        A = np.matmul(np.abs(Ut)[None, None], Wa)                      # L H T d
        a2 = np.linalg.norm(A, axis=-1)
    return 2.0 ** -14 * a2 + 2.0 ** -20 * np.linalg.norm(R, axis=-1)


def check_codes(u_gpu, u_ref, sc_gpu, sc_ref, rotated, tol_row, bits, d, max_frac=1e-2):
    """Every code and scale of the GPU equals the oracle's, or is a boundary
    case within the bound: u (G x 64) codes, sc (G,) bf16 scale bits, rotated
    (G x 64) the oracle's fp32 rotated residual, tol_row (rows,) the bound per
    row (d / 64 groups per row).  Returns (code mismatches, scale mismatches)."""
    G = u_ref.shape[0]
    tol = np.repeat(np.asarray(tol_row, dtype=np.float64).ravel(), d // 64)
    assert tol.shape[0] == G
    qm = (1 << (bits - 1)) - 1
    x32 = np.asarray(rotated, dtype=np.float32)
    # scales: the oracle's fp32 absmax / qmax near a bf16 rounding midpoint
    bad_s = np.nonzero(np.asarray(sc_gpu) != np.asarray(sc_ref))[0]
    for g in bad_s:
        s32 = float(np.float32(np.max(np.abs(x32[g]))) / np.float32(qm))
        lo, hi = sorted((float(oquant.bf16_bits_to_f32(sc_gpu[g])), float(oquant.bf16_bits_to_f32(sc_ref[g]))))
        assert abs(int(sc_gpu[g]) - int(sc_ref[g])) == 1, ("scale differs by more than one bf16 step", g)
        mid = 0.5 * (lo + hi)
        assert abs(s32 - mid) <= tol[g] / qm + 2.0 ** -24 * abs(s32), ("scale mismatch off a boundary", g, s32, mid)
    # codes in groups with equal scales: the oracle's scaled value near k + 1/2
    same = np.ones(G, dtype=bool)
    same[bad_s] = False
    scale = oquant.bf16_bits_to_f32(np.asarray(sc_ref, dtype=np.uint16)).astype(np.float64)
    mism = (np.asarray(u_gpu) != np.asarray(u_ref)) & same[:, None]
    gi, ei = np.nonzero(mism)
    if gi.size:
        ug = np.asarray(u_gpu)[gi, ei].astype(np.int64)
        ur = np.asarray(u_ref)[gi, ei].astype(np.int64)
        assert np.all(np.abs(ug - ur) == 1), "a code differs by more than one step"
        inv = (np.float32(1.0) / oquant.bf16_bits_to_f32(np.asarray(sc_ref, dtype=np.uint16)[gi])).astype(np.float32)
        y = (x32[gi, ei] * inv).astype(np.float64)
        mid = np.minimum(ug, ur) - (1 << (bits - 1)) + 0.5
        dist = np.abs(y - mid)
        allowed = tol[gi] / scale[gi] + 2.0 ** -22 * (np.abs(y) + 1.0)
        assert np.all(dist <= allowed), ("code mismatch off a rounding boundary",
                                          float(np.max(dist / allowed)), int(np.argmax(dist / allowed)))
    n_codes = int(np.sum(mism))
    assert n_codes <= max_frac * u_ref.size and bad_s.size <= max_frac * G
    return n_codes, int(bad_s.size)
