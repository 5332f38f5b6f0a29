// Symmetric eigensolver for small dense matrices (n <= kTriMaxN) in five
// launches that hand over through a per-matrix workspace (tri_ws):
// k_eig_tridiag (step 1) and k_eig_polish (step 5, output) run one workgroup
// of 1024 threads per matrix with the matrix resident in LDS; k_eig_wy forms
// the compact-WY T of each reflector block (a wave per block); k_eig_trivec
// (steps 2 and 3) runs a group of 16 lanes per eigenvalue over the whole chip;
// k_eig_backtr (step 4) runs a workgroup per 32 columns of each matrix.
//
//   1. Householder tridiagonalization Q^T A Q = T (Golub & Van Loan, Matrix
//      Computations, sec. 8.3.1) in panels of 32 columns: within a panel the
//      trailing matrix is left as stored and corrected on the fly by the
//      panel's V and W (the latrd form), then updated once on fp32 MFMA;
//      the reflectors stay in the rows of A;
//   2. every eigenvalue of T by multisection on Sturm counts (sec. 8.4.1),
//      16 lanes per eigenvalue, to a relative width of 2 eps;
//   3. every eigenvector of T from a twisted factorization of T - lambda I
//      (Dhillon & Parlett, Orthogonal eigenvectors and relative gaps, 2004):
//      forward and backward LDL^T pivots, the twist index where |gamma| is
//      smallest, and the two one-sided recurrences from it;
//   4. V = Q Z with the reflectors applied 32 at a time in compact WY form
//      (Schreiber & Van Loan 1989) on fp32 MFMA;
//   5. Newton-Schulz polar steps V <- V (3 I - V^T V) / 2 (at most 3, until
//      V^T V is within 4e-6 of I, or one step after it was within 1e-3),
//      which restore the orthogonality that vectors of close eigenvalues lose.
// When V^T V is far from I (numerically repeated eigenvalues: the twisted
// vectors coincide) the matrix is flagged in sweeps_out and the Jacobi kernel,
// launched right after in retry mode, solves it instead.
//
// Output convention (shared with the Jacobi kernel): eigenvalues descending,
// eigenvector columns sign-normalised so that the entry of largest magnitude
// (first such row) is positive.
#include <float.h>

#include <algorithm>

#include "dev_common.h"
#include "plan_kernels.h"
#include "ktimer.h"

namespace jolt {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
// row stride of the panel's V and W: with an even stride every per-step
// access pattern over them meets each LDS bank at most twice per wave
constexpr int kPanelStride = 34;

// Per-matrix workspace between the launches (floats; eig_tri_ws_bytes gives
// its size): A after the reduction (n x n, row-major, reflector j in row j),
// Z^T (row k = the eigenvector of the k-th smallest eigenvalue of T, later
// the back-transformed V^T), both with rows of np = n rounded up to 4 floats
// (16-byte aligned), the compact-WY T of each block of 32 reflectors (32 x 32
// row-major, zero below the diagonal), d, e (e_{n-1} = 0), tau, the
// eigenvalues of T ascending, and a fail flag.
struct TriWs {
    float *a, *zt, *tb, *d, *e, *tau, *lam;
    int *flag;
    float *ex;          // wide solver only: E of the polish steps (n x np)
    int np;
};
__device__ __forceinline__ int tri_blocks(int n) { return (max(n - 2, 0) + 31) >> 5; }
__device__ __forceinline__ TriWs tri_ws(float *base, int n) {
    TriWs w;
    w.np = n > kTriMaxN ? (n + 15) & ~15 : (n + 3) & ~3;
    const size_t nn = (size_t)n * w.np;
    w.a = base;
    w.zt = base + nn;
    w.tb = w.zt + nn;
    w.d = w.tb + 1024 * tri_blocks(n);
    w.e = w.d + n;
    w.tau = w.e + n;
    w.lam = w.tau + n;
    w.flag = reinterpret_cast<int *>(w.lam + n);
    w.ex = w.lam + n + 4;
    return w;
}

// Reads rows [0, rows) of float4 columns [0, c4) of a global matrix (row
// stride gs floats, rows 16-byte aligned) with B loads of each thread in
// flight before their LDS stores: st(r, c, v) stores the float4 of row r at
// columns 4c .. 4c + 3.  NT threads take part.
template <int NT, int B, typename St>
__device__ __forceinline__ void load_rows4(const float *g, int gs, int rows, int c4, int tid, St st) {
    const int total = rows * c4;
    for (int e0 = tid; e0 < total; e0 += NT * B) {
        float4 v[B];
#pragma unroll
        for (int u = 0; u < B; ++u) {
            const int e = min(e0 + NT * u, total - 1), r = e / c4, c = e - r * c4;
            v[u] = *reinterpret_cast<const float4 *>(g + (size_t)r * gs + 4 * c);
        }
#pragma unroll
        for (int u = 0; u < B; ++u) {
            const int e = e0 + NT * u;
            if (e < total) {
                const int r = e / c4, c = e - r * c4;
                st(r, c, v[u]);
            }
        }
    }
}


// C (n x n) tile (tm, tn) of sum_k A(m, k) B(k, n) on v_mfma_f32_32x32x2f32, with
// A(m, k) = a[k * lda_k + m * lda_m] and B(k, n) = b[k * ld + n]; out of range
// entries read as zero.
__device__ __forceinline__ f32x16 mfma_tile(const float *a, int lda_k, int lda_m, const float *b, int ld, int n,
                                            int tm, int tn, int lane) {
    f32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
    const int m = tm * 32 + (lane & 31), col = tn * 32 + (lane & 31), kh = lane >> 5;
    const bool mv = m < n, cv = col < n;
    const int mc = min(m, n - 1), cc = min(col, n - 1);
    // four K steps per iteration over a multiple of 8 (the masks zero the
    // padding), so that a batch of loads is in flight before its MFMAs: the
    // compiler does not unroll loops with a runtime count around MFMAs
    for (int k0 = 0; k0 < n; k0 += 8) {
        float av[4], bv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int kk = k0 + 2 * u + kh, kc = min(kk, n - 1);
            const bool kv = kk < n;
            av[u] = ld_or_zero(a, kc * lda_k + mc * lda_m, mv && kv);
            bv[u] = ld_or_zero(b, kc * ld + cc, cv && kv);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av[u], bv[u], acc, 0, 0, 0);
    }
    return acc;
}

// Tile (tm, tn) of V + V E on fp32 MFMA.  Both factors stay in fp32: a
// rounded V would put error vectors outside V's span into every column, and
// the next polar step would spread them into the accurate columns.
__device__ __forceinline__ f32x16 ns_tile(const float *V, const float *E, int ld, int n, int tm, int tn, int lane) {
    f32x16 acc = mfma_tile(V, 1, ld, E, ld, n, tm, tn, lane);
    const int c = tn * 32 + (lane & 31), cc = min(c, n - 1);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int row = tm * 32 + frag_row(lane, q);
        acc[q] += ld_or_zero(V, min(row, n - 1) * ld + cc, row < n && c < n);
    }
    return acc;
}

// write the (up to) two 32 x 32 tiles a wave owns (tiles wid and wid + 16)
__device__ __forceinline__ void store_tiles(float *dst, const f32x16 &a0, const f32x16 &a1, int ld, int n, int nt,
                                            int ntiles, int wid, int lane) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int t = wid + u * kWaves;
        if (t >= ntiles) continue;
        const int tm = t / nt, tn = t % nt, col = tn * 32 + (lane & 31);
        const f32x16 &a = u ? a1 : a0;
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
            const int row = tm * 32 + frag_row(lane, jj);
            if (row < n && col < n) dst[row * ld + col] = a[jj];
        }
    }
}

}  // namespace

// Column c = lane % 32 of T for a full block of 32 reflectors, in registers:
// solves (diag(1 / tau) + strict_upper(G)) t = e_c from the last row up and
// stores T(i, c), i <= c, at D[c * ld + i].  On entry G(i, r), i < r, is at
// D[r * ld + i].
__device__ __forceinline__ void wblock_t_full(float *D, int ld, const float *tau, int c, int lane) {
    float x[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = i == c ? 1.f : 0.f;
#pragma unroll
    for (int r = 31; r >= 0; --r) {
        const float xr = tau[r] * x[r];
        x[r] = xr;
        const float *Gc = D + r * ld;
#pragma unroll
        for (int i = 0; i < r; ++i) x[i] = fmaf(-Gc[i], xr, x[i]);
        // row r is finished here, and the next row's loads start after it: no
        // loaded value is kept live across rows
#pragma unroll
        for (int g = 0; g < 32; g += 8)
            asm volatile("" : "+v"(x[g]), "+v"(x[g + 1]), "+v"(x[g + 2]), "+v"(x[g + 3]), "+v"(x[g + 4]),
                         "+v"(x[g + 5]), "+v"(x[g + 6]), "+v"(x[g + 7])::"memory");
    }
    wave_lds_sync();
    if (lane < 32)
#pragma unroll
        for (int i = 0; i < 32; ++i)
            if (i <= c) D[c * ld + i] = x[i];
}

template <class B>
__global__ __launch_bounds__(kThreads) void k_eig_tridiag(B batch, int ld, int boff, int poff) {
    extern __shared__ float sm[];
    __shared__ float sd[kTriMaxN], se[kTriMaxN], stau[kTriMaxN];
    __shared__ float sx0[kTriMaxN], sx1[kTriMaxN], sp[kTriMaxN], sy[64];
    const JacItem &it = batch.it[blockIdx.x];
    const int n = it.n;
    // the wave index as a scalar: loops and branches on it stay uniform
    const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    float *A = sm;          // A[r * ld + c]; the reflectors in its rows after the reduction
    float *B1 = sm + boff;  // the panel's V and W
    constexpr int PS = kPanelStride;
    float *Vp = B1, *Wp = B1 + poff;

    // (A + A^T) / 2, eight entries of each thread in flight
    for (int e0 = tid; e0 < n * n; e0 += 8 * kThreads) {
        float x[8], y[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int e = min(e0 + u * kThreads, n * n - 1), r = e / n, c = e - r * n;
            x[u] = it.a[(size_t)r * it.lda + c];
            y[u] = it.a[(size_t)c * it.lda + r];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int e = e0 + u * kThreads;
            if (e < n * n) {
                const int r = e / n, c = e - r * n;
                A[r * ld + c] = 0.5f * (x[u] + y[u]);
            }
        }
    }

    // ---------------------------------------------------------------- 1. tridiagonalize
    // Blocked Householder reduction (Golub & Van Loan sec. 8.3.1 in the
    // panel form of LAPACK's latrd): within a panel of up to 32 columns the
    // trailing matrix is not updated; step j works on the current column
    //   x = A(j:, j) - V(j:, :jj) W(j, :jj)^T - W(j:, :jj) V(j, :jj)^T,
    // reflects x(j+1:) onto beta e_1 with H = I - tau v v^T (v unnormalised,
    // tau = 2 / v^T v), and appends v to V and
    //   w = p - (tau p^T v / 2) v,  p = tau (A22 - V W^T - W V^T) v
    // to W, with p^T v = tau (v^T A22 v - 2 (W^T v) . (V^T v)).  At the end of
    // the panel A22 -= V W^T + W V^T on MFMA.  Reflector j is kept in row j.
    float *sxa = sx0, *sxb = sx1;
    // Within a panel A22 is read-only, so each lane keeps its share in
    // registers for the panel's steps: lane l32 of half h of wave w holds
    // A(R_p, C_u), R_p = 2 w + h + 32 p, C_u = l32 + 32 u (p, u < 5).
    const int l32 = lane & 31, half = lane >> 5, hw = 2 * wid + half;
    for (int p0 = 0; p0 + 2 < n; p0 += 32) {
        const int nb = min(32, n - 2 - p0);
        __syncthreads();
        for (int r = p0 + tid; r < n; r += kThreads) sxa[r] = A[p0 * ld + r];
        float areg[5][5];
#pragma unroll
        for (int pp = 0; pp < 5; ++pp)
#pragma unroll
            for (int u = 0; u < 5; ++u) {
                const int R = hw + 32 * pp, C = l32 + 32 * u;
                areg[pp][u] = ld_or_zero(A, min(R, n - 1) * ld + min(C, n - 1), R < n && C < n);
            }
        for (int e = tid; e < (n - p0) * 32; e += kThreads) {
            const int r = p0 + (e >> 5), m = e & 31;
            Vp[r * PS + m] = 0.f;
            Wp[r * PS + m] = 0.f;
        }
        if (tid < 64) sy[tid] = 0.f;
        __syncthreads();
        for (int jj = 0; jj < nb; ++jj) {
            const int j = p0 + jj, s = n - j - 1;
            float part = 0.f;
#pragma unroll
            for (int t = 0; t < 3; ++t) {
                const int c = 1 + lane + 64 * t;
                const float x = ld_or_zero(sxa, j + 1 + min(c, s - 1), c < s);
                part = fmaf(x, x, part);
            }
            const float xn2 = wave_sum(part);     // identical in every wave
            const float x0 = sxa[j + 1];
            float beta = x0, v0 = 0.f, tau = 0.f;
            if (xn2 > 0.f) {
                const float alpha = sqrtf(x0 * x0 + xn2);
                beta = x0 >= 0.f ? -alpha : alpha;
                v0 = x0 - beta;
                tau = 2.f * __builtin_amdgcn_rcpf(v0 * v0 + xn2);
            }
            if (tid == 0) {
                sd[j] = sxa[j];
                se[j] = beta;
                stau[j] = tau;
            }
            for (int c = tid; c < s; c += kThreads) {
                const float vc = c == 0 ? v0 : sxa[j + 1 + c];
                Vp[(j + 1 + c) * PS + jj] = vc;
                A[j * ld + j + 1 + c] = vc;
            }
            // v in registers at the lanes' columns (zero outside j+1..n-1)
            float vr[5];
#pragma unroll
            for (int u = 0; u < 5; ++u) {
                const int C = l32 + 32 * u;
                vr[u] = C == j + 1 ? v0 : ld_or_zero(sxa, min(C, n - 1), C > j + 1 && C < n);
            }
            // sp = A22 v from the register copy (the panel's updates are not
            // applied to A22 yet): 5 products per row, then the sum over the
            // 32 lanes of the half (rows of 16 by DPP, then the lower row's
            // total from its lane 15 into the upper row)
            {
                float acc[5];
#pragma unroll
                for (int pp = 0; pp < 5; ++pp) {
                    float t = 0.f;
#pragma unroll
                    for (int u = 0; u < 5; ++u) t = fmaf(areg[pp][u], vr[u], t);
                    acc[pp] = t;
                }
#pragma unroll
                for (int pp = 0; pp < 5; ++pp) {
                    acc[pp] = group16_sum(acc[pp]);
                    acc[pp] += dpp_move<kDppRowBcast15>(acc[pp]);
                }
                if (l32 == 16)
#pragma unroll
                    for (int pp = 0; pp < 5; ++pp) {
                        const int R = hw + 32 * pp;
                        if (R > j && R < n) sp[R - j - 1] = acc[pp];
                    }
            }
            // sy[m] = (W^T v)_m, sy[32 + m] = (V^T v)_m: half-wave hw takes
            // outputs hw and hw + 32 of the 2 jj, over the same lane columns
#pragma unroll
            for (int oo = 0; oo < 2; ++oo) {
                const int o = hw + 32 * oo;
                if (o < 2 * jj) {
                    const float *vec = o < jj ? Wp + o : Vp + (o - jj);
                    float acc = 0.f;
#pragma unroll
                    for (int u = 0; u < 5; ++u) {
                        const int C = l32 + 32 * u;
                        acc = fmaf(ld_or_zero(vec, min(C, n - 1) * PS, C > j && C < n), vr[u], acc);
                    }
                    acc = group16_sum(acc);
                    acc += dpp_move<kDppRowBcast15>(acc);
                    if (l32 == 16) sy[o < jj ? o : 32 + (o - jj)] = acc;
                }
            }
            __syncthreads();
            // p = tau (A22 v - V W^T v - W V^T v), w = p - hk v, and the next column
            // x = A(:, j+1) - V W(j+1, :)^T - W V(j+1, :)^T; 4 lanes per row share
            // the sums over the panel's previous columns m (m = l4 mod 4)
            float kp = 0.f;
#pragma unroll
            for (int t = 0; t < 3; ++t) {
                const int c = lane + 64 * t, cc = min(c, s - 1);
                const float vc = c == 0 ? v0 : sxa[j + 1 + cc];
                kp = fmaf(ld_or_zero(sp, cc, c < s), vc, kp);
            }
            kp = wave_sum(kp);
            const bool next = jj + 1 < nb;
            // waves past the last row skip; all 8 sums over m are issued at once
            // (the panel's V, W and the dot slots past jj hold zeros, and
            // column jj of row j+1 is masked: it is written in this part)
            if (16 * wid < s) {
                const int l4 = tid & 3, c = tid >> 2, r = j + 1 + c, rc = min(r, n - 1);
                const bool live = c < s;
                float cw = 0.f, cx = 0.f, cw1 = 0.f, yy = 0.f;
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const int m = l4 + 4 * t;
                    const bool on = m < jj;
                    const float y1 = sy[m], y2 = sy[32 + m];
                    const float bv = ld_or_zero(Vp, (j + 1) * PS + m, on);
                    const float bw = ld_or_zero(Wp, (j + 1) * PS + m, on);
                    const float rv = Vp[rc * PS + m], rw = Wp[rc * PS + m];
                    yy = fmaf(y1, y2, yy);
                    cw1 = fmaf(bv, y1, fmaf(bw, y2, cw1));
                    cw = fmaf(rv, y1, fmaf(rw, y2, cw));
                    cx = fmaf(rv, bw, fmaf(rw, bv, cx));
                }
                cw = group4_sum(cw);
                cx = group4_sum(cx);
                cw1 = group4_sum(cw1);
                yy = group4_sum(yy);
                const float hk = 0.5f * tau * (tau * (kp - 2.f * yy));
                if (live && l4 == 0) {
                    const float vc = c == 0 ? v0 : sxa[r];
                    const float w = tau * (sp[c] - cw) - hk * vc;
                    Wp[r * PS + jj] = w;
                    if (next) {
                        const float w0 = tau * (sp[0] - cw1) - hk * v0;
                        sxb[r] = A[(j + 1) * ld + r] - cx - fmaf(vc, w0, w * v0);
                    }
                }
            }
            float *t = sxa;
            sxa = sxb;
            sxb = t;
            __syncthreads();
        }
        // trailing update A22 -= V W^T + W V^T (rows, columns >= q0), K = 2 nb
        const int q0 = p0 + nb;
        const int tt = (n - q0 + 31) >> 5, ntl = tt * tt;
        for (int t = wid; t < ntl; t += kWaves) {
            const int R0 = q0 + 32 * (t / tt), C0 = q0 + 32 * (t % tt);
            const int rr = R0 + (lane & 31), cc = C0 + (lane & 31), kh = lane >> 5;
            const int rc = min(rr, n - 1), ccl = min(cc, n - 1);
            f32x16 acc;
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int row = R0 + frag_row(lane, q);
                acc[q] = ld_or_zero(A, min(row, n - 1) * ld + ccl, row < n && cc < n);
            }
            for (int k0 = 0; k0 < 2 * nb; k0 += 2) {
                const int k = k0 + kh;
                const bool first = k < nb;
                const int m = first ? k : k - nb;
                const float a = -ld_or_zero(first ? Vp : Wp, rc * PS + m, rr < n);
                const float b = ld_or_zero(first ? Wp : Vp, ccl * PS + m, cc < n);
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
            }
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int row = R0 + frag_row(lane, q);
                if (row < n && cc < n) A[row * ld + cc] = acc[q];
            }
        }
    }
    __syncthreads();
    if (tid == 0) {
        if (n >= 2) {
            sd[n - 2] = A[(n - 2) * ld + n - 2];
            se[n - 2] = A[(n - 2) * ld + n - 1];
        }
        sd[n - 1] = A[(n - 1) * ld + n - 1];
    }
    __syncthreads();

    // hand over to k_eig_trivec and k_eig_backtr: A (reflectors in its rows),
    // T = (d, e) and tau; the fail flag starts clear
    const TriWs w = tri_ws(it.tw, n);
    for (int e = tid; e < n * w.np; e += kThreads) {
        const int r = e / w.np, c = e - r * w.np;
        w.a[e] = c < n ? A[r * ld + c] : 0.f;
    }
    for (int i = tid; i < n; i += kThreads) {
        w.d[i] = sd[i];
        w.e[i] = i + 1 < n ? se[i] : 0.f;
        w.tau[i] = i + 2 < n ? stau[i] : 0.f;
    }
    if (tid == 0) *w.flag = 0;
}

// ---------------------------------------------------------------- 1 (wide). tridiagonalize, 140 < n <= 272
// The same blocked reduction for matrices too large for LDS: the whole matrix
// stays in the registers of a 512-thread workgroup (two waves per SIMD, so up
// to 256 registers per lane) for the entire reduction.  Lane l32 of half h of
// wave w (hw = 2 w + h) holds A(R_p, C_u), R_p = hw + 16 p (p < 17), C_u =
// l32 + 32 u (u < 9).  Per panel the 32 panel columns go to LDS (Xp), the
// steps run as in k_eig_tridiag with the matrix-vector products from the
// registers, and the panel's rank-64 update A22 -= V W^T + W V^T is applied in
// the registers.  Reflectors go straight to the workspace rows.
constexpr int kWThreads = 512;
constexpr int kWRows = 17;
constexpr int kWCols = 9;
constexpr int kXpPitch = 33;
constexpr size_t kWTriLds = ((size_t)kWideMaxN * (kXpPitch + 2 * kPanelStride) + 6 * kWideMaxN + 64) * 4;

template <class B>
__global__ __launch_bounds__(kWThreads) void k_eig_tridiag_w(B batch) {
    extern __shared__ float sm[];
    const JacItem &it = batch.it[blockIdx.x];
    const int n = it.n;
    const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hw = 2 * wid + (lane >> 5);
    constexpr int PS = kPanelStride;
    float *Xp = sm;                              // panel columns: Xp[r * 33 + m] = A(r, p0 + m)
    float *Vp = Xp + kWideMaxN * kXpPitch;       // the panel's V and W
    float *Wp = Vp + kWideMaxN * PS;
    float *sx0 = Wp + kWideMaxN * PS, *sx1 = sx0 + kWideMaxN, *sp = sx1 + kWideMaxN;
    float *sd = sp + kWideMaxN, *se = sd + kWideMaxN, *stau = se + kWideMaxN, *sy = stau + kWideMaxN;
    const TriWs w = tri_ws(it.tw, n);

    // (A + A^T) / 2 into the registers
    float areg[kWRows][kWCols];
#pragma unroll
    for (int pp = 0; pp < kWRows; ++pp)
#pragma unroll
        for (int u = 0; u < kWCols; ++u) {
            const int R = hw + 16 * pp, C = l32 + 32 * u;
            const bool ok = R < n && C < n;
            const int Rc = min(R, n - 1), Cc = min(C, n - 1);
            const float x = it.a[(size_t)Rc * it.lda + Cc], y = it.a[(size_t)Cc * it.lda + Rc];
            areg[pp][u] = ok ? 0.5f * (x + y) : 0.f;
        }

    float *sxa = sx0, *sxb = sx1;
    for (int p0 = 0; p0 + 2 < n; p0 += 32) {
        const int nb = min(32, n - 2 - p0);
        const int up = p0 >> 5;
        __syncthreads();
        // the panel's columns from the registers (column block up of every lane)
#pragma unroll
        for (int pp = 0; pp < kWRows; ++pp) {
            const int R = hw + 16 * pp;
            float v = 0.f;
#pragma unroll
            for (int u = 0; u < kWCols; ++u) v = u == up ? areg[pp][u] : v;
            if (R < n && R >= p0) Xp[R * kXpPitch + l32] = v;
        }
        for (int e = tid; e < (n - p0) * 32; e += kWThreads) {
            const int r = p0 + (e >> 5), m = e & 31;
            Vp[r * PS + m] = 0.f;
            Wp[r * PS + m] = 0.f;
        }
        if (tid < 64) sy[tid] = 0.f;
        __syncthreads();
        for (int r = p0 + tid; r < n; r += kWThreads) sxa[r] = Xp[r * kXpPitch];
        __syncthreads();
        for (int jj = 0; jj < nb; ++jj) {
            const int j = p0 + jj, s = n - j - 1;
            float part = 0.f;
#pragma unroll
            for (int t = 0; t < 5; ++t) {
                const int c = 1 + lane + 64 * t;
                const float x = ld_or_zero(sxa, j + 1 + min(c, s - 1), c < s);
                part = fmaf(x, x, part);
            }
            const float xn2 = wave_sum(part);
            const float x0 = sxa[j + 1];
            float beta = x0, v0 = 0.f, tau = 0.f;
            if (xn2 > 0.f) {
                const float alpha = sqrtf(x0 * x0 + xn2);
                beta = x0 >= 0.f ? -alpha : alpha;
                v0 = x0 - beta;
                tau = 2.f * __builtin_amdgcn_rcpf(v0 * v0 + xn2);
            }
            if (tid == 0) {
                sd[j] = sxa[j];
                se[j] = beta;
                stau[j] = tau;
            }
            for (int c = tid; c < s; c += kWThreads) {
                const float vc = c == 0 ? v0 : sxa[j + 1 + c];
                Vp[(j + 1 + c) * PS + jj] = vc;
                w.a[(size_t)j * w.np + j + 1 + c] = vc;
            }
            float vr[kWCols];
#pragma unroll
            for (int u = 0; u < kWCols; ++u) {
                const int C = l32 + 32 * u;
                vr[u] = C == j + 1 ? v0 : ld_or_zero(sxa, min(C, n - 1), C > j + 1 && C < n);
            }
            // sp = A22 v from the registers: 9 products per row, then the sum over
            // the 32 lanes of the half (rows of 16 by DPP, the lower row's total
            // from its lane 15 into the upper row)
#pragma unroll
            for (int pp = 0; pp < kWRows; ++pp) {
                float t = 0.f;
#pragma unroll
                for (int u = 0; u < kWCols; ++u) t = fmaf(areg[pp][u], vr[u], t);
                t = group16_sum(t);
                t += dpp_move<kDppRowBcast15>(t);
                const int R = hw + 16 * pp;
                if (l32 == 16 && R > j && R < n) sp[R - j - 1] = t;
            }
            // sy[m] = (W^T v)_m, sy[32 + m] = (V^T v)_m: half-wave hw takes outputs
            // hw + 16 oo of the 2 jj
#pragma unroll
            for (int oo = 0; oo < 4; ++oo) {
                const int o = hw + 16 * oo;
                if (o < 2 * jj) {
                    const float *vec = o < jj ? Wp + o : Vp + (o - jj);
                    float acc = 0.f;
#pragma unroll
                    for (int u = 0; u < kWCols; ++u) {
                        const int C = l32 + 32 * u;
                        acc = fmaf(ld_or_zero(vec, min(C, n - 1) * PS, C > j && C < n), vr[u], acc);
                    }
                    acc = group16_sum(acc);
                    acc += dpp_move<kDppRowBcast15>(acc);
                    if (l32 == 16) sy[o < jj ? o : 32 + (o - jj)] = acc;
                }
            }
            __syncthreads();
            float kp = 0.f;
#pragma unroll
            for (int t = 0; t < 5; ++t) {
                const int c = lane + 64 * t, cc = min(c, s - 1);
                const float vc = c == 0 ? v0 : sxa[j + 1 + cc];
                kp = fmaf(ld_or_zero(sp, cc, c < s), vc, kp);
            }
            kp = wave_sum(kp);
            const bool next = jj + 1 < nb;
            // w and the next column, 4 lanes per row, 128 rows per pass
            for (int cb = 0; cb < s; cb += kWThreads / 4) {
                if (cb + 16 * wid >= s) break;
                const int l4 = tid & 3, c = cb + (tid >> 2), r = j + 1 + c, rc = min(r, n - 1);
                const bool live = c < s;
                float cw = 0.f, cx = 0.f, cw1 = 0.f, yy = 0.f;
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const int m = l4 + 4 * t;
                    const bool on = m < jj;
                    const float y1 = sy[m], y2 = sy[32 + m];
                    const float bv = ld_or_zero(Vp, (j + 1) * PS + m, on);
                    const float bw = ld_or_zero(Wp, (j + 1) * PS + m, on);
                    const float rv = Vp[rc * PS + m], rw = Wp[rc * PS + m];
                    yy = fmaf(y1, y2, yy);
                    cw1 = fmaf(bv, y1, fmaf(bw, y2, cw1));
                    cw = fmaf(rv, y1, fmaf(rw, y2, cw));
                    cx = fmaf(rv, bw, fmaf(rw, bv, cx));
                }
                cw = group4_sum(cw);
                cx = group4_sum(cx);
                cw1 = group4_sum(cw1);
                yy = group4_sum(yy);
                const float hk = 0.5f * tau * (tau * (kp - 2.f * yy));
                if (live && l4 == 0) {
                    const float vc = c == 0 ? v0 : sxa[r];
                    const float wv = tau * (sp[c] - cw) - hk * vc;
                    Wp[r * PS + jj] = wv;
                    if (next) {
                        const float w0 = tau * (sp[0] - cw1) - hk * v0;
                        sxb[r] = Xp[r * kXpPitch + jj + 1] - cx - fmaf(vc, w0, wv * v0);
                    }
                }
            }
            float *t = sxa;
            sxa = sxb;
            sxb = t;
            __syncthreads();
        }
        // A22 -= V W^T + W V^T in the registers, rows and columns >= q0
        const int q0 = p0 + nb;
        for (int m = 0; m < nb; ++m) {
            float cv[kWCols], cwv[kWCols];
#pragma unroll
            for (int u = 0; u < kWCols; ++u) {
                const int C = l32 + 32 * u;
                const bool ok = C >= q0 && C < n;
                cv[u] = ld_or_zero(Vp, min(C, n - 1) * PS + m, ok);
                cwv[u] = ld_or_zero(Wp, min(C, n - 1) * PS + m, ok);
            }
#pragma unroll
            for (int pp = 0; pp < kWRows; ++pp) {
                if (16 * pp + 15 < q0) continue;
                const int R = hw + 16 * pp;
                const bool ok = R >= q0 && R < n;
                const float rv = ld_or_zero(Vp, min(R, n - 1) * PS + m, ok);
                const float rw = ld_or_zero(Wp, min(R, n - 1) * PS + m, ok);
#pragma unroll
                for (int u = 0; u < kWCols; ++u) areg[pp][u] = fmaf(-rv, cwv[u], fmaf(-rw, cv[u], areg[pp][u]));
            }
        }
    }
    __syncthreads();
    // the trailing 2 x 2 block from the registers
#pragma unroll
    for (int pp = 0; pp < kWRows; ++pp)
#pragma unroll
        for (int u = 0; u < kWCols; ++u) {
            const int R = hw + 16 * pp, C = l32 + 32 * u;
            if (R == n - 2 && C == n - 2) sd[n - 2] = areg[pp][u];
            if (R == n - 2 && C == n - 1) se[n - 2] = areg[pp][u];
            if (R == n - 1 && C == n - 1) sd[n - 1] = areg[pp][u];
        }
    __syncthreads();
    for (int i = tid; i < n; i += kWThreads) {
        w.d[i] = sd[i];
        w.e[i] = i + 1 < n ? se[i] : 0.f;
        w.tau[i] = i + 2 < n ? stau[i] : 0.f;
    }
    if (tid == 0) *w.flag = 0;
}

// ---------------------------------------------------------------- 2 + 3. eigenpairs of T
// Every eigenpair of the tridiagonal T = (d, e) that k_eig_tridiag left in the
// workspace, a group of 16 lanes per eigenvalue k (the k-th smallest), four
// groups per wave, so that a batch spreads over the chip:
//   2. multisection on Sturm counts (Golub & Van Loan sec. 8.4.1): the group's
//      16 lanes count at the 16 inner points of 17 equal sections of the
//      interval [a, b) that holds it (count(a) <= k < count(b), count(x) =
//      #{i : q_i(x) < 0}); the interval shrinks to the section that starts
//      below the first point whose count exceeds k, to a relative width of
//      2 eps (floored at eps ||T|| / 1024: vectors of close eigenvalues stay
//      near orthogonal only with accurate shifts);
//   3. the eigenvector from a twisted factorization of T - lambda I (Dhillon &
//      Parlett, Orthogonal eigenvectors and relative gaps, 2004): lanes 0 and 1
//      of the group run the forward and backward LDL^T pivots side by side,
//      the group finds the twist index r where |gamma| is smallest (the first
//      such index) and the factors of the one-sided recurrences, lanes 0 and 1
//      run their products up and down from z_r = 1, and the group normalises.
// The sequential recurrences read LDS in batches of 8.  Writes lambda_k and
// row k of Z^T; sets the fail flag when a vector overflows.
constexpr int kVecWaves = 1;                          // one-wave workgroups spread evenly
constexpr int kVecGroup = 16;                           // lanes per eigenvalue
constexpr int kVecPerWave = 64 / kVecGroup;
// sizes for matrices of order <= NMAX (kTriMaxN or kWideMaxN)
template <int NMAX>
struct VecDims {
    static constexpr int kVecPad = NMAX + 24;           // room for the batch reads past the end
    // LDS in floats of one k_eig_trivec workgroup (the eigenpair arrays) and of
    // one k_eig_wy workgroup (a block's G / T buffer and its tau)
    static constexpr int kLdsEig = 4 * kVecPad + kVecPerWave * 2 * NMAX;
    static constexpr int kLdsWy = 32 * 33 + 32;
};

// T of reflector block b for k_eig_backtr, one wave (the T role of
// k_eig_trivec): G = Y^T Y of the block's 32 reflectors (Y(r, i) = v_{b0+i}(r),
// zero for r <= b0 + i), then (diag(1 / tau) + strict_upper(G)) T = I column
// by column (wblock_t_full).  A partial last block is padded with zero
// reflectors of tau = 0, whose rows and columns of T come out zero.
// The reflectors are read straight from the workspace rows (reflector i of the
// block is row b0 + i, 16-byte aligned): lane (i, kh) loads 4 consecutive
// entries of row i and supplies the K index kh of two consecutive MFMA steps.
template <int NMAX>
__device__ void wy_block(const TriWs &w, int n, int b, float *lds, int lane) {
    const int mref = max(n - 2, 0), b0 = 32 * b, nbk = min(32, mref - b0);
    float *D = lds;                     // G(i, c), i < c, then T(i, c), i <= c, at D[c * 33 + i]
    float *taus = D + 32 * 33;
    if (lane < 32) taus[lane] = lane < nbk ? w.tau[b0 + lane] : 0.f;
    const int m32 = lane & 31, kh = lane >> 5;
    const bool iv = m32 < nbk;
    const float *yrow = w.a + (size_t)(b0 + (iv ? m32 : 0)) * w.np;
    f32x16 g = {};
    for (int k0 = b0; k0 < n; k0 += 4) {            // k0 + 3 < np: rows are n rounded up to 4
        const float4 v = *reinterpret_cast<const float4 *>(yrow + k0);
        const float e0 = kh ? v.y : v.x, e1 = kh ? v.w : v.z;
        const int r0 = k0 + kh, r1 = k0 + 2 + kh;
        const float y0 = iv && r0 > b0 + m32 && r0 < n ? e0 : 0.f;
        const float y1 = iv && r1 > b0 + m32 && r1 < n ? e1 : 0.f;
        g = __builtin_amdgcn_mfma_f32_32x32x2f32(y0, y0, g, 0, 0, 0);
        g = __builtin_amdgcn_mfma_f32_32x32x2f32(y1, y1, g, 0, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int r = frag_row(lane, q);
        if (r < m32) D[m32 * 33 + r] = g[q];
    }
    wave_lds_sync();
    wblock_t_full(D, 33, taus, m32, lane);
    wave_lds_sync();
    float *tb = w.tb + 1024 * b;
    for (int e = lane; e < 1024; e += 64) {
        const int i = e >> 5, c = e & 31;
        tb[e] = i <= c ? D[c * 33 + i] : 0.f;
    }
}

// The compact-WY T blocks for k_eig_backtr, one wave per block of 32 reflectors
// (a launch of its own: its LDS, which the eigenpair workgroups do not need,
// would otherwise be reserved for every one of them and cut their occupancy).
template <int NMAX, class B>
__global__ __launch_bounds__(64) void k_eig_wy(B batch) {
    __shared__ __attribute__((aligned(16))) float lds[VecDims<NMAX>::kLdsWy];
    const JacItem &it = batch.it[blockIdx.y];
    const int n = it.n;
    const TriWs w = tri_ws(it.tw, n);
    if ((int)blockIdx.x < tri_blocks(n)) wy_block<NMAX>(w, n, blockIdx.x, lds, threadIdx.x & 63);
}

template <int NMAX, class B>
__global__ __launch_bounds__(64 * kVecWaves) void k_eig_trivec(B batch) {
    constexpr int kTriMaxN = NMAX, kVecPad = VecDims<NMAX>::kVecPad;
    __shared__ __attribute__((aligned(16))) float lds[VecDims<NMAX>::kLdsEig];
    const JacItem &it = batch.it[blockIdx.y];
    const int n = it.n;
    const TriWs w = tri_ws(it.tw, n);
    const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    constexpr int kPerBlock = kVecWaves * kVecPerWave;
    if ((int)blockIdx.x * kPerBlock >= n) return;
    float *sd = lds, *se = sd + kVecPad;
    float2 *sde = reinterpret_cast<float2 *>(se + kVecPad);      // {d_i, e_{i-1}^2}
    // [wave][group][2][kTriMaxN]: the pivots, then the eigenvector in their place
    float *piv = reinterpret_cast<float *>(sde + kVecPad);
    for (int i = tid; i < kVecPad; i += 64 * kVecWaves) {
        const float di = i < n ? w.d[i] : 0.f, em = i > 0 && i < n ? w.e[i - 1] : 0.f;
        sd[i] = di;
        se[i] = i < n ? w.e[i] : 0.f;
        sde[i] = make_float2(di, em * em);
    }
    __syncthreads();
    const int g = lane / kVecGroup, q = lane % kVecGroup;
    const int kw = blockIdx.x * kPerBlock + wid * kVecPerWave;     // the wave's first eigenvalue
    if (kw >= n) return;
    const int k = kw + g;
    const bool kv = k < n;

    float glo = FLT_MAX, ghi = -FLT_MAX;
    for (int i = lane; i < n; i += 64) {
        const float rad = (i > 0 ? fabsf(se[i - 1]) : 0.f) + (i + 1 < n ? fabsf(se[i]) : 0.f);
        glo = fminf(glo, sd[i] - rad);
        ghi = fmaxf(ghi, sd[i] + rad);
    }
    glo = wave_min(glo);
    ghi = wave_max(ghi);
    const float eps = FLT_EPSILON;
    const float tnorm = fmaxf(fmaxf(fabsf(glo), fabsf(ghi)), FLT_MIN);
    const float pivmin = fmaxf(FLT_MIN, tnorm * eps * eps);
    const float floor_tol = eps * tnorm * (1.f / 1024.f);
    // a and b are the same in the lanes of a group; lane q counts at a + (q + 1) (b - a) / 17
    float a = glo - (4.f * eps * tnorm + pivmin), b = ghi + (4.f * eps * tnorm + pivmin);
    const unsigned long long gmask = 0xFFFFull << (kVecGroup * g);
    for (int round = 0; round < 24; ++round) {
        const bool open = kv && b - a > 2.f * eps * fmaxf(fabsf(a), fabsf(b)) + floor_tol;
        if (!__ballot(open)) break;
        const float wd = (b - a) * (1.f / (kVecGroup + 1));
        const float x = a + wd * (float)(q + 1);
        // q_i = (d_i - x) - e_{i-1}^2 / q_{i-1}; a |q_i| below pivmin counts as -pivmin
        int cnt = 0;
        float qv = 1.f;
        auto step = [&](float2 de) {
            qv = fmaf(-de.y, __builtin_amdgcn_rcpf(qv), de.x - x);
            if (fabsf(qv) < pivmin) qv = -pivmin;
            cnt += (int)(__float_as_uint(qv) >> 31);
        };
        // batches of 8 from LDS, alternating between two register sets so that
        // one is read while the other is used (reads past n hit the padding)
        float2 ba[8], bb[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) ba[u] = sde[u];
        int i0 = 0;
        for (; i0 + 16 <= n; i0 += 16) {
#pragma unroll
            for (int u = 0; u < 8; ++u) bb[u] = sde[i0 + 8 + u];
#pragma unroll
            for (int u = 0; u < 8; ++u) step(ba[u]);
#pragma unroll
            for (int u = 0; u < 8; ++u) ba[u] = sde[i0 + 16 + u];
#pragma unroll
            for (int u = 0; u < 8; ++u) step(bb[u]);
        }
        if (i0 + 8 <= n) {
#pragma unroll
            for (int u = 0; u < 8; ++u) bb[u] = sde[i0 + 8 + u];
#pragma unroll
            for (int u = 0; u < 8; ++u) step(ba[u]);
#pragma unroll
            for (int u = 0; u < 7; ++u)
                if (i0 + 8 + u < n) step(bb[u]);
        } else {
#pragma unroll
            for (int u = 0; u < 7; ++u)
                if (i0 + u < n) step(ba[u]);
        }
        // first point of the group past the k-th eigenvalue (kVecGroup if none)
        const unsigned long long past = (__ballot(cnt > k) & gmask) >> (kVecGroup * g);
        const int m = past ? __ffsll((long long)past) - 1 : kVecGroup;
        if (open) {
            const float na = m > 0 ? a + wd * (float)m : a;
            const float nb = m < kVecGroup ? a + wd * (float)(m + 1) : b;
            a = na;
            b = nb;
        }
    }
    const float lam = 0.5f * (a + b);

    // pivots of T - lam I = L+ D+ L+^T (lane 0 of the group, i upwards) and
    // U- D- U-^T (lane 1, i downwards), both in step order s: step s of lane 1
    // takes row n-1-s (d from sde[n-1-s], e^2 of the pair below it from
    // sde[n-s], none at step 0), and P[1][s] = D-_{n-1-s}
    float *P = piv + (wid * kVecPerWave + g) * 2 * kTriMaxN;
    if (kv && q < 2) {
        float *ps = P + q * kTriMaxN;
        const float *sdx = reinterpret_cast<const float *>(sde), *sdy = sdx + 1;
        // float offsets of row x(s) = s or n-1-s and of the e^2 entry e(s) = s or n-s
        const int x0 = q ? 2 * (n - 1) : 0, e0 = q ? 2 * n : 0, dx = q ? -2 : 2;
        float p = 1.f;     // step 0 has e^2 = 0: p = d - lam
        auto step = [&](float xv, float ev) {
            p = fmaf(-ev, __builtin_amdgcn_rcpf(p), xv - lam);
            if (fabsf(p) < pivmin) p = -pivmin;
            return p;
        };
        int s0 = 0;
        for (; s0 + 8 <= n; s0 += 8) {
            float xv[8], ev[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                xv[u] = sdx[x0 + dx * (s0 + u)];
                ev[u] = sdy[e0 + dx * (s0 + u)];
            }
            if (s0 == 0) ev[0] = 0.f;
#pragma unroll
            for (int u = 0; u < 8; ++u) ps[s0 + u] = step(xv[u], ev[u]);
        }
        for (; s0 < n; ++s0) ps[s0] = step(sdx[x0 + dx * s0], s0 == 0 ? 0.f : sdy[e0 + dx * s0]);
    }
    wave_lds_sync();
    // twist index r: the first i where |gamma_i| is smallest, gamma_i =
    // D+_i + D-_i - (d_i - lam) for i < n - 1 and gamma_{n-1} = D+_{n-1}; each
    // lane of the group takes i = q mod 16, then the group reduces (value,
    // index) pairs
    float best = FLT_MAX;
    int r = n - 1;
    if (kv) {
        for (int i = q; i < n; i += kVecGroup) {
            const float gv = i == n - 1 ? fabsf(P[i]) : fabsf(P[i] + P[kTriMaxN + n - 1 - i] - (sd[i] - lam));
            if (gv < best || (gv == best && i < r)) {
                best = gv;
                r = i;
            }
        }
    }
#pragma unroll
    for (int off = 1; off < kVecGroup; off <<= 1) {
        const float ob = __shfl_xor(best, off);
        const int orr = __shfl_xor(r, off);
        if (ob < best || (ob == best && orr < r)) {
            best = ob;
            r = orr;
        }
    }
    // z_r = 1; z_i = f_i z_{i+1} above r with f_i = -(e_i / D+_i), z_i = f_i z_{i-1}
    // below with f_i = -(e_{i-1} / D-_i): the factors by the whole group, the
    // running products by lanes 0 (up) and 1 (down).  Each factor and product
    // takes the place of the pivot it came from: z_i at P[i] for i <= r and at
    // P[1][n-1-i] for i > r, so both lanes walk their half downwards.
    if (kv) {
        for (int i = q; i < n; i += kVecGroup) {
            if (i < r) {
                P[i] = -(se[i] * __builtin_amdgcn_rcpf(P[i]));
            } else if (i > r) {
                float *pb = P + kTriMaxN + n - 1 - i;
                *pb = -(se[i - 1] * __builtin_amdgcn_rcpf(*pb));
            } else {
                P[r] = 1.f;
            }
        }
    }
    wave_lds_sync();
    if (kv && q < 2) {
        float *zb = P + q * kTriMaxN;
        const int len = q == 0 ? r : n - 1 - r;
        int j = q == 0 ? r - 1 : n - 2 - r;      // the first entry of the walk
        float zz = 1.f;
        int s0 = 0;
        for (; s0 + 8 <= len; s0 += 8) {
            float fv[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) fv[u] = zb[j - u];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                zz = fv[u] * zz;
                zb[j - u] = zz;
            }
            j -= 8;
        }
        for (; s0 < len; ++s0, --j) {
            zz = zb[j] * zz;
            zb[j] = zz;
        }
    }
    wave_lds_sync();
    auto zval = [&](int i) { return i <= r ? P[i] : P[kTriMaxN + n - 1 - i]; };
    float ss = 0.f;
    if (kv)
        for (int i = q; i < n; i += kVecGroup) {
            const float zi = zval(i);
            ss += zi * zi;
        }
    const float nrm = group16_sum(ss);
    if (!kv) return;
    if (!(nrm < FLT_MAX) && q == 0) *w.flag = 1;
    const float inv = 1.f / sqrtf(nrm);
    for (int i = q; i < w.np; i += kVecGroup) w.zt[(size_t)k * w.np + i] = i < n ? zval(i) * inv : 0.f;
    if (q == 0) w.lam[k] = lam;
}

// ---------------------------------------------------------------- 4. V = Q Z
// Q = H_0 H_1 ... H_{n-3} applied to Z a block of 32 reflectors at a time,
// last block first, in compact WY form: H_b0 ... H_b0+31 = I - Y T Y^T
// (Schreiber & Van Loan's storage-efficient WY, T from the T role of
// k_eig_trivec), Z <- Z - Y (T (Y^T Z)).  Columns of Z are independent, so one
// workgroup takes a chunk of 32 columns of one matrix: per block, its waves
// split the rows of S = Y^T Z_c, wave 0 forms M = T S, and the waves update
// the row tiles Z_c -= Y M.  V_c goes back over Z_c^T in the workspace.
constexpr int kBtWaves = 4;
constexpr int kTile = 32 * 33;                          // a 32 x 32 LDS tile, row pitch 33
template <class B>
__global__ __launch_bounds__(64 * kBtWaves) void k_eig_backtr(B batch, int ldy) {
    extern __shared__ float sm[];
    const JacItem &it = batch.it[blockIdx.y];
    const int n = it.n, c0 = 32 * blockIdx.x;
    if (c0 >= n) return;
    const TriWs w = tri_ws(it.tw, n);
    if (*w.flag) return;                                // k_eig_polish reports it
    const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int m32 = lane & 31, kh = lane >> 5;
    const int mref = max(n - 2, 0), nblk = tri_blocks(n), nt = (n + 31) >> 5;
    float *Ys = sm;                      // Ys[j * ldy + r] = v_j(r) for r > j (row j of A)
    float *Ts = Ys + mref * ldy;         // T_b(i, k) at Ts[b * kTile + i * 33 + k]
    float *Zc = Ts + nblk * kTile;       // Z(r, c0 + m) at Zc[r * 33 + m]
    float *Pt = Zc + n * 33;             // partial S of wave w: S(i, m) at Pt[w * kTile + i * 33 + m]
    float *Mt = Pt + kBtWaves * kTile;   // M(k, m) at Mt[k * 33 + m]
    constexpr int NT = 64 * kBtWaves;
    const int c4 = w.np >> 2, ncol = min(32, n - c0);
    load_rows4<NT, 8>(w.a, w.np, mref, c4, tid, [&](int r, int c, float4 v) {
        float *d = Ys + r * ldy + 4 * c;
        d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
    });
    load_rows4<NT, 8>(w.tb, 32, 32 * nblk, 8, tid, [&](int r, int c, float4 v) {
        float *d = Ts + (r >> 5) * kTile + (r & 31) * 33 + 4 * c;
        d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
    });
    // Z(r, c0 + m) = Z^T(c0 + m, r); columns past n read as zero
    for (int e = tid; e < (32 - ncol) * n; e += NT) {
        const int m = ncol + e / n, r = e - (e / n) * n;
        Zc[r * 33 + m] = 0.f;
    }
    load_rows4<NT, 8>(w.zt + (size_t)c0 * w.np, w.np, ncol, c4, tid, [&](int m, int c, float4 v) {
        const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (4 * c + i < n) Zc[(4 * c + i) * 33 + m] = vv[i];
    });
    __syncthreads();
    // Y(r, b0 + i): reflector b0 + i at row r, zero unless b0 + i < mref and b0 + i < r < n
    auto Y = [&](int b0, int r, int i) {
        const int j = b0 + i;
        return ld_or_zero(Ys, min(j, mref - 1) * ldy + min(r, n - 1), j < mref && r > j && r < n);
    };
    for (int b = nblk - 1; b >= 0; --b) {
        const int b0 = 32 * b;
        // S = Y_b^T Z_c over rows b0 + 1 .. n - 1, split in runs of 8 rows over the waves
        {
            const int rows = n - 1 - b0, per = ((rows + 8 * kBtWaves - 1) / (8 * kBtWaves)) * 8;
            const int r0 = b0 + 1 + wid * per, r1 = min(n, r0 + per);
            f32x16 acc = {};
            for (int k0 = r0; k0 < r1; k0 += 8) {
                float ya[4], zb[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int r = k0 + 2 * u + kh;
                    const bool ok = r < r1;
                    ya[u] = ok ? Y(b0, r, m32) : 0.f;
                    zb[u] = ld_or_zero(Zc, min(r, n - 1) * 33 + m32, ok);
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(ya[u], zb[u], acc, 0, 0, 0);
            }
#pragma unroll
            for (int q = 0; q < 16; ++q) Pt[wid * kTile + frag_row(lane, q) * 33 + m32] = acc[q];
        }
        __syncthreads();
        if (wid == 0) {
            // M = T_b S, S the sum of the partials (T_b is upper triangular)
            const float *T = Ts + b * kTile;
            f32x16 acc = {};
#pragma unroll
            for (int k0 = 0; k0 < 32; k0 += 8) {
                float ta[4], sb[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int k = k0 + 2 * u + kh;
                    ta[u] = T[m32 * 33 + k];
                    float sv = 0.f;
#pragma unroll
                    for (int v = 0; v < kBtWaves; ++v) sv += Pt[v * kTile + k * 33 + m32];
                    sb[u] = sv;
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(ta[u], sb[u], acc, 0, 0, 0);
            }
#pragma unroll
            for (int q = 0; q < 16; ++q) Mt[frag_row(lane, q) * 33 + m32] = acc[q];
        }
        __syncthreads();
        // Z_c -= Y_b M on the row tiles that Y_b touches (rows > b0)
        for (int rt = b + wid; rt < nt; rt += kBtWaves) {
            f32x16 acc;
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int row = 32 * rt + frag_row(lane, q);
                acc[q] = ld_or_zero(Zc, min(row, n - 1) * 33 + m32, row < n);
            }
#pragma unroll
            for (int k0 = 0; k0 < 32; k0 += 8) {
                float ya[4], mb[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int k = k0 + 2 * u + kh;
                    ya[u] = -Y(b0, 32 * rt + m32, k);
                    mb[u] = Mt[k * 33 + m32];
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(ya[u], mb[u], acc, 0, 0, 0);
            }
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int row = 32 * rt + frag_row(lane, q);
                if (row < n) Zc[row * 33 + m32] = acc[q];
            }
        }
        __syncthreads();
    }
    for (int e = tid; e < ncol * n; e += NT) {
        const int m = e / n, r = e - m * n;
        w.zt[(size_t)(c0 + m) * w.np + r] = Zc[r * 33 + m];
    }
}

// The back-transform for the wide solver: the reflectors are read straight
// from the workspace rows (L2-resident; all of them would not fit in LDS next to
// the columns of Z), the block's T through LDS.
template <class B>
__global__ __launch_bounds__(64 * kBtWaves) void k_eig_backtr_w(B batch) {
    extern __shared__ float sm[];
    const JacItem &it = batch.it[blockIdx.y];
    const int n = it.n, c0 = 32 * blockIdx.x;
    if (c0 >= n) return;
    const TriWs w = tri_ws(it.tw, n);
    if (*w.flag) return;                                // k_eig_polish_w reports it
    const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int m32 = lane & 31, kh = lane >> 5;
    const int mref = max(n - 2, 0), nblk = tri_blocks(n), nt = (n + 31) >> 5;
    float *Ts = sm;                      // T_b(i, k) at Ts[i * 33 + k]
    float *Zc = Ts + kTile;              // Z(r, c0 + m) at Zc[r * 33 + m]
    float *Pt = Zc + n * 33;             // partial S of wave w
    float *Mt = Pt + kBtWaves * kTile;   // M(k, m) at Mt[k * 33 + m]
    constexpr int NT = 64 * kBtWaves;
    const int c4 = w.np >> 2, ncol = min(32, n - c0);
    for (int e = tid; e < (32 - ncol) * n; e += NT) {
        const int m = ncol + e / n, r = e - (e / n) * n;
        Zc[r * 33 + m] = 0.f;
    }
    load_rows4<NT, 8>(w.zt + (size_t)c0 * w.np, w.np, ncol, c4, tid, [&](int m, int c, float4 v) {
        const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (4 * c + i < n) Zc[(4 * c + i) * 33 + m] = vv[i];
    });
    for (int b = nblk - 1; b >= 0; --b) {
        const int b0 = 32 * b, nbk = min(32, mref - b0);
        __syncthreads();
        load_rows4<NT, 8>(w.tb + 1024 * b, 32, 32, 8, tid, [&](int r, int c, float4 v) {
            float *d = Ts + r * 33 + 4 * c;
            d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
        });
        __syncthreads();
        // Y(r, i): reflector b0 + i at row r (workspace row b0 + i), zero unless
        // i < nbk and b0 + i < r < n
        const float *ya0 = w.a + (size_t)b0 * w.np;
        auto Y = [&](int r, int i) {
            return ld_or_zero(ya0, min(i, nbk - 1) * w.np + min(r, n - 1), i < nbk && r > b0 + i && r < n);
        };
        {
            const int rows = n - 1 - b0, per = ((rows + 8 * kBtWaves - 1) / (8 * kBtWaves)) * 8;
            const int r0 = b0 + 1 + wid * per, r1 = min(n, r0 + per);
            f32x16 acc = {};
            for (int k0 = r0; k0 < r1; k0 += 8) {
                float ya[4], zb[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int r = k0 + 2 * u + kh;
                    const bool ok = r < r1;
                    ya[u] = ok ? Y(r, m32) : 0.f;
                    zb[u] = ld_or_zero(Zc, min(r, n - 1) * 33 + m32, ok);
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(ya[u], zb[u], acc, 0, 0, 0);
            }
#pragma unroll
            for (int q = 0; q < 16; ++q) Pt[wid * kTile + frag_row(lane, q) * 33 + m32] = acc[q];
        }
        __syncthreads();
        if (wid == 0) {
            f32x16 acc = {};
#pragma unroll
            for (int k0 = 0; k0 < 32; k0 += 8) {
                float ta[4], sb[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int k = k0 + 2 * u + kh;
                    ta[u] = Ts[m32 * 33 + k];
                    float sv = 0.f;
#pragma unroll
                    for (int v = 0; v < kBtWaves; ++v) sv += Pt[v * kTile + k * 33 + m32];
                    sb[u] = sv;
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(ta[u], sb[u], acc, 0, 0, 0);
            }
#pragma unroll
            for (int q = 0; q < 16; ++q) Mt[frag_row(lane, q) * 33 + m32] = acc[q];
        }
        __syncthreads();
        for (int rt = b + wid; rt < nt; rt += kBtWaves) {
            f32x16 acc;
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int row = 32 * rt + frag_row(lane, q);
                acc[q] = ld_or_zero(Zc, min(row, n - 1) * 33 + m32, row < n);
            }
#pragma unroll
            for (int k0 = 0; k0 < 32; k0 += 8) {
                float ya[4], mb[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int k = k0 + 2 * u + kh;
                    ya[u] = -Y(32 * rt + m32, k);
                    mb[u] = Mt[k * 33 + m32];
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(ya[u], mb[u], acc, 0, 0, 0);
            }
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int row = 32 * rt + frag_row(lane, q);
                if (row < n) Zc[row * 33 + m32] = acc[q];
            }
        }
    }
    __syncthreads();
    for (int e = tid; e < ncol * n; e += NT) {
        const int m = e / n, r = e - m * n;
        w.zt[(size_t)(c0 + m) * w.np + r] = Zc[r * 33 + m];
    }
}

// C(m, c) = sum_k a[m lda + k] b[c ldb + k] for tile (tm, tn), both operands
// rows in k padded with zeros to a multiple of 8 past n, 16-byte aligned rows:
// four K steps per pair of float4 loads (lane half kh takes k0 + 4 kh + u on
// both operands, so the hardware's K pairing cancels)
__device__ __forceinline__ f32x16 mfma_tile_rr(const float *a, int lda, const float *b, int ldb, int n, int tm,
                                               int tn, int lane) {
    f32x16 acc = {};
    const int kh = lane >> 5;
    const int mc = min(tm * 32 + (lane & 31), n - 1), cc = min(tn * 32 + (lane & 31), n - 1);
    const float *ap = a + (size_t)mc * lda + 4 * kh, *bp = b + (size_t)cc * ldb + 4 * kh;
    for (int k0 = 0; k0 < n; k0 += 8) {
        const float4 av = *reinterpret_cast<const float4 *>(ap + k0);
        const float4 bv = *reinterpret_cast<const float4 *>(bp + k0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av.x, bv.x, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av.y, bv.y, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av.z, bv.z, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av.w, bv.w, acc, 0, 0, 0);
    }
    return acc;
}

// Newton-Schulz polish and output for the wide solver, one workgroup per
// matrix, on the workspace: Z^T (rows = vectors) in zt, E = (I - Z^T Z) / 2 in
// ex (both triangles, zero padded), the next Z^T in the reflector rows (no
// longer needed), the two swapping roles every step.  The same step rule as
// k_eig_polish; a matrix it cannot make orthonormal reports kEigWideFail in
// sweeps_out (its output is written as it stands).
template <class B>
__global__ __launch_bounds__(kThreads) void k_eig_polish_w(B batch) {
    __shared__ float sred[kWaves];
    const JacItem &it = batch.it[blockIdx.x];
    const int n = it.n;
    const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const TriWs w = tri_ws(it.tw, n);
    if (*w.flag) {
        if (tid == 0) *it.sweeps_out = kEigWideFail;
        return;
    }
    const int np = w.np, nt = (n + 31) >> 5, ntiles = nt * nt, ntri = nt * (nt + 1) / 2;
    float *Z = w.zt, *Z2 = w.a, *E = w.ex;
    for (int e = tid; e < n * (np - n); e += kThreads) {
        const int r = e / (np - n), c = n + e - r * (np - n);
        E[(size_t)r * np + c] = 0.f;
        Z2[(size_t)r * np + c] = 0.f;
    }
    bool failed = false;
    for (int step = 0;; ++step) {
        float dev = 0.f;
        for (int t = wid; t < ntri; t += kWaves) {
            int tt = t, tm = 0;
            while (tt >= nt - tm) {
                tt -= nt - tm;
                ++tm;
            }
            const int tn = tm + tt, col = tn * 32 + (lane & 31);
            const f32x16 g = mfma_tile_rr(Z, np, Z, np, n, tm, tn, lane);
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) {
                const int row = tm * 32 + frag_row(lane, jj);
                if (row < n && col < n) {
                    const float id = row == col ? 1.f : 0.f;
                    const float gv = g[jj];
                    dev = fmaxf(dev, fabsf(gv - id));
                    if (!(gv == gv)) dev = FLT_MAX;
                    const float ev = 0.5f * (id - gv);
                    E[(size_t)row * np + col] = ev;
                    E[(size_t)col * np + row] = ev;
                }
            }
        }
        dev = wave_max(dev);
        if (lane == 0) sred[wid] = dev;
        __syncthreads();
        float devmax = 0.f;
#pragma unroll
        for (int v = 0; v < kWaves; ++v) devmax = fmaxf(devmax, sred[v]);
        __syncthreads();
        if (devmax <= 4e-6f) break;
        if (step == 3 || !(devmax <= 0.3f)) {
            failed = !(devmax <= 1e-4f);
            break;
        }
        // Z2 = Z + E Z (E symmetric: the rows of Z^T (I + E))
        for (int t = wid; t < ntiles; t += kWaves) {
            const int tm = t / nt, tn = t % nt;
            const int kh = lane >> 5, cc = min(tn * 32 + (lane & 31), n - 1), col = tn * 32 + (lane & 31);
            const int mc = min(tm * 32 + (lane & 31), n - 1);
            f32x16 acc;
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int row = tm * 32 + frag_row(lane, q);
                acc[q] = ld_or_zero(Z, min(row, n - 1) * np + cc, row < n && col < n);
            }
            const float *ap = E + (size_t)mc * np + 4 * kh;
            for (int k0 = 0; k0 < n; k0 += 8) {
                const float4 av = *reinterpret_cast<const float4 *>(ap + k0);
                float bv[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int k = k0 + 4 * kh + u;
                    bv[u] = ld_or_zero(Z, min(k, n - 1) * np + cc, k < n);
                }
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av.x, bv[0], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av.y, bv[1], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av.z, bv[2], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av.w, bv[3], acc, 0, 0, 0);
            }
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int row = tm * 32 + frag_row(lane, q);
                if (row < n && col < n) Z2[(size_t)row * np + col] = acc[q];
            }
        }
        __syncthreads();
        float *t = Z;
        Z = Z2;
        Z2 = t;
        if (devmax <= 1e-3f) break;
    }
    // output: eigenvalue k (ascending) -> column n - 1 - k, sign so that the
    // entry of largest magnitude (first such row) is positive
    for (int k = tid; k < n; k += kThreads) {
        const float *zr = Z + (size_t)k * np;
        int best = 0;
        float bm = -1.f;
        for (int r = 0; r < n; ++r) {
            const float v = fabsf(zr[r]);
            if (v > bm) {
                bm = v;
                best = r;
            }
        }
        const float sg = zr[best] < 0.f ? -1.f : 1.f;
        const int col = n - 1 - k;
        it.lam[col] = w.lam[k];
        for (int r = 0; r < n; ++r) it.vec[(size_t)r * it.ldv + col] = sg * zr[r];
    }
    if (tid == 0) *it.sweeps_out = failed ? kEigWideFail : 0;
}

// ---------------------------------------------------------------- 5 and output
// Newton-Schulz polish and the output of one matrix per workgroup, V loaded
// from the workspace.
template <class B>
__global__ __launch_bounds__(kThreads) void k_eig_polish(B batch, int ld, int boff) {
    extern __shared__ float sm[];
    __shared__ float slam[kTriMaxN];
    __shared__ float sred[2 * kWaves];
    const JacItem &it = batch.it[blockIdx.x];
    const int n = it.n;
    const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    float *A = sm;          // E of the polish steps
    float *V = sm + boff;   // V[r * ld + c]
    const TriWs w = tri_ws(it.tw, n);
    if (*w.flag) {
        if (tid == 0) *it.sweeps_out = kEigRetry;
        return;
    }
    load_rows4<kThreads, 4>(w.zt, w.np, n, w.np >> 2, tid, [&](int k, int c, float4 v) {
        const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (4 * c + i < n) V[(4 * c + i) * ld + k] = vv[i];
    });
    for (int i = tid; i < n; i += kThreads) slam[i] = w.lam[i];
    __syncthreads();
    const int nt = (n + 31) >> 5, ntiles = nt * nt;

    // ---------------------------------------------------------------- 5. Newton-Schulz steps
    // V <- V (3 I - V^T V) / 2 = V + V E with E = (I - V^T V) / 2.  V^T V is
    // symmetric: its upper tiles are formed and E goes to both triangles of
    // the A buffer; V + V E is formed with V E as the small term.
    const int ntri = nt * (nt + 1) / 2;     // <= kWaves for n <= 160
    for (int step = 0;; ++step) {
        float dev = 0.f;
        if (wid < ntri) {
            int t = wid, tm = 0;
            while (t >= nt - tm) {
                t -= nt - tm;
                ++tm;
            }
            const int tn = tm + t, col = tn * 32 + (lane & 31);
            const f32x16 g = mfma_tile(V, ld, 1, V, ld, n, tm, tn, lane);
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) {
                const int row = tm * 32 + frag_row(lane, jj);
                if (row < n && col < n) {
                    const float id = row == col ? 1.f : 0.f;
                    const float gv = g[jj];
                    dev = fmaxf(dev, fabsf(gv - id));
                    if (!(gv == gv)) dev = FLT_MAX;
                    const float e = 0.5f * (id - gv);
                    A[row * ld + col] = e;
                    A[col * ld + row] = e;
                }
            }
        }
        dev = wave_max(dev);
        if (lane == 0) sred[wid] = dev;
        __syncthreads();
        float devmax = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) devmax = fmaxf(devmax, sred[w]);
        if (devmax <= 4e-6f) break;
        if (step == 3 || !(devmax <= 0.3f)) {
            if (!(devmax <= 1e-4f)) {
                if (tid == 0) *it.sweeps_out = kEigRetry;
                return;
            }
            break;
        }
        f32x16 acc0 = {}, acc1 = {};
        if (wid < ntiles) acc0 = ns_tile(V, A, ld, n, wid / nt, wid % nt, lane);
        if (wid + kWaves < ntiles) acc1 = ns_tile(V, A, ld, n, (wid + kWaves) / nt, (wid + kWaves) % nt, lane);
        __syncthreads();
        store_tiles(V, acc0, acc1, ld, n, nt, ntiles, wid, lane);
        __syncthreads();
        // a polar step maps a deviation d of V^T V from I to at most
        // 3 d^2 / 4 + d^3 / 4: from d <= 1e-3 that is below 1e-6 (plus fp32
        // rounding of the step), so the result is taken without another check
        if (devmax <= 1e-3f) break;
    }
    const float *W = V;

    // ---------------------------------------------------------------- output
    if (tid < n) {
        const int k = tid, col = n - 1 - k;
        int best = 0;
        float bm = -1.f;
        for (int r = 0; r < n; ++r) {
            const float v = fabsf(W[r * ld + k]);
            if (v > bm) {
                bm = v;
                best = r;
            }
        }
        const float sg = W[best * ld + k] < 0.f ? -1.f : 1.f;
        it.lam[col] = slam[k];
        for (int r = 0; r < n; ++r) it.vec[(size_t)r * it.ldv + col] = sg * W[r * ld + k];
    }
    if (tid == 0) *it.sweeps_out = 0;
}

static hipError_t allow_lds(const void *fn) {
    hipFuncAttributes fa;
    hipError_t e = hipFuncGetAttributes(&fa, fn);
    if (e == hipSuccess)
        e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024 - (int)fa.sharedSizeBytes);
    return e;
}
template <class B>
static hipError_t allow_lds_tri() {
    static hipError_t state = hipErrorNotReady;
    if (state == hipErrorNotReady) {
        hipError_t e = allow_lds(reinterpret_cast<const void *>(k_eig_tridiag<B>));
        if (e == hipSuccess) e = allow_lds(reinterpret_cast<const void *>(k_eig_backtr<B>));
        if (e == hipSuccess) e = allow_lds(reinterpret_cast<const void *>(k_eig_polish<B>));
        state = e;
    }
    return state;
}

// dynamic LDS layout of k_eig_tridiag and k_eig_polish for a batch of order
// <= maxN (floats): [A: maxN x ld | B1: max(maxN x ld, 2 maxN x kPanelStride)]
struct TriLayout { int ld, boff, poff; size_t bytes; };
static TriLayout tri_layout(int maxN) {
    TriLayout L;
    L.ld = maxN | 1;
    L.boff = maxN * L.ld;
    L.poff = maxN * kPanelStride;
    const int b1 = std::max(maxN * L.ld, 2 * maxN * kPanelStride);
    L.bytes = (size_t)(L.boff + b1) * sizeof(float);
    return L;
}

template <class B>
static hipError_t launch_eig_wide(const B &b, int count, int maxN, hipStream_t s) {
    static hipError_t state = hipErrorNotReady;
    if (state == hipErrorNotReady) {
        hipError_t e = allow_lds(reinterpret_cast<const void *>(k_eig_tridiag_w<B>));
        if (e == hipSuccess) e = allow_lds(reinterpret_cast<const void *>(k_eig_backtr_w<B>));
        state = e;
    }
    if (state != hipSuccess) return state;
    {
        KTimeScope kts("k_eig_tridiag", s);
        hipLaunchKernelGGL(k_eig_tridiag_w<B>, dim3(count), dim3(kWThreads), kWTriLds, s, b);
        if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    }
    const int nblk = (std::max(maxN - 2, 0) + 31) / 32;
    {
        KTimeScope kts("k_eig_trivec", s);
        constexpr int per = kVecWaves * kVecPerWave;
        const int eig_blocks = (maxN + per - 1) / per;
        hipLaunchKernelGGL((k_eig_wy<kWideMaxN, B>), dim3(std::max(nblk, 1), count), dim3(64), 0, s, b);
        hipLaunchKernelGGL((k_eig_trivec<kWideMaxN, B>), dim3(eig_blocks, count), dim3(64 * kVecWaves), 0, s, b);
        if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    }
    {
        KTimeScope kts("k_eig_backtr", s);
        const size_t lds = ((size_t)kTile + (size_t)maxN * 33 + (size_t)(kBtWaves + 1) * kTile) * sizeof(float);
        hipLaunchKernelGGL(k_eig_backtr_w<B>, dim3((maxN + 31) / 32, count), dim3(64 * kBtWaves), lds, s, b);
        if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    }
    KTimeScope kts("k_eig_polish", s);
    hipLaunchKernelGGL(k_eig_polish_w<B>, dim3(count), dim3(kThreads), 0, s, b);
    return hipGetLastError();
}

template <class B>
static hipError_t eig_tri(const JacItem *items, int count, const B &b, int maxN, hipStream_t s) {
    if (count <= 0) return hipSuccess;
    if (maxN > kWideMaxN) return hipErrorInvalidValue;
    if (maxN > kTriMaxN) {
        for (int i = 0; i < count; ++i)
            if (!items[i].sweeps_out || !items[i].tw || items[i].n > maxN || items[i].n <= kTriMaxN)
                return hipErrorInvalidValue;
        return launch_eig_wide(b, count, maxN, s);
    }
    for (int i = 0; i < count; ++i)
        if (!items[i].sweeps_out || !items[i].tw || items[i].n > maxN) return hipErrorInvalidValue;
    if (hipError_t e = allow_lds_tri<B>(); e != hipSuccess) return e;
    const TriLayout L = tri_layout(maxN);
    {
        KTimeScope kts("k_eig_tridiag", s);
        hipLaunchKernelGGL(k_eig_tridiag<B>, dim3(count), dim3(kThreads), L.bytes, s, b, L.ld, L.boff, L.poff);
        if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    }
    const int nblk = (std::max(maxN - 2, 0) + 31) / 32;
    {
        KTimeScope kts("k_eig_trivec", s);
        constexpr int per = kVecWaves * kVecPerWave;
        const int eig_blocks = (maxN + per - 1) / per;
        hipLaunchKernelGGL((k_eig_wy<kTriMaxN, B>), dim3(std::max(nblk, 1), count), dim3(64), 0, s, b);
        hipLaunchKernelGGL((k_eig_trivec<kTriMaxN, B>), dim3(eig_blocks, count), dim3(64 * kVecWaves), 0, s, b);
        if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    }
    {
        KTimeScope kts("k_eig_backtr", s);
        const int ldy = ((maxN + 3) & ~3) | 1;         // odd, and room for the padded rows
        const size_t lds = ((size_t)std::max(maxN - 2, 0) * ldy + (size_t)nblk * kTile + (size_t)maxN * 33 +
                            (size_t)(kBtWaves + 1) * kTile) * sizeof(float);
        hipLaunchKernelGGL(k_eig_backtr<B>, dim3((maxN + 31) / 32, count), dim3(64 * kBtWaves), lds, s, b, ldy);
        if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    }
    KTimeScope kts("k_eig_polish", s);
    hipLaunchKernelGGL(k_eig_polish<B>, dim3(count), dim3(kThreads), L.bytes, s, b, L.ld, L.boff);
    return hipGetLastError();
}
hipError_t launch_eig_tridiag(const JacBatch &b, int maxN, hipStream_t s) {
    return eig_tri(b.it, b.n, b, maxN, s);
}
hipError_t launch_eig_tridiag(const JacItem *host, const JacTable &dev, int maxN, hipStream_t s) {
    return eig_tri(host, dev.n, dev, maxN, s);
}

}  // namespace jolt
