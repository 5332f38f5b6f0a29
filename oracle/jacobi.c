/*
 * ORACLE (test infrastructure only) -- two-sided Jacobi eigensolver, fp64.
 *
 * Both Tucker factors of "A JoLT for the KV cache" (paper landing page,
 * abstract: partial Tucker along the token and feature modes; exact token-mode
 * SVD) are eigenvectors of symmetric Gram matrices.  This is the classical
 * Jacobi method (Golub & Van Loan, Matrix Computations, 4th ed., sec. 8.5):
 * every rotation zeroes one off-diagonal pair a[p][q] = a[q][p] with the
 * symmetric 2x2 Schur decomposition
 *     tau = (a_qq - a_pp) / (2 a_pq),  t = sign(tau) / (|tau| + sqrt(1 + tau^2)),
 *     c = 1 / sqrt(1 + t^2),  s = t c,   J = [[c, s], [-s, c]] on (p, q),
 * and A <- J^T A J, V <- V J.  A sweep visits every pair once in the
 * round-robin ("parallel") ordering of Golub & Van Loan sec. 8.5.5: each of
 * the n-1 rounds pairs all indices disjointly, so the round's rotations
 * commute and are applied together, 2x2 block by 2x2 block:
 *     A[{p_i,q_i}][{p_j,q_j}] <- J_i^T A[{p_i,q_i}][{p_j,q_j}] J_j.
 * Sweeps stop once off(A) <= tol * ||A||_F, or after max_sweeps.
 *
 * A: n x n row-major symmetric (overwritten).  The eigenvectors are returned
 * transposed (row i of Vt = eigenvector i); w receives the unsorted
 * eigenvalues.  Returns the number of sweeps used, or -1 if not converged.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>

static double off_norm2(int n, const double *A) {
    double s = 0.0;
    for (int i = 0; i < n; ++i)
        for (int j = 0; j < n; ++j)
            if (i != j) s += A[(size_t)i * n + j] * A[(size_t)i * n + j];
    return s;
}

int oracle_jacobi_eigh(int n, double *A, double *Vt, double *w, int max_sweeps, double tol) {
    double fro2 = 0.0;
    for (size_t i = 0; i < (size_t)n * n; ++i) fro2 += A[i] * A[i];
    memset(Vt, 0, sizeof(double) * (size_t)n * n);
    for (int i = 0; i < n; ++i) Vt[(size_t)i * n + i] = 1.0;
    int m = n + (n & 1);            /* even count; index n is a dummy when n is odd */
    int half = m / 2;
    int *pos = (int *)malloc(sizeof(int) * m);
    int *P = (int *)malloc(sizeof(int) * half);
    int *Q = (int *)malloc(sizeof(int) * half);
    double *C = (double *)malloc(sizeof(double) * half);
    double *S = (double *)malloc(sizeof(double) * half);
    for (int i = 0; i < m; ++i) pos[i] = i;
    int sweeps = 0, converged = 0;
    for (; sweeps <= max_sweeps; ++sweeps) {
        if (off_norm2(n, A) <= tol * tol * fro2) { converged = 1; break; }
        if (sweeps == max_sweeps) break;
        for (int round = 0; round < m - 1; ++round) {
            /* pairs of this round and their rotations */
            int np = 0;
            for (int i = 0; i < half; ++i) {
                int p = pos[i], q = pos[m - 1 - i];
                if (p > q) { int t = p; p = q; q = t; }
                if (q >= n) continue;                 /* paired with the dummy */
                double apq = A[(size_t)p * n + q];
                double c = 1.0, s = 0.0;
                if (apq != 0.0) {
                    double app = A[(size_t)p * n + p], aqq = A[(size_t)q * n + q];
                    double tau = (aqq - app) / (2.0 * apq);
                    double t = (tau >= 0.0) ? 1.0 / (tau + sqrt(1.0 + tau * tau))
                                            : -1.0 / (-tau + sqrt(1.0 + tau * tau));
                    c = 1.0 / sqrt(1.0 + t * t);
                    s = t * c;
                }
                P[np] = p; Q[np] = q; C[np] = c; S[np] = s; ++np;
            }
            /* A <- J^T A J, block by block */
            for (int i = 0; i < np; ++i) {
                double *rp = A + (size_t)P[i] * n, *rq = A + (size_t)Q[i] * n;
                double ci = C[i], si = S[i];
                for (int j = 0; j < np; ++j) {
                    int pj = P[j], qj = Q[j];
                    double cj = C[j], sj = S[j];
                    double b00 = rp[pj], b01 = rp[qj], b10 = rq[pj], b11 = rq[qj];
                    double m00 = cj * b00 - sj * b01, m01 = sj * b00 + cj * b01;
                    double m10 = cj * b10 - sj * b11, m11 = sj * b10 + cj * b11;
                    rp[pj] = ci * m00 - si * m10; rp[qj] = ci * m01 - si * m11;
                    rq[pj] = si * m00 + ci * m10; rq[qj] = si * m01 + ci * m11;
                }
                /* rows paired with the dummy index (odd n): only the column
                   rotation of the real pairs applies to them */
            }
            if (n & 1) {
                /* the index paired with the dummy: its row gets the column rotations */
                int lone = -1;
                for (int i = 0; i < half; ++i) {
                    int p = pos[i], q = pos[m - 1 - i];
                    if (p == n) lone = q;
                    if (q == n) lone = p;
                }
                if (lone >= 0) {
                    double *rl = A + (size_t)lone * n;
                    for (int j = 0; j < np; ++j) {
                        double a = rl[P[j]], b = rl[Q[j]];
                        rl[P[j]] = C[j] * a - S[j] * b;
                        rl[Q[j]] = S[j] * a + C[j] * b;
                    }
                    for (int j = 0; j < np; ++j) {
                        double *rp = A + (size_t)P[j] * n, *rq = A + (size_t)Q[j] * n;
                        double a = rp[lone], b = rq[lone];
                        rp[lone] = C[j] * a - S[j] * b;
                        rq[lone] = S[j] * a + C[j] * b;
                    }
                }
            }
            for (int i = 0; i < np; ++i) {
                A[(size_t)P[i] * n + Q[i]] = 0.0;
                A[(size_t)Q[i] * n + P[i]] = 0.0;
                double *vp = Vt + (size_t)P[i] * n, *vq = Vt + (size_t)Q[i] * n;
                double c = C[i], s = S[i];
                for (int k = 0; k < n; ++k) {
                    double a = vp[k], b = vq[k];
                    vp[k] = c * a - s * b;
                    vq[k] = s * a + c * b;
                }
            }
            /* next round: keep pos[0], rotate pos[1..m-1] by one place */
            int last = pos[m - 1];
            for (int i = m - 1; i > 1; --i) pos[i] = pos[i - 1];
            pos[1] = last;
        }
    }
    for (int i = 0; i < n; ++i) w[i] = A[(size_t)i * n + i];
    free(pos); free(P); free(Q); free(C); free(S);
    return converged ? sweeps : -1;
}
