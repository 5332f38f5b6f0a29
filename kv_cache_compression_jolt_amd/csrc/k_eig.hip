// Symmetric eigensolver for small dense matrices (n <= kTriMaxN), one
// workgroup of 1024 threads per matrix, all of it resident in LDS.
//
//   1. Householder tridiagonalization Q^T A Q = T (Golub & Van Loan, Matrix
//      Computations, sec. 8.3.1), with Q accumulated in the same steps;
//   2. every eigenvalue of T by bisection on Sturm counts (sec. 8.4.1), one
//      lane per eigenvalue, to a relative width of 2 eps;
//   3. every eigenvector of T from a twisted factorization of T - lambda I
//      (Dhillon & Parlett, Orthogonal eigenvectors and relative gaps, 2004):
//      forward and backward LDL^T pivots, the twist index where |gamma| is
//      smallest, and the two one-sided recurrences from it;
//   4. V = Q Z on fp32 MFMA;
//   5. Newton-Schulz polar steps V <- V (3 I - V^T V) / 2 (at most 3, until
//      V^T V is within 4e-6 of I), which restore the orthogonality that vectors
//      of close eigenvalues lose.
// When V^T V is far from I (numerically repeated eigenvalues: the twisted
// vectors coincide) the matrix is flagged in sweeps_out and the Jacobi kernel,
// launched right after in retry mode, solves it instead.
//
// Output convention (shared with the Jacobi kernel): eigenvalues descending,
// eigenvector columns sign-normalised so that the entry of largest magnitude
// (first such row) is positive.
#include <float.h>

#include "dev_common.h"
#include "plan_kernels.h"
#include "ktimer.h"

namespace jolt {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kRowBatch = 5;           // rows per wave per load batch in the rank-2 update


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
    for (int k0 = 0; k0 < n; k0 += 2) {
        const int kk = k0 + kh;
        const bool kv = kk < n;
        const float av = (mv && kv) ? a[kk * lda_k + m * lda_m] : 0.f;
        const float bv = (cv && kv) ? b[kk * ld + col] : 0.f;
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc, 0, 0, 0);
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

__global__ __launch_bounds__(kThreads) void k_eig_tridiag(JacBatch batch, int ld, int boff) {
    extern __shared__ float sm[];
    __shared__ float sd[kTriMaxN], se[kTriMaxN], slam[kTriMaxN];
    __shared__ __align__(8) float sbuf[2 * kTriMaxN + 2];
    __shared__ float sred[2 * kWaves];
    __shared__ int s_fail;
    const JacItem &it = batch.it[blockIdx.x];
    const int n = it.n;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    float *A = sm;          // A[r * ld + c]; later Z, then M, then the final vectors
    float *Qt = sm + boff;  // Qt[c * ld + r] = Q[r][c]; later V = Q Z (row-major)
    float *sp = sbuf, *su = sbuf + kTriMaxN;

    JOLT_PROBE(0);
    if (tid == 0) s_fail = 0;
    for (int e = tid; e < n * n; e += kThreads) {
        const int r = e / n, c = e - r * n;
        A[r * ld + c] = 0.5f * (it.a[(size_t)r * it.lda + c] + it.a[(size_t)c * it.lda + r]);
        Qt[r * ld + c] = (r == c) ? 1.f : 0.f;
    }

    // ---------------------------------------------------------------- 1. tridiagonalize
    // Step j reflects x = A[j+1:, j] (read as row j, A stays exactly symmetric)
    // onto beta e_1 with H = I - tau v v^T, v = x - beta e_1 (unnormalised),
    // tau = 2 / v^T v.  Then p = tau A22 v, w = p - (tau p^T v / 2) v,
    // A22 -= v w^T + w v^T and Q[:, j+1:] -= tau (Q[:, j+1:] v) v^T.
    const int rl = lane & 15, q4 = lane >> 4;
    JOLT_PROBE(1);
    for (int j = 0; j + 2 < n; ++j) {
        __syncthreads();
        const int s = n - j - 1;
        const float *rowj = A + j * ld + j + 1;
        float part = 0.f;
        for (int c = 1 + lane; c < s; c += 64) {
            const float x = rowj[c];
            part += x * x;
        }
        const float xn2 = wave_sum(part);     // identical in every wave
        const float x0 = rowj[0];
        float beta = x0, v0 = 0.f, tau = 0.f;
        if (xn2 > 0.f) {
            const float alpha = sqrtf(x0 * x0 + xn2);
            beta = x0 >= 0.f ? -alpha : alpha;
            v0 = x0 - beta;
            tau = 2.f / (v0 * v0 + xn2);
        }
        if (tid == 0) {
            sd[j] = A[j * ld + j];
            se[j] = beta;
        }
        if (tau == 0.f) continue;             // x already a multiple of e_1

        // p (rows of A22, read as columns by symmetry) and u = Q[:, j+1:] v:
        // 16 rows per wave pass, 4 lanes per row splitting the sum
        const int ngp = (s + 15) >> 4, ngu = (n + 15) >> 4;
        for (int g = wid; g < ngp + ngu; g += kWaves) {
            const bool isp = g < ngp;
            const int r = (isp ? g : g - ngp) * 16 + rl;
            const int rows = isp ? s : n;
            float acc = 0.f;
            if (r < rows) {
                const float *col = isp ? (A + (j + 1) * ld + j + 1 + r) : (Qt + (j + 1) * ld + r);
                // 8 independent products in flight per lane
                float a8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
                int c = q4;
                for (; c + 28 < s; c += 32) {
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        const int cc = c + 4 * u;
                        a8[u] = fmaf(col[cc * ld], cc == 0 ? v0 : rowj[cc], a8[u]);
                    }
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int cc = c + 4 * u;
                    if (cc < s) a8[u] = fmaf(col[cc * ld], cc == 0 ? v0 : rowj[cc], a8[u]);
                }
                acc = ((a8[0] + a8[1]) + (a8[2] + a8[3])) + ((a8[4] + a8[5]) + (a8[6] + a8[7]));
            }
            acc += __shfl_xor(acc, 16);
            acc += __shfl_xor(acc, 32);
            if (q4 == 0 && r < rows) {
                if (isp) sp[r] = tau * acc;
                else su[r] = acc;
            }
        }
        __syncthreads();

        float kp = 0.f;
        for (int c = lane; c < s; c += 64) kp = fmaf(sp[c], c == 0 ? v0 : rowj[c], kp);
        const float hk = 0.5f * tau * wave_sum(kp);
        float vr[3], wr[3], ur[3];
#pragma unroll
        for (int t = 0; t < 3; ++t) {
            const int r = lane + 64 * t;
            vr[t] = r < s ? (r == 0 ? v0 : rowj[r]) : 0.f;
            wr[t] = r < s ? sp[r] - hk * vr[t] : 0.f;
            ur[t] = r < n ? su[r] : 0.f;
        }
        // rows c = wid + 16 g of A22 and of Q^T: all loads of a batch of rows
        // first, then the updates (one LDS round trip per batch)
        for (int c0 = wid; c0 < s; c0 += kWaves * kRowBatch) {
            float av[kRowBatch][3], qv[kRowBatch][3], vcs[kRowBatch], wcs[kRowBatch];
#pragma unroll
            for (int g = 0; g < kRowBatch; ++g) {
                const int c = c0 + kWaves * g;
                const bool ok = c < s;
                const float vc = ok ? (c == 0 ? v0 : rowj[c]) : 0.f;
                vcs[g] = vc;
                wcs[g] = ok ? sp[c] - hk * vc : 0.f;
#pragma unroll
                for (int t = 0; t < 3; ++t) {
                    const int r = lane + 64 * t;
                    av[g][t] = (ok && r < s) ? A[(j + 1 + c) * ld + j + 1 + r] : 0.f;
                    qv[g][t] = (ok && r < n) ? Qt[(j + 1 + c) * ld + r] : 0.f;
                }
            }
#pragma unroll
            for (int g = 0; g < kRowBatch; ++g) {
                const int c = c0 + kWaves * g;
                if (c >= s) continue;
                const float vc = vcs[g], wc = wcs[g], tv = tau * vc;
                // (v_c w_r) + (w_c v_r): the same two products and one sum as the
                // mirrored entry, so A keeps exact symmetry (no contraction)
#pragma unroll
                for (int t = 0; t < 3; ++t) {
                    const int r = lane + 64 * t;
                    if (r < s) A[(j + 1 + c) * ld + j + 1 + r] = av[g][t] - (vc * wr[t] + wc * vr[t]);
                    if (r < n) Qt[(j + 1 + c) * ld + r] = fmaf(-tv, ur[t], qv[g][t]);
                }
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

    // ---------------------------------------------------------------- 2. eigenvalues
    JOLT_PROBE(2);
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
    const float lo = glo - (4.f * eps * tnorm + pivmin), hi = ghi + (4.f * eps * tnorm + pivmin);
    // relative width 2 eps |lambda|, floored at eps ||T|| / 1024 (vectors of
    // close eigenvalues stay near orthogonal only with accurate shifts)
    const float floor_tol = eps * tnorm * (1.f / 1024.f);
    float2 *sde = reinterpret_cast<float2 *>(sbuf);    // {d_i, e_{i-1}^2}
    for (int i = tid; i < n; i += kThreads) sde[i] = make_float2(sd[i], i > 0 ? se[i - 1] * se[i - 1] : 0.f);
    __syncthreads();
    if (tid < n) {
        // the tid-th smallest eigenvalue: count(x) = #{i : q_i(x) < 0}
        float a = lo, b = hi;
        for (int iter = 0; iter < 64 && b - a > 2.f * eps * fmaxf(fabsf(a), fabsf(b)) + floor_tol; ++iter) {
            const float x = 0.5f * (a + b);
            int cnt = 0;
            float qv = 1.f;
            for (int i = 0; i < n; ++i) {
                const float2 de = sde[i];
                qv = (de.x - x) - de.y * __builtin_amdgcn_rcpf(qv);
                if (fabsf(qv) < pivmin) qv = -pivmin;
                cnt += qv < 0.f;
            }
            if (cnt > tid) b = x;
            else a = x;
        }
        slam[tid] = 0.5f * (a + b);
    }
    __syncthreads();

    // ---------------------------------------------------------------- 3. vectors of T
    JOLT_PROBE(3);
    float *Z = A;      // Z[i * ld + k]: column k belongs to the k-th smallest eigenvalue
    if (tid < n) {
        const int k = tid;
        const float lam = slam[k];
        float dp = sd[0] - lam;
        if (fabsf(dp) < pivmin) dp = -pivmin;
        Z[k] = dp;
        for (int i = 1; i < n; ++i) {
            dp = (sd[i] - lam) - sde[i].y / dp;
            if (fabsf(dp) < pivmin) dp = -pivmin;
            Z[i * ld + k] = dp;
        }
        float dm = sd[n - 1] - lam;
        if (fabsf(dm) < pivmin) dm = -pivmin;
        float best = fabsf(Z[(n - 1) * ld + k]);
        int r = n - 1;
        for (int i = n - 2; i >= 0; --i) {
            dm = (sd[i] - lam) - sde[i + 1].y / dm;
            if (fabsf(dm) < pivmin) dm = -pivmin;
            const float g = fabsf(Z[i * ld + k] + dm - (sd[i] - lam));
            if (g <= best) {
                best = g;
                r = i;
            }
        }
        // z_r = 1; z_i = -(e_i / D+_i) z_{i+1} above r; z_{i+1} = -(e_i / D-_{i+1}) z_i below
        float nrm = 1.f, z = 1.f;
        for (int i = r - 1; i >= 0; --i) {
            z = -(se[i] / Z[i * ld + k]) * z;
            Z[i * ld + k] = z;
            nrm += z * z;
        }
        dm = sd[n - 1] - lam;
        if (fabsf(dm) < pivmin) dm = -pivmin;
        if (r < n - 1) Z[(n - 1) * ld + k] = dm;
        for (int i = n - 2; i > r; --i) {
            dm = (sd[i] - lam) - sde[i + 1].y / dm;
            if (fabsf(dm) < pivmin) dm = -pivmin;
            Z[i * ld + k] = dm;
        }
        Z[r * ld + k] = 1.f;
        z = 1.f;
        for (int i = r; i + 1 < n; ++i) {
            z = -(se[i] / Z[(i + 1) * ld + k]) * z;
            Z[(i + 1) * ld + k] = z;
            nrm += z * z;
        }
        if (!(nrm < FLT_MAX)) s_fail = 1;
        const float inv = 1.f / sqrtf(nrm);
        for (int i = 0; i < n; ++i) Z[i * ld + k] *= inv;
    }
    __syncthreads();

    if (s_fail) {
        if (tid == 0) *it.sweeps_out = kEigRetry;
        return;
    }

    // ---------------------------------------------------------------- 4. V = Q Z
    JOLT_PROBE(4);
    const int nt = (n + 31) >> 5, ntiles = nt * nt;
    float *V = Qt;     // V[r * ld + c], kept in the Q buffer from here on
    {
        f32x16 acc0 = {}, acc1 = {};
        if (wid < ntiles) acc0 = mfma_tile(Qt, ld, 1, Z, ld, n, wid / nt, wid % nt, lane);
        if (wid + kWaves < ntiles) acc1 = mfma_tile(Qt, ld, 1, Z, ld, n, (wid + kWaves) / nt, (wid + kWaves) % nt, lane);
        __syncthreads();
        store_tiles(V, acc0, acc1, ld, n, nt, ntiles, wid, lane);
    }
    __syncthreads();

    // ---------------------------------------------------------------- 5. Newton-Schulz steps
    JOLT_PROBE(5);
    // G = V^T V and M = (3 I - G) / 2 (M in the Z buffer); V <- V M
    for (int step = 0;; ++step) {
        float dev = 0.f;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int t = wid + u * kWaves;
            if (t >= ntiles) continue;
            const int tm = t / nt, tn = t % nt, col = tn * 32 + (lane & 31);
            const f32x16 g = mfma_tile(V, ld, 1, V, ld, n, tm, tn, lane);
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) {
                const int row = tm * 32 + frag_row(lane, jj);
                if (row < n && col < n) {
                    const float id = row == col ? 1.f : 0.f;
                    const float gv = g[jj];
                    dev = fmaxf(dev, fabsf(gv - id));
                    if (!(gv == gv)) dev = FLT_MAX;
                    A[row * ld + col] = 1.5f * id - 0.5f * gv;
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
        // V M: A(m, k) = V[m][k], read down the rows of V
        f32x16 acc0 = {}, acc1 = {};
        if (wid < ntiles) acc0 = mfma_tile(V, 1, ld, A, ld, n, wid / nt, wid % nt, lane);
        if (wid + kWaves < ntiles) acc1 = mfma_tile(V, 1, ld, A, ld, n, (wid + kWaves) / nt, (wid + kWaves) % nt, lane);
        __syncthreads();
        store_tiles(V, acc0, acc1, ld, n, nt, ntiles, wid, lane);
        __syncthreads();
    }
    const float *W = V;

    // ---------------------------------------------------------------- output
    JOLT_PROBE(6);
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

static hipError_t allow_lds_tri() {
    static hipError_t state = hipErrorNotReady;
    if (state == hipErrorNotReady) {
        const void *fn = reinterpret_cast<const void *>(k_eig_tridiag);
        hipFuncAttributes fa;
        hipError_t e = hipFuncGetAttributes(&fa, fn);
        if (e == hipSuccess)
            e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                    160 * 1024 - (int)fa.sharedSizeBytes);
        state = e;
    }
    return state;
}

size_t eig_tridiag_lds_bytes(int maxN) {
    const int ld = maxN | 1;
    return (size_t)2 * maxN * ld * sizeof(float);
}

hipError_t launch_eig_tridiag(const JacBatch &b, int maxN, hipStream_t s) {
    if (b.n <= 0) return hipSuccess;
    if (maxN > kTriMaxN) return hipErrorInvalidValue;
    for (int i = 0; i < b.n; ++i)
        if (!b.it[i].sweeps_out || b.it[i].n > maxN) return hipErrorInvalidValue;
    if (hipError_t e = allow_lds_tri(); e != hipSuccess) return e;
    KTimeScope kts("k_eig_tridiag", s);
    const int ld = maxN | 1;
    hipLaunchKernelGGL(k_eig_tridiag, dim3(b.n), dim3(kThreads), eig_tridiag_lds_bytes(maxN), s, b, ld, maxN * ld);
    return hipGetLastError();
}

}  // namespace jolt
