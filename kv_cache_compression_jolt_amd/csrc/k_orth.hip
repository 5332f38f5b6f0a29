// Orthonormalization kernels of the randomized range finder (CholeskyQR:
// Q = Y L^{-T} with G = Y^T Y + shift I = L L^T).
//
// k_chol_inv: the inverse Cholesky factor, blocked (32 x 32 blocks, one
// workgroup per matrix, everything in one LDS square).  For each block column
// J (Golub & Van Loan, Matrix Computations, sec. 4.2.8):
//   one wave factors the diagonal block, G_JJ = L_JJ L_JJ^T, and inverts it;
//   the panel L_IJ = G_IJ L_JJ^{-T} (I > J) and the trailing update
//   G_IK -= L_IJ L_KJ^T (J < K <= I) run as fp32 MFMA tiles, one per wave.
// Then the off-diagonal blocks of X = L^{-1}, one block diagonal at a time:
//   X_IJ = -X_II sum_{K=J}^{I-1} L_IK X_KJ.
// Storage: L in the lower triangle, X^T in the strict upper triangle (block
// (J, I) above the diagonal holds X_IJ^T), diag(X) in a side array.
// Pivots are clamped at the shift floor, so rank-deficient sketches still give
// a usable basis.
//
// k_apply_linv: Q = L^{-1} Y for a 64-column block of Y (all k rows), on fp32
// MFMA; the block is staged in LDS first, so the product can overwrite Y.
#include <float.h>

#include <algorithm>

#include "dev_common.h"
#include "plan_kernels.h"
#include "ktimer.h"

namespace jolt {

// Factor and invert the 32 x 32 diagonal block at B (row stride ld) with one
// wave, in registers: lane i < 32 holds row i, and the entries a step needs
// from other rows come by v_readlane (lane indices are compile-time constants
// after unrolling).  Only the lower triangle is meaningful; updates that land
// above the diagonal are never read.  Writes L to the lower triangle, X =
// L^{-1} transposed into the strict upper triangle and diag(X) to dx.
__device__ __forceinline__ float lane_val(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

__device__ __forceinline__ void diag_block(float *B, int ld, float *dx, float shift, int lane) {
    const int i = lane & 31;
    float row[32];
#pragma unroll
    for (int c = 0; c < 32; ++c) row[c] = B[i * ld + c];
    // right-looking Cholesky of the block
#pragma unroll
    for (int jj = 0; jj < 32; ++jj) {
        const float piv = sqrtf(fmaxf(lane_val(row[jj], jj), shift)), rp = 1.f / piv;
        const float li = row[jj] * rp;
#pragma unroll
        for (int c = jj + 1; c < 32; ++c) row[c] = fmaf(-li, lane_val(row[jj], c) * rp, row[c]);
        row[jj] = i == jj ? piv : li;
    }
    // X = L^{-1} by forward substitution, lane c owning column c
    float x[32];
#pragma unroll
    for (int r = 0; r < 32; ++r) {
        float s = r == i ? 1.f : 0.f;
#pragma unroll
        for (int m = 0; m < r; ++m) s = fmaf(-lane_val(row[m], r), x[m], s);
        x[r] = s / lane_val(row[r], r);
    }
    if (lane < 32) {
#pragma unroll
        for (int c = 0; c < 32; ++c)
            if (c <= i) B[i * ld + c] = row[c];
#pragma unroll
        for (int r = 0; r < 32; ++r)
            if (r > i) B[i * ld + r] = x[r];        // X(r, i) at B[i][r]
        dx[i] = x[i];
    }
}

// X_JJ(r, c) for the diagonal block at J0 (lower triangular, stored transposed)
__device__ __forceinline__ float x_diag(const float *S, int ld, const float *dx, int J0, int r, int c) {
    return c < r ? S[(J0 + c) * ld + J0 + r] : (c == r ? dx[J0 + r] : 0.f);
}

__global__ __launch_bounds__(512) void k_chol_inv(CholBatch batch, int ld) {
    extern __shared__ float S[];
    __shared__ float dx[kCholInverseMaxK];
    __shared__ float s_red[8];
    const CholItem &it = batch.it[blockIdx.x];
    if (!it.inverse) return;
    const int k = it.k, nb = (k + 31) >> 5, P = nb * 32;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    constexpr int NW = 8;
    JOLT_PROBE(0);
    float tr = 0.f;
    for (int i = tid; i < k; i += 512) tr += it.g[(size_t)i * it.ld + i];
    tr = wave_sum(tr);
    if (lane == 0) s_red[wid] = tr;
    __syncthreads();
    float trace = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) trace += s_red[w];
    float shift = it.rel_shift * trace / (float)k;
    if (!(shift > 0.f)) shift = FLT_MIN;
    // lower triangle of G (+ shift I); padding rows and columns are the identity
    for (int r = wid; r < P; r += NW) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int c = lane + 64 * u;
            if (c >= P) continue;
            float v = 0.f;
            if (r < k && c < k) {
                if (c <= r) v = it.g[(size_t)r * it.ld + c] + (r == c ? shift : 0.f);
            } else if (r == c) {
                v = 1.f;
            }
            S[r * ld + c] = v;
        }
    }
    __syncthreads();

    const int m32 = lane & 31, kh = lane >> 5;
    for (int J = 0; J < nb; ++J) {
        const int J0 = 32 * J;
        JOLT_PROBE(1 + 3 * J);
        if (wid == 0) diag_block(S + J0 * ld + J0, ld, dx + J0, shift, lane);
        __syncthreads();
        JOLT_PROBE(2 + 3 * J);
        // panel: L_IJ = G_IJ X_JJ^T, in place over G_IJ
        for (int t = wid; t < nb - 1 - J; t += NW) {
            const int I0 = 32 * (J + 1 + t);
            f32x16 acc = {};
#pragma unroll 4
            for (int k0 = 0; k0 < 32; k0 += 2) {
                const int kk = k0 + kh;
                const float a = S[(I0 + m32) * ld + J0 + kk];
                const float b = x_diag(S, ld, dx, J0, m32, kk);     // X_JJ^T(kk, n) = X_JJ(n, kk)
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
            }
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) S[(I0 + frag_row(lane, jj)) * ld + J0 + m32] = acc[jj];
        }
        __syncthreads();
        JOLT_PROBE(3 + 3 * J);
        // trailing: G_IK -= L_IJ L_KJ^T for J < K <= I
        const int rem = nb - 1 - J, pairs = rem * (rem + 1) / 2;
        for (int t = wid; t < pairs; t += NW) {
            int I = 0;
            while ((I + 1) * (I + 2) / 2 <= t) ++I;
            const int K = t - I * (I + 1) / 2;
            const int I0 = 32 * (J + 1 + I), K0 = 32 * (J + 1 + K);
            f32x16 acc;
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) acc[jj] = S[(I0 + frag_row(lane, jj)) * ld + K0 + m32];
#pragma unroll 4
            for (int k0 = 0; k0 < 32; k0 += 2) {
                const int kk = k0 + kh;
                const float a = -S[(I0 + m32) * ld + J0 + kk];
                const float b = S[(K0 + m32) * ld + J0 + kk];
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
            }
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) S[(I0 + frag_row(lane, jj)) * ld + K0 + m32] = acc[jj];
        }
        __syncthreads();
    }
    // off-diagonal blocks of X, block diagonal d = I - J
    JOLT_PROBE(20);
    for (int d = 1; d < nb; ++d) {
        for (int t = wid; t < nb - d; t += NW) {
            const int J0 = 32 * t, I0 = 32 * (t + d);
            f32x16 acc = {};
            for (int K = t; K < t + d; ++K) {
                const int K0 = 32 * K;
#pragma unroll 4
                for (int k0 = 0; k0 < 32; k0 += 2) {
                    const int kk = k0 + kh;
                    const float a = S[(I0 + m32) * ld + K0 + kk];                           // L_IK(m, kk)
                    const float b = K == t ? x_diag(S, ld, dx, J0, kk, m32)                  // X_JJ(kk, n)
                                           : S[(J0 + m32) * ld + K0 + kk];                   // X_KJ(kk, n)
                    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
                }
            }
            // T goes where X_IJ^T will live (block (J, I) above the diagonal)
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) S[(J0 + m32) * ld + I0 + frag_row(lane, jj)] = acc[jj];
            f32x16 x = {};
#pragma unroll 4
            for (int k0 = 0; k0 < 32; k0 += 2) {
                const int kk = k0 + kh;
                const float a = -x_diag(S, ld, dx, I0, m32, kk);                             // -X_II(m, kk)
                const float b = S[(J0 + m32) * ld + I0 + kk];                                // T(kk, n)
                x = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, x, 0, 0, 0);
            }
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) S[(J0 + m32) * ld + I0 + frag_row(lane, jj)] = x[jj];
        }
        __syncthreads();
    }
    JOLT_PROBE(21);
    // L^{-1}: X(i, c) = S[c][i] below the diagonal, dx on it
    for (int i = wid; i < k; i += NW) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int c = lane + 64 * u;
            if (c >= k) continue;
            it.l[(size_t)i * it.ld + c] = c < i ? S[c * ld + i] : (c == i ? dx[i] : 0.f);
        }
    }
}

// One wave per 32-row block tm of Q (K = 32 (tm + 1): X is lower triangular).
// X is staged in LDS once per workgroup (zero outside the k x k triangle; read
// from global memory when it does not fit), and the workgroup walks column
// blocks of 64 (cb = blockIdx.x, + gridDim.x, ...): each block of Y (all P
// rows, zero past k and len) goes through LDS, the next one is loaded into
// registers while the current one is multiplied.
constexpr int kApplyYS = 68;                // row stride of a staged Y block

template <bool XLDS>
__global__ __launch_bounds__(64 * kCholInverseMaxK / 32) void k_apply_linv(TrsmBatch batch, int ldx) {
    extern __shared__ float sh[];
    const TrsmItem &it = batch.it[blockIdx.y];
    const int k = it.k, ntm = (k + 31) >> 5, P = 32 * ntm, nthr = 64 * ntm;
    const int ncb = (it.len + 63) >> 6;
    if ((int)blockIdx.x >= ncb || (int)threadIdx.x >= nthr) return;      // whole waves leave together
    const int tid = threadIdx.x, lane = tid & 63, tm = tid >> 6;
    const int m32 = lane & 31, kh = lane >> 5, m = 32 * tm + m32, mc = min(m, k - 1);
    float *ys = sh;                             // [P][kApplyYS]
    float *xs = sh + P * kApplyYS;              // [P][ldx] when XLDS
    if constexpr (XLDS) {
        for (int e = tid; e < P * P / 4; e += nthr) {
            const int r = e / (P / 4), c = 4 * (e % (P / 4));
            const bool ok = r < k && c < k;
            float4 v = *reinterpret_cast<const float4 *>(it.l + (size_t)(ok ? r : 0) * it.ld + (ok ? c : 0));
            if (!ok) v = make_float4(0.f, 0.f, 0.f, 0.f);
            float *d = xs + r * ldx + c;
            d[0] = c < k ? v.x : 0.f;
            d[1] = c + 1 < k ? v.y : 0.f;
            d[2] = c + 2 < k ? v.z : 0.f;
            d[3] = c + 3 < k ? v.w : 0.f;
        }
    }
    // staging of a Y block: P rows x 16 float4 = exactly 8 pieces per thread
    constexpr int kPer = 8;
    float4 stg[kPer];
    auto load_y = [&](int cb) {
        const int c0 = cb * 64;
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
            const int p = tid + nthr * q;
            const int r = p >> 4, c = c0 + 4 * (p & 15);
            const bool ok = r < k && c < it.len;     // len is a multiple of 4
            const float4 v = *reinterpret_cast<const float4 *>(it.y + (size_t)(ok ? r : 0) * it.ldy + (ok ? c : 0));
            stg[q] = ok ? v : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };
    auto store_y = [&]() {
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
            const int p = tid + nthr * q;
            *reinterpret_cast<float4 *>(ys + (p >> 4) * kApplyYS + 4 * (p & 15)) = stg[q];
        }
    };
    const int kend = 32 * (tm + 1);
    const float *xrow = XLDS ? xs + m * ldx : it.l + (size_t)mc * it.ld;
    int cb = blockIdx.x;
    load_y(cb);
    for (;;) {
        __syncthreads();                        // the previous block's reads of ys are done
        store_y();
        __syncthreads();
        const int next = cb + gridDim.x;
        if (next < ncb) load_y(next);
        f32x16 acc0 = {}, acc1 = {};
#pragma unroll 8
        for (int k0 = 0; k0 < kend; k0 += 2) {
            const int kk = k0 + kh;
            const float a = XLDS ? xrow[kk] : ld_or_zero(xrow, min(kk, k - 1), m < k && kk < k);
            acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, ys[kk * kApplyYS + m32], acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, ys[kk * kApplyYS + 32 + m32], acc1, 0, 0, 0);
        }
        const int c0 = cb * 64;
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
            const int row = 32 * tm + frag_row(lane, jj);
            if (row < k) {
                if (c0 + m32 < it.len) it.q[(size_t)row * it.ldy + c0 + m32] = acc0[jj];
                if (c0 + 32 + m32 < it.len) it.q[(size_t)row * it.ldy + c0 + 32 + m32] = acc1[jj];
            }
        }
        if (next >= ncb) break;
        cb = next;
    }
}

static hipError_t allow_lds(const void *fn) {
    hipFuncAttributes fa;
    hipError_t e = hipFuncGetAttributes(&fa, fn);
    if (e != hipSuccess) return e;
    return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024 - (int)fa.sharedSizeBytes);
}
static hipError_t orth_lds_attrs() {
    static hipError_t state = hipErrorNotReady;
    if (state == hipErrorNotReady) {
        hipError_t e = allow_lds(reinterpret_cast<const void *>(k_chol_inv));
        if (e == hipSuccess) e = allow_lds(reinterpret_cast<const void *>(k_apply_linv<true>));
        if (e == hipSuccess) e = allow_lds(reinterpret_cast<const void *>(k_apply_linv<false>));
        state = e;
    }
    return state;
}

hipError_t launch_chol_inv(const CholBatch &b, int maxK, hipStream_t s) {
    if (b.n <= 0) return hipSuccess;
    if (maxK > kCholInverseMaxK) return hipErrorInvalidValue;
    if (hipError_t e = orth_lds_attrs(); e != hipSuccess) return e;
    KTimeScope kts("k_chol_inv", s);
    const int P = (maxK + 31) / 32 * 32, ld = P + 1;
    hipLaunchKernelGGL(k_chol_inv, dim3(b.n), dim3(512), (size_t)P * ld * sizeof(float), s, b, ld);
    return hipGetLastError();
}

hipError_t launch_apply_linv(const TrsmBatch &b, int maxK, int maxLen, hipStream_t s) {
    if (b.n <= 0) return hipSuccess;
    if (maxK > kCholInverseMaxK) return hipErrorInvalidValue;
    for (int i = 0; i < b.n; ++i)
        if (b.it[i].len % 4 || b.it[i].ldy % 4 || b.it[i].ld % 4) return hipErrorInvalidValue;
    if (hipError_t e = orth_lds_attrs(); e != hipSuccess) return e;
    KTimeScope kts("k_apply_linv", s);
    const int ntm = (maxK + 31) / 32, P = 32 * ntm, ldx = P + 1;
    const size_t ylds = (size_t)P * kApplyYS * sizeof(float);
    const size_t xlds = (size_t)P * ldx * sizeof(float);
    const bool xin = ylds + xlds <= 150 * 1024;
    // about two workgroups per CU over the batch; each walks its column blocks
    const int ncb = (maxLen + 63) / 64;
    const int gx = std::max(1, std::min(ncb, (512 + b.n - 1) / b.n));
    if (xin) hipLaunchKernelGGL(k_apply_linv<true>, dim3(gx, b.n), dim3(64 * ntm), ylds + xlds, s, b, ldx);
    else hipLaunchKernelGGL(k_apply_linv<false>, dim3(gx, b.n), dim3(64 * ntm), ylds, s, b, ldx);
    return hipGetLastError();
}

}  // namespace jolt
