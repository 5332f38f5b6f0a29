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
// wave, in registers.  Lanes 0..31 run the right-looking Cholesky on row
// i = lane of the block; lanes 32..63 run the forward substitution L X = I for
// column i = lane - 32 of X = L^{-1}.  Both follow one instruction stream, two
// columns (a 2 x 2 pivot block) per step:
//   L(j,j) = sqrt(a), L(j+1,j) = b / L(j,j), L(j+1,j+1) = sqrt(c - L(j+1,j)^2)
// from the current a = A(j,j), b = A(j+1,j), c = A(j+1,j+1); a lane's
// multipliers are m0 = v[j] / L(j,j) and m1 = (v[j+1] - m0 L(j+1,j)) / L(j+1,j+1)
// (L(i,j), L(i,j+1) on a factor lane, X(j,i), X(j+1,i) on a substitution lane),
// and every later entry takes v[c] -= m0 L(c,j) + m1 L(c,j+1), where L(c,.) are
// factor lane c's multipliers.  Columns j+2 and j+3 (the next pivot block's)
// get them by v_readlane at once; for the later columns the step writes its
// two columns of L to cb (LDS) and issues the broadcast reads, and the next
// step applies them, so the read latency overlaps the next pivot block.  The
// shift enters only through the pivots: the first nvalid diagonal entries get
// it (the rest is padding, already the identity), and pivots are clamped at the
// shift floor.  L itself is not kept (later steps use X_JJ and the
// off-diagonal blocks only): the substitution lanes store X transposed over
// the whole block, X(r, i) at B[i][r] (zero for r < i).
__device__ __forceinline__ float lane_val(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

__device__ __forceinline__ void diag_block(float *B, int ld, float *cb, float shift, int nvalid, int lane) {
    const int i = lane & 31;
    const bool fac = lane < 32;
    float v[32], lp0[32], lp1[32], mp0 = 0.f, mp1 = 0.f;
#pragma unroll
    for (int c = 0; c < 32; ++c) {
        const float g = B[i * ld + c];
        v[c] = fac ? g : (c == i ? 1.f : 0.f);
        lp0[c] = lp1[c] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < 32; j += 2) {
        const float a = fmaxf(lane_val(v[j], j) + (j < nvalid ? shift : 0.f), shift);
        const float b = lane_val(v[j], j + 1);
        const float c1 = lane_val(v[j + 1], j + 1) + (j + 1 < nvalid ? shift : 0.f);
        const float ra = __builtin_amdgcn_rsqf(a);
        const float l10 = b * ra;
        const float rc = __builtin_amdgcn_rsqf(fmaxf(fmaf(-l10, l10, c1), shift));
        const float m0 = v[j] * ra;
        const float m1 = fmaf(-m0, l10, v[j + 1]) * rc;
        float *col = cb + 128 * (j / 2);
        col[lane] = m0;
        col[64 + lane] = m1;
        if (j + 2 < 32) {
            const float p0 = lane_val(m0, j + 2), p1 = lane_val(m1, j + 2);
            const float q0 = lane_val(m0, j + 3), q1 = lane_val(m1, j + 3);
            v[j + 2] = fmaf(-m1, p1, fmaf(-m0, p0, v[j + 2]));
            v[j + 3] = fmaf(-m1, q1, fmaf(-m0, q0, v[j + 3]));
        }
        // the previous pivot block's update of columns j + 2 .. 31
#pragma unroll
        for (int c = j + 2; c < 32; ++c)
            if (j >= 2) v[c] = fmaf(-mp1, lp1[c], fmaf(-mp0, lp0[c], v[c]));
#pragma unroll
        for (int c = j + 4; c < 32; ++c) {
            lp0[c] = col[c];
            lp1[c] = col[64 + c];
        }
        mp0 = m0;
        mp1 = m1;
        v[j] = m0;
        v[j + 1] = m1;
        // one step at a time: without this the scheduler reorders the updates
        // column by column and keeps every broadcast value live
#pragma unroll
        for (int g = 0; g < 32; g += 8)
            asm volatile("" : "+v"(v[g]), "+v"(v[g + 1]), "+v"(v[g + 2]), "+v"(v[g + 3]), "+v"(v[g + 4]),
                         "+v"(v[g + 5]), "+v"(v[g + 6]), "+v"(v[g + 7]));
    }
    if (!fac) {
#pragma unroll
        for (int r = 0; r < 32; ++r) B[i * ld + r] = v[r];
    }
}

// X_JJ(r, c) for the diagonal block at J0 (lower triangular, stored transposed)
__device__ __forceinline__ float x_diag(const float *S, int ld, int J0, int r, int c) {
    const float u = S[(J0 + c) * ld + J0 + r];
    return c <= r ? u : 0.f;
}

// One 32 x 32 MFMA tile product over a 32-wide K block: acc += A B with
// A(m, kk) = a(m, kk) and B(kk, n) = b(kk, n) read from LDS by the caller's
// accessors (m, n = lane & 31; kk = k0 + lane / 32).
template <class FA, class FB>
__device__ __forceinline__ void tile_kblock(f32x16 &acc, int lane, FA a, FB b) {
    const int m32 = lane & 31, kh = lane >> 5;
#pragma unroll 4
    for (int k0 = 0; k0 < 32; k0 += 2) {
        const int kk = k0 + kh;
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a(m32, kk), b(kk, m32), acc, 0, 0, 0);
    }
}

// Blocked over 32 x 32 blocks, one workgroup per matrix, right-looking.  Step J:
//   A: the panel L_IJ = G_IJ X_JJ^T (I > J) and block row J of X,
//      X_JK = -X_JJ R_JK (K < J), in parallel over waves;
//   B: the trailing update G_IK -= L_IJ L_KJ^T (J < K <= I) and the
//      accumulation R_IK += L_IJ X_JK (I > J, K <= J), where R_IK =
//      sum_{M=K}^{I-1} L_IM X_MK is kept in block (K, I) above the diagonal
//      (the slot of X_IK^T); meanwhile wave 0 updates block (J+1, J+1) first
//      and factors it, so the next step's diagonal block is ready at the
//      barrier.
__global__ __launch_bounds__(512) void k_chol_inv(CholBatch batch, int ld) {
    extern __shared__ float S[];
    __shared__ float cb[32 * 64];
    const CholItem &it = batch.it[blockIdx.x];
    if (!it.inverse) return;
    const int k = it.k, nb = (k + 31) >> 5, P = nb * 32;
    // the wave index as a scalar: loops and branches on it stay uniform
    const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    constexpr int NW = 8;
    float shift = 0.f;                          // used by wave 0 only
    JOLT_PROBE(0);
    if (wid == 0) {
        // wave 0: shift = rel_shift * trace(G) / k, then block (0, 0) straight
        // from G (identity in the padding), while the other waves fill LDS
        float tr = 0.f;
        for (int r = lane; r < k; r += 64) tr += it.g[(size_t)r * it.ld + r];
        tr = wave_sum(tr);
        shift = it.rel_shift * tr / (float)k;
        if (!(shift > 0.f)) shift = FLT_MIN;
        const int i = lane & 31;
#pragma unroll
        for (int c = 0; c < 32; ++c) {
            const bool ok = i < k && c < k;
            const float g = it.g[ok ? (size_t)i * it.ld + c : 0];
            S[i * ld + c] = ok ? g : (i == c ? 1.f : 0.f);        // both half-waves write the same value
        }
        wave_lds_sync();
        diag_block(S, ld, cb, shift, k, lane);
    } else {
        // the rest of G, with the identity in the padding rows and columns
        // (float4 loads: rows of G are 16-byte aligned, it.ld is a multiple of 4)
        constexpr int kFill = 64 * (NW - 1);
        constexpr int kPer = (kCholInverseMaxK * kCholInverseMaxK / 4 + kFill - 1) / kFill;
        const int q4 = P / 4, n4 = P * q4, t = tid - 64;
        float4 stg[kPer];
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int e = t + kFill * u;
            const int r = e / q4, c = 4 * (e - r * q4);
            const bool ok = e < n4 && r < k && c < k && (r >= 32 || c >= 32);
            stg[u] = *reinterpret_cast<const float4 *>(it.g + (ok ? (size_t)r * it.ld + c : 0));
        }
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int e = t + kFill * u;
            if (e >= n4) break;
            const int r = e / q4, c = 4 * (e - r * q4);
            if (r < 32 && c < 32) continue;
            const float w[4] = {stg[u].x, stg[u].y, stg[u].z, stg[u].w};
#pragma unroll
            for (int h = 0; h < 4; ++h)
                S[r * ld + c + h] = (r < k && c + h < k) ? w[h] : (r == c + h ? 1.f : 0.f);
        }
    }
    auto LDSv = [&](int r, int c) { return S[r * ld + c]; };
    for (int J = 0; J < nb; ++J) {
        const int J0 = 32 * J;
        __syncthreads();                        // diagonal block J factored, R_JK complete
        JOLT_PROBE(1 + 2 * J);
        const int npanel = nb - 1 - J;
        for (int t = wid; t < npanel + J; t += NW) {
            f32x16 acc = {};
            if (t < npanel) {
                // L_IJ = G_IJ X_JJ^T, in place over G_IJ
                const int I0 = 32 * (J + 1 + t);
                tile_kblock(acc, lane, [&](int m, int kk) { return LDSv(I0 + m, J0 + kk); },
                            [&](int kk, int n) { return x_diag(S, ld, J0, n, kk); });
                wave_lds_sync();
#pragma unroll
                for (int jj = 0; jj < 16; ++jj) S[(I0 + frag_row(lane, jj)) * ld + J0 + (lane & 31)] = acc[jj];
            } else {
                // X_JK = -X_JJ R_JK, over R_JK in block (K, J) (stored transposed)
                const int K0 = 32 * (t - npanel);
                tile_kblock(acc, lane, [&](int m, int kk) { return -x_diag(S, ld, J0, m, kk); },
                            [&](int kk, int n) { return LDSv(K0 + n, J0 + kk); });
                wave_lds_sync();
#pragma unroll
                for (int jj = 0; jj < 16; ++jj) S[(K0 + (lane & 31)) * ld + J0 + frag_row(lane, jj)] = acc[jj];
            }
        }
        __syncthreads();
        JOLT_PROBE(2 + 2 * J);
        if (npanel == 0) break;
        const int J1 = J0 + 32;
        if (wid == 0) {
            // look-ahead: block (J+1, J+1) of the trailing update, then its factorization
            f32x16 acc;
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) acc[jj] = S[(J1 + frag_row(lane, jj)) * ld + J1 + (lane & 31)];
            tile_kblock(acc, lane, [&](int m, int kk) { return -LDSv(J1 + m, J0 + kk); },
                        [&](int kk, int n) { return LDSv(J1 + n, J0 + kk); });
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) S[(J1 + frag_row(lane, jj)) * ld + J1 + (lane & 31)] = acc[jj];
            wave_lds_sync();
            diag_block(S + J1 * ld + J1, ld, cb, shift, k - J1, lane);
        } else {
            const int ntrail = npanel * (npanel + 1) / 2 - 1, nacc = npanel * (J + 1);
            for (int t = wid - 1; t < ntrail + nacc; t += NW - 1) {
                f32x16 acc;
                if (t < ntrail) {
                    // G_IK -= L_IJ L_KJ^T, pairs after (J+1, J+1) in row-major order
                    int a = 0, pr = t + 1;
                    while ((a + 1) * (a + 2) / 2 <= pr) ++a;
                    const int I0 = J1 + 32 * a, K0 = J1 + 32 * (pr - a * (a + 1) / 2);
#pragma unroll
                    for (int jj = 0; jj < 16; ++jj) acc[jj] = S[(I0 + frag_row(lane, jj)) * ld + K0 + (lane & 31)];
                    tile_kblock(acc, lane, [&](int m, int kk) { return -LDSv(I0 + m, J0 + kk); },
                                [&](int kk, int n) { return LDSv(K0 + n, J0 + kk); });
#pragma unroll
                    for (int jj = 0; jj < 16; ++jj) S[(I0 + frag_row(lane, jj)) * ld + K0 + (lane & 31)] = acc[jj];
                } else {
                    // R_IK += L_IJ X_JK (the first term, K = J, starts the sum)
                    const int u = t - ntrail, I0 = J1 + 32 * (u / (J + 1)), K = u % (J + 1), K0 = 32 * K;
#pragma unroll
                    for (int jj = 0; jj < 16; ++jj)
                        acc[jj] = K == J ? 0.f : S[(K0 + (lane & 31)) * ld + I0 + frag_row(lane, jj)];
                    if (K == J)
                        tile_kblock(acc, lane, [&](int m, int kk) { return LDSv(I0 + m, J0 + kk); },
                                    [&](int kk, int n) { return x_diag(S, ld, J0, kk, n); });
                    else
                        tile_kblock(acc, lane, [&](int m, int kk) { return LDSv(I0 + m, J0 + kk); },
                                    [&](int kk, int n) { return LDSv(K0 + n, J0 + kk); });
#pragma unroll
                    for (int jj = 0; jj < 16; ++jj) S[(K0 + (lane & 31)) * ld + I0 + frag_row(lane, jj)] = acc[jj];
                }
            }
        }
    }
    JOLT_PROBE(21);
    // L^{-1}: X(i, c) = S[c][i] on and below the diagonal; four rows per wave
    // in flight (in-bounds loads, then selects)
    for (int i0 = wid; i0 < k; i0 += 4 * NW) {
        float val[4][3];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int i = min(i0 + q * NW, P - 1);
#pragma unroll
            for (int u = 0; u < 3; ++u) {
                const int c = min(lane + 64 * u, P - 1);
                const float x = S[c * ld + i];
                val[q][u] = c <= i ? x : 0.f;
            }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int i = i0 + q * NW;
#pragma unroll
            for (int u = 0; u < 3; ++u) {
                const int c = lane + 64 * u;
                if (i < k && c < k) it.l[(size_t)i * it.ld + c] = val[q][u];
            }
        }
    }
    JOLT_PROBE(22);
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
            if (it.qh) {
                // bf16 copies for the next sketch pass, every row (rows k .. P - 1 are zero)
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int col = c0 + 32 * u + m32;
                    if (col >= it.len) continue;
                    const float v = u ? acc1[jj] : acc0[jj];
                    const uint16_t hv = f32_to_bf16(v);
                    it.qh[(size_t)row * it.ldy + col] = hv;
                    if (it.ql) it.ql[(size_t)row * it.ldy + col] = f32_to_bf16(v - bf16_to_f32(hv));
                }
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
    for (int i = 0; i < b.n; ++i)
        if (b.it[i].ld % 4 || b.it[i].ld < b.it[i].k) return hipErrorInvalidValue;    // float4 rows of G
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
    // about one workgroup per CU over the batch; each walks its column blocks (L^-1 is
    // staged once per workgroup, so fewer, longer workgroups read less of it)
    const int ncb = (maxLen + 63) / 64;
    const int gx = std::max(1, std::min(ncb, (256 + b.n - 1) / b.n));
    if (xin) hipLaunchKernelGGL(k_apply_linv<true>, dim3(gx, b.n), dim3(64 * ntm), ylds + xlds, s, b, ldx);
    else hipLaunchKernelGGL(k_apply_linv<false>, dim3(gx, b.n), dim3(64 * ntm), ylds, s, b, ldx);
    return hipGetLastError();
}

}  // namespace jolt
