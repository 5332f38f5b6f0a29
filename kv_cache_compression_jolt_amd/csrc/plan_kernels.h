// Launch interfaces of the plan-stage kernels (factorisation of the cache).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "jolt_internal.h"

namespace jolt {

// X-pass "A M": out[c][t] = sum_kk X(t, kk) M(c, kk), kk = (lh, f) over all heads and
// layers, X(t, kk) = x[lh][t][f].  M(c, kk) = m + c * m_c + (kk / d) * m_blk + kk % d.
struct XmItem {
    const void *x;
    const void *m;
    float *out;          // [ncols][ldo], or split s at out + s * ncols * ldo
    int64_t m_c, m_blk;
    int T, LH, ncols, ldo;
    int lh_split, nsplit;   // K split: (layer, head) blocks per split, number of splits
};
struct XmBatch { XmItem it[kMaxBatch]; int n; };
hipError_t launch_xm(const XmBatch &b, int dtype, int d, int maxT, int maxCols, int maxSplit, hipStream_t s);

// X-pass "Q^T A": out[s][c][lh d + f] = sum_{t in split s} q[c][t] x[lh][t][f]
// (q in the X dtype; an optional second operand ql is added: hi + lo split).
struct XtqItem {
    const void *x;
    const void *qh;
    const void *ql;      // may be null
    float *out;          // [nsplit][ncols][LH d]
    int T, LH, ncols, ldq, tsplit, nsplit;
};
struct XtqBatch { XtqItem it[kMaxBatch]; int n; };
hipError_t launch_xtq(const XtqBatch &b, int dtype, int d, int maxLH, int maxSplit, int maxCols, hipStream_t s);

// feature Gram partials: out[p][f1][f2] = sum over rows of chunk p of x[r][f1] x[r][f2]
struct GramItem {
    const void *x;
    float *out;          // [P][d][d]
    int64_t rows;
    int chunk, P;
};
struct GramBatch { GramItem it[kMaxBatch]; int n; };
hipError_t launch_gram_rows(const GramBatch &b, int dtype, int d, int maxP, hipStream_t s);

// generic batched fp32 GEMM with element strides and split-K partial outputs
// C[bi](i, j) (+split s) = sum_{k in split s} A[bi](i, k) B[bi](k, j); bi < nb is an
// inner batch with its own base strides (a_z, b_z, c_z).
struct GemmItem {
    const float *a, *b;
    float *c;
    int64_t a_i, a_k, b_k, b_j, c_i, c_j, c_split;
    int64_t a_z, b_z, c_z;
    int M, N, K, kchunk, nsplit, nb;
};
struct GemmBatch { GemmItem it[kMaxBatch]; int n; };
hipError_t launch_gemm(const GemmBatch &b, int maxM, int maxN, int maxSplit, int maxNb, hipStream_t s);
// The same product on the bf16 MFMA with both operands split into hi + lo
// planes (about 2^-16 relative per product), for products whose operands are
// well conditioned; operands need unit stride along their row index or K
// (others go to launch_gemm).
hipError_t launch_gemm_split(const GemmBatch &b, int maxM, int maxN, int maxSplit, int maxNb, hipStream_t s);

// Symmetric Gram of the rows of Y (k x len, row stride ldy): part[s][r][c] = sum
// over the columns t of split s (chunk columns each) of y[r][t] y[c][t], for
// r, c < kp (rows >= k count as zero); both triangles are written.
struct SymGramItem {
    const float *y;
    float *part;          // [nsplit][kp][kp]
    int k, kp, len, ldy, chunk, nsplit;
};
struct SymGramBatch { SymGramItem it[kMaxBatch]; int n; };
constexpr int kSymGramMaxK = 192;
constexpr int kSymGramWideK = 288;
hipError_t launch_sym_gram(const SymGramBatch &b, int maxK, int maxSplit, hipStream_t s);

// out[i] = sum_s part[s * stride + i], i < count (fixed order); optional double trace
struct ReduceItem {
    const float *part;
    float *out;
    int64_t stride, count;
    int nsplit;
};
struct ReduceBatch { ReduceItem it[kMaxBatch]; int n; };
hipError_t launch_reduce(const ReduceBatch &b, int64_t maxCount, hipStream_t s);

// Cholesky of G + shift I (k x k, ld) -> lower L written to l (k x k, ld), zeros above
struct CholItem {
    const float *g;
    float *l;            // L, or L^{-1} when inverse != 0 (k <= kCholWideMaxK)
    int k, ld;
    float rel_shift;     // shift = rel_shift * trace(G) / k
    int inverse;
    float *work;         // k > kCholInverseMaxK: P x P device scratch (P = k rounded up to 32)
};
struct CholBatch { CholItem it[kSolverBatch]; int n; };
hipError_t launch_cholesky(const CholBatch &b, int maxK, hipStream_t s);

// rows 0..k-1 of y[k][len] <- L^{-1} y   (forward substitution, in place allowed)
struct TrsmItem {
    const float *l;
    const float *y;
    float *q;
    int k, ld, len, ldy;
    uint16_t *qh, *ql;   // optional bf16 copies of q (hi, and lo = q - hi), all kp rows (apply only)
};
struct TrsmBatch { TrsmItem it[kMaxBatch]; int n; };
hipError_t launch_trsm(const TrsmBatch &b, int maxK, int maxLen, hipStream_t s);
// y <- X y with X = L^{-1} lower triangular (in place; k <= 600)
hipError_t launch_apply_linv(const TrsmBatch &b, int maxK, int maxLen, hipStream_t s);
constexpr int kCholInverseMaxK = 192;     // the inverse factor's working square in LDS
constexpr int kCholWideMaxK = 288;        // ... or in the item's work buffer
// the fused elimination behind launch_cholesky for the inverse != 0 items
hipError_t launch_chol_inv(const CholBatch &b, int maxK, hipStream_t s);

// symmetric eigen-decomposition by parallel-order two-sided Jacobi in LDS (n <= 142)
// vec[r][c] = component r of eigenvector c, eigenvalues descending, sign-normalised.
struct JacItem {
    const float *a;
    float *vec;
    float *lam;
    int n, lda, ldv;
    int raw;             // 1: eigenpairs in Jacobi order (no sort / sign change)
    int *sweeps_out;     // sweeps used, or -1 if the cap was hit
    float *tw;           // tridiagonal solver only: eig_tri_ws_bytes(n) of device workspace
};
struct JacBatch { JacItem it[kSolverBatch]; int n; };
constexpr int kJacobiMaxN = 142;
// retry_only: solve only the items whose sweeps_out holds kEigRetry
hipError_t launch_jacobi_lds(const JacBatch &b, int maxN, int max_sweeps, hipStream_t s, int retry_only = 0);

// Householder tridiagonal eigensolver for n <= kTriMaxN (same outputs as the
// Jacobi kernel; sweeps_out is required and receives 0, or kEigRetry when the
// matrix must be handed to the Jacobi kernel; every item needs its own tw of
// eig_tri_ws_bytes(n), 16-byte aligned, which the three launches share)
constexpr int kTriMaxN = 140;
// the wide variant of the same four-launch solver (140 < n <= kWideMaxN): the
// reduction keeps the matrix in registers and the polish works in the
// workspace; it has no Jacobi hand-back (a matrix it cannot make orthonormal
// reports -1 in sweeps_out, results written)
constexpr int kWideMaxN = 272;
constexpr int kEigRetry = -2;
constexpr int kEigWideFail = -3;    // the wide solver's sweeps_out when it could not finish
// row pitch (floats) of the solver's n x n workspace matrices
inline int eig_tri_np(int n) { return n > kTriMaxN ? (n + 15) / 16 * 16 : (n + 3) / 4 * 4; }
inline size_t eig_tri_ws_bytes(int n) {
    const size_t blocks = ((n > 2 ? n - 2 : 0) + 31) / 32;
    const size_t np = (size_t)eig_tri_np(n);
    const size_t ex = n > kTriMaxN ? (size_t)n * np : 0;      // the wide polish's E
    return (((size_t)2 * n * np + 1024 * blocks + 4 * (size_t)n + 4 + ex) * 4 + 255) / 256 * 256;
}
hipError_t launch_eig_tridiag(const JacBatch &b, int maxN, hipStream_t s);

// A solver batch whose item table is in device memory, for any number of
// items in one launch (a by-value batch is limited by the kernel-argument
// size): the kernels read it.it[blockIdx] exactly as from a by-value batch.
// The launchers take the host copy of the items too, for their checks and
// sizes; launch_put_table copies a table to device memory in stream order.
template <typename Item> struct DevTable {
    const Item *it;
    int n;
};
typedef DevTable<JacItem> JacTable;
typedef DevTable<CholItem> CholTable;
typedef DevTable<SymGramItem> SymGramTable;
// every item of a plan group in one launch
hipError_t launch_sym_gram(const SymGramItem *host, const SymGramTable &dev, int maxK, int maxSplit, hipStream_t s);
hipError_t launch_eig_tridiag(const JacItem *host, const JacTable &dev, int maxN, hipStream_t s);
hipError_t launch_jacobi_lds(const JacItem *host, const JacTable &dev, int maxN, int max_sweeps, hipStream_t s,
                             int retry_only = 0);
hipError_t launch_chol_inv(const CholItem *host, const CholTable &dev, int maxK, hipStream_t s);
// bytes (a multiple of 4) from host memory to dev (4-byte aligned), through
// kernel arguments: the host memory may be reused as soon as this returns
hipError_t launch_put_table(const void *host, size_t bytes, void *dev, hipStream_t s);

// block Jacobi state of one large symmetric matrix (N = padded size, multiple of 128)
struct EigItem {
    const float *g;      // input n x n (ld ldg)
    float *a, *t;        // N x N working matrix and its permuted copy
    float *v, *vt;       // N x N rotations and its permuted copy
    float *norms;        // [2]: off-diagonal and total sum of squares
    float *vec, *lam;    // outputs: n x n (ld ldv) and n
    int n, N, ldg, ldv;
};
struct EigBatch { EigItem it[kMaxBatch]; int n; };
struct BlockPerm { int src[32]; };
hipError_t launch_eig_init(const EigBatch &b, int maxN, hipStream_t s);
hipError_t launch_block_permute(const EigBatch &b, const BlockPerm &p, int maxN, hipStream_t s);
hipError_t launch_offnorm(const EigBatch &b, hipStream_t s);
hipError_t launch_eig_finish(const EigBatch &b, int maxN, hipStream_t s);

// batched small kernels (one launch for all items of a chunk)
struct SmallItem {
    const float *in;     // trace: G (d x d); energy: core; to_bf16: source
    float *out32;        // energy: E; gen_omega: fp32 Omega^T
    double *out64;       // trace
    uint16_t *hi, *lo;   // to_bf16 / gen_omega (bf16 Omega^T)
    int64_t count;       // elements (to_bf16, gen_omega: kp * n)
    uint64_t key;        // gen_omega
    int a, b, c;         // trace: d; energy: LH, rt_max, d; gen_omega: k, kp, (n in count / kp)
};
struct SmallBatch { SmallItem it[kMaxBatch]; int n; };
hipError_t launch_trace_batch(const SmallBatch &b, hipStream_t s);
hipError_t launch_energy_batch(const SmallBatch &b, int64_t maxCount, hipStream_t s);

// captured energy on the candidate grid, in fp64:
// S[i][j] = sum_{r < step (i+1), f < step (j+1)} E[r][f] (E rows of length d),
// and s_fixed = sum_{r < frt, f < frf} E[r][f] when frt > 0
struct GridItem {
    const float *E;
    double *S, *s_fixed;
    int d, step, nr, nf, frt, frf;
};
struct GridBatch { GridItem it[kMaxBatch]; int n; };
hipError_t launch_energy_grid(const GridBatch &b, hipStream_t s);
hipError_t launch_to_bf16_batch(const SmallBatch &b, int64_t maxCount, hipStream_t s);
hipError_t launch_gen_omega_batch(const SmallBatch &b, int64_t maxCount, hipStream_t s);

// elementwise conversions
hipError_t launch_to_bf16(const float *in, uint16_t *hi, uint16_t *lo, int64_t count, hipStream_t s);
hipError_t launch_transpose(const float *in, float *out, int rows, int cols, int ldi, int ldo, hipStream_t s);
hipError_t launch_zero(void *p, size_t bytes, hipStream_t s);

// stored parameters -> payload (rounded to the item dtype) + header
struct StoreItem {
    const float *ut;     // [rt_max][T]
    const float *uf;     // [d][d]
    const float *core;   // [LH][rt_max][d]
    uint8_t *pay;
    size_t off_ut, off_uf, off_core;
    int T, d, LH, rt_max, rt, rf;
    uint32_t header[16];
};
struct StoreBatch { StoreItem it[kMaxBatch]; int n; };
hipError_t launch_store(const StoreBatch &b, int dtype, hipStream_t s);

}  // namespace jolt
