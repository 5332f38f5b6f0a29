// jolt_plan: factor every item, then allocate (r_t, r_f, b) with the single dual.
//
// Per item ("A JoLT for the KV cache", landing page abstract; author page abstract):
//   feature factor  U_f = eigenvectors of G_f = sum over (layer, head, token) of x x^T
//   token factor    exact:      eigenvectors of A A^T (A = token unfolding, T x L H d)
//                   randomized: FlashJoLT range finder (Halko, Martinsson & Tropp,
//                               SIAM Review 2011, Alg. 4.4 + Alg. 5.1): Y = A Omega,
//                               Q = orth(Y); q times Q = orth(A orth(A^T Q));
//                               B = Q^T A; W = B B^T = U~ L U~^T; U_t = Q U~
//   core            C_lh = U_t^T X_lh U_f, energy E[i][j] = sum_lh C_lh[i][j]^2, ||X||^2
// then one sync, the distortion / byte tables on the host and the dual (planner.cpp).
//
// orth() is shifted Cholesky QR (Fukaya et al. 2020): G = Y Y^T + s I = L L^T,
// Q = L^{-1} Y (rows are the basis vectors), once for the intermediate bases
// and twice for the final one.
#include <algorithm>
#include <chrono>
#include <cmath>
#include <cstdio>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "api_internal.h"
#include "jolt_internal.h"
#include "plan_kernels.h"
#include "planner.h"

namespace jolt {

namespace {

struct Bump {
    size_t off = 0;
    size_t take(size_t bytes) {
        const size_t o = off;
        off = align_up(off + std::max<size_t>(bytes, 1), 256);
        return o;
    }
};

// Device item tables of a plan group's solver launches (feature eigensolver,
// token eigensolver, CholeskyQR), in the group scratch after the items'.
constexpr int kTableItems = kPlanGroup;
struct Tables {
    size_t feat, tok, chol, sg;
};
inline Tables reserve_tables(Bump &b) {
    const size_t bytes = (size_t)kTableItems * std::max(sizeof(JacItem), sizeof(CholItem));
    Tables t;
    t.feat = b.take(bytes);
    t.tok = b.take(bytes);
    t.chol = b.take(bytes);
    t.sg = b.take((size_t)kTableItems * sizeof(SymGramItem));
    return t;
}

struct Dims {
    int L, H, T, d, LH, n;       // n = L H d
    int e;                        // element bytes of the item dtype
    int k, kp;                    // sketch width and its 32-padding
    int rt_max, rf_max, rtp32;
    int xs_split, xs_tsplit;      // Q^T A passes: splits over tokens
    int gf_P, gf_chunk;           // feature Gram partial sums
    int gT_split, gT_chunk;       // Gram of a T-long basis
    int gN_split, gN_chunk;       // Gram of an n-long basis
    int xm_split, xm_lh;          // A M passes: K split over (layer, head) blocks
};

struct Scratch {
    size_t omt, yt, ypart, qh, ql, zt, zb, xpart, gpart, gram, lmat, csq, wmat, vmat, lamk, sweeps;
    size_t gfpart, gf, pmat, gt, vt, lamT, uh, ul;
    size_t eA, eT, eV, eVT, eR, eRlam, eNorm, eSw;     // block Jacobi (n > 142)
    size_t etri, ftri;      // tridiagonal solver workspaces (token, feature); SIZE_MAX if unused
    int eN;                                             // padded size, 0 if unused
};

// size of the eigenproblem solved for the token factor
int token_eig_n(const jolt_config &cfg, const Dims &D) {
    return cfg.mode == JOLT_TOKEN_RANDOMIZED ? D.k : D.T;
}

int clampi(int v, int lo, int hi) { return std::max(lo, std::min(hi, v)); }

// Splits of the symmetric Grams over whole 64-column chunks, at most cap.
void set_gram_splits(Dims &D, int cap) {
    D.gT_split = clampi(D.T / 64, 1, cap);
    D.gT_chunk = round_up((D.T + D.gT_split - 1) / D.gT_split, 64);
    D.gT_split = (D.T + D.gT_chunk - 1) / D.gT_chunk;
    D.gN_split = clampi(D.n / 64, 1, cap);
    D.gN_chunk = round_up((D.n + D.gN_split - 1) / D.gN_split, 64);
    D.gN_split = (D.n + D.gN_chunk - 1) / D.gN_chunk;
}

Dims dims_for(const jolt_config &cfg, const jolt_item &it, int rt_max, int rf_max) {
    Dims D;
    D.L = it.L; D.H = it.H; D.T = it.T; D.d = it.d;
    D.LH = it.L * it.H;
    D.n = D.LH * it.d;
    D.e = elem_bytes(it.dtype);
    D.rt_max = rt_max; D.rf_max = rf_max;
    D.rtp32 = round_up(std::max(rt_max, 1), 32);
    D.k = (cfg.mode == JOLT_TOKEN_RANDOMIZED) ? rt_max + cfg.oversample : 0;
    D.kp = round_up(std::max(D.k, 1), 32);
    // Q^T A: about one workgroup per CU, as for A M below (ceil(n / 256) feature
    // tiles per item, 16 items per launch); a split adds a reduction pass
    D.xs_split = clampi(256 / std::max(1, ((D.n + 255) / 256) * kMaxBatch), 1, std::max(1, D.T / 64));
    D.xs_tsplit = round_up((D.T + D.xs_split - 1) / D.xs_split, 64);
    D.xs_split = (D.T + D.xs_tsplit - 1) / D.xs_tsplit;
    const int64_t rows = (int64_t)D.LH * D.T;
    D.gf_P = (int)std::min<int64_t>(64, std::max<int64_t>(1, rows / 512));
    D.gf_chunk = round_up((int)((rows + D.gf_P - 1) / D.gf_P), 64);
    D.gf_P = (int)((rows + D.gf_chunk - 1) / D.gf_chunk);
    // symmetric Grams of k-row panels: up to 16 splits of whole 64-column chunks
    // (16 items x 16 splits fill the CUs)
    set_gram_splits(D, 16);
    // about one workgroup per CU: ceil(T / 256) token tiles per item, 16 items per launch
    D.xm_split = clampi(256 / std::max(1, ((D.T + 255) / 256) * kMaxBatch), 1, 8);
    D.xm_split = std::min(D.xm_split, D.LH);
    D.xm_lh = (D.LH + D.xm_split - 1) / D.xm_split;
    D.xm_split = (D.LH + D.xm_lh - 1) / D.xm_lh;
    return D;
}

void reserve_scratch(const jolt_config &cfg, const Dims &D, Bump &b, Scratch &s) {
    std::memset(&s, 0, sizeof s);
    const size_t T = D.T, n = D.n, kp = D.kp, d = D.d;
    s.gfpart = b.take((size_t)D.gf_P * d * d * 4);
    s.gf = b.take(d * d * 4);
    if (cfg.mode == JOLT_TOKEN_RANDOMIZED) {
        s.omt = b.take(kp * n * D.e);
        s.yt = b.take(kp * T * 4);
        s.ypart = D.xm_split > 1 ? b.take((size_t)D.xm_split * kp * T * 4) : 0;
        if (D.e == 2) {
            s.qh = b.take(kp * T * 2);
            s.ql = b.take(kp * T * 2);
            s.zb = b.take(kp * n * 2);
        }
        s.zt = b.take(kp * n * 4);
        s.xpart = b.take((size_t)D.xs_split * kp * n * 4);
        s.gpart = b.take((size_t)std::max(D.gT_split, D.gN_split) * kp * kp * 4);
        s.gram = b.take(kp * kp * 4);
        s.lmat = b.take(kp * kp * 4);
        s.csq = D.k > kCholInverseMaxK ? b.take(kp * kp * 4) : 0;     // the inverse factor's working square
        s.wmat = b.take(kp * kp * 4);
        s.vmat = b.take(kp * kp * 4);
        s.lamk = b.take(kp * 4);
        s.pmat = b.take((size_t)D.rt_max * n * 4);
    } else {
        s.gt = b.take(T * T * 4);
        s.vt = b.take(T * T * 4);
        s.lamT = b.take(T * 4);
        s.uh = b.take((size_t)D.rtp32 * T * D.e);
        if (D.e == 2) s.ul = b.take((size_t)D.rtp32 * T * 2);
        s.xpart = b.take((size_t)D.xs_split * D.rtp32 * n * 4);
        s.pmat = b.take((size_t)D.rtp32 * n * 4);
    }
    s.sweeps = b.take(16);
    const int ne = token_eig_n(cfg, D);
    // the token and feature eigenproblems run at the same time on two streams
    s.etri = ne <= kWideMaxN ? b.take(eig_tri_ws_bytes(ne)) : SIZE_MAX;
    s.ftri = D.d <= kWideMaxN ? b.take(eig_tri_ws_bytes(D.d)) : SIZE_MAX;
    s.eN = 0;
    if (ne > kJacobiMaxN) {     // block Jacobi: above kWideMaxN, and the wide solver's fallback
        const size_t N = (size_t)round_up(ne, 128), P = N / 128;
        s.eN = (int)N;
        s.eA = b.take(N * N * 4);
        s.eT = b.take(N * N * 4);
        s.eV = b.take(N * N * 4);
        s.eVT = b.take(N * N * 4);
        s.eR = b.take(P * 128 * 128 * 4);
        s.eRlam = b.take(P * 128 * 4);
        s.eNorm = b.take(16);
        s.eSw = b.take(P * 4);
    }
}

struct Ctx {
    jolt_handle h;
    hipStream_t st;
    int dtype, d;
};

#define HIPCHK(expr, where)                                   \
    do {                                                      \
        hipError_t e_ = (expr);                               \
        if (e_ != hipSuccess) return hip_fail(c.h, e_, where); \
    } while (0)

}  // namespace

// ------------------------------------------------------------------ config and layout
jolt_status check_config(jolt_handle h, const jolt_config &cfg, const jolt_item *items, int n) {
    if (cfg.mode != JOLT_TOKEN_EXACT && cfg.mode != JOLT_TOKEN_RANDOMIZED) return fail(h, JOLT_E_INVALID, "mode");
    if (cfg.group_size != 64) return fail(h, JOLT_E_UNSUPPORTED, "group_size must be 64");
    if (cfg.rank_step < 1) return fail(h, JOLT_E_INVALID, "rank_step must be >= 1");
    if (cfg.rt_max < 0 || cfg.rt_max > 256) return fail(h, JOLT_E_INVALID, "rt_max must be in [0, 256]");
    if (cfg.oversample < 0 || cfg.power_iters < 0 || cfg.power_iters > 8) return fail(h, JOLT_E_INVALID, "p / q");
    if (cfg.bits_mask == 0 || (cfg.bits_mask & ~0x1FDu)) return fail(h, JOLT_E_INVALID, "bits_mask: b in {0, 2..8}");
    if (cfg.budget_bytes >= 0) {
        if (!(cfg.delta_b[0] == 1.0)) return fail(h, JOLT_E_INVALID, "delta_b[0] must be 1");
        for (int b = 2; b <= 8; ++b)
            if ((cfg.bits_mask >> b) & 1u)
                if (!(cfg.delta_b[b] > 0.0) || !std::isfinite(cfg.delta_b[b]))
                    return fail(h, JOLT_E_INVALID, "delta_b[%d] must be positive", b);
    } else {
        if (cfg.fixed_rt < 0 || cfg.fixed_rf < 0 || cfg.fixed_rt > cfg.rt_max ||
            cfg.fixed_bits < 0 || cfg.fixed_bits == 1 || cfg.fixed_bits > 8)
            return fail(h, JOLT_E_INVALID, "fixed ranks / bits");
    }
    for (int i = 0; i < n; ++i) {
        const jolt_item &it = items[i];
        if (it.T % 64) return fail(h, JOLT_E_UNSUPPORTED, "plan: T must be a multiple of 64");
        const int rf_max = cfg.rf_max ? cfg.rf_max : it.d;
        if (rf_max > it.d || rf_max < 0) return fail(h, JOLT_E_INVALID, "rf_max > d");
        if (cfg.budget_bytes < 0 && cfg.fixed_rf > rf_max) return fail(h, JOLT_E_INVALID, "fixed_rf > rf_max");
        if (cfg.rt_max > it.T) return fail(h, JOLT_E_INVALID, "rt_max > T");
        if (cfg.mode == JOLT_TOKEN_RANDOMIZED) {
            const int k = cfg.rt_max + cfg.oversample;
            if (k < 1 || k > it.T || k > it.L * it.H * it.d)
                return fail(h, JOLT_E_INVALID, "sketch width rt_max + oversample must be in [1, min(T, L H d)]");
            if (k > 2048) return fail(h, JOLT_E_UNSUPPORTED, "sketch width above 2048 not supported");
        } else {
            if (it.T > 2048) return fail(h, JOLT_E_UNSUPPORTED, "exact mode: T above 2048 not supported (T x T eigensolve)");
        }
    }
    return JOLT_OK;
}

jolt_status plan_layout(const jolt_config &cfg, const jolt_item *items, int n, PlanLayout *out) {
    jolt_status s = check_config(nullptr, cfg, items, n);
    if (s) return s;
    PlanLayout pl;
    pl.rt_max = cfg.rt_max;
    pl.rf_max = n > 0 ? (cfg.rf_max ? cfg.rf_max : items[0].d) : 0;
    pl.k = cfg.mode == JOLT_TOKEN_RANDOMIZED ? cfg.rt_max + cfg.oversample : 0;
    pl.kp = round_up(std::max(pl.k, 1), 32);
    Bump b;
    pl.item.resize(n);
    // host-bound results of all items in one block, per item:
    // [S grid (grid_nr x grid_nf doubles) | S at the fixed ranks | ||X||^2 | status]
    const size_t rt1 = std::max(pl.rt_max, 1);
    pl.step = std::max(cfg.rank_step, 1);
    pl.grid_nr = pl.rt_max / pl.step;
    pl.grid_nf = pl.rf_max / pl.step;
    const size_t cells = std::max(pl.grid_nr * pl.grid_nf, 1);
    pl.readback_stride = align_up(cells * 8 + 8 + 8 + 16, 256);
    pl.readback = b.take(pl.readback_stride * std::max(n, 1));
    for (int i = 0; i < n; ++i) {
        const jolt_item &it = items[i];
        const size_t rt = rt1, T = it.T, d = it.d, LH = (size_t)it.L * it.H;
        FactorOffsets &o = pl.item[i];
        o.ut = b.take(rt * T * 4);
        o.uf = b.take(d * d * 4);
        const size_t nlam = std::max<size_t>(std::max<size_t>(rt, 256),
                                             std::max<size_t>(round_up(pl.k, 32), cfg.mode == JOLT_TOKEN_EXACT ? T : 0));
        o.lam_t = b.take(nlam * 4);
        o.lam_f = b.take(d * 4);
        o.core = b.take(LH * rt * d * 4);
        o.energy = b.take(rt * d * 4);
        o.grid = pl.readback + i * pl.readback_stride;
        o.sfixed = o.grid + cells * 8;
        o.normx2 = o.sfixed + 8;
        o.sweeps = o.normx2 + 8;
    }
    pl.scratch = b.off;
    size_t worst = 0;
    for (int c0 = 0; c0 < n; c0 += kPlanGroup) {
        Bump sb;
        for (int i = c0; i < std::min(n, c0 + kPlanGroup); ++i) {
            Dims D = dims_for(cfg, items[i], pl.rt_max, pl.rf_max);
            Scratch S;
            reserve_scratch(cfg, D, sb, S);
        }
        reserve_tables(sb);
        worst = std::max(worst, sb.off);
    }
    pl.scratch_bytes = worst;
    pl.total = pl.scratch + worst;
    *out = pl;
    return JOLT_OK;
}

// ------------------------------------------------------------------ device pipeline
namespace {


// ------------------------------------------------------------------ eigensolvers
// Symmetric eigen-decompositions (descending, sign-normalised eigenvectors).
// n <= 272: the Householder-tridiagonal solver (k_eig.hip), n <= 140 with the
// Jacobi kernel for the matrices it hands back.
// n > 272: block Jacobi over 64-wide blocks (see k_plan.hip): every round the
// pair sub-matrices (128 x 128) are diagonalised in LDS and the rotations are
// applied to the whole matrix and to V with the fp32 GEMM; sweeps repeat until
// off(A) <= 4e-6 ||A||_F (checked on the host once per sweep).
struct EigReq {
    const float *g;
    int ldg, n;
    float *vec;
    int ldv;
    float *lam;
    int *sw;
    const Scratch *S;
    float *tw;       // tridiagonal solver workspace (n <= kTriMaxN)
};

int rr_pos_host(int i, int round, int m) {
    if (i == 0) return 0;
    return 1 + (((i - 1 - round) % (m - 1)) + (m - 1)) % (m - 1);
}

jolt_status eig_block(const Ctx &c, const std::vector<EigReq> &reqs, int N, uint8_t *scr, int max_sweeps,
                      bool *noconv) {
    auto F = [&](size_t off) { return reinterpret_cast<float *>(scr + off); };
    EigBatch eb{};
    for (const EigReq &r : reqs) {
        EigItem &e = eb.it[eb.n++];
        e.g = r.g; e.ldg = r.ldg; e.n = r.n; e.N = N;
        e.a = F(r.S->eA); e.t = F(r.S->eT); e.v = F(r.S->eV); e.vt = F(r.S->eVT);
        e.norms = F(r.S->eNorm); e.vec = r.vec; e.ldv = r.ldv; e.lam = r.lam;
    }
    HIPCHK(launch_eig_init(eb, N, c.st), "eig init");
    const int NB = N / 64, P = N / 128;
    std::vector<int> cur(NB), desired(NB);
    for (int b = 0; b < NB; ++b) cur[b] = b;
    const float tol2 = 4e-6f * 4e-6f;
    float prev = 1.f;
    bool converged = false;
    const int inner_sweeps = 4;
    for (int sweep = 0; sweep < max_sweeps && !converged; ++sweep) {
        for (int round = 0; round < NB - 1; ++round) {
            for (int p = 0; p < NB / 2; ++p) {
                desired[2 * p] = rr_pos_host(p, round, NB);
                desired[2 * p + 1] = rr_pos_host(NB - 1 - p, round, NB);
            }
            BlockPerm bp{};
            for (int b = 0; b < NB; ++b)
                for (int q = 0; q < NB; ++q)
                    if (cur[q] == desired[b]) bp.src[b] = q;
            HIPCHK(launch_block_permute(eb, bp, N, c.st), "eig permute");
            for (int i = 0; i < eb.n; ++i) {
                std::swap(eb.it[i].a, eb.it[i].t);
                std::swap(eb.it[i].v, eb.it[i].vt);
            }
            cur = desired;
            // pair sub-problems
            JacBatch jb{};
            for (size_t i = 0; i < reqs.size(); ++i) {
                for (int p = 0; p < P; ++p) {
                    JacItem &j = jb.it[jb.n++];
                    j.a = eb.it[i].a + (size_t)128 * p * N + 128 * p;
                    j.lda = N;
                    j.vec = F(reqs[i].S->eR) + (size_t)p * 128 * 128;
                    j.ldv = 128;
                    j.lam = F(reqs[i].S->eRlam) + 128 * p;
                    j.n = 128;
                    j.raw = 1;
                    j.sweeps_out = reinterpret_cast<int *>(scr + reqs[i].S->eSw) + p;
                    if (jb.n == kSolverBatch) {
                        HIPCHK(launch_jacobi_lds(jb, 128, inner_sweeps, c.st), "eig pairs");
                        jb.n = 0;
                    }
                }
            }
            HIPCHK(launch_jacobi_lds(jb, 128, inner_sweeps, c.st), "eig pairs");
            // A <- J^T A J (rows into t, then columns back into a), V <- V J
            GemmBatch rows{}, cols{}, vup{};
            for (size_t i = 0; i < reqs.size(); ++i) {
                const float *R = F(reqs[i].S->eR);
                EigItem &e = eb.it[i];
                GemmItem &g = rows.it[rows.n++];
                g.a = R; g.a_i = 1; g.a_k = 128; g.a_z = 128 * 128;
                g.b = e.a; g.b_k = N; g.b_j = 1; g.b_z = (int64_t)128 * N;
                g.c = e.t; g.c_i = N; g.c_j = 1; g.c_z = (int64_t)128 * N; g.c_split = 0;
                g.M = 128; g.N = N; g.K = 128; g.kchunk = 128; g.nsplit = 1; g.nb = P;
                GemmItem &h = cols.it[cols.n++];
                h.a = e.t; h.a_i = N; h.a_k = 1; h.a_z = 128;
                h.b = R; h.b_k = 128; h.b_j = 1; h.b_z = 128 * 128;
                h.c = e.a; h.c_i = N; h.c_j = 1; h.c_z = 128; h.c_split = 0;
                h.M = N; h.N = 128; h.K = 128; h.kchunk = 128; h.nsplit = 1; h.nb = P;
                GemmItem &v = vup.it[vup.n++];
                v = h;
                v.a = e.v; v.c = e.vt;
            }
            HIPCHK(launch_gemm(rows, 128, N, 1, P, c.st), "eig rows");
            HIPCHK(launch_gemm(cols, N, 128, 1, P, c.st), "eig cols");
            HIPCHK(launch_gemm(vup, N, 128, 1, P, c.st), "eig vectors");
            for (int i = 0; i < eb.n; ++i) std::swap(eb.it[i].v, eb.it[i].vt);
        }
        HIPCHK(launch_offnorm(eb, c.st), "eig offnorm");
        // stop at the tolerance, or once the off-diagonal norm stops falling
        // (quadratic convergence has reached the fp32 rounding floor); every
        // item's two norms come back in one synchronisation per sweep
        float *nr = nullptr;
        HIPCHK(sweep_buffer(c.h, &nr), "eig norms");
        for (int i = 0; i < eb.n; ++i)
            HIPCHK(hipMemcpyAsync(nr + 2 * i, eb.it[i].norms, 2 * sizeof(float), hipMemcpyDeviceToHost, c.st),
                   "eig norms");
        HIPCHK(hipStreamSynchronize(c.st), "eig norms");
        float worst = 0.f;
        for (int i = 0; i < eb.n; ++i) {
            const float rel2 = nr[2 * i + 1] > 0.f ? nr[2 * i] / nr[2 * i + 1] : 0.f;
            worst = std::max(worst, rel2);
        }
        if (getenv("JOLT_DEBUG")) fprintf(stderr, "libjolt: block Jacobi N=%d sweep %d off %.3e\n", N, sweep, sqrtf(worst));
        if (worst <= tol2) converged = true;
        else if (sweep > 0 && worst > 0.25f * prev) {
            converged = true;
            if (worst > 1e-8f && noconv) *noconv = true;       // stalled above 1e-4 relative
        }
        prev = worst;
    }
    if (!converged && noconv) *noconv = true;
    HIPCHK(launch_eig_finish(eb, N, c.st), "eig finish");
    return JOLT_OK;
}

// table: device memory for the item tables of this call's tridiagonal
// solves (one launch each for all the n <= kTriMaxN matrices and all the wide
// ones; kTableItems items in all), else slices of kSolverBatch by value
jolt_status eig_all(const Ctx &c, const std::vector<EigReq> &reqs, uint8_t *scr, int max_sweeps, bool *noconv,
                    bool wide_ok, JacItem *table) {
    JacBatch jb{};
    int maxN = 0, maxT = 0, maxW = 0;
    std::vector<JacItem> tri, wide;
    std::vector<std::vector<EigReq>> large;
    std::vector<int> largeN;
    for (const EigReq &r : reqs) {
        JacItem j{};
        j.a = r.g; j.lda = r.ldg; j.vec = r.vec; j.ldv = r.ldv; j.lam = r.lam; j.n = r.n; j.sweeps_out = r.sw;
        j.raw = 0;
        if (wide_ok && r.n <= kWideMaxN && r.n > kTriMaxN && r.sw && r.tw) {
            // the wide tridiagonal solver for kTriMaxN < n <= kWideMaxN
            j.tw = r.tw;
            wide.push_back(j);
            maxW = std::max(maxW, r.n);
        } else if (r.n <= kTriMaxN && r.sw && r.tw) {
            // tridiagonal solver first, Jacobi for what it hands back
            j.tw = r.tw;
            tri.push_back(j);
            maxT = std::max(maxT, r.n);
        } else if (r.n <= kJacobiMaxN) {
            jb.it[jb.n++] = j;
            maxN = std::max(maxN, r.n);
            if (jb.n == kSolverBatch) {
                HIPCHK(launch_jacobi_lds(jb, maxN, max_sweeps, c.st), "eig");
                jb.n = 0;
                maxN = 0;
            }
        } else {
            const int N = round_up(r.n, 128);
            size_t g = 0;
            while (g < largeN.size() && largeN[g] != N) ++g;
            if (g == largeN.size()) { largeN.push_back(N); large.emplace_back(); }
            large[g].push_back(r);
        }
    }
    HIPCHK(launch_jacobi_lds(jb, maxN, max_sweeps, c.st), "eig");
    auto solve = [&](const std::vector<JacItem> &v, JacItem *dev, int maxn, bool retry) -> jolt_status {
        if (v.empty()) return JOLT_OK;
        if (table && dev + v.size() <= table + kTableItems) {
            HIPCHK(launch_put_table(v.data(), v.size() * sizeof(JacItem), dev, c.st), "eig table");
            const JacTable t{dev, (int)v.size()};
            HIPCHK(launch_eig_tridiag(v.data(), t, maxn, c.st), "eig (tridiagonal)");
            if (retry) HIPCHK(launch_jacobi_lds(v.data(), t, maxn, max_sweeps, c.st, 1), "eig (Jacobi retry)");
            return JOLT_OK;
        }
        for (size_t s0 = 0; s0 < v.size(); s0 += kSolverBatch) {
            JacBatch b{};
            for (size_t i = s0; i < std::min(v.size(), s0 + kSolverBatch); ++i) b.it[b.n++] = v[i];
            HIPCHK(launch_eig_tridiag(b, maxn, c.st), "eig (tridiagonal)");
            if (retry) HIPCHK(launch_jacobi_lds(b, maxn, max_sweeps, c.st, 1), "eig (Jacobi retry)");
        }
        return JOLT_OK;
    };
    if (jolt_status s = solve(tri, table, maxT, true)) return s;
    if (jolt_status s = solve(wide, table ? table + tri.size() : nullptr, maxW, false)) return s;
    for (size_t g = 0; g < large.size(); ++g)
        for (size_t s0 = 0; s0 < large[g].size(); s0 += kMaxBatch) {
            const std::vector<EigReq> part(large[g].begin() + s0,
                                           large[g].begin() + std::min(large[g].size(), s0 + kMaxBatch));
            jolt_status s = eig_block(c, part, largeN[g], scr, max_sweeps, noconv);
            if (s) return s;
        }
    return JOLT_OK;
}

// Grams of k-row panels (part[s] = partial sums of split s): the symmetric
// kernel up to kSymGramMaxK rows, the generic GEMM beyond
hipError_t panel_grams(const SymGramBatch &gb, int maxK, int maxS, hipStream_t st) {
    if (maxK <= kSymGramWideK) return launch_sym_gram(gb, maxK, maxS, st);
    GemmBatch g{};
    for (int i = 0; i < gb.n; ++i) {
        const SymGramItem &s = gb.it[i];
        GemmItem &m = g.it[g.n++];
        m.a = s.y; m.b = s.y; m.c = s.part;
        m.a_i = s.ldy; m.a_k = 1; m.b_k = 1; m.b_j = s.ldy;
        m.c_i = s.kp; m.c_j = 1; m.c_split = (int64_t)s.kp * s.kp;
        m.a_z = m.b_z = m.c_z = 0;
        m.M = s.k; m.N = s.k; m.K = s.len; m.kchunk = s.chunk; m.nsplit = s.nsplit; m.nb = 1;
    }
    return launch_gemm(g, maxK, maxK, maxS, 1, st);
}

// Launches in slices of at most CAP items: fill(batch, i) appends item i (or
// nothing), go(batch) launches a non-empty batch.
template <class Batch, int CAP, class Fill, class Go>
hipError_t sliced(int n, Fill &&fill, Go &&go) {
    for (int s0 = 0; s0 < n; s0 += CAP) {
        Batch b{};
        b.n = 0;
        for (int i = s0; i < std::min(n, s0 + CAP); ++i) fill(b, i);
        if (b.n == 0) continue;
        if (hipError_t e = go(b); e != hipSuccess) return e;
    }
    return hipSuccess;
}

// Orthonormalizes the rows of each y in place (passes of shifted CholeskyQR).
// With hi (and lo) given, the last pass also writes bf16 copies of the result
// when the L^-1 apply runs (k <= kCholWideMaxK); *bf reports whether it did.
// table: device memory for the Cholesky item table (kTableItems items).
// Symmetric Grams of the k-row panels g[i].y: by-value launches of kMaxBatch
// items, or, given a device table (groups of more items), one launch for all
// of them (the table written first when put).
hipError_t sym_grams(const Ctx &c, const std::vector<SymGramItem> &g, SymGramItem *tab, bool put) {
    int maxK = 0, maxS = 0;
    for (const SymGramItem &i : g) {
        maxK = std::max(maxK, i.k);
        maxS = std::max(maxS, i.nsplit);
    }
    const int nb = (int)g.size();
    if (tab && maxK <= kSymGramWideK) {
        if (put)
            if (hipError_t e = launch_put_table(g.data(), g.size() * sizeof(SymGramItem), tab, c.st); e != hipSuccess)
                return e;
        return launch_sym_gram(g.data(), SymGramTable{tab, nb}, maxK, maxS, c.st);
    }
    return sliced<SymGramBatch, kMaxBatch>(
        nb, [&](SymGramBatch &b, int i) { b.it[b.n++] = g[i]; },
        [&](const SymGramBatch &b) { return panel_grams(b, maxK, maxS, c.st); });
}

// direct: an item whose Gram is a single launch-table split goes straight to
// gram (no partials, no reduction)
jolt_status orth_rows(const Ctx &c, int nb, float **y, float **gram, float **gpart, float **lmat, float **csq,
                      const int *k, const int *kp, const int *len, const int *split, const int *chunk, int passes,
                      CholItem *table, uint16_t *const *hi = nullptr, uint16_t *const *lo = nullptr,
                      bool *bf = nullptr, SymGramItem *sg_tab = nullptr) {
    if (bf) *bf = false;
    std::vector<CholItem> chol;
    int maxK = 0, maxLen = 0, maxS = 0;
    int64_t maxCount = 0;
    for (int i = 0; i < nb; ++i) {
        maxK = std::max(maxK, k[i]);
        maxLen = std::max(maxLen, len[i]);
        maxS = std::max(maxS, split[i]);
        maxCount = std::max<int64_t>(maxCount, (int64_t)kp[i] * kp[i]);
    }
    std::vector<SymGramItem> gi(nb);
    std::vector<char> direct(nb);
    for (int i = 0; i < nb; ++i) {
        direct[i] = sg_tab && split[i] == 1 && maxK <= kSymGramWideK;
        SymGramItem &g = gi[i];
        g.y = y[i]; g.part = direct[i] ? gram[i] : gpart[i]; g.k = k[i]; g.kp = kp[i]; g.len = len[i];
        g.ldy = len[i]; g.chunk = chunk[i]; g.nsplit = split[i];
    }
    for (int pass = 0; pass < passes; ++pass) {
        const bool last = pass + 1 == passes;
        HIPCHK(sym_grams(c, gi, sg_tab, pass == 0), "orth gram");
        HIPCHK((sliced<ReduceBatch, kMaxBatch>(
                   nb,
                   [&](ReduceBatch &b, int i) {
                       if (direct[i]) return;
                       ReduceItem &r = b.it[b.n++];
                       r.part = gpart[i]; r.out = gram[i]; r.stride = (int64_t)kp[i] * kp[i];
                       r.count = (int64_t)kp[i] * kp[i]; r.nsplit = split[i];
                   },
                   [&](const ReduceBatch &b) { return launch_reduce(b, maxCount, c.st); })),
               "orth reduce");
        if (maxK <= kCholWideMaxK && table && nb <= kTableItems) {
            // every matrix in one launch, from a device table written once per call
            if (pass == 0) {
                chol.resize(nb);
                for (int i = 0; i < nb; ++i) {
                    CholItem &ch = chol[i];
                    ch = CholItem{};
                    ch.g = gram[i]; ch.l = lmat[i]; ch.k = k[i]; ch.ld = kp[i]; ch.rel_shift = 1.0f / 1048576.0f;
                    ch.inverse = 1;
                    ch.work = csq[i];
                }
                HIPCHK(launch_put_table(chol.data(), nb * sizeof(CholItem), table, c.st), "cholesky table");
            }
            HIPCHK(launch_chol_inv(chol.data(), CholTable{table, nb}, maxK, c.st), "orth cholesky");
        } else {
            HIPCHK((sliced<CholBatch, kSolverBatch>(
                       nb,
                       [&](CholBatch &b, int i) {
                           CholItem &ch = b.it[b.n++];
                           ch.g = gram[i]; ch.l = lmat[i]; ch.k = k[i]; ch.ld = kp[i];
                           ch.rel_shift = 1.0f / 1048576.0f;
                           ch.inverse = k[i] <= kCholWideMaxK;
                           ch.work = csq[i];
                       },
                       [&](const CholBatch &b) { return launch_cholesky(b, maxK, c.st); })),
                   "orth cholesky");
        }
        HIPCHK((sliced<TrsmBatch, kMaxBatch>(
                   nb,
                   [&](TrsmBatch &b, int i) {
                       TrsmItem &t = b.it[b.n++];
                       t.l = lmat[i]; t.y = y[i]; t.q = y[i]; t.k = k[i]; t.ld = kp[i]; t.len = len[i];
                       t.ldy = len[i];
                       if (hi && last) {
                           t.qh = hi[i];
                           t.ql = lo ? lo[i] : nullptr;
                       }
                   },
                   [&](const TrsmBatch &b) {
                       return maxK <= kCholWideMaxK ? launch_apply_linv(b, maxK, maxLen, c.st)
                                                    : launch_trsm(b, maxK, maxLen, c.st);
                   })),
               "orth L^-1 Y");
        if (bf && hi && last && maxK <= kCholWideMaxK) *bf = true;
    }
    return JOLT_OK;
}

// One group of up to kPlanGroup items: every stage runs for all of them
// before the next, with launches of kMaxBatch items for the streaming kernels
// (item tables as kernel arguments) and one launch for all the group's
// matrices of each one-workgroup-per-matrix solver (item tables in device
// memory), whose launches of a few matrices would leave most CUs idle.
jolt_status run_group_body(const Ctx &c, const jolt_config &cfg, const PlanLayout &pl, const jolt_item *items,
                           int i0, int nb, const void *const *x_dev, uint8_t *ws, bool *noconv, bool wide_ok,
                           hipStream_t *forked) {
    const int max_sweeps = cfg.max_sweeps > 0 ? cfg.max_sweeps : 30;
    const int d = c.d, dt = c.dtype;
    const bool bf = dt == JOLT_BF16;
    std::vector<Dims> D(nb);
    std::vector<Scratch> S(nb);
    Bump sb;
    // symmetric Grams: a group of more items than one by-value launch holds
    // launches all of them at once from a device table, split over columns only
    // as far as needed to fill the CUs (not at all from 256 items on: no
    // partial Grams and no reduction pass)
    const bool sg_tab = nb > kMaxBatch;
    for (int i = 0; i < nb; ++i) {
        D[i] = dims_for(cfg, items[i0 + i], pl.rt_max, pl.rf_max);
        if (sg_tab) set_gram_splits(D[i], clampi((256 + nb - 1) / nb, 1, 16));
        reserve_scratch(cfg, D[i], sb, S[i]);
    }
    const Tables tabs = reserve_tables(sb);
    uint8_t *scr = ws + pl.scratch;
    JacItem *tab_feat = reinterpret_cast<JacItem *>(scr + tabs.feat);
    JacItem *tab_tok = reinterpret_cast<JacItem *>(scr + tabs.tok);
    CholItem *tab_chol = reinterpret_cast<CholItem *>(scr + tabs.chol);
    SymGramItem *tab_sg = sg_tab ? reinterpret_cast<SymGramItem *>(scr + tabs.sg) : nullptr;
    HIPCHK(launch_zero(ws + pl.item[i0].grid, pl.readback_stride * nb, c.st), "zero readback");
    auto P = [&](size_t off) { return scr + off; };
    auto F = [&](size_t off) { return reinterpret_cast<float *>(scr + off); };
    auto W = [&](size_t off) { return ws + off; };
    const FactorOffsets *fo = pl.item.data() + i0;
    int maxT = 0, maxLH = 0;
    for (int i = 0; i < nb; ++i) {
        maxT = std::max(maxT, D[i].T);
        maxLH = std::max(maxLH, D[i].LH);
    }

    // the feature eigenproblems run on the side stream too, next to the token ones
    std::vector<EigReq> feigs, eigs;
    for (int i = 0; i < nb; ++i)
        feigs.push_back(EigReq{F(S[i].gf), d, d, reinterpret_cast<float *>(W(fo[i].uf)), d,
                               reinterpret_cast<float *>(W(fo[i].lam_f)), reinterpret_cast<int *>(W(fo[i].sweeps)),
                               &S[i], S[i].ftri != SIZE_MAX ? F(S[i].ftri) : nullptr});
    // ---- feature Gram, ||X||^2 and the feature eigenproblems, on the side
    // stream: forked when the token eigenproblems start (one workgroup per
    // matrix leaves most CUs and HBM idle for this), joined before the core,
    // their first consumer.  (Forked at the start instead, the Gram pass and
    // the first sketch pass took turns on HBM and the CUs: no faster.)
    hipStream_t side;
    hipEvent_t fork, join;
    HIPCHK(side_stream(c.h, &side, &fork, &join), "side stream");
    auto feature_gram = [&]() -> jolt_status {
        HIPCHK(hipEventRecord(fork, c.st), "fork");
        HIPCHK(hipStreamWaitEvent(side, fork, 0), "fork");
        *forked = side;
        int maxP = 0;
        for (int i = 0; i < nb; ++i) maxP = std::max(maxP, D[i].gf_P);
        HIPCHK((sliced<GramBatch, kMaxBatch>(
                   nb,
                   [&](GramBatch &b, int i) {
                       GramItem &g = b.it[b.n++];
                       g.x = x_dev[i0 + i]; g.out = F(S[i].gfpart);
                       g.rows = (int64_t)D[i].LH * D[i].T; g.chunk = D[i].gf_chunk; g.P = D[i].gf_P;
                   },
                   [&](const GramBatch &b) { return launch_gram_rows(b, dt, d, maxP, side); })),
               "feature gram");
        HIPCHK((sliced<ReduceBatch, kMaxBatch>(
                   nb,
                   [&](ReduceBatch &b, int i) {
                       ReduceItem &r = b.it[b.n++];
                       r.part = F(S[i].gfpart); r.out = F(S[i].gf); r.stride = (int64_t)d * d;
                       r.count = (int64_t)d * d; r.nsplit = D[i].gf_P;
                   },
                   [&](const ReduceBatch &b) { return launch_reduce(b, (int64_t)d * d, side); })),
               "feature gram reduce");
        HIPCHK((sliced<SmallBatch, kMaxBatch>(
                   nb,
                   [&](SmallBatch &b, int i) {
                       SmallItem &t = b.it[b.n++];
                       t.in = F(S[i].gf); t.out64 = reinterpret_cast<double *>(W(fo[i].normx2)); t.a = d;
                   },
                   [&](const SmallBatch &b) { return launch_trace_batch(b, side); })),
               "trace");
        const Ctx cs{c.h, side, c.dtype, c.d};
        // kept on the side stream: the solver streams are the token eigenproblems'
        if (jolt_status es = eig_all(cs, feigs, scr, max_sweeps, noconv, wide_ok, tab_feat)) return es;
        HIPCHK(hipEventRecord(join, side), "join");
        return JOLT_OK;
    };

    if (cfg.mode == JOLT_TOKEN_RANDOMIZED) {
        std::vector<float *> yv(nb), zv(nb), gram(nb), gpart(nb), lmat(nb), csq(nb);
        std::vector<int> kk(nb), kpp(nb), lenT(nb), lenN(nb), sT(nb), cT(nb), sN(nb), cN(nb);
        int64_t maxOm = 0;
        for (int i = 0; i < nb; ++i) maxOm = std::max<int64_t>(maxOm, (int64_t)D[i].kp * D[i].n);
        HIPCHK((sliced<SmallBatch, kMaxBatch>(
                   nb,
                   [&](SmallBatch &b, int i) {
                       const jolt_item &it = items[i0 + i];
                       SmallItem &o = b.it[b.n++];
                       o.hi = bf ? reinterpret_cast<uint16_t *>(P(S[i].omt)) : nullptr;
                       o.out32 = bf ? nullptr : F(S[i].omt);
                       o.key = item_key(it.seed, it.item_id); o.a = D[i].k; o.b = D[i].kp;
                       o.count = (int64_t)D[i].kp * D[i].n;
                   },
                   [&](const SmallBatch &b) { return launch_gen_omega_batch(b, maxOm, c.st); })),
               "omega");
        for (int i = 0; i < nb; ++i) {
            yv[i] = F(S[i].yt); zv[i] = F(S[i].zt); gram[i] = F(S[i].gram); gpart[i] = F(S[i].gpart);
            lmat[i] = F(S[i].lmat);
            csq[i] = S[i].csq ? F(S[i].csq) : nullptr;
            kk[i] = D[i].k; kpp[i] = D[i].kp; lenT[i] = D[i].T; lenN[i] = D[i].n;
            sT[i] = D[i].gT_split; cT[i] = D[i].gT_chunk; sN[i] = D[i].gN_split; cN[i] = D[i].gN_chunk;
        }
        auto xm = [&](bool first) -> jolt_status {
            int maxC = 0, maxS = 0;
            int64_t maxCount = 0;
            for (int i = 0; i < nb; ++i) {
                maxC = std::max(maxC, D[i].kp);
                maxS = std::max(maxS, D[i].xm_split);
                maxCount = std::max<int64_t>(maxCount, (int64_t)D[i].kp * D[i].T);
            }
            HIPCHK((sliced<XmBatch, kMaxBatch>(
                       nb,
                       [&](XmBatch &b, int i) {
                           XmItem &x = b.it[b.n++];
                           x.x = x_dev[i0 + i];
                           x.m = first ? (const void *)P(S[i].omt)
                                       : (bf ? (const void *)P(S[i].zb) : (const void *)P(S[i].zt));
                           x.m_c = D[i].n; x.m_blk = d;
                           x.T = D[i].T; x.LH = D[i].LH; x.ncols = D[i].kp; x.ldo = D[i].T;
                           x.lh_split = D[i].xm_lh; x.nsplit = D[i].xm_split;
                           x.out = x.nsplit > 1 ? F(S[i].ypart) : F(S[i].yt);
                       },
                       [&](const XmBatch &b) { return launch_xm(b, dt, d, maxT, maxC, maxS, c.st); })),
                   "sketch A M");
            HIPCHK((sliced<ReduceBatch, kMaxBatch>(
                       nb,
                       [&](ReduceBatch &b, int i) {
                           if (D[i].xm_split <= 1) return;
                           ReduceItem &r = b.it[b.n++];
                           r.part = F(S[i].ypart); r.out = F(S[i].yt);
                           r.stride = (int64_t)D[i].kp * D[i].T; r.count = r.stride; r.nsplit = D[i].xm_split;
                       },
                       [&](const ReduceBatch &b) { return launch_reduce(b, maxCount, c.st); })),
                   "sketch reduce");
            return JOLT_OK;
        };
        auto xtq = [&](bool hilo) -> jolt_status {
            int maxS = 0, maxC = 0;
            int64_t maxCount = 0;
            for (int i = 0; i < nb; ++i) {
                maxS = std::max(maxS, D[i].xs_split);
                maxC = std::max(maxC, D[i].kp);
                maxCount = std::max<int64_t>(maxCount, (int64_t)D[i].kp * D[i].n);
            }
            HIPCHK((sliced<XtqBatch, kMaxBatch>(
                       nb,
                       [&](XtqBatch &b, int i) {
                           XtqItem &x = b.it[b.n++];
                           x.x = x_dev[i0 + i];
                           x.qh = bf ? (const void *)P(S[i].qh) : (const void *)P(S[i].yt);
                           x.ql = (bf && hilo) ? (const void *)P(S[i].ql) : nullptr;
                           x.T = D[i].T; x.LH = D[i].LH; x.ncols = D[i].kp; x.ldq = D[i].T;
                           x.tsplit = D[i].xs_tsplit; x.nsplit = D[i].xs_split;
                           x.out = x.nsplit == 1 ? F(S[i].zt) : F(S[i].xpart);
                       },
                       [&](const XtqBatch &b) { return launch_xtq(b, dt, d, maxLH, maxS, maxC, c.st); })),
                   "sketch Q^T A");
            HIPCHK((sliced<ReduceBatch, kMaxBatch>(
                       nb,
                       [&](ReduceBatch &b, int i) {
                           if (D[i].xs_split <= 1) return;
                           ReduceItem &r = b.it[b.n++];
                           r.part = F(S[i].xpart); r.out = F(S[i].zt);
                           r.stride = (int64_t)D[i].kp * D[i].n; r.count = r.stride; r.nsplit = D[i].xs_split;
                       },
                       [&](const ReduceBatch &b) { return launch_reduce(b, maxCount, c.st); })),
                   "sketch reduce");
            return JOLT_OK;
        };
        auto to_bf = [&](bool from_y, bool lo) -> jolt_status {
            if (!bf) return JOLT_OK;
            int64_t maxC = 0;
            for (int i = 0; i < nb; ++i)
                maxC = std::max<int64_t>(maxC, (int64_t)D[i].kp * (from_y ? D[i].T : D[i].n));
            HIPCHK((sliced<SmallBatch, kMaxBatch>(
                       nb,
                       [&](SmallBatch &b, int i) {
                           SmallItem &t = b.it[b.n++];
                           t.in = from_y ? F(S[i].yt) : F(S[i].zt);
                           t.hi = reinterpret_cast<uint16_t *>(from_y ? P(S[i].qh) : P(S[i].zb));
                           t.lo = (from_y && lo) ? reinterpret_cast<uint16_t *>(P(S[i].ql)) : nullptr;
                           t.count = (int64_t)D[i].kp * (from_y ? D[i].T : D[i].n);
                       },
                       [&](const SmallBatch &b) { return launch_to_bf16_batch(b, maxC, c.st); })),
                   "to bf16");
            return JOLT_OK;
        };
        jolt_status s;
        // bf16 copies for the sketch passes come from the last L^-1 apply of each
        // orthonormalization when it can write them (conv), else from to_bf
        std::vector<uint16_t *> qhv(nb), qlv(nb), zbv(nb);
        for (int i = 0; i < nb; ++i) {
            qhv[i] = bf ? reinterpret_cast<uint16_t *>(P(S[i].qh)) : nullptr;
            qlv[i] = bf ? reinterpret_cast<uint16_t *>(P(S[i].ql)) : nullptr;
            zbv[i] = bf ? reinterpret_cast<uint16_t *>(P(S[i].zb)) : nullptr;
        }
        uint16_t *const *qh_out = bf ? qhv.data() : nullptr;
        bool conv = false;
        if ((s = xm(true))) return s;                                                        // Y = A Omega
        if ((s = orth_rows(c, nb, yv.data(), gram.data(), gpart.data(), lmat.data(), csq.data(), kk.data(),
                           kpp.data(), lenT.data(), sT.data(), cT.data(), cfg.power_iters > 0 ? 1 : 2, tab_chol, qh_out,
                           (bf && cfg.power_iters == 0) ? qlv.data() : nullptr, &conv, tab_sg)))
            return s;
        for (int q = 0; q < cfg.power_iters; ++q) {
            if (!conv && (s = to_bf(true, false))) return s;
            if ((s = xtq(false))) return s;                                                 // Z = A^T Q
            if ((s = orth_rows(c, nb, zv.data(), gram.data(), gpart.data(), lmat.data(), csq.data(), kk.data(),
                               kpp.data(), lenN.data(), sN.data(), cN.data(), 1, tab_chol, bf ? zbv.data() : nullptr, nullptr,
                               &conv, tab_sg)))
                return s;
            if (!conv && (s = to_bf(false, false))) return s;
            if ((s = xm(false))) return s;                                                  // Y = A Z
            const bool last = q + 1 == cfg.power_iters;
            if ((s = orth_rows(c, nb, yv.data(), gram.data(), gpart.data(), lmat.data(), csq.data(), kk.data(),
                               kpp.data(), lenT.data(), sT.data(), cT.data(), last ? 2 : 1, tab_chol, qh_out,
                               (bf && last) ? qlv.data() : nullptr, &conv, tab_sg)))
                return s;
        }
        if (!conv && (s = to_bf(true, true))) return s;
        if ((s = xtq(true))) return s;                                                      // B = Q^T A (hi + lo)
        // W = B B^T, eig
        {
            int maxK = 0, maxS = 0;
            int64_t maxCount = 0;
            for (int i = 0; i < nb; ++i) {
                maxK = std::max(maxK, D[i].k);
                maxS = std::max(maxS, D[i].gN_split);
                maxCount = std::max<int64_t>(maxCount, (int64_t)D[i].kp * D[i].kp);
            }
            std::vector<SymGramItem> gw(nb);
            std::vector<char> direct(nb);
            for (int i = 0; i < nb; ++i) {
                direct[i] = tab_sg && D[i].gN_split == 1 && maxK <= kSymGramWideK;
                SymGramItem &g = gw[i];
                g.y = zv[i]; g.part = direct[i] ? F(S[i].wmat) : gpart[i]; g.k = D[i].k; g.kp = D[i].kp;
                g.len = D[i].n; g.ldy = D[i].n; g.chunk = D[i].gN_chunk; g.nsplit = D[i].gN_split;
            }
            HIPCHK(sym_grams(c, gw, tab_sg, true), "B B^T");
            HIPCHK((sliced<ReduceBatch, kMaxBatch>(
                       nb,
                       [&](ReduceBatch &b, int i) {
                           if (direct[i]) return;
                           ReduceItem &r = b.it[b.n++];
                           r.part = gpart[i]; r.out = F(S[i].wmat); r.stride = (int64_t)D[i].kp * D[i].kp;
                           r.count = r.stride; r.nsplit = D[i].gN_split;
                       },
                       [&](const ReduceBatch &b) { return launch_reduce(b, maxCount, c.st); })),
                   "B B^T reduce");
            for (int i = 0; i < nb; ++i)
                eigs.push_back(EigReq{F(S[i].wmat), D[i].kp, D[i].k, F(S[i].vmat), D[i].kp,
                                      reinterpret_cast<float *>(W(fo[i].lam_t)),
                                      reinterpret_cast<int *>(W(fo[i].sweeps)) + 1, &S[i],
                                      S[i].etri != SIZE_MAX ? F(S[i].etri) : nullptr});
            if ((s = feature_gram())) return s;
            jolt_status es = eig_all(c, eigs, scr, max_sweeps, noconv, wide_ok, tab_tok);
            if (es) return es;
        }
        // U_t^T = U~^T Q, P = U~^T B, lambda_t
        if (pl.rt_max > 0) {
            int maxN = 0, maxNn = 0;
            for (int i = 0; i < nb; ++i) {
                maxN = std::max(maxN, D[i].T);
                maxNn = std::max(maxNn, D[i].n);
            }
            HIPCHK((sliced<GemmBatch, kMaxBatch>(
                       nb,
                       [&](GemmBatch &b, int i) {
                           GemmItem &g = b.it[b.n++];
                           g.a = F(S[i].vmat); g.b = yv[i]; g.c = reinterpret_cast<float *>(W(fo[i].ut));
                           g.a_i = 1; g.a_k = D[i].kp; g.b_k = D[i].T; g.b_j = 1; g.c_i = D[i].T; g.c_j = 1;
                           g.c_split = 0; g.a_z = g.b_z = g.c_z = 0;
                           g.M = pl.rt_max; g.N = D[i].T; g.K = D[i].k; g.kchunk = D[i].k; g.nsplit = 1; g.nb = 1;
                       },
                       [&](const GemmBatch &b) { return launch_gemm_split(b, pl.rt_max, maxN, 1, 1, c.st); })),
                   "U_t");
            HIPCHK((sliced<GemmBatch, kMaxBatch>(
                       nb,
                       [&](GemmBatch &b, int i) {
                           GemmItem &q = b.it[b.n++];
                           q.a = F(S[i].vmat); q.b = zv[i]; q.c = F(S[i].pmat);
                           q.a_i = 1; q.a_k = D[i].kp; q.b_k = D[i].n; q.b_j = 1; q.c_i = D[i].n; q.c_j = 1;
                           q.c_split = 0; q.a_z = q.b_z = q.c_z = 0;
                           q.M = pl.rt_max; q.N = D[i].n; q.K = D[i].k; q.kchunk = D[i].k; q.nsplit = 1; q.nb = 1;
                       },
                       [&](const GemmBatch &b) { return launch_gemm_split(b, pl.rt_max, maxNn, 1, 1, c.st); })),
                   "P");
        }
    } else {
        // exact token factor: eigenvectors of G_t = A A^T (T x T)
        int maxC = 0;
        for (int i = 0; i < nb; ++i) maxC = std::max(maxC, D[i].T);
        HIPCHK((sliced<XmBatch, kMaxBatch>(
                   nb,
                   [&](XmBatch &b, int i) {
                       XmItem &x = b.it[b.n++];
                       x.x = x_dev[i0 + i]; x.m = x_dev[i0 + i]; x.out = F(S[i].gt);
                       x.m_c = d; x.m_blk = (int64_t)D[i].T * d;
                       x.T = D[i].T; x.LH = D[i].LH; x.ncols = D[i].T; x.ldo = D[i].T;
                       x.lh_split = D[i].LH; x.nsplit = 1;
                   },
                   [&](const XmBatch &b) { return launch_xm(b, dt, d, maxT, maxC, 1, c.st); })),
               "token Gram");
        for (int i = 0; i < nb; ++i)
            eigs.push_back(EigReq{F(S[i].gt), D[i].T, D[i].T, F(S[i].vt), D[i].T,
                                  reinterpret_cast<float *>(W(fo[i].lam_t)),
                                  reinterpret_cast<int *>(W(fo[i].sweeps)) + 1, &S[i],
                                  S[i].etri != SIZE_MAX ? F(S[i].etri) : nullptr});
        if (jolt_status fs = feature_gram()) return fs;
        jolt_status es = eig_all(c, eigs, scr, max_sweeps, noconv, wide_ok, tab_tok);
        if (es) return es;
        // U_t^T rows = leading eigenvectors; P = U_t^T A (hi + lo split for bf16 caches)
        int maxS = 0, maxCols = 0;
        int64_t maxCount = 0;
        for (int i = 0; i < nb; ++i) {
            float *ut = reinterpret_cast<float *>(W(fo[i].ut));
            HIPCHK(launch_transpose(F(S[i].vt), ut, D[i].T, pl.rt_max, D[i].T, D[i].T, c.st), "U_t");
            const int64_t rows_pad = (int64_t)D[i].rtp32 * D[i].T;
            if (bf) {
                HIPCHK(launch_zero(P(S[i].uh), rows_pad * 2, c.st), "zero");
                HIPCHK(launch_zero(P(S[i].ul), rows_pad * 2, c.st), "zero");
                HIPCHK(launch_to_bf16(ut, reinterpret_cast<uint16_t *>(P(S[i].uh)),
                                      reinterpret_cast<uint16_t *>(P(S[i].ul)), (int64_t)pl.rt_max * D[i].T, c.st),
                       "U_t split");
            } else {
                HIPCHK(launch_zero(P(S[i].uh), rows_pad * 4, c.st), "zero");
                HIPCHK(hipMemcpyAsync(P(S[i].uh), ut, (size_t)pl.rt_max * D[i].T * 4, hipMemcpyDeviceToDevice, c.st),
                       "U_t copy");
            }
            maxS = std::max(maxS, D[i].xs_split);
            maxCols = std::max(maxCols, D[i].rtp32);
            maxCount = std::max<int64_t>(maxCount, (int64_t)D[i].rtp32 * D[i].n);
        }
        if (pl.rt_max > 0) {
            HIPCHK((sliced<XtqBatch, kMaxBatch>(
                       nb,
                       [&](XtqBatch &b, int i) {
                           XtqItem &x = b.it[b.n++];
                           x.x = x_dev[i0 + i]; x.qh = P(S[i].uh); x.ql = bf ? (const void *)P(S[i].ul) : nullptr;
                           x.T = D[i].T; x.LH = D[i].LH; x.ncols = D[i].rtp32; x.ldq = D[i].T;
                           x.tsplit = D[i].xs_tsplit; x.nsplit = D[i].xs_split;
                           x.out = x.nsplit == 1 ? F(S[i].pmat) : F(S[i].xpart);
                       },
                       [&](const XtqBatch &b) { return launch_xtq(b, dt, d, maxLH, maxS, maxCols, c.st); })),
                   "U_t^T A");
            HIPCHK((sliced<ReduceBatch, kMaxBatch>(
                       nb,
                       [&](ReduceBatch &b, int i) {
                           if (D[i].xs_split <= 1) return;
                           ReduceItem &r = b.it[b.n++];
                           r.part = F(S[i].xpart); r.out = F(S[i].pmat);
                           r.stride = (int64_t)D[i].rtp32 * D[i].n; r.count = r.stride; r.nsplit = D[i].xs_split;
                       },
                       [&](const ReduceBatch &b) { return launch_reduce(b, maxCount, c.st); })),
                   "U_t^T A reduce");
        }
    }

    // core[lh] = P[:, lh d : lh d + d] U_f, energy
    HIPCHK(hipStreamWaitEvent(c.st, join, 0), "join");
    if (pl.rt_max > 0) {
        int maxNb = 0;
        for (int i = 0; i < nb; ++i) maxNb = std::max(maxNb, D[i].LH);
        HIPCHK((sliced<GemmBatch, kMaxBatch>(
                   nb,
                   [&](GemmBatch &b, int i) {
                       GemmItem &g = b.it[b.n++];
                       g.a = F(S[i].pmat); g.b = reinterpret_cast<const float *>(W(fo[i].uf));
                       g.c = reinterpret_cast<float *>(W(fo[i].core));
                       g.a_i = D[i].n; g.a_k = 1; g.b_k = d; g.b_j = 1; g.c_i = d; g.c_j = 1; g.c_split = 0;
                       g.a_z = d; g.b_z = 0; g.c_z = (int64_t)pl.rt_max * d;
                       g.M = pl.rt_max; g.N = d; g.K = d; g.kchunk = d; g.nsplit = 1; g.nb = D[i].LH;
                   },
                   [&](const GemmBatch &b) { return launch_gemm_split(b, pl.rt_max, d, 1, maxNb, c.st); })),
               "core");
        HIPCHK((sliced<SmallBatch, kMaxBatch>(
                   nb,
                   [&](SmallBatch &b, int i) {
                       SmallItem &t = b.it[b.n++];
                       t.in = reinterpret_cast<const float *>(W(fo[i].core));
                       t.out32 = reinterpret_cast<float *>(W(fo[i].energy));
                       t.a = D[i].LH; t.b = pl.rt_max; t.c = d;
                   },
                   [&](const SmallBatch &b) { return launch_energy_batch(b, (int64_t)pl.rt_max * d, c.st); })),
               "energy");
        HIPCHK((sliced<GridBatch, kMaxBatch>(
                   nb,
                   [&](GridBatch &b, int i) {
                       GridItem &g = b.it[b.n++];
                       g.E = reinterpret_cast<const float *>(W(fo[i].energy));
                       g.S = reinterpret_cast<double *>(W(fo[i].grid));
                       g.s_fixed = reinterpret_cast<double *>(W(fo[i].sfixed));
                       g.d = d; g.step = pl.step; g.nr = pl.grid_nr; g.nf = pl.grid_nf;
                       g.frt = cfg.budget_bytes < 0 ? std::min(cfg.fixed_rt, pl.rt_max) : 0;
                       g.frf = cfg.budget_bytes < 0 ? std::min(cfg.fixed_rf, d) : 0;
                   },
                   [&](const GridBatch &b) { return launch_energy_grid(b, c.st); })),
               "energy grid");
    }
    return JOLT_OK;
}

// One group of the plan.  Work forked onto the side stream reads the inputs
// and writes the workspace, so an error waits for that stream before
// returning: everything launched has finished when jolt_plan returns.
jolt_status run_group(const Ctx &c, const jolt_config &cfg, const PlanLayout &pl, const jolt_item *items, int i0,
                      int nb, const void *const *x_dev, uint8_t *ws, bool *noconv, bool wide_ok) {
    hipStream_t forked = nullptr;
    jolt_status s = run_group_body(c, cfg, pl, items, i0, nb, x_dev, ws, noconv, wide_ok, &forked);
    if (s != JOLT_OK) drain_streams(c.h);
    return s;
}

}  // namespace

// ------------------------------------------------------------------ parameter store (jolt_compress)
jolt_status store_params(jolt_handle h, const PlanLayout &pl, const jolt_item *items, int n, const jolt_alloc *alloc,
                         const void *plan_ws, void *const *payload_dev, hipStream_t st) {
    const uint8_t *ws = static_cast<const uint8_t *>(plan_ws);
    StoreBatch b{};
    b.n = 0;
    const int dt = items[0].dtype;
    for (int i = 0; i < n; ++i) {
        const jolt_item &it = items[i];
        PayloadLayout p = payload_layout(it, alloc[i].rt, alloc[i].rf, alloc[i].bits);
        StoreItem &s = b.it[b.n++];
        s.ut = reinterpret_cast<const float *>(ws + pl.item[i].ut);
        s.uf = reinterpret_cast<const float *>(ws + pl.item[i].uf);
        s.core = reinterpret_cast<const float *>(ws + pl.item[i].core);
        s.pay = static_cast<uint8_t *>(payload_dev[i]);
        s.off_ut = p.ut; s.off_uf = p.uf; s.off_core = p.core;
        s.T = it.T; s.d = it.d; s.LH = it.L * it.H; s.rt_max = pl.rt_max; s.rt = p.rt; s.rf = p.rf;
        jolt_alloc a = alloc[i];
        uint8_t hdr[64];
        make_header(it, a, hdr);
        std::memcpy(s.header, hdr, 64);
        if (b.n == kMaxBatch || i == n - 1) {
            hipError_t e = launch_store(b, dt, st);
            if (e != hipSuccess) return hip_fail(h, e, "store params");
            b.n = 0;
        }
    }
    return JOLT_OK;
}

}  // namespace jolt

using namespace jolt;

// The allocation from a plan's host copy of its readback block (energy grids,
// ||X||^2, eigensolver status): fixed ranks, or the single dual under
// cfg.budget_bytes.  Shared by jolt_plan and jolt_replan.
static jolt_status allocate_from_readback(jolt_handle h, const jolt_config &cfg, const jolt_item *items, int n,
                                          const PlanLayout &pl, const uint8_t *rb, jolt_alloc *alloc_host,
                                          double *lambda_out, bool *noconv) {
    static const bool debug = getenv("JOLT_DEBUG") != nullptr;
    const int rt_max = pl.rt_max;
    const size_t cells = (size_t)std::max(pl.grid_nr * pl.grid_nf, 1);
    std::vector<const double *> grid(n);
    std::vector<double> nx2(n), sfix(n);
    for (int i = 0; i < n; ++i) {
        grid[i] = reinterpret_cast<const double *>(rb + (pl.item[i].grid - pl.readback));
        (void)cells;
        std::memcpy(&sfix[i], rb + (pl.item[i].sfixed - pl.readback), 8);
        std::memcpy(&nx2[i], rb + (pl.item[i].normx2 - pl.readback), 8);
        int sw[2];
        std::memcpy(sw, rb + (pl.item[i].sweeps - pl.readback), 8);
        if (sw[0] < 0 || sw[1] < 0) *noconv = true;
        if (debug) fprintf(stderr, "libjolt: item %d eig sweeps feature %d token %d\n", i, sw[0], sw[1]);
    }

    const int rf_max = pl.rf_max;
    if (cfg.budget_bytes < 0) {
        for (int i = 0; i < n; ++i) {
            jolt_alloc &a = alloc_host[i];
            a.rt = cfg.fixed_rt; a.rf = cfg.fixed_rf; a.bits = cfg.fixed_bits; a.reserved = 0;
            if (a.rt == 0 || a.rf == 0) a.rt = a.rf = 0;
            a.bytes = jolt_item_bytes(&items[i], a.rt, a.rf, a.bits);
            const double S = (a.rt == 0 || a.rf == 0) ? 0.0 : sfix[i];
            a.distortion = std::max(0.0, nx2[i] - S);
        }
        if (lambda_out) *lambda_out = -1.0;
        return JOLT_OK;
    }
    DualTables &dt = dual_tables(h);
    if (dt.rt_max != rt_max || dt.rf_max != rf_max || dt.step != pl.step || dt.grid_nf != pl.grid_nf ||
        dt.bits_mask != cfg.bits_mask || dt.dtype != items[0].dtype || dt.d != items[0].d ||
        pl.step != cfg.rank_step) {
        dt = DualTables{};
        dt.rt_max = rt_max; dt.rf_max = rf_max; dt.step = pl.step; dt.grid_nf = pl.grid_nf;
        dt.bits_mask = cfg.bits_mask; dt.dtype = items[0].dtype; dt.d = items[0].d;
        dt.cand = candidate_grid(rt_max, rf_max, cfg.rank_step, cfg.bits_mask);
        dt.cell.resize(dt.cand.size());
        for (size_t j = 0; j < dt.cand.size(); ++j)
            dt.cell[j] = (dt.cand[j].rt == 0 || dt.cand[j].rf == 0)
                             ? -1 : (dt.cand[j].rt / pl.step - 1) * pl.grid_nf + (dt.cand[j].rf / pl.step - 1);
    }
    const std::vector<Cand> &cand = dt.cand;
    const int nc = (int)cand.size();
    // byte tables and their order, shared by the items of one shape (dtype and d
    // are common to the call; L, H, T may differ).  Kept for at most 64 shapes
    // between calls, so callers whose T changes every call do not grow the cache.
    if (dt.shapes.size() > 64) dt.shapes.clear();
    std::vector<int> shape_of(n);
    for (int i = 0; i < n; ++i) {
        int k = 0;
        while (k < (int)dt.shapes.size() &&
               !(dt.shapes[k].L == items[i].L && dt.shapes[k].H == items[i].H && dt.shapes[k].T == items[i].T))
            ++k;
        if (k == (int)dt.shapes.size()) {
            std::vector<int64_t> B(nc);
            for (int j = 0; j < nc; ++j) B[j] = jolt_item_bytes(&items[i], cand[j].rt, cand[j].rf, cand[j].bits);
            dt.shapes.push_back(DualTables::Shape{items[i].L, items[i].H, items[i].T, sorted_cands(cand, dt.cell.data(), B.data())});
        }
        shape_of[i] = k;
    }
    std::vector<const SortedCands *> scp(n);
    for (int i = 0; i < n; ++i) scp[i] = &dt.shapes[shape_of[i]].sc;
    std::vector<int> choice(n);
    std::vector<double> dist(n);
    double lam = 0.0;
    jolt_status s = allocate_sorted(n, scp.data(), grid.data(), nx2.data(), cfg.delta_b, cfg.budget_bytes, choice.data(),
                        dist.data(), &lam);
    for (int i = 0; i < n; ++i) {
        const Cand &cc = cand[choice[i]];
        alloc_host[i].rt = cc.rt; alloc_host[i].rf = cc.rf; alloc_host[i].bits = cc.bits; alloc_host[i].reserved = 0;
        alloc_host[i].bytes = jolt_item_bytes(&items[i], cc.rt, cc.rf, cc.bits);
        alloc_host[i].distortion = dist[i];
    }
    if (lambda_out) *lambda_out = lam;
    if (s == JOLT_E_INFEASIBLE) return fail(h, s, "budget below the sum of minimum item bytes");
    return JOLT_OK;
}

extern "C" jolt_status jolt_plan(jolt_handle h, const jolt_config *cfg, const jolt_item *items, int32_t n,
                                 const void *const *x_dev, void *plan_ws, size_t plan_ws_bytes, void *stream,
                                 jolt_alloc *alloc_host, double *lambda_out) {
    if (!h || !cfg) return JOLT_E_INVALID;
    clear_err(h);
    jolt_status s = check_items_uniform(h, items, n);
    if (s) return s;
    if (n == 0) return JOLT_OK;
    if (!x_dev || !plan_ws || !alloc_host) return fail(h, JOLT_E_INVALID, "NULL array");
    for (int i = 0; i < n; ++i)
        if (!x_dev[i]) return fail(h, JOLT_E_INVALID, "x_dev[%d] is NULL", i);
    s = check_config(h, *cfg, items, n);
    if (s) return s;
    PlanLayout pl;
    s = plan_layout(*cfg, items, n, &pl);
    if (s) return fail(h, s, "layout");
    if (plan_ws_bytes < pl.total)
        return fail(h, JOLT_E_WORKSPACE, "plan workspace: need %zu bytes, have %zu", pl.total, plan_ws_bytes);
    hipStream_t st = static_cast<hipStream_t>(stream);
    uint8_t *ws = static_cast<uint8_t *>(plan_ws);
    Ctx c{h, st, items[0].dtype, items[0].d};
    bool noconv = false;
    // JOLT_TIMING=1: host-side phase times of this call on stderr
    static const bool timing = getenv("JOLT_TIMING") != nullptr;
    static const bool debug = getenv("JOLT_DEBUG") != nullptr;
    const auto t_start = std::chrono::steady_clock::now();
    for (int c0 = 0; c0 < n; c0 += kPlanGroup) {
        const int nb = std::min(kPlanGroup, n - c0);
        s = run_group(c, *cfg, pl, items, c0, nb, x_dev, ws, &noconv, true);
        if (s) return s;
    }
    // energy tables, ||X||^2 and sweep counters back to the host (the one synchronisation)
    const int rt_max = pl.rt_max;
    const size_t rb_bytes = pl.readback_stride * n;
    uint8_t *rb = nullptr;
    hipError_t e = readback_buffer(h, rb_bytes, &rb);
    if (e == hipSuccess) e = hipMemcpyAsync(rb, ws + pl.readback, rb_bytes, hipMemcpyDeviceToHost, st);
    const auto t_launched = std::chrono::steady_clock::now();
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(h, e, "plan");
    // a chunk whose wide eigensolves did not all finish (numerically repeated
    // eigenvalues) is planned again with block Jacobi for them, then read back
    // again: the only case with more than one synchronisation
    {
        bool again = false;
        for (int c0 = 0; c0 < n; c0 += kPlanGroup) {
            const int nb = std::min(kPlanGroup, n - c0);
            bool redo = false;
            for (int i = c0; i < c0 + nb; ++i) {
                int sw[2];
                std::memcpy(sw, rb + (pl.item[i].sweeps - pl.readback), 8);
                redo |= sw[0] == kEigWideFail || sw[1] == kEigWideFail;
            }
            if (!redo) continue;
            if (debug) fprintf(stderr, "libjolt: items %d..%d planned again with block Jacobi\n", c0, c0 + nb - 1);
            s = run_group(c, *cfg, pl, items, c0, nb, x_dev, ws, &noconv, false);
            if (s) return s;
            again = true;
        }
        if (again) {
            e = hipMemcpyAsync(rb, ws + pl.readback, rb_bytes, hipMemcpyDeviceToHost, st);
            if (e == hipSuccess) e = hipStreamSynchronize(st);
            if (e != hipSuccess) return hip_fail(h, e, "plan (block Jacobi fallback)");
        }
    }
    const auto t_synced = std::chrono::steady_clock::now();
    auto report = [&]() {
        if (!timing) return;
        auto us = [](std::chrono::steady_clock::time_point a, std::chrono::steady_clock::time_point b) {
            return std::chrono::duration<double, std::micro>(b - a).count();
        };
        const auto t_end = std::chrono::steady_clock::now();
        fprintf(stderr, "libjolt plan: launch %.1f us, wait for device %.1f us, tables + dual %.1f us\n",
                us(t_start, t_launched), us(t_launched, t_synced), us(t_synced, t_end));
    };
    jolt_status ds = allocate_from_readback(h, *cfg, items, n, pl, rb, alloc_host, lambda_out, &noconv);
    report();
    if (ds) return ds;
    if (noconv) return fail(h, JOLT_E_NOCONV, "eigensolver hit its sweep cap");
    return JOLT_OK;
}

extern "C" jolt_status jolt_replan(jolt_handle h, const jolt_config *cfg, const jolt_item *items, int32_t n,
                                   const void *plan_ws, size_t plan_ws_bytes, void *stream, jolt_alloc *alloc_host,
                                   double *lambda_out) {
    if (!h || !cfg) return JOLT_E_INVALID;
    clear_err(h);
    jolt_status s = check_items_uniform(h, items, n);
    if (s) return s;
    if (n == 0) return JOLT_OK;
    if (!plan_ws || !alloc_host) return fail(h, JOLT_E_INVALID, "NULL array");
    if (cfg->budget_bytes < 0) return fail(h, JOLT_E_INVALID, "replan: budget_bytes must be >= 0");
    s = check_config(h, *cfg, items, n);
    if (s) return s;
    PlanLayout pl;
    s = plan_layout(*cfg, items, n, &pl);
    if (s) return fail(h, s, "layout");
    if (plan_ws_bytes < pl.total)
        return fail(h, JOLT_E_WORKSPACE, "plan workspace: need %zu bytes, have %zu", pl.total, plan_ws_bytes);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const size_t rb_bytes = pl.readback_stride * n;
    uint8_t *rb = nullptr;
    hipError_t e = readback_buffer(h, rb_bytes, &rb);
    if (e == hipSuccess)
        e = hipMemcpyAsync(rb, static_cast<const uint8_t *>(plan_ws) + pl.readback, rb_bytes, hipMemcpyDeviceToHost,
                           st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(h, e, "replan");
    bool noconv = false;
    s = allocate_from_readback(h, *cfg, items, n, pl, rb, alloc_host, lambda_out, &noconv);
    if (s) return s;
    if (noconv) return fail(h, JOLT_E_NOCONV, "eigensolver hit its sweep cap");
    return JOLT_OK;
}
