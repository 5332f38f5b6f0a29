// Host planner: byte accounting, distortion tables and the single-Lagrangian-dual
// allocation of (token rank, feature rank, residual bits).
//
// Method ("A JoLT for the KV cache": author page abstract, landing page abstract;
// podcast section "The Core Mechanism"): one Lagrangian dual allocates the Tucker
// ranks and the residual bit-widths together, per layer group and separately for
// K and V, under one byte budget, instead of pre-splitting the budget.
//
// For a dual value lambda every item independently takes the candidate that
// minimises D + lambda * bytes (ties: fewer bytes, then smaller r_t, r_f, b).
// Only vertices of the lower convex hull of an item's (bytes, D) points can win;
// between consecutive vertices the choice flips at slope s = dD / dbytes.  Total
// bytes is a non-increasing step function of lambda, so lambda* (the least lambda
// whose allocation fits the budget) is 0 or one of the slopes; it is found by
// bisection over the sorted slopes.  All arithmetic is fp64 / int64; the build
// uses -ffp-contract=off so the slope and hull tests round the same way every time.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <numeric>
#include <thread>
#include <vector>

#include "planner.h"

namespace jolt {

int64_t item_bytes_impl(int L, int H, int T, int d, int e, int rt, int rf, int bits) {
    if (rt == 0 || rf == 0) rt = rf = 0;
    const int64_t N = (int64_t)L * H * T * d;
    int64_t params = (int64_t)e * ((int64_t)T * rt + (int64_t)d * rf + (int64_t)L * H * rt * rf);
    int64_t resid = bits > 0 ? (N * bits / 8 + 2 * N / 64) : 0;
    return params + resid;
}

std::vector<Cand> candidate_grid(int rt_max, int rf_max, int step, uint32_t bits_mask) {
    // generated in (rt, rf, bits) order: the rank-0 candidates first, one per bit width
    std::vector<Cand> out;
    for (int b = 0; b <= 8; ++b)
        if (bits_mask & (1u << b)) out.push_back({0, 0, b});
    for (int rt = step; rt <= rt_max; rt += step)
        for (int rf = step; rf <= rf_max; rf += step)
            for (int b = 0; b <= 8; ++b)
                if (bits_mask & (1u << b)) out.push_back({rt, rf, b});
    return out;
}

std::vector<int> byte_order(int nc, const Cand *cand, const int64_t *B) {
    std::vector<int> order(nc);
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) {
        if (B[a] != B[b]) return B[a] < B[b];
        if (cand[a].rt != cand[b].rt) return cand[a].rt < cand[b].rt;
        if (cand[a].rf != cand[b].rf) return cand[a].rf < cand[b].rf;
        return cand[a].bits < cand[b].bits;
    });
    return order;
}

namespace {

struct ItemHull {
    std::vector<int> v;        // positions in byte order, bytes ascending
    std::vector<double> d;     // distortion at v[j]
    std::vector<double> s;     // slope between v[j] and v[j+1] (decreasing)
};

// Lower convex hull of the (bytes, distortion) points of one item, given in
// byte order (equal bytes in the order (rt, rf, bits)): B[p] and D(p) at
// position p.  The points that matter form a staircase: of each run of equal
// bytes the point of least D (ties: the earliest), kept only where D falls
// strictly below every point kept so far.  Each staircase point goes onto the
// monotone chain as it is found; a later point of the same bytes and lower D
// first takes the earlier one off the end of the chain (it pops at least what
// that one popped, so the chain is the one over the final staircase).  h is
// reused: its vectors keep their capacity from call to call.
template <typename DF>
void build_hull(int nc, const int64_t *B, DF D, ItemHull &h) {
    h.v.clear();
    h.d.clear();
    h.s.clear();
    double run = 0.0;
    for (int p = 0; p < nc; ++p) {
        const double di = D(p);
        if (!h.v.empty()) {
            if (!(di < run)) continue;
            if (B[h.v.back()] == B[p]) {
                h.v.pop_back();
                h.d.pop_back();
            }
        }
        run = di;
        while (h.v.size() >= 2) {
            const int o = h.v[h.v.size() - 2], a = h.v.back();
            const double dO = h.d[h.d.size() - 2], dA = h.d.back();
            const double cross = (double)(B[a] - B[o]) * (di - dO) - (dA - dO) * (double)(B[p] - B[o]);
            if (cross <= 0.0) {
                h.v.pop_back();
                h.d.pop_back();
            } else {
                break;
            }
        }
        h.v.push_back(p);
        h.d.push_back(di);
    }
    for (size_t j = 0; j + 1 < h.v.size(); ++j) h.s.push_back((h.d[j] - h.d[j + 1]) / (double)(B[h.v[j + 1]] - B[h.v[j]]));
}

// per-thread hulls, kept between calls for their capacity
std::vector<ItemHull> &hull_scratch(int n) {
    thread_local std::vector<ItemHull> hulls;
    if ((int)hulls.size() < n) hulls.resize(n);
    return hulls;
}

// vertex chosen at lambda: v[J], J = #{j : s_j > lambda}
int vertex_at(const ItemHull &h, double lam) {
    int J = 0;
    for (double s : h.s) J += (s > lam);
    return h.v[J];
}

// the single dual over the items' hulls (B_i: item i's bytes in byte order):
// lambda* and each item's chosen position
jolt_status dual(int n, const std::vector<ItemHull> &hulls, const int64_t *const *B, int64_t budget, int *pos,
                 double *lambda_out) {
    int64_t min_total = 0;
    for (int i = 0; i < n; ++i) min_total += B[i][hulls[i].v[0]];
    if (min_total > budget) {
        for (int i = 0; i < n; ++i) pos[i] = hulls[i].v[0];
        if (lambda_out) *lambda_out = INFINITY;
        return JOLT_E_INFEASIBLE;
    }
    // lambda* is 0 when taking every hull edge fits.  Otherwise it is the
    // largest hull slope sigma at which the minimum bytes plus the bytes of
    // every edge of slope >= sigma exceed the budget: walking the distinct
    // slopes from the largest down, the first whose edges no longer fit.  The
    // allocation at sigma takes the edges of slope > sigma only, and those fit.
    // sigma is found by a weighted selection over all the items' edges:
    // partition the range around a pivot slope into (> p, == p, < p) and keep
    // the part that holds the crossing; every edge of one slope stays together.
    struct Edge {
        double s;
        int64_t w;
    };
    thread_local std::vector<Edge> E;
    E.clear();
    for (int i = 0; i < n; ++i) {
        const ItemHull &h = hulls[i];
        for (size_t j = 0; j < h.s.size(); ++j) E.push_back(Edge{h.s[j], B[i][h.v[j + 1]] - B[i][h.v[j]]});
    }
    double lam = 0.0;
    int64_t base = min_total;                           // bytes of the edges above the range, plus the minimum
    size_t lo = 0, hi = E.size();
    while (lo < hi) {
        const double a = E[lo].s, b = E[lo + (hi - lo) / 2].s, c = E[hi - 1].s;
        const double p = std::max(std::min(a, b), std::min(std::max(a, b), c));   // median of three
        size_t m1 = lo, k = lo, m2 = hi;
        while (k < m2) {
            if (E[k].s > p) std::swap(E[k++], E[m1++]);
            else if (E[k].s < p) std::swap(E[k], E[--m2]);
            else ++k;
        }
        int64_t w_gt = 0, w_eq = 0;
        for (size_t q = lo; q < m1; ++q) w_gt += E[q].w;
        for (size_t q = m1; q < m2; ++q) w_eq += E[q].w;
        if (base + w_gt > budget) {
            hi = m1;                                    // the crossing lies among the slopes > p
        } else if (base + w_gt + w_eq > budget) {
            lam = p;
            break;
        } else {
            base += w_gt + w_eq;
            lo = m2;
        }
    }
    for (int i = 0; i < n; ++i) pos[i] = vertex_at(hulls[i], lam);
    if (lambda_out) *lambda_out = lam;
    return JOLT_OK;
}

}  // namespace

jolt_status allocate(int n, const int32_t *n_cand, const Cand *const *cand, const double *const *D,
                     const int64_t *const *B, int64_t budget, int *choice, double *lambda_out,
                     const int *const *order) {
    std::vector<ItemHull> &hulls = hull_scratch(n);
    std::vector<std::vector<int>> own(n);
    std::vector<std::vector<int64_t>> Bs(n);
    std::vector<const int64_t *> bp(n);
    std::vector<const int *> op(n);
    for (int i = 0; i < n; ++i) {
        if (n_cand[i] <= 0) return JOLT_E_INVALID;
        if (order && order[i]) {
            op[i] = order[i];
        } else {
            own[i] = byte_order(n_cand[i], cand[i], B[i]);
            op[i] = own[i].data();
        }
        Bs[i].resize(n_cand[i]);
        for (int p = 0; p < n_cand[i]; ++p) Bs[i][p] = B[i][op[i][p]];
        bp[i] = Bs[i].data();
        const double *Di = D[i];
        const int *oi = op[i];
        build_hull(n_cand[i], bp[i], [&](int p) { return Di[oi[p]]; }, hulls[i]);
    }
    std::vector<int> pos(n);
    const jolt_status s = dual(n, hulls, bp.data(), budget, pos.data(), lambda_out);
    for (int i = 0; i < n; ++i) choice[i] = op[i][pos[i]];
    return s;
}

jolt_status allocate_sorted(int n, const SortedCands *const *sc, const double *const *grid, const double *normx2,
                            const double *delta, int64_t budget, int *choice, double *distortion,
                            double *lambda_out) {
    std::vector<ItemHull> &hulls = hull_scratch(n);
    std::vector<const int64_t *> bp(n);
    for (int i = 0; i < n; ++i) {
        if (sc[i]->B.empty()) return JOLT_E_INVALID;
        bp[i] = sc[i]->B.data();
    }
    auto hull_of = [&](int i) {
        const SortedCands &c = *sc[i];
        const double *g = grid[i], nx2 = normx2[i];
        const int *cell = c.cell.data();
        const uint8_t *bits = c.bits.data();
        // D = delta_b max(0, ||X||^2 - S), S the captured energy of the cell (0 at rank 0)
        build_hull((int)c.B.size(), bp[i], [&](int p) {
            const double S = cell[p] < 0 ? 0.0 : g[cell[p]];
            return delta[bits[p]] * std::max(0.0, nx2 - S);
        }, hulls[i]);
    };
    // The hulls are independent: a large call builds them on a few threads,
    // each over a contiguous run of items (the result does not depend on it).
    const int workers = std::min({(int)std::max(1u, std::thread::hardware_concurrency()), 8, (n + 31) / 32});
    if (workers <= 1) {
        for (int i = 0; i < n; ++i) hull_of(i);
    } else {
        std::vector<std::thread> pool;
        pool.reserve(workers - 1);
        const int per = (n + workers - 1) / workers;
        for (int w = 1; w < workers; ++w)
            pool.emplace_back([&, w]() {
                for (int i = w * per; i < std::min(n, (w + 1) * per); ++i) hull_of(i);
            });
        for (int i = 0; i < std::min(n, per); ++i) hull_of(i);
        for (std::thread &t : pool) t.join();
    }
    std::vector<int> pos(n);
    const jolt_status s = dual(n, hulls, bp.data(), budget, pos.data(), lambda_out);
    for (int i = 0; i < n; ++i) {
        const SortedCands &c = *sc[i];
        const int p = pos[i];
        choice[i] = c.cand[p];
        const double S = c.cell[p] < 0 ? 0.0 : grid[i][c.cell[p]];
        distortion[i] = delta[c.bits[p]] * std::max(0.0, normx2[i] - S);
    }
    return s;
}

SortedCands sorted_cands(const std::vector<Cand> &cand, const int *cell, const int64_t *B) {
    SortedCands s;
    const std::vector<int> order = byte_order((int)cand.size(), cand.data(), B);
    const size_t nc = cand.size();
    s.B.resize(nc);
    s.cell.resize(nc);
    s.bits.resize(nc);
    s.cand.resize(nc);
    for (size_t p = 0; p < nc; ++p) {
        const int j = order[p];
        s.B[p] = B[j];
        s.cell[p] = cell[j];
        s.bits[p] = (uint8_t)cand[j].bits;
        s.cand[p] = j;
    }
    return s;
}

}  // namespace jolt
