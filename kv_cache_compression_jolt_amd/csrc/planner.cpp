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
    std::vector<int> v;        // candidate indices, bytes ascending
    std::vector<double> s;     // slope between v[j] and v[j+1] (decreasing)
};

struct Pt {
    int64_t B;
    double D;
    int rt, rf, bits, idx;
};

// `order`: candidate indices by (bytes, rt, rf, bits)
ItemHull build_hull(int nc, const int *order, const double *D, const int64_t *B) {
    // staircase: per byte count the point of least D (ties: the earliest in
    // order, i.e. smaller rt, rf, bits), kept only where D strictly falls
    std::vector<int> stair;
    stair.reserve(nc);
    for (int p = 0; p < nc;) {
        int best = order[p], q = p + 1;
        for (; q < nc && B[order[q]] == B[best]; ++q)
            if (D[order[q]] < D[best]) best = order[q];
        p = q;
        if (!stair.empty() && !(D[best] < D[stair.back()])) continue;
        stair.push_back(best);
    }
    ItemHull h;
    h.v.reserve(stair.size());
    h.s.reserve(stair.size());
    for (int i : stair) {
        while (h.v.size() >= 2) {
            const int o = h.v[h.v.size() - 2], a = h.v.back();
            const double cross = (double)(B[a] - B[o]) * (D[i] - D[o]) - (D[a] - D[o]) * (double)(B[i] - B[o]);
            if (cross <= 0.0) h.v.pop_back();
            else break;
        }
        h.v.push_back(i);
    }
    for (size_t j = 0; j + 1 < h.v.size(); ++j) {
        const int a = h.v[j], b = h.v[j + 1];
        h.s.push_back((D[a] - D[b]) / (double)(B[b] - B[a]));
    }
    return h;
}

// vertex chosen at lambda: v[J], J = #{j : s_j > lambda}
int vertex_at(const ItemHull &h, double lam) {
    int J = 0;
    for (double s : h.s) J += (s > lam);
    return h.v[J];
}

}  // namespace

jolt_status allocate(int n, const int32_t *n_cand, const Cand *const *cand, const double *const *D,
                     const int64_t *const *B, int64_t budget, int *choice, double *lambda_out,
                     const int *const *order) {
    std::vector<ItemHull> hulls(n);
    int64_t min_total = 0;
    for (int i = 0; i < n; ++i) {
        if (n_cand[i] <= 0) return JOLT_E_INVALID;
        if (order && order[i]) {
            hulls[i] = build_hull(n_cand[i], order[i], D[i], B[i]);
        } else {
            const std::vector<int> o = byte_order(n_cand[i], cand[i], B[i]);
            hulls[i] = build_hull(n_cand[i], o.data(), D[i], B[i]);
        }
        min_total += B[i][hulls[i].v[0]];
    }
    if (min_total > budget) {
        for (int i = 0; i < n; ++i) choice[i] = hulls[i].v[0];
        if (lambda_out) *lambda_out = INFINITY;
        return JOLT_E_INFEASIBLE;
    }
    // lambda* is 0 when taking every hull edge fits; else the least hull slope
    // sigma whose allocation (every edge of slope > sigma taken) fits.  The
    // distinct slopes are walked from the largest down by merging the items'
    // hulls (each in decreasing slope order): total(sigma_1) is the minimum,
    // and total(sigma_{k+1}) adds the edges of slope exactly sigma_k.
    double lam = 0.0;
    {
        std::vector<size_t> next(n, 0);
        auto next_slope = [&]() {
            double m = -1.0;                            // slopes are positive
            for (int i = 0; i < n; ++i)
                if (next[i] < hulls[i].s.size()) m = std::max(m, hulls[i].s[next[i]]);
            return m;
        };
        int64_t tot = min_total;                        // total(sg)
        double fit = 0.0;
        double sg = next_slope();
        while (sg > 0.0 && tot <= budget) {
            fit = sg;
            for (int i = 0; i < n; ++i) {
                const ItemHull &h = hulls[i];
                for (; next[i] < h.s.size() && h.s[next[i]] == sg; ++next[i])
                    tot += B[i][h.v[next[i] + 1]] - B[i][h.v[next[i]]];
            }
            sg = next_slope();
        }
        lam = (sg <= 0.0 && tot <= budget) ? 0.0 : fit;
    }
    for (int i = 0; i < n; ++i) choice[i] = vertex_at(hulls[i], lam);
    if (lambda_out) *lambda_out = lam;
    return JOLT_OK;
}

void distortion_table(const double *grid /* captured energy S at (rt, rf) = (step (i+1), step (j+1)) */, int nf,
                      int step, double normx2, const double *delta, const std::vector<Cand> &cand, double *D) {
    for (size_t i = 0; i < cand.size(); ++i) {
        const Cand &c = cand[i];
        const double S = (c.rt == 0 || c.rf == 0) ? 0.0 : grid[(size_t)(c.rt / step - 1) * nf + (c.rf / step - 1)];
        D[i] = delta[c.bits] * std::max(0.0, normx2 - S);
    }
}

void distortion_table_cells(const double *grid, const int *cell, double normx2, const double *delta,
                            const std::vector<Cand> &cand, double *D) {
    for (size_t i = 0; i < cand.size(); ++i) {
        const double S = cell[i] < 0 ? 0.0 : grid[cell[i]];
        D[i] = delta[cand[i].bits] * std::max(0.0, normx2 - S);
    }
}

}  // namespace jolt
