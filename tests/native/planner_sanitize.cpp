// Host-dual driver for the sanitizer build (tests/test_host_sanitize.py): the
// planner's allocate() on arbitrary (bytes, distortion) tables and
// allocate_sorted() on captured-energy grids, at sizes from 0 to 300 items,
// with tied bytes and distortions, zero-byte candidates and infeasible, tight
// and loose budgets.  Each result is checked against the dual's contract:
// choices in range, the bytes within the budget when feasible, every item's
// choice minimal in D + lambda * bytes at the returned lambda, and the
// minimum-byte choices when the budget is infeasible.  Exit status 0 when every
// check holds; AddressSanitizer / UndefinedBehaviorSanitizer abort otherwise.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <vector>

#include "planner.h"

using namespace jolt;

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64() {                 // SplitMix64
    uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
static int rnd(int lo, int hi) { return lo + (int)(next_u64() % (uint64_t)(hi - lo + 1)); }
static double rndf() { return (double)(next_u64() >> 11) * (1.0 / 9007199254740992.0); }

static int failures = 0;
#define CHECK(c, ...)                                   \
    do {                                                \
        if (!(c)) {                                     \
            ++failures;                                 \
            std::fprintf(stderr, __VA_ARGS__);          \
            std::fprintf(stderr, "\n");                 \
        }                                               \
    } while (0)

// the contract of one dual result over per-item tables
static void check_result(const char *tag, int n, const std::vector<int> &nc, const std::vector<std::vector<double>> &D,
                         const std::vector<std::vector<int64_t>> &B, int64_t budget, jolt_status s,
                         const std::vector<int> &choice, double lam) {
    int64_t total = 0, min_total = 0;
    for (int i = 0; i < n; ++i) {
        CHECK(choice[i] >= 0 && choice[i] < nc[i], "%s: item %d choice %d of %d", tag, i, choice[i], nc[i]);
        if (choice[i] < 0 || choice[i] >= nc[i]) return;
        total += B[i][choice[i]];
        int64_t mb = B[i][0];
        for (int j = 1; j < nc[i]; ++j) mb = std::min(mb, B[i][j]);
        min_total += mb;
    }
    if (s == JOLT_E_INFEASIBLE) {
        CHECK(min_total > budget, "%s: infeasible with min bytes %lld <= budget %lld", tag, (long long)min_total,
              (long long)budget);
        for (int i = 0; i < n; ++i) {
            int64_t mb = B[i][0];
            for (int j = 1; j < nc[i]; ++j) mb = std::min(mb, B[i][j]);
            CHECK(B[i][choice[i]] == mb, "%s: infeasible item %d not at its minimum bytes", tag, i);
        }
        return;
    }
    CHECK(s == JOLT_OK, "%s: status %d", tag, (int)s);
    CHECK(total <= budget, "%s: bytes %lld > budget %lld", tag, (long long)total, (long long)budget);
    CHECK(lam >= 0.0 && std::isfinite(lam), "%s: lambda %g", tag, lam);
    for (int i = 0; i < n; ++i) {
        const double mine = D[i][choice[i]] + lam * (double)B[i][choice[i]];
        for (int j = 0; j < nc[i]; ++j) {
            const double other = D[i][j] + lam * (double)B[i][j];
            CHECK(mine <= other + 1e-9 * (std::fabs(mine) + std::fabs(other) + 1.0),
                  "%s: item %d choice %d (%.17g) beaten by %d (%.17g) at lambda %.17g", tag, i, choice[i], mine, j,
                  other, lam);
        }
    }
}

static int64_t pick_budget(int64_t lo, int64_t hi) {
    switch (rnd(0, 5)) {
        case 0: return lo - rnd(1, 1000);          // infeasible
        case 1: return lo;                         // tight
        case 2: return hi + rnd(0, 1000);          // loose
        default: return lo + (int64_t)((double)(hi - lo) * rndf());
    }
}

static void tables_trial(int trial) {
    const int n = trial == 0 ? 0 : rnd(1, trial % 7 == 0 ? 300 : 24);
    std::vector<int> nc(n);
    std::vector<std::vector<double>> D(n);
    std::vector<std::vector<int64_t>> B(n);
    std::vector<std::vector<Cand>> cand(n);
    int64_t lo = 0, hi = 0;
    for (int i = 0; i < n; ++i) {
        nc[i] = rnd(1, 40);
        D[i].resize(nc[i]);
        B[i].resize(nc[i]);
        cand[i].resize(nc[i]);
        int64_t mn = INT64_MAX, mx = 0;
        for (int j = 0; j < nc[i]; ++j) {
            B[i][j] = rnd(0, 3) == 0 ? (int64_t)rnd(0, 4) * 1000 : (int64_t)rnd(0, 1 << 20);   // tied bytes
            D[i][j] = rnd(0, 4) == 0 ? (double)rnd(0, 3) : 1e3 * rndf();                     // tied distortions
            cand[i][j] = Cand{8 * rnd(0, 32), 8 * rnd(0, 16), rnd(0, 4)};
            mn = std::min(mn, B[i][j]);
            mx = std::max(mx, B[i][j]);
        }
        lo += mn;
        hi += mx;
    }
    const int64_t budget = pick_budget(lo, hi);
    std::vector<const Cand *> cp(n);
    std::vector<const double *> dp(n);
    std::vector<const int64_t *> bp(n);
    for (int i = 0; i < n; ++i) {
        cp[i] = cand[i].data();
        dp[i] = D[i].data();
        bp[i] = B[i].data();
    }
    std::vector<int> choice(n, -1);
    double lam = -1.0;
    const jolt_status s = allocate(n, nc.data(), cp.data(), dp.data(), bp.data(), budget, choice.data(), &lam);
    char tag[64];
    std::snprintf(tag, sizeof tag, "tables trial %d (n %d)", trial, n);
    check_result(tag, n, nc, D, B, budget, s, choice, lam);
}

static void grid_trial(int trial) {
    const int step = 8, rt_max = 8 * rnd(1, 32), rf_max = 8 * rnd(1, 16);
    const uint32_t mask = rnd(0, 1) ? 0x1Du : 0x1FDu;         // b in {0, 2, 3, 4} or {0, 2..8}
    const std::vector<Cand> cand = candidate_grid(rt_max, rf_max, step, mask);
    const int nc = (int)cand.size(), nr = rt_max / step, nf = rf_max / step;
    std::vector<int> cell(nc);
    for (int j = 0; j < nc; ++j)
        cell[j] = (cand[j].rt == 0 || cand[j].rf == 0) ? -1 : (cand[j].rt / step - 1) * nf + (cand[j].rf / step - 1);
    const int n = rnd(1, trial % 5 == 0 ? 300 : 20);
    const int L = rnd(1, 4), H = rnd(1, 8), T = 64 * rnd(4, 64), d = 128;
    std::vector<int64_t> Bc(nc);
    for (int j = 0; j < nc; ++j) Bc[j] = item_bytes_impl(L, H, T, d, 2, cand[j].rt, cand[j].rf, cand[j].bits);
    const SortedCands sc = sorted_cands(cand, cell.data(), Bc.data());
    double delta[9];
    for (int b = 0; b < 9; ++b) delta[b] = b == 0 ? 1.0 : std::ldexp(1.2, -2 * b);
    std::vector<std::vector<double>> grid(n, std::vector<double>((size_t)nr * nf));
    std::vector<double> nx2(n);
    for (int i = 0; i < n; ++i) {
        // captured energy: prefix sums of a non-negative table, below ||X||^2
        std::vector<double> e((size_t)nr * nf);
        for (auto &v : e) v = rnd(0, 6) == 0 ? 0.0 : rndf();
        for (int r = 0; r < nr; ++r)
            for (int f = 0; f < nf; ++f) {
                double v = e[(size_t)r * nf + f];
                if (r) v += grid[i][(size_t)(r - 1) * nf + f];
                if (f) v += grid[i][(size_t)r * nf + f - 1];
                if (r && f) v -= grid[i][(size_t)(r - 1) * nf + f - 1];
                grid[i][(size_t)r * nf + f] = v;
            }
        nx2[i] = grid[i].back() * (1.0 + rndf());
    }
    std::vector<std::vector<double>> D(n, std::vector<double>(nc));
    std::vector<std::vector<int64_t>> B(n, Bc);
    std::vector<int> ncv(n, nc);
    int64_t lo = 0, hi = 0;
    for (int i = 0; i < n; ++i) {
        int64_t mn = INT64_MAX, mx = 0;
        for (int j = 0; j < nc; ++j) {
            const double S = cell[j] < 0 ? 0.0 : grid[i][cell[j]];
            D[i][j] = delta[cand[j].bits] * std::max(0.0, nx2[i] - S);
            mn = std::min(mn, Bc[j]);
            mx = std::max(mx, Bc[j]);
        }
        lo += mn;
        hi += mx;
    }
    const int64_t budget = pick_budget(lo, hi);
    std::vector<const SortedCands *> scp(n, &sc);
    std::vector<const double *> gp(n);
    for (int i = 0; i < n; ++i) gp[i] = grid[i].data();
    std::vector<int> choice(n, -1);
    std::vector<double> dist(n, -1.0);
    double lam = -1.0;
    const jolt_status s =
        allocate_sorted(n, scp.data(), gp.data(), nx2.data(), delta, budget, choice.data(), dist.data(), &lam);
    char tag[64];
    std::snprintf(tag, sizeof tag, "grid trial %d (n %d, %d candidates)", trial, n, nc);
    check_result(tag, n, ncv, D, B, budget, s, choice, lam);
    for (int i = 0; i < n && s == JOLT_OK; ++i)
        CHECK(dist[i] == D[i][choice[i]], "%s: item %d distortion %.17g, table %.17g", tag, i, dist[i],
              D[i][choice[i]]);
}

int main() {
    for (int t = 0; t < 2000; ++t) tables_trial(t);
    for (int t = 0; t < 400; ++t) grid_trial(t);
    std::printf("planner sanitize: %d failures\n", failures);
    return failures ? 1 : 0;
}
