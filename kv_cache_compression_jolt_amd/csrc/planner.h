// Host planner declarations (pure host code).
#pragma once
#include <stdint.h>

#include <vector>

#include "../../include/libjolt.h"

namespace jolt {

struct Cand {
    int32_t rt, rf, bits;
};

int64_t item_bytes_impl(int L, int H, int T, int d, int e, int rt, int rf, int bits);
std::vector<Cand> candidate_grid(int rt_max, int rf_max, int step, uint32_t bits_mask);
// candidate indices sorted by (bytes, rt, rf, bits)
std::vector<int> byte_order(int nc, const Cand *cand, const int64_t *B);
// order[i] (optional, may be null or hold nulls): item i's byte_order, when the
// caller shares one among items of the same shape
jolt_status allocate(int n, const int32_t *n_cand, const Cand *const *cand, const double *const *D,
                     const int64_t *const *B, int64_t budget, int *choice, double *lambda_out,
                     const int *const *order = nullptr);
// One item shape's candidates in byte order (as byte_order): bytes, grid cell
// (-1: rank 0), bits and candidate index at each position.
struct SortedCands {
    std::vector<int64_t> B;
    std::vector<int> cell;
    std::vector<uint8_t> bits;
    std::vector<int> cand;
};
SortedCands sorted_cands(const std::vector<Cand> &cand, const int *cell, const int64_t *B);
// allocate() with each item's distortions formed from its captured-energy grid
// position by position in byte order, D = delta_b max(0, ||X||^2 - S(cell))
// with S = 0 at rank 0 (no table): choice[i] is a candidate index,
// distortion[i] its distortion
jolt_status allocate_sorted(int n, const SortedCands *const *sc, const double *const *grid, const double *normx2,
                            const double *delta, int64_t budget, int *choice, double *distortion,
                            double *lambda_out);

}  // namespace jolt
