// Payload format and plan-workspace layout (pure host computations).
#pragma once
#include <stddef.h>
#include <stdint.h>

#include <vector>

#include "../../include/libjolt.h"

namespace jolt {

constexpr uint32_t kMagic = 0x544C4F4Au;   // "JOLT"
constexpr uint16_t kVersion = 1;

struct PayloadLayout {
    size_t ut, uf, core, scales, codes, total;
    size_t ut_bytes, uf_bytes, core_bytes, scales_bytes, codes_bytes;
    int rt, rf, bits;
};

inline int elem_bytes(int dtype) { return dtype == JOLT_F32 ? 4 : 2; }
PayloadLayout payload_layout(const jolt_item &it, int rt, int rf, int bits);
void make_header(const jolt_item &it, const jolt_alloc &a, uint8_t out[64]);

// Per-item factor storage inside plan_ws, followed by per-chunk scratch.
struct FactorOffsets {
    size_t ut, uf, lam_t, lam_f, core, energy, grid, sfixed, normx2, sweeps;
};
struct PlanLayout {
    int rt_max, rf_max, k, kp;              // k = sketch width (randomized) ; kp = padded
    int step, grid_nr, grid_nf;              // candidate rank step; captured-energy grid (rt_max / step) x (rf_max / step)
    std::vector<FactorOffsets> item;
    // host-bound results, one block per item: captured-energy grid S (fp64) |
    // S at the fixed ranks | ||X||^2 | eigensolver status
    size_t readback, readback_stride;
    size_t scratch;                          // start of the scratch region
    size_t scratch_bytes;                    // per chunk
    size_t total;
};
jolt_status plan_layout(const jolt_config &cfg, const jolt_item *items, int n, PlanLayout *out);
size_t codec_ws_bytes_for(const jolt_item *items, int n, const int *rt);

}  // namespace jolt
