// Decode attention over stored factors: launch interface (k_attn.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "jolt_internal.h"

namespace jolt {

// One layer group's K and V payload sections, the queries and outputs, and
// this group's two workspace regions.
struct AttnGroup {
    int L, H, T, d;
    int rtk, rfk, bk, rtpk;          // K item: ranks, residual bits, r_t rounded up to 16
    int rtv, rfv, bv, rtpv;          // V item
    int splits, per_split;           // token ranges (per_split a multiple of 256)
    uint32_t sk[4], sv[4];           // rotation signs (bit f set: s_f = -1)
    float isd;                       // 1 / sqrt(d)
    const void *ut_k, *uf_k, *core_k, *ut_v, *uf_v, *core_v;
    const uint16_t *scales_k, *scales_v;
    const uint8_t *codes_k, *codes_v;
    const float *q;                  // [L][hq][d]
    float *out;                      // [L][hq][d]
    float *lse;                      // [L][hq]
    float *ws_prep;                  // [L][hq][rtpk + d]
    float *ws_part;                  // [splits][L][hq][2 + rtpv + d]
};
struct AttnBatch {
    AttnGroup it[kMaxBatch];
    int n;
    int hq;                          // query heads per layer
    float scale;                     // softmax scale
};
hipError_t launch_attention(const AttnBatch &b, int dtype, hipStream_t s);

}  // namespace jolt
