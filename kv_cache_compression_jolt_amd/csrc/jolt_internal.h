// Internal declarations shared by the libjolt host code and kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/libjolt.h"

namespace jolt {

constexpr int kMaxBatch = 16;      // items per launch (kernel-argument tables)
constexpr int kSolverBatch = 64;   // items per launch of the one-workgroup-per-matrix solvers
constexpr int kPlanGroup = 256;    // items a plan takes through its stages together
constexpr int kGroup = 64;

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline int round_up(int v, int a) { return (v + a - 1) / a * a; }

// ---------------------------------------------------------------- codec
// One item for the fused residual kernels.  `wt` is W~ transposed and sign
// folded: wt[lh][f][k] = s_f * round(C~_lh U~_f^T)[k][f], k padded to rtp
// (multiple of 16) with zeros.
struct CodecItem {
    const void *x;          // encode input  X[LH][T][D]
    void *out;              // decode output X~[LH][T][D]
    const void *ut;         // payload U~_t [T][rt]
    const void *wt;         // [LH][D][rtp] (bf16: hi plane, then the lo plane)
    uint16_t *scales;       // payload scales, (LH T D / 64) bf16
    uint8_t *codes;         // payload codes, (LH T D / 64) * 8 bits bytes
    int T, LH, rt, rtp;
    uint32_t sign_bits[4];  // bit f set -> s_f = -1
};
struct CodecBatch {
    CodecItem it[kMaxBatch];
    int n;
};

// W~ construction from payload parameters
struct WtItem {
    const void *uf;         // payload U~_f [D][rf]
    const void *core;       // payload C~ [LH][rt][rf]
    void *wt;               // out [LH][D][rtp] (bf16: hi plane, then the lo plane)
    int LH, rt, rf, rtp;
    uint32_t sign_bits[4];
};
struct WtBatch {
    WtItem it[kMaxBatch];
    int n;
};

hipError_t launch_encode(const CodecBatch &b, int dtype, int D, int bits, int maxT, int maxLH,
                         hipStream_t s);
hipError_t launch_decode(const CodecBatch &b, int dtype, int D, int bits, int maxT, int maxLH,
                         hipStream_t s);
hipError_t launch_build_wt(const WtBatch &b, int dtype, int D, int maxLH, int maxRtp, hipStream_t s);
// the encoder's W~ of bf16 caches: rotated, in the encoder's row order
hipError_t launch_build_wt_rot(const WtBatch &b, int D, int maxLH, int maxRtp, hipStream_t s);

// test hooks
hipError_t launch_rotate(const float *in, float *out, int64_t rows, int d, const uint32_t *sign_bits,
                         int inverse, hipStream_t s);
hipError_t launch_quantize_pack(const float *rot, int64_t rows, int d, int bits, uint8_t *codes,
                                uint16_t *scales, hipStream_t s);
hipError_t launch_unpack_dequant(const uint8_t *codes, const uint16_t *scales, int64_t rows, int d,
                                 int bits, float *out, hipStream_t s);
hipError_t launch_rademacher(uint64_t key, uint32_t stream, uint64_t first, int64_t count, float *out,
                             hipStream_t s);

// host helpers
void sign_bits_for(uint64_t seed, uint32_t item_id, int d, uint32_t out[4]);

}  // namespace jolt
