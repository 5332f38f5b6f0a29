// fp32 values as bf16 hi + lo pairs, for products of split operands on the
// bf16 MFMA (hi hi + hi lo + lo hi).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace jolt {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two values split into bf16 hi = RNE(v) and lo = RNE(v - hi), packed in pairs
// (element 0 in the low half): the hardware's paired conversion, which rounds
// to nearest even as a software round-to-nearest-even does for finite values.
// |v - hi - lo| <= 2^-18 |v|.
__device__ __forceinline__ void split_bf16x2(float a, float b, uint32_t &hi, uint32_t &lo) {
    const f32x2 f = {a, b};
    const bf16x2 h = __builtin_convertvector(f, bf16x2);
    const bf16x2 l = __builtin_convertvector(f - __builtin_convertvector(h, f32x2), bf16x2);
    hi = __builtin_bit_cast(uint32_t, h);
    lo = __builtin_bit_cast(uint32_t, l);
}

}  // namespace jolt
