// Device-side helpers shared by the libjolt kernels (gfx950 / CDNA4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace jolt {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- bf16 bits
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(((uint32_t)b) << 16);
}
// fp32 -> bf16 round to nearest even (finite values)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float round_bf16(float f) { return bf16_to_f32(f32_to_bf16(f)); }
// two fp32 -> two bf16 (a in the low half) in one conversion instruction; round
// to nearest even, the same bits as f32_to_bf16 for finite values
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16_pair(float a, float b) {
    const f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// ---------------------------------------------------------------- counter RNG
// SplitMix64 output function (Steele, Lea & Flood 2014), used as a counter hash.
__host__ __device__ __forceinline__ uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
// key of an item's streams
__host__ __device__ __forceinline__ uint64_t item_key(uint64_t seed, uint32_t item_id) {
    return mix64(mix64(seed) + (uint64_t)item_id);
}
// +1 / -1 for counter `idx` of stream `stream`: bit 63 of the hash set -> -1
__host__ __device__ __forceinline__ float rademacher(uint64_t key, uint32_t stream, uint64_t idx) {
    uint64_t w = mix64(key + ((uint64_t)stream << 56) + idx);
    return (w >> 63) ? -1.0f : 1.0f;
}

// ---------------------------------------------------------------- MFMA fragments
// A 32x32 output tile of v_mfma_f32_32x32x16_bf16 / _32x32x2f32: lane l holds
// column n = l % 32 and rows m = 8*(j/4) + 4*(l/32) + (j%4), j = 0..15.
// Operand fragments: lane l holds row (A) / column (B) l % 32 and the 8
// consecutive K indices k0 + 8*(l/32) + i, i = 0..7 (the same K mapping on
// both operands, so any hardware K permutation cancels).
struct FragBF16 { bf16x8 v; };
struct FragF32 { float v[8]; };

__device__ __forceinline__ FragBF16 load_frag(const uint16_t *p) {
    FragBF16 f;
    uint4 raw = *reinterpret_cast<const uint4 *>(p);
    f.v = __builtin_bit_cast(bf16x8, raw);
    return f;
}
__device__ __forceinline__ FragF32 load_frag(const float *p) {
    FragF32 f;
    float4 a = *reinterpret_cast<const float4 *>(p);
    float4 b = *reinterpret_cast<const float4 *>(p + 4);
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
    f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
    return f;
}
// element-wise load of min(8, count) values (count may be <= 0), zero fill; any alignment
__device__ __forceinline__ FragBF16 load_frag_n(const uint16_t *p, int count) {
    uint16_t e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) e[i] = (i < count) ? p[i] : (uint16_t)0;
    FragBF16 f;
    f.v = __builtin_bit_cast(bf16x8, e);
    return f;
}
__device__ __forceinline__ FragF32 load_frag_n(const float *p, int count) {
    FragF32 f;
#pragma unroll
    for (int i = 0; i < 8; ++i) f.v[i] = (i < count) ? p[i] : 0.f;
    return f;
}
__device__ __forceinline__ FragBF16 zero_frag(const uint16_t *) { FragBF16 f; f.v = bf16x8{}; return f; }
__device__ __forceinline__ FragF32 zero_frag(const float *) {
    FragF32 f;
#pragma unroll
    for (int i = 0; i < 8; ++i) f.v[i] = 0.f;
    return f;
}
__device__ __forceinline__ void mfma(const FragBF16 &a, const FragBF16 &b, f32x16 &acc) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mfma(const FragF32 &a, const FragF32 &b, f32x16 &acc) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.v[i], b.v[i], acc, 0, 0, 0);
}

// p[i] where ok, else 0: the load is always issued, so i must address the
// buffer even where ok is false; a select, not a branch, drops the value
__device__ __forceinline__ float ld_or_zero(const float *p, int i, bool ok) {
    const float v = p[i];
    return ok ? v : 0.f;
}

// Orders one wave's LDS stores before its later LDS loads of other lanes'
// values (no workgroup barrier: only the calling wave takes part).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Scheduling hint for an unrolled run of N LDS fragment reads, each feeding M
// MFMAs: the reads are issued AHEAD in front of the MFMAs, then one read per
// M MFMAs, so that AHEAD reads are in flight while the MFMAs run (without it
// the scheduler puts each read right before its MFMA and waits for it there).
// VM > 0: VM global loads of the same region are issued first of all, so that
// they are in flight together.  PRE > 0: PRE MFMAs of the region that need none
// of the reads (and of the loads) come next, while the loads are in flight,
// with the first AHEAD reads issued in front of them.
template <int N, int M, int AHEAD, int VM = 0, int PRE = 0>
__device__ __forceinline__ void sched_reads_ahead() {
    constexpr int A = AHEAD < N ? AHEAD : N;
    if constexpr (VM > 0) __builtin_amdgcn_sched_group_barrier(0x020, VM, 0);   // VMEM reads
    __builtin_amdgcn_sched_group_barrier(0x100, A, 0);          // DS reads
    if constexpr (PRE > 0) __builtin_amdgcn_sched_group_barrier(0x008, PRE, 0);
#pragma unroll
    for (int i = 0; i < N - A; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, M, 0);      // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, M * A, 0);
}

// ---------------------------------------------------------------- wave reductions
// Sums within aligned lane groups of 4, 8 and 16 use DPP lane moves inside a
// row of 16 lanes (quad permutes, then the half-row and row mirrors), which
// cost a VALU op each instead of an LDS-crossbar round trip.  Every lane of a
// group ends with the same value: each step adds a pair in both orders.
template <int Ctrl>
__device__ __forceinline__ float dpp_move(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), Ctrl, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;          // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;          // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;   // lane i <- 7 - i within 8
constexpr int kDppMirror = 0x140;       // lane i <- 15 - i within 16
constexpr int kDppRowBcast15 = 0x142;   // rows 1 and 3 <- lane 15 of the row below

__device__ __forceinline__ float group4_sum(float v) {
    v += dpp_move<kDppXor1>(v);
    return v + dpp_move<kDppXor2>(v);
}
__device__ __forceinline__ float group8_sum(float v) {
    v = group4_sum(v);
    return v + dpp_move<kDppHalfMirror>(v);
}
__device__ __forceinline__ float group16_sum(float v) {
    v = group8_sum(v);
    return v + dpp_move<kDppMirror>(v);
}
__device__ __forceinline__ float lane_bcast(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
// whole-wave sum: row sums, then the four rows read out and added in a fixed
// order (the result is wave-uniform)
__device__ __forceinline__ float wave_sum(float v) {
    v = group16_sum(v);
    return (lane_bcast(v, 0) + lane_bcast(v, 16)) + (lane_bcast(v, 32) + lane_bcast(v, 48));
}
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp_move<kDppXor1>(v));
    v = fmaxf(v, dpp_move<kDppXor2>(v));
    v = fmaxf(v, dpp_move<kDppHalfMirror>(v));
    v = fmaxf(v, dpp_move<kDppMirror>(v));
    return fmaxf(fmaxf(lane_bcast(v, 0), lane_bcast(v, 16)), fmaxf(lane_bcast(v, 32), lane_bcast(v, 48)));
}
__device__ __forceinline__ float wave_min(float v) {
    v = fminf(v, dpp_move<kDppXor1>(v));
    v = fminf(v, dpp_move<kDppXor2>(v));
    v = fminf(v, dpp_move<kDppHalfMirror>(v));
    v = fminf(v, dpp_move<kDppMirror>(v));
    return fminf(fminf(lane_bcast(v, 0), lane_bcast(v, 16)), fminf(lane_bcast(v, 32), lane_bcast(v, 48)));
}

// ---------------------------------------------------------------- XCD-aware block ids
// The GPU deals workgroups round-robin over its 8 XCDs (each with its own L2).
// xcd_block() permutes the linear workgroup id so that each XCD gets one
// contiguous range of logical workgroups: neighbours in (x, y, z) order, which
// share operands (the same item, the same layer-head), then hit the same L2.
// Grids whose size is not a multiple of 8 keep the identity order.
struct Block3 { int x, y, z; };
__device__ __forceinline__ Block3 xcd_block() {
    constexpr int kXcd = 8;
    const int gx = gridDim.x, gy = gridDim.y;
    const int total = gx * gy * gridDim.z;
    int w = blockIdx.x + gx * (blockIdx.y + gy * blockIdx.z);
    if (total % kXcd == 0) w = (w % kXcd) * (total / kXcd) + w / kXcd;
    Block3 b;
    b.x = w % gx;
    b.y = (w / gx) % gy;
    b.z = w / (gx * gy);
    return b;
}

__device__ __forceinline__ int frag_row(int lane, int j) { return 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3); }

template <typename T> struct Elem;
template <> struct Elem<uint16_t> { typedef FragBF16 Frag; static constexpr int bytes = 2; };
template <> struct Elem<float> { typedef FragF32 Frag; static constexpr int bytes = 4; };

__device__ __forceinline__ float to_f32(uint16_t v) { return bf16_to_f32(v); }
__device__ __forceinline__ float to_f32(float v) { return v; }

}  // namespace jolt
