// Residual codec kernels for gfx950: the fused residual -> rotate -> quantize ->
// pack encoder, the fused decoder, W~ construction, and the plain per-row /
// per-group kernels behind the test hooks.
//
// Method ("A JoLT for the KV cache", landing page abstract; author page
// abstract): the truncation residual of the partial Tucker approximation is
// rotated by a Johnson-Lindenstrauss rotation and quantized to a few bits.
// Here the rotation of a (layer, head, token) row of d features is
// r' = (1/sqrt d) H_d (s o r) (Sylvester Hadamard, seeded signs s); each group
// of 64 rotated values gets a bf16 absmax scale and b-bit symmetric codes,
// packed as one little-endian bit stream per group (element j in bits
// [b j, b j + b)).  The residual is taken against the reconstruction the
// decoder forms from the stored parameters: X^_lh = U~_t W~_lh, W~_lh =
// C~_lh U~_f^T kept to fp32 precision (for bf16 caches as a hi + lo pair of
// bf16 planes, each of them an MFMA operand).
//
// Register layout of the fused kernels.  A wave owns 32 tokens of one (layer,
// head).  X^ is an MFMA product D[f][t] = sum_k W~t[f][k] U~_t[t][k]
// (v_mfma_f32_32x32x16_bf16, or 32x32x2f32 for fp32 caches); lane l then
// holds token l % 32 and, for each 32-feature block mf, features
// f = 32 mf + 8 (j / 4) + 4 (l / 32) + (j % 4), j = 0..15.  Six of the
// log2(d) butterfly stages are in-register; the stage over feature bit 2
// (the lane half) uses v_permlane32_swap on register pairs that differ in the
// top feature bit, which leaves each lane holding one whole 64-group
// (d = 128) or half of it (d = 64).  Group absmax and packing are then
// in-lane, and each lane stores its group's codes contiguously.
#include <algorithm>

#include "dev_common.h"
#include "jolt_internal.h"
#include "ktimer.h"

namespace jolt {

// ------------------------------------------------------------------ helpers
__device__ __forceinline__ uint32_t pack_lowbytes(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    // [a.b0, b.b0, c.b0, d.b0]
    uint32_t p01 = __builtin_amdgcn_perm(b, a, 0x0c0c0400u);
    uint32_t p23 = __builtin_amdgcn_perm(d, c, 0x0c0c0400u);
    return __builtin_amdgcn_perm(p23, p01, 0x05040100u);
}

// swap lanes 32..63 of x with lanes 0..31 of y
__device__ __forceinline__ void swap_halves(float &x, float &y) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    x = __uint_as_float(r[0]);
    y = __uint_as_float(r[1]);
}

// Pack NE codes (magic-float bit patterns whose low byte is the code) of
// width BITS into the little-endian stream words w[BITS * NE / 32].
template <int BITS, int NE>
__device__ __forceinline__ void pack_codes(const uint32_t *t, uint32_t *w) {
    constexpr int NW = BITS * NE / 32;
    if constexpr (BITS == 8) {
#pragma unroll
        for (int k = 0; k < NW; ++k) w[k] = pack_lowbytes(t[4 * k], t[4 * k + 1], t[4 * k + 2], t[4 * k + 3]);
    } else if constexpr (BITS == 4) {
#pragma unroll
        for (int k = 0; k < NW; ++k) {
            const uint32_t *s = t + 8 * k;
            uint32_t ev = pack_lowbytes(s[0], s[2], s[4], s[6]);
            uint32_t od = pack_lowbytes(s[1], s[3], s[5], s[7]);
            w[k] = ev | (od << 4);
        }
    } else if constexpr (BITS == 2) {
#pragma unroll
        for (int k = 0; k < NW; ++k) {
            const uint32_t *s = t + 16 * k;
            uint32_t b0 = pack_lowbytes(s[0], s[4], s[8], s[12]);
            uint32_t b1 = pack_lowbytes(s[1], s[5], s[9], s[13]);
            uint32_t b2 = pack_lowbytes(s[2], s[6], s[10], s[14]);
            uint32_t b3 = pack_lowbytes(s[3], s[7], s[11], s[15]);
            w[k] = b0 | (b1 << 2) | (b2 << 4) | (b3 << 6);
        }
    } else {
#pragma unroll
        for (int k = 0; k < NW; ++k) w[k] = 0;
#pragma unroll
        for (int e = 0; e < NE; ++e) {
            const uint32_t u = t[e] & ((1u << BITS) - 1u);
            const int pos = BITS * e;
            w[pos >> 5] |= u << (pos & 31);
            if ((pos & 31) + BITS > 32) w[(pos >> 5) + 1] |= u >> (32 - (pos & 31));
        }
    }
}

// Unpack NE codes of width BITS from w into floats q = u - 2^(BITS-1).
template <int BITS, int NE>
__device__ __forceinline__ void unpack_codes(const uint32_t *w, float *u) {
    constexpr int NW = BITS * NE / 32;
    if constexpr (BITS == 8) {
#pragma unroll
        for (int k = 0; k < NW; ++k)
#pragma unroll
            for (int i = 0; i < 4; ++i) u[4 * k + i] = (float)((w[k] >> (8 * i)) & 0xFFu);
    } else if constexpr (BITS == 4) {
#pragma unroll
        for (int k = 0; k < NW; ++k) {
            const uint32_t lo = w[k] & 0x0F0F0F0Fu, hi = (w[k] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                u[8 * k + 2 * i] = (float)((lo >> (8 * i)) & 0xFFu);
                u[8 * k + 2 * i + 1] = (float)((hi >> (8 * i)) & 0xFFu);
            }
        }
    } else if constexpr (BITS == 2) {
#pragma unroll
        for (int k = 0; k < NW; ++k)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint32_t v = (w[k] >> (2 * r)) & 0x03030303u;
#pragma unroll
                for (int i = 0; i < 4; ++i) u[16 * k + 4 * i + r] = (float)((v >> (8 * i)) & 0xFFu);
            }
    } else {
#pragma unroll
        for (int e = 0; e < NE; ++e) {
            const int pos = BITS * e;
            uint32_t v = w[pos >> 5] >> (pos & 31);
            if ((pos & 31) + BITS > 32) v |= w[(pos >> 5) + 1] << (32 - (pos & 31));
            u[e] = (float)(v & ((1u << BITS) - 1u));
        }
    }
}

template <typename T> struct Store;
template <> struct Store<uint16_t> {
    // round to bf16 (RNE) pairs
    static __device__ __forceinline__ void put4(uint8_t *dst, float a, float b, float c, float d) {
        uint2 v;
        v.x = (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
        v.y = (uint32_t)f32_to_bf16(c) | ((uint32_t)f32_to_bf16(d) << 16);
        *reinterpret_cast<uint2 *>(dst) = v;
    }
    static __device__ __forceinline__ void get4(const uint8_t *src, float *o) {
        uint2 v = *reinterpret_cast<const uint2 *>(src);
        o[0] = __uint_as_float(v.x << 16);
        o[1] = __uint_as_float(v.x & 0xFFFF0000u);
        o[2] = __uint_as_float(v.y << 16);
        o[3] = __uint_as_float(v.y & 0xFFFF0000u);
    }
    static constexpr uint32_t kSignBit = 0x8000u;
    static constexpr int kPerDword = 2;
};
template <> struct Store<float> {
    static __device__ __forceinline__ void put4(uint8_t *dst, float a, float b, float c, float d) {
        uint2 *p = reinterpret_cast<uint2 *>(dst);
        p[0] = make_uint2(__float_as_uint(a), __float_as_uint(b));
        p[1] = make_uint2(__float_as_uint(c), __float_as_uint(d));
    }
    static __device__ __forceinline__ void get4(const uint8_t *src, float *o) {
        const uint2 *p = reinterpret_cast<const uint2 *>(src);
        uint2 a = p[0], b = p[1];
        o[0] = __uint_as_float(a.x); o[1] = __uint_as_float(a.y);
        o[2] = __uint_as_float(b.x); o[3] = __uint_as_float(b.y);
    }
    static constexpr uint32_t kSignBit = 0x80000000u;
    static constexpr int kPerDword = 1;
};

// XOR mask that flips the signs of the features held by a 16-byte chunk
template <typename T>
__device__ __forceinline__ uint4 chunk_sign_mask(const uint32_t *sign_bits, int chunk) {
    constexpr int per = 16 / sizeof(T);          // features per chunk
    uint32_t m[4] = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < per; ++i) {
        const int f = chunk * per + i;
        const uint32_t s = (sign_bits[f >> 5] >> (f & 31)) & 1u;
        const int dw = i / Store<T>::kPerDword;
        const int sh = (i % Store<T>::kPerDword) * 16;
        m[dw] |= (s * Store<T>::kSignBit) << sh;
    }
    return make_uint4(m[0], m[1], m[2], m[3]);
}

// Features f0 .. f0 + 3 (f0 a multiple of 4) of one row (bytes), with the
// rotation signs applied, as floats.
template <typename T>
__device__ __forceinline__ void get4_signed(const uint8_t *row, const uint32_t *sign_bits, int f0, float *o);
template <>
__device__ __forceinline__ void get4_signed<uint16_t>(const uint8_t *row, const uint32_t *sign_bits, int f0, float *o) {
    uint2 v = *reinterpret_cast<const uint2 *>(row + 2 * f0);
    const uint32_t n = (sign_bits[f0 >> 5] >> (f0 & 31)) & 0xFu;
    v.x ^= ((n & 1u) << 15) | ((n & 2u) << 30);
    v.y ^= ((n & 4u) << 13) | ((n & 8u) << 28);
    o[0] = __uint_as_float(v.x << 16);
    o[1] = __uint_as_float(v.x & 0xFFFF0000u);
    o[2] = __uint_as_float(v.y << 16);
    o[3] = __uint_as_float(v.y & 0xFFFF0000u);
}
template <>
__device__ __forceinline__ void get4_signed<float>(const uint8_t *row, const uint32_t *sign_bits, int f0, float *o) {
    uint4 v = *reinterpret_cast<const uint4 *>(row + 4 * f0);
    const uint32_t n = (sign_bits[f0 >> 5] >> (f0 & 31)) & 0xFu;
    v.x ^= (n & 1u) << 31;
    v.y ^= (n & 2u) << 30;
    v.z ^= (n & 4u) << 29;
    v.w ^= (n & 8u) << 28;
    o[0] = __uint_as_float(v.x);
    o[1] = __uint_as_float(v.y);
    o[2] = __uint_as_float(v.z);
    o[3] = __uint_as_float(v.w);
}

// Stores a, b, c, d as features f0 .. f0 + 3 of one row (bytes), in the
// storage type (bf16 by RNE), with the rotation signs applied.
template <typename T>
__device__ __forceinline__ void put4_signed(uint8_t *row, const uint32_t *sign_bits, int f0, float a, float b,
                                            float c, float d);
template <>
__device__ __forceinline__ void put4_signed<uint16_t>(uint8_t *row, const uint32_t *sign_bits, int f0, float a,
                                                      float b, float c, float d) {
    const uint32_t n = (sign_bits[f0 >> 5] >> (f0 & 31)) & 0xFu;
    uint2 v;
    v.x = ((uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16)) ^ (((n & 1u) << 15) | ((n & 2u) << 30));
    v.y = ((uint32_t)f32_to_bf16(c) | ((uint32_t)f32_to_bf16(d) << 16)) ^ (((n & 4u) << 13) | ((n & 8u) << 28));
    *reinterpret_cast<uint2 *>(row + 2 * f0) = v;
}
template <>
__device__ __forceinline__ void put4_signed<float>(uint8_t *row, const uint32_t *sign_bits, int f0, float a, float b,
                                                   float c, float d) {
    const uint32_t n = (sign_bits[f0 >> 5] >> (f0 & 31)) & 0xFu;
    uint4 v = make_uint4(__float_as_uint(a) ^ ((n & 1u) << 31), __float_as_uint(b) ^ ((n & 2u) << 30),
                         __float_as_uint(c) ^ ((n & 4u) << 29), __float_as_uint(d) ^ ((n & 8u) << 28));
    *reinterpret_cast<uint4 *>(row + 4 * f0) = v;
}

// ------------------------------------------------------------------ X^ via MFMA
// acc[mf] += sum_k wt[f][k] * ut[t][k], f = 32 mf + row, t = token of the lane;
// for bf16, wt is the hi plane and wlo (same layout) the lo plane of W~.  The
// lane's fragments of its U~_t row (global memory) are loaded KB at a time, all
// in flight before the MFMAs that use them.
template <typename T>
__device__ __forceinline__ typename Elem<T>::Frag frag_or_zero(const T *p, bool ok);
template <>
__device__ __forceinline__ FragBF16 frag_or_zero<uint16_t>(const uint16_t *p, bool ok) {
    uint4 raw = *reinterpret_cast<const uint4 *>(p);
    if (!ok) raw = make_uint4(0, 0, 0, 0);
    FragBF16 f;
    f.v = __builtin_bit_cast(bf16x8, raw);
    return f;
}
template <>
__device__ __forceinline__ FragF32 frag_or_zero<float>(const float *p, bool ok) {
    FragF32 f = load_frag(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) f.v[i] = ok ? f.v[i] : 0.f;
    return f;
}

template <typename T, int NMF>
__device__ __forceinline__ void xhat_mfma(const T *wt, const T *wlo, int rtp, const T *ut, int rt, int tok, bool tv,
                                          int lane, f32x16 *acc) {
    const int ln = lane & 31, h = lane >> 5;
    const bool vec = (rt & 7) == 0;        // rows of U~_t are 16-byte aligned
    constexpr int KB = sizeof(T) == 2 ? 8 : 4;
    const T *urow = ut + (size_t)(tv ? tok : 0) * rt;
    for (int k0b = 0; k0b < rt; k0b += 16 * KB) {
        typename Elem<T>::Frag b[KB];
#pragma unroll
        for (int q = 0; q < KB; ++q) {
            const int kk = k0b + 16 * q + 8 * h;
            const bool ok = tv && kk < rt;
            // in-bounds address (rt >= 8 whenever vec and the loop runs), zero where !ok
            b[q] = vec ? frag_or_zero(urow + min(kk, rt - 8), ok)
                       : (ok ? load_frag_n(urow + kk, rt - kk) : zero_frag(ut));
        }
#pragma unroll
        for (int q = 0; q < KB; ++q) {
            const int kk = k0b + 16 * q + 8 * h;
            if (k0b + 16 * q >= rt) break;
#pragma unroll
            for (int mf = 0; mf < NMF; ++mf) {
                typename Elem<T>::Frag a = load_frag(wt + (size_t)(32 * mf + ln) * rtp + kk);
                mfma(a, b[q], acc[mf]);
                if constexpr (sizeof(T) == 2) {
                    typename Elem<T>::Frag al = load_frag(wlo + (size_t)(32 * mf + ln) * rtp + kk);
                    mfma(al, b[q], acc[mf]);
                }
            }
        }
    }
}

// W~ of one (layer, head) as the X^ MFMA reads it: straight from global memory,
// or (WL) staged once per workgroup into dynamic LDS as [planes][D][rtp + 16 B],
// the workgroup's waves all reading that copy.  Every thread of the workgroup
// must call this (the LDS variant ends with a barrier).
template <typename T>
struct WtView {
    const T *hi, *lo;
    int pitch;
};
template <typename T, int D, int NW, bool WL>
__device__ __forceinline__ WtView<T> wt_view(const CodecItem &it, int lh) {
    const T *g = reinterpret_cast<const T *>(it.wt);
    WtView<T> v;
    if constexpr (!WL) {
        v.hi = g + (size_t)lh * D * it.rtp;
        v.lo = g + ((size_t)it.LH + lh) * D * it.rtp;
        v.pitch = it.rtp;
    } else {
        extern __shared__ __attribute__((aligned(16))) uint8_t wt_lds[];
        constexpr int PER = 16 / sizeof(T), PLANES = sizeof(T) == 2 ? 2 : 1;
        T *w = reinterpret_cast<T *>(wt_lds);
        const int WP = it.rtp + PER, ppr = it.rtp / PER, total = PLANES * D * ppr;
        // batches of KB 16-byte pieces per thread, all loads of a batch in flight
        // before its stores (pieces past the end load piece 0 and are not stored)
        constexpr int KB = 8;
        for (int p0 = threadIdx.x; p0 < total; p0 += 64 * NW * KB) {
            uint4 x[KB];
#pragma unroll
            for (int b = 0; b < KB; ++b) {
                const int p = p0 + 64 * NW * b, q = p < total ? p : 0;
                const int pl = q / (D * ppr), rem = q - pl * D * ppr, f = rem / ppr, c = (rem - f * ppr) * PER;
                x[b] = *reinterpret_cast<const uint4 *>(g + ((size_t)(pl * it.LH + lh) * D + f) * it.rtp + c);
            }
#pragma unroll
            for (int b = 0; b < KB; ++b) {
                const int p = p0 + 64 * NW * b;
                if (p >= total) break;
                const int pl = p / (D * ppr), rem = p - pl * D * ppr, f = rem / ppr, c = (rem - f * ppr) * PER;
                *reinterpret_cast<uint4 *>(w + ((size_t)pl * D + f) * WP + c) = x[b];
            }
        }
        __syncthreads();
        v.hi = w;
        v.lo = w + (size_t)D * WP;
        v.pitch = WP;
    }
    return v;
}

template <typename T, int D>
struct Tile {
    static constexpr int RB = D * (int)sizeof(T);   // row bytes
    static constexpr int NMF = D / 32;
};

// ------------------------------------------------------------------ fused encoder
template <typename T, int D, int BITS, int NWV, bool WL>
__global__ __launch_bounds__(64 * NWV) void k_encode(CodecBatch batch) {
    typedef Tile<T, D> TL;
    constexpr int NMF = TL::NMF;
    constexpr int HALF = NMF / 2;
    constexpr int NE = 32 * NMF / 2 * 2 / 2;       // values per lane: 64 (d=128) or 32 (d=64)
    static_assert(NE == 16 * NMF, "layout");
    const Block3 blk = xcd_block();
    const CodecItem &it = batch.it[blk.z];
    const int lh = blk.y;
    if (lh >= it.LH || blk.x * 32 * NWV >= it.T) return;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int ln = lane & 31, h = lane >> 5;
    const int t0 = blk.x * 32 * NWV + wave * 32;
    const int tok = t0 + ln;
    const bool tv = tok < it.T;

    // -(s o x) in the MFMA layout (the lane's features 32 mf + 8 jb + 4 h + c
    // of its token), loaded before the W~ staging so that the load latency
    // overlaps it; an invalid token reads row 0 and stores nothing.  The X^
    // products (signs folded into wt) accumulate onto it, leaving -(s o r).
    const uint8_t *xrow = reinterpret_cast<const uint8_t *>(it.x) + ((size_t)lh * it.T + (tv ? tok : 0)) * TL::RB;
    f32x16 acc[NMF];
#pragma unroll
    for (int mf = 0; mf < NMF; ++mf)
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) {
            float xv[4];
            get4_signed<T>(xrow, it.sign_bits, 32 * mf + 8 * jb + 4 * h, xv);
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[mf][4 * jb + c] = -xv[c];
        }
    const WtView<T> wv = wt_view<T, D, NWV, WL>(it, lh);
    xhat_mfma<T, NMF>(wv.hi, wv.lo, wv.pitch, reinterpret_cast<const T *>(it.ut), it.rt, tok, tv, lane, acc);
    float r[NMF][16];
#pragma unroll
    for (int mf = 0; mf < NMF; ++mf)
#pragma unroll
        for (int j = 0; j < 16; ++j) r[mf][j] = acc[mf][j];

    // in-register Hadamard stages: feature bits 0, 1, 3, 4 (j bits) and the mf bits
#pragma unroll
    for (int jbit = 1; jbit < 16; jbit <<= 1)
#pragma unroll
        for (int mf = 0; mf < NMF; ++mf)
#pragma unroll
            for (int j = 0; j < 16; ++j)
                if (!(j & jbit)) {
                    const float a = r[mf][j], b = r[mf][j | jbit];
                    r[mf][j] = a + b;
                    r[mf][j | jbit] = a - b;
                }
#pragma unroll
    for (int mbit = 1; mbit < NMF; mbit <<= 1)
#pragma unroll
        for (int mf = 0; mf < NMF; ++mf)
            if (!(mf & mbit))
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const float a = r[mf][j], b = r[mf | mbit][j];
                    r[mf][j] = a + b;
                    r[mf | mbit][j] = a - b;
                }

    // feature bit 2 across lane halves; afterwards the lane half is the top
    // feature bit and y[e] holds in-group element e (+ 32 h for d = 64).  The
    // butterflies so far ran on -r; the negative 1/sqrt(d) restores the sign
    // exactly (negation commutes with every rounding here).
    const float isd = (D == 128) ? -0.08838834764831845f : -0.125f;
    float y[NE];
#pragma unroll
    for (int mp = 0; mp < HALF; ++mp)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            float u = r[mp][j], w = r[mp + HALF][j];
            swap_halves(u, w);
            const int e = (j & 3) + 8 * (j >> 2) + 32 * mp;
            y[e] = (u + w) * isd;
            y[e + 4] = (u - w) * isd;
        }

    // group absmax, bf16 scale, codes
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < NE; ++e) amax = fmaxf(amax, fabsf(y[e]));
    if (D == 64) amax = fmaxf(amax, __shfl_xor(amax, 32));
    constexpr float qmax = (float)((1 << (BITS - 1)) - 1);
    const float s32 = amax / qmax;
    const uint16_t sbits = f32_to_bf16(s32);
    const float scale = bf16_to_f32(sbits);
    const float inv = (scale == 0.f) ? 0.f : 1.0f / scale;
    constexpr float magic = 12582912.0f + (float)(1 << (BITS - 1));
    uint32_t tq[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e) {
        float v = y[e] * inv;
        v = fminf(fmaxf(v, -qmax), qmax);
        tq[e] = __float_as_uint(v + magic);
    }
    constexpr int NW = BITS * NE / 32;
    uint32_t w[NW];
    pack_codes<BITS, NE>(tq, w);
    if (tv) {
        const size_t row = (size_t)lh * it.T + tok;
        const size_t grp = row * (D / 64) + (D == 128 ? h : 0);
        uint8_t *dst = it.codes + grp * 8 * BITS + (D == 64 ? h * 4 * BITS : 0);
        if constexpr (NW % 2 == 0) {
#pragma unroll
            for (int k = 0; k < NW; k += 2) *reinterpret_cast<uint2 *>(dst + 4 * k) = make_uint2(w[k], w[k + 1]);
        } else {
#pragma unroll
            for (int k = 0; k < NW; ++k) *reinterpret_cast<uint32_t *>(dst + 4 * k) = w[k];
        }
        if (D == 128 || h == 0) it.scales[grp] = sbits;
    }
}

// ------------------------------------------------------------------ fused decoder
template <typename T, int D, int BITS, int NWV, bool WL>
__global__ __launch_bounds__(64 * NWV) void k_decode(CodecBatch batch) {
    typedef Tile<T, D> TL;
    constexpr int NMF = TL::NMF;
    constexpr int HALF = NMF / 2;
    constexpr int NE = 16 * NMF;
    const Block3 blk = xcd_block();
    const CodecItem &it = batch.it[blk.z];
    const int lh = blk.y;
    if (lh >= it.LH || blk.x * 32 * NWV >= it.T) return;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int ln = lane & 31, h = lane >> 5;
    const int t0 = blk.x * 32 * NWV + wave * 32;
    const int tok = t0 + ln;
    const bool tv = tok < it.T;

    // the lane's codes and scale first, so that their loads overlap the W~
    // staging and the X^ products
    constexpr int NCW = BITS > 0 ? BITS * NE / 32 : 1;
    uint32_t w[NCW];
    uint16_t sbits = 0;
    if constexpr (BITS > 0) {
        const size_t row = (size_t)lh * it.T + (tv ? tok : 0);
        const size_t grp = row * (D / 64) + (D == 128 ? h : 0);
        const uint8_t *src = it.codes + grp * 8 * BITS + (D == 64 ? h * 4 * BITS : 0);
        if constexpr (NCW % 2 == 0) {
#pragma unroll
            for (int k = 0; k < NCW; k += 2) {
                uint2 v = *reinterpret_cast<const uint2 *>(src + 4 * k);
                w[k] = v.x; w[k + 1] = v.y;
            }
        } else {
#pragma unroll
            for (int k = 0; k < NCW; ++k) w[k] = *reinterpret_cast<const uint32_t *>(src + 4 * k);
        }
        sbits = it.scales[grp];
    }

    const WtView<T> wv = wt_view<T, D, NWV, WL>(it, lh);

    // rotated-back residual first, straight into the accumulators of the X^
    // products (the MFMA layout), so that it and the products are never live
    // at the same time
    f32x16 acc[NMF];
    if constexpr (BITS > 0) {
        // codes of the lane's group (or half group) -> scaled values
        const float isd = (D == 128) ? 0.08838834764831845f : 0.125f;
        const float sc = bf16_to_f32(sbits) * isd;
        const float off = (float)(1 << (BITS - 1));
        float y[NE];
        unpack_codes<BITS, NE>(w, y);
#pragma unroll
        for (int e = 0; e < NE; ++e) y[e] = fmaf(y[e], sc, -off * sc);
        // back to the register pairs of the swap stage: y[e], e = (j&3) + 4 sd + 8 (j>>2) + 32 mp
        // in-register stages over the in-group bits (incl. feature bit 2 = sd)
#pragma unroll
        for (int bit = 1; bit < NE; bit <<= 1)
#pragma unroll
            for (int e = 0; e < NE; ++e)
                if (!(e & bit)) {
                    const float a = y[e], b = y[e | bit];
                    y[e] = a + b;
                    y[e | bit] = a - b;
                }
        // top feature bit across lane halves; lane half becomes feature bit 2 again
#pragma unroll
        for (int mp = 0; mp < HALF; ++mp)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int e = (j & 3) + 8 * (j >> 2) + 32 * mp;
                float u = y[e], v = y[e + 4];
                swap_halves(u, v);
                acc[mp][j] = u + v;
                acc[mp + HALF][j] = u - v;
            }
    } else {
#pragma unroll
        for (int mf = 0; mf < NMF; ++mf) acc[mf] = f32x16{};
    }
    // s o X~ = rotated-back residual + s o X^
    xhat_mfma<T, NMF>(wv.hi, wv.lo, wv.pitch, reinterpret_cast<const T *>(it.ut), it.rt, tok, tv, lane, acc);

    // stored from the MFMA layout (the lane's features 32 mf + 8 jb + 4 h + c
    // of its token) with the signs
    if (tv) {
        uint8_t *orow = reinterpret_cast<uint8_t *>(it.out) + ((size_t)lh * it.T + tok) * TL::RB;
#pragma unroll
        for (int mf = 0; mf < NMF; ++mf)
#pragma unroll
            for (int jb = 0; jb < 4; ++jb) {
                const int j = 4 * jb;
                put4_signed<T>(orow, it.sign_bits, 32 * mf + 8 * jb + 4 * h, acc[mf][j], acc[mf][j + 1],
                               acc[mf][j + 2], acc[mf][j + 3]);
            }
    }
}

// ------------------------------------------------------------------ W~ construction
// wt[lh][f][k] = s_f * sum_j core[lh][k][j] * uf[f][j] for k < rt, 0 for rt <= k < rtp;
// bf16: hi plane round(v) and, LH D rtp elements further, lo plane round(v - hi).
// One wave per (32 features, 32 ranks) tile: D[m = f][n = k] with K = j.
template <typename T>
__global__ __launch_bounds__(64) void k_build_wt(WtBatch batch, int D) {
    const Block3 blk = xcd_block();
    const WtItem &it = batch.it[blk.z];
    const int lh = blk.y;
    const int f0 = (blk.x % (D / 32)) * 32, k0 = (blk.x / (D / 32)) * 32;
    if (lh >= it.LH || k0 >= it.rtp) return;
    const int lane = threadIdx.x, ln = lane & 31, h = lane >> 5;
    const T *uf = reinterpret_cast<const T *>(it.uf);
    const T *core = reinterpret_cast<const T *>(it.core) + (size_t)lh * it.rt * it.rf;
    f32x16 acc = f32x16{};
    const int kr = k0 + ln;
    const T *ua = uf + (size_t)(f0 + ln) * it.rf;
    const T *cb = core + (size_t)(kr < it.rt ? kr : 0) * it.rf;
    if (it.rf % 16 == 0) {
        // whole fragments: 16-byte loads, all of a row's fragments in flight together
        for (int j0 = 0; j0 < it.rf; j0 += 64) {
            typename Elem<T>::Frag a[4], b[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int jj = j0 + 16 * u + 8 * h;
                if (jj < it.rf) {
                    a[u] = load_frag(ua + jj);
                    b[u] = load_frag(cb + jj);
                }
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (j0 + 16 * u < it.rf) mfma(a[u], kr < it.rt ? b[u] : zero_frag(core), acc);
        }
    } else {
        for (int j0 = 0; j0 < it.rf; j0 += 16) {
            const int jj = j0 + 8 * h;
            typename Elem<T>::Frag a = load_frag_n(ua + jj, it.rf - jj);
            typename Elem<T>::Frag b = (kr < it.rt) ? load_frag_n(cb + jj, it.rf - jj) : zero_frag(core);
            mfma(a, b, acc);
        }
    }
    T *wt = reinterpret_cast<T *>(it.wt) + (size_t)lh * D * it.rtp;
    if (kr < it.rtp) {
#pragma unroll
        for (int jr = 0; jr < 16; ++jr) {
            const int f = f0 + frag_row(lane, jr);
            const bool neg = (it.sign_bits[f >> 5] >> (f & 31)) & 1u;
            float v = (kr < it.rt) ? acc[jr] : 0.f;
            if (sizeof(T) == 2) {
                uint16_t b = f32_to_bf16(v);
                uint16_t bl = f32_to_bf16(v - bf16_to_f32(b));
                if (neg) {
                    b ^= 0x8000u;
                    bl ^= 0x8000u;
                }
                reinterpret_cast<uint16_t *>(wt)[(size_t)f * it.rtp + kr] = b;
                reinterpret_cast<uint16_t *>(wt)[((size_t)it.LH * D + f) * it.rtp + kr] = bl;
            } else {
                reinterpret_cast<float *>(wt)[(size_t)f * it.rtp + kr] = neg ? -v : v;
            }
        }
    }
}

// ------------------------------------------------------------------ test-hook kernels
// One thread per row: plain Hadamard butterflies.
__global__ void k_rotate_rows(const float *in, float *out, int64_t rows, int d, uint32_t s0, uint32_t s1,
                              uint32_t s2, uint32_t s3, int inverse) {
    const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= rows) return;
    const uint32_t sb[4] = {s0, s1, s2, s3};
    float v[128];
    for (int f = 0; f < d; ++f) {
        const float x = in[r * d + f];
        const bool neg = (sb[f >> 5] >> (f & 31)) & 1u;
        v[f] = (!inverse && neg) ? -x : x;
    }
    for (int hs = 1; hs < d; hs <<= 1)
        for (int i = 0; i < d; ++i)
            if (!(i & hs)) {
                const float a = v[i], b = v[i | hs];
                v[i] = a + b;
                v[i | hs] = a - b;
            }
    const float isd = 1.0f / sqrtf((float)d);
    for (int f = 0; f < d; ++f) {
        const bool neg = (sb[f >> 5] >> (f & 31)) & 1u;
        const float x = v[f] * isd;
        out[r * d + f] = (inverse && neg) ? -x : x;
    }
}

// One thread per 64-group: the quantizer definition step by step.
__global__ void k_quant_pack_groups(const float *x, int64_t groups, int bits, uint8_t *codes, uint16_t *scales) {
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= groups) return;
    const float *p = x + g * 64;
    float amax = 0.f;
    for (int j = 0; j < 64; ++j) amax = fmaxf(amax, fabsf(p[j]));
    const float qmax = (float)((1 << (bits - 1)) - 1);
    const float s32 = amax / qmax;
    const uint16_t sb = f32_to_bf16(s32);
    const float scale = bf16_to_f32(sb);
    const float inv = 1.0f / scale;
    uint64_t st[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int j = 0; j < 64; ++j) {
        float q = 0.f;
        if (scale != 0.f) {
            const float yv = p[j] * inv;
            q = fminf(fmaxf(rintf(yv), -qmax), qmax);
        }
        const uint64_t u = (uint64_t)((int)q + (1 << (bits - 1)));
        const int pos = bits * j;
        st[pos >> 6] |= u << (pos & 63);
        if ((pos & 63) + bits > 64) st[(pos >> 6) + 1] |= u >> (64 - (pos & 63));
    }
    uint64_t *dst = reinterpret_cast<uint64_t *>(codes + g * 8 * bits);
    for (int k = 0; k < bits; ++k) dst[k] = st[k];
    scales[g] = sb;
}

__global__ void k_unpack_dequant_groups(const uint8_t *codes, const uint16_t *scales, int64_t groups, int bits,
                                        float *out) {
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= groups) return;
    const uint64_t *src = reinterpret_cast<const uint64_t *>(codes + g * 8 * bits);
    uint64_t st[9];
    for (int k = 0; k < bits; ++k) st[k] = src[k];
    st[bits] = 0;
    const float scale = bf16_to_f32(scales[g]);
    for (int j = 0; j < 64; ++j) {
        const int pos = bits * j;
        uint64_t v = st[pos >> 6] >> (pos & 63);
        if ((pos & 63) + bits > 64) v |= st[(pos >> 6) + 1] << (64 - (pos & 63));
        const int u = (int)(v & ((1u << bits) - 1u));
        out[g * 64 + j] = (float)(u - (1 << (bits - 1))) * scale;
    }
}

__global__ void k_rademacher_fill(uint64_t key, uint32_t stream, uint64_t first, int64_t count, float *out) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= count) return;
    out[i] = rademacher(key, stream, first + (uint64_t)i);
}

// ------------------------------------------------------------------ launchers
// Workgroups of NW waves x 32 tokens of one (layer, head).  bf16: 8 waves; fp32:
// 4.  W~ goes through LDS when it fits: 68 KiB for d = 128, r_tp = 128
// bf16 (hi + lo planes), so two workgroups share a CU.
template <typename T, int D>
struct CodecShape {
    static constexpr int NW = sizeof(T) == 2 ? 8 : 4;
    static size_t wt_lds(int maxRtp) {
        return (size_t)(sizeof(T) == 2 ? 2 : 1) * D * (maxRtp + 16 / sizeof(T)) * sizeof(T);
    }
    // W~ staged in LDS when it fits (the kernels use no other LDS)
    static bool wl(int maxRtp) { return wt_lds(maxRtp) <= 160 * 1024; }
};

template <void (*K)(CodecBatch)>
static hipError_t codec_launch(dim3 grid, int threads, size_t lds, hipStream_t s, const CodecBatch &b) {
    const auto k = K;
    if (lds > 64 * 1024) {
        // raised once per kernel (one instantiation, and so one static, per kernel)
        static hipError_t state = hipErrorNotReady;
        if (state == hipErrorNotReady) {
            hipFuncAttributes fa;
            hipError_t e = hipFuncGetAttributes(&fa, reinterpret_cast<const void *>(k));
            if (e == hipSuccess)
                e = hipFuncSetAttribute(reinterpret_cast<const void *>(k), hipFuncAttributeMaxDynamicSharedMemorySize,
                                        160 * 1024 - (int)fa.sharedSizeBytes);
            state = e;
        }
        if (state != hipSuccess) return state;
    }
    hipLaunchKernelGGL(k, grid, dim3(threads), lds, s, b);
    return hipGetLastError();
}

template <typename T, int D, int BITS>
static hipError_t encode_one(const CodecBatch &b, int maxT, int maxLH, int maxRtp, hipStream_t s) {
    using CS = CodecShape<T, D>;
    dim3 grid((maxT + 32 * CS::NW - 1) / (32 * CS::NW), maxLH, b.n);
    if (CS::wl(maxRtp)) return codec_launch<k_encode<T, D, BITS, CS::NW, true>>(grid, 64 * CS::NW, CS::wt_lds(maxRtp), s, b);
    return codec_launch<k_encode<T, D, BITS, CS::NW, false>>(grid, 64 * CS::NW, 0, s, b);
}
template <typename T, int D, int BITS>
static hipError_t decode_one(const CodecBatch &b, int maxT, int maxLH, int maxRtp, hipStream_t s) {
    using CS = CodecShape<T, D>;
    dim3 grid((maxT + 32 * CS::NW - 1) / (32 * CS::NW), maxLH, b.n);
    if (CS::wl(maxRtp)) return codec_launch<k_decode<T, D, BITS, CS::NW, true>>(grid, 64 * CS::NW, CS::wt_lds(maxRtp), s, b);
    return codec_launch<k_decode<T, D, BITS, CS::NW, false>>(grid, 64 * CS::NW, 0, s, b);
}

template <typename T, int D>
static hipError_t encode_bits(const CodecBatch &b, int bits, int maxT, int maxLH, int maxRtp, hipStream_t s) {
    switch (bits) {
        case 2: return encode_one<T, D, 2>(b, maxT, maxLH, maxRtp, s);
        case 3: return encode_one<T, D, 3>(b, maxT, maxLH, maxRtp, s);
        case 4: return encode_one<T, D, 4>(b, maxT, maxLH, maxRtp, s);
        case 5: return encode_one<T, D, 5>(b, maxT, maxLH, maxRtp, s);
        case 6: return encode_one<T, D, 6>(b, maxT, maxLH, maxRtp, s);
        case 7: return encode_one<T, D, 7>(b, maxT, maxLH, maxRtp, s);
        case 8: return encode_one<T, D, 8>(b, maxT, maxLH, maxRtp, s);
        default: return hipErrorInvalidValue;
    }
}
template <typename T, int D>
static hipError_t decode_bits(const CodecBatch &b, int bits, int maxT, int maxLH, int maxRtp, hipStream_t s) {
    switch (bits) {
        case 0: return decode_one<T, D, 0>(b, maxT, maxLH, maxRtp, s);
        case 2: return decode_one<T, D, 2>(b, maxT, maxLH, maxRtp, s);
        case 3: return decode_one<T, D, 3>(b, maxT, maxLH, maxRtp, s);
        case 4: return decode_one<T, D, 4>(b, maxT, maxLH, maxRtp, s);
        case 5: return decode_one<T, D, 5>(b, maxT, maxLH, maxRtp, s);
        case 6: return decode_one<T, D, 6>(b, maxT, maxLH, maxRtp, s);
        case 7: return decode_one<T, D, 7>(b, maxT, maxLH, maxRtp, s);
        case 8: return decode_one<T, D, 8>(b, maxT, maxLH, maxRtp, s);
        default: return hipErrorInvalidValue;
    }
}

static int max_rtp(const CodecBatch &b) {
    int m = 0;
    for (int i = 0; i < b.n; ++i) m = std::max(m, b.it[i].rtp);
    return m;
}

hipError_t launch_encode(const CodecBatch &b, int dtype, int D, int bits, int maxT, int maxLH, hipStream_t s) {
    if (b.n <= 0) return hipSuccess;
    KTimeScope kts("k_encode", s);
    const int r = max_rtp(b);
    if (dtype == JOLT_BF16)
        return D == 128 ? encode_bits<uint16_t, 128>(b, bits, maxT, maxLH, r, s)
                        : encode_bits<uint16_t, 64>(b, bits, maxT, maxLH, r, s);
    return D == 128 ? encode_bits<float, 128>(b, bits, maxT, maxLH, r, s)
                    : encode_bits<float, 64>(b, bits, maxT, maxLH, r, s);
}
hipError_t launch_decode(const CodecBatch &b, int dtype, int D, int bits, int maxT, int maxLH, hipStream_t s) {
    if (b.n <= 0) return hipSuccess;
    KTimeScope kts("k_decode", s);
    const int r = max_rtp(b);
    if (dtype == JOLT_BF16)
        return D == 128 ? decode_bits<uint16_t, 128>(b, bits, maxT, maxLH, r, s)
                        : decode_bits<uint16_t, 64>(b, bits, maxT, maxLH, r, s);
    return D == 128 ? decode_bits<float, 128>(b, bits, maxT, maxLH, r, s)
                    : decode_bits<float, 64>(b, bits, maxT, maxLH, r, s);
}
hipError_t launch_build_wt(const WtBatch &b, int dtype, int D, int maxLH, int maxRtp, hipStream_t s) {
    if (b.n <= 0 || maxRtp <= 0) return hipSuccess;
    KTimeScope kts("k_build_wt", s);
    dim3 grid((D / 32) * ((maxRtp + 31) / 32), maxLH, b.n);
    if (dtype == JOLT_BF16) hipLaunchKernelGGL(k_build_wt<uint16_t>, grid, dim3(64), 0, s, b, D);
    else hipLaunchKernelGGL(k_build_wt<float>, grid, dim3(64), 0, s, b, D);
    return hipGetLastError();
}
hipError_t launch_rotate(const float *in, float *out, int64_t rows, int d, const uint32_t *sb, int inverse,
                         hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_rotate_rows, dim3((unsigned)((rows + 127) / 128)), dim3(128), 0, s, in, out, rows, d,
                       sb[0], sb[1], sb[2], sb[3], inverse);
    return hipGetLastError();
}
hipError_t launch_quantize_pack(const float *rot, int64_t rows, int d, int bits, uint8_t *codes, uint16_t *scales,
                                hipStream_t s) {
    const int64_t groups = rows * d / 64;
    if (groups <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_quant_pack_groups, dim3((unsigned)((groups + 127) / 128)), dim3(128), 0, s, rot, groups,
                       bits, codes, scales);
    return hipGetLastError();
}
hipError_t launch_unpack_dequant(const uint8_t *codes, const uint16_t *scales, int64_t rows, int d, int bits,
                                 float *out, hipStream_t s) {
    const int64_t groups = rows * d / 64;
    if (groups <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_unpack_dequant_groups, dim3((unsigned)((groups + 127) / 128)), dim3(128), 0, s, codes,
                       scales, groups, bits, out);
    return hipGetLastError();
}
hipError_t launch_rademacher(uint64_t key, uint32_t stream, uint64_t first, int64_t count, float *out,
                             hipStream_t s) {
    if (count <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_rademacher_fill, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, s, key, stream,
                       first, count, out);
    return hipGetLastError();
}

}  // namespace jolt
