// Decode attention over the stored factors of a compressed layer group (the
// method's decode kernel evaluates attention directly over the stored factors,
// without forming the dense K and V: "A JoLT for the KV cache", paper landing
// page, abstract).
//
// For a query q of query head j on KV head h = j / G of layer l, with the K
// item's stored U_t, U_f, core C and rotated residual codes:
//   k_t = U_t[t] (C_lh U_f^T) + s o (1/sqrt d) H r'_t,   r'_t = dequant(codes_t)
//   scale (q . k_t) = U_t[t] . z + q' . r'_t,  z = scale C_lh (U_f^T q),
//                                             q' = scale (1/sqrt d) H (s o q)
// (H is symmetric), so a score costs r_t + d products on the stored data.  For
// the V item, with weights p_t of the softmax,
//   sum_t p_t v_t = (sum_t p_t U_t[t]) C_lh U_f^T + s o (1/sqrt d) H sum_t p_t r'_t,
// so the values are accumulated as an r_t-vector and a d-vector in the
// factor and rotated domains, and mapped to features once per head.
//
// Three launches: k_att_prep (z and q' per query head), k_att_split (a
// workgroup per (token range, layer-head, group): scores, softmax in chunks of
// 256 tokens with a running maximum, the two value accumulators), and
// k_att_combine (merges the ranges: max, rescaled sums; applies C U_f^T and the
// inverse rotation; divides; writes o and the log-sum-exp).
#include <float.h>

#include <algorithm>

#include "dev_common.h"
#include "attn.h"
#include "ktimer.h"

namespace jolt {

namespace {

constexpr int kChunk = 256;           // tokens per softmax chunk (one per thread)
constexpr int kSplitThreads = 256;

template <typename T> __device__ __forceinline__ float ld_param(const T *p, size_t i);
template <> __device__ __forceinline__ float ld_param<uint16_t>(const uint16_t *p, size_t i) {
    return bf16_to_f32(p[i]);
}
template <> __device__ __forceinline__ float ld_param<float>(const float *p, size_t i) { return p[i]; }

__device__ __forceinline__ bool sign_neg(const uint32_t *sb, int f) { return (sb[f >> 5] >> (f & 31)) & 1u; }

// (H x)[f] for the Sylvester Hadamard matrix, H[f][i] = (-1)^popcount(f & i)
__device__ __forceinline__ float hadamard_row(const float *x, int d, int f) {
    float acc = 0.f;
    for (int i = 0; i < d; ++i) acc += (__popc(f & i) & 1) ? -x[i] : x[i];
    return acc;
}

// q - 2^(b-1) of element j of group `grp` (b-bit little-endian stream)
__device__ __forceinline__ float code_q(const uint8_t *codes, size_t grp, int j, int bits) {
    const uint32_t *w = reinterpret_cast<const uint32_t *>(codes + grp * 8 * (size_t)bits);
    const int pos = bits * j, wi = pos >> 5, sh = pos & 31;
    uint32_t v = w[wi] >> sh;
    if (sh + bits > 32) v |= w[wi + 1] << (32 - sh);
    return (float)(int)(v & ((1u << bits) - 1u)) - (float)(1 << (bits - 1));
}

}  // namespace

// ---------------------------------------------------------------- prep
// One workgroup of d threads per (query head, layer, group): z (rt_K, padded
// with zeros to rtp_K) and q' (d), scaled, into the workspace.
template <typename T>
__global__ __launch_bounds__(128) void k_att_prep(AttnBatch batch) {
    const AttnGroup &g = batch.it[blockIdx.y];
    const int lq = blockIdx.x, l = lq / batch.hq, j = lq % batch.hq;
    if (l >= g.L) return;
    const int d = g.d, f = threadIdx.x, h = j / (batch.hq / g.H), lh = l * g.H + h;
    __shared__ float qs[128], u[128];
    const float *q = g.q + ((size_t)l * batch.hq + j) * d;
    float *z = g.ws_prep + ((size_t)l * batch.hq + j) * (g.rtpk + d);
    float *qr = z + g.rtpk;
    if (f < d) qs[f] = q[f];
    __syncthreads();
    if (g.bk > 0 && f < d) {
        float acc = 0.f;
        for (int i = 0; i < d; ++i) {
            const float x = sign_neg(g.sk, i) ? -qs[i] : qs[i];
            acc += (__popc(f & i) & 1) ? -x : x;
        }
        qr[f] = batch.scale * g.isd * acc;
    }
    const T *uf = reinterpret_cast<const T *>(g.uf_k), *core = reinterpret_cast<const T *>(g.core_k);
    if (f < g.rfk) {
        float acc = 0.f;
        for (int i = 0; i < d; ++i) acc = fmaf(ld_param(uf, (size_t)i * g.rfk + f), qs[i], acc);
        u[f] = acc;
    }
    __syncthreads();
    for (int r = f; r < g.rtpk; r += blockDim.x) {
        float acc = 0.f;
        if (r < g.rtk)
            for (int c = 0; c < g.rfk; ++c) acc = fmaf(ld_param(core, ((size_t)lh * g.rtk + r) * g.rfk + c), u[c], acc);
        z[r] = batch.scale * acc;
    }
}

// ---------------------------------------------------------------- split
// One workgroup per (token range, layer-head, group), kSplitThreads threads;
// the range is walked in chunks of 256 tokens.  Per chunk, thread t scores
// token t for the G query heads of this KV head; the chunk's weights go through
// LDS to the value accumulators (thread r: sum_t p U_t^V[t][r]; thread f < d:
// sum_t p r'^V_t[f]), which are rescaled whenever the running maximum grows.
template <typename T, int G>
__global__ __launch_bounds__(kSplitThreads) void k_att_split(AttnBatch batch) {
    const AttnGroup &g = batch.it[blockIdx.z];
    const int lh = blockIdx.y, split = blockIdx.x;
    if (lh >= g.L * g.H || split >= g.splits) return;
    const int l = lh / g.H, h = lh % g.H, d = g.d, tid = threadIdx.x;
    extern __shared__ float sm[];
    float *zs = sm;                                   // [G][rtpk]
    float *qs = zs + G * g.rtpk;                      // [G][d]
    float *ps = qs + G * d;                           // [G][kChunk]
    __shared__ float red[G][kSplitThreads / 64];
    __shared__ float cmax[G];
    for (int e = tid; e < G * (g.rtpk + d); e += kSplitThreads) {
        const int gg = e / (g.rtpk + d), r = e - gg * (g.rtpk + d);
        const float *src = g.ws_prep + ((size_t)l * batch.hq + h * G + gg) * (g.rtpk + d);
        if (r < g.rtpk) zs[gg * g.rtpk + r] = src[r];
        else qs[gg * d + (r - g.rtpk)] = src[r];
    }
    const T *utk = reinterpret_cast<const T *>(g.ut_k), *utv = reinterpret_cast<const T *>(g.ut_v);
    const int per = g.per_split, tb = split * per, te = min(g.T, tb + per);
    float m_run[G], l_run[G], av[G], bv[G];
#pragma unroll
    for (int gg = 0; gg < G; ++gg) {
        m_run[gg] = -FLT_MAX;
        l_run[gg] = 0.f;
        av[gg] = 0.f;
        bv[gg] = 0.f;
    }
    const int lane = tid & 63, wid = tid >> 6;
    for (int c0 = tb; c0 < te; c0 += kChunk) {
        __syncthreads();                              // previous chunk's weights consumed
        const int t = c0 + tid;
        const bool tv = t < te;
        float s[G];
#pragma unroll
        for (int gg = 0; gg < G; ++gg) s[gg] = 0.f;
        if (tv) {
            const size_t row = (size_t)t;
            for (int r = 0; r < g.rtk; ++r) {
                const float uv = ld_param(utk, row * g.rtk + r);
#pragma unroll
                for (int gg = 0; gg < G; ++gg) s[gg] = fmaf(uv, zs[gg * g.rtpk + r], s[gg]);
            }
            if (g.bk > 0) {
                const size_t grow = ((size_t)lh * g.T + t) * (d / 64);
                for (int gi = 0; gi < d / 64; ++gi) {
                    const float sc = bf16_to_f32(g.scales_k[grow + gi]);
                    for (int jj = 0; jj < 64; ++jj) {
                        const float v = code_q(g.codes_k, grow + gi, jj, g.bk) * sc;
#pragma unroll
                        for (int gg = 0; gg < G; ++gg) s[gg] = fmaf(v, qs[gg * d + gi * 64 + jj], s[gg]);
                    }
                }
            }
        }
        // chunk maximum per head
#pragma unroll
        for (int gg = 0; gg < G; ++gg) {
            const float w = wave_max(tv ? s[gg] : -FLT_MAX);
            if (lane == 0) red[gg][wid] = w;
        }
        __syncthreads();
        if (tid < G) {
            float m = red[tid][0];
            for (int w = 1; w < kSplitThreads / 64; ++w) m = fmaxf(m, red[tid][w]);
            cmax[tid] = m;
        }
        __syncthreads();
#pragma unroll
        for (int gg = 0; gg < G; ++gg) {
            const float mn = fmaxf(m_run[gg], cmax[gg]);
            const float alpha = __expf(m_run[gg] - mn);       // 0 on the first chunk
            m_run[gg] = mn;
            l_run[gg] *= alpha;
            av[gg] *= alpha;
            bv[gg] *= alpha;
            ps[gg * kChunk + tid] = tv ? __expf(s[gg] - mn) : 0.f;
        }
        __syncthreads();
        // chunk weight sums (every thread keeps the same running sum)
#pragma unroll
        for (int gg = 0; gg < G; ++gg) {
            const float w = wave_sum(ps[gg * kChunk + tid]);
            if (lane == 0) red[gg][wid] = w;
        }
        __syncthreads();
#pragma unroll
        for (int gg = 0; gg < G; ++gg) {
            float sum = 0.f;
            for (int w = 0; w < kSplitThreads / 64; ++w) sum += red[gg][w];
            l_run[gg] += sum;
        }
        const int nt = min(kChunk, te - c0);
        // factor-domain value accumulator: thread r < rt_V
        if (tid < g.rtv) {
            for (int tt = 0; tt < nt; ++tt) {
                const float uv = ld_param(utv, (size_t)(c0 + tt) * g.rtv + tid);
#pragma unroll
                for (int gg = 0; gg < G; ++gg) av[gg] = fmaf(ps[gg * kChunk + tt], uv, av[gg]);
            }
        }
        // rotated-residual value accumulator: thread f < d
        if (g.bv > 0 && tid < d) {
            const int gi = tid >> 6, jj = tid & 63;
            for (int tt = 0; tt < nt; ++tt) {
                const size_t grp = ((size_t)lh * g.T + c0 + tt) * (d / 64) + gi;
                const float v = code_q(g.codes_v, grp, jj, g.bv) * bf16_to_f32(g.scales_v[grp]);
#pragma unroll
                for (int gg = 0; gg < G; ++gg) bv[gg] = fmaf(ps[gg * kChunk + tt], v, bv[gg]);
            }
        }
    }
    // partials of this range: [m, l, a (rtpv), b (d)] per query head
#pragma unroll
    for (int gg = 0; gg < G; ++gg) {
        float *o = g.ws_part + (((size_t)split * g.L + l) * batch.hq + h * G + gg) * (2 + g.rtpv + d);
        if (tid == 0) {
            o[0] = m_run[gg];
            o[1] = l_run[gg];
        }
        if (tid < g.rtpv) o[2 + tid] = tid < g.rtv ? av[gg] : 0.f;
        if (tid < d) o[2 + g.rtpv + tid] = bv[gg];
    }
}

// ---------------------------------------------------------------- combine
// One workgroup of d threads per (query head, layer, group).
template <typename T>
__global__ __launch_bounds__(128) void k_att_combine(AttnBatch batch) {
    const AttnGroup &g = batch.it[blockIdx.y];
    const int lq = blockIdx.x, l = lq / batch.hq, j = lq % batch.hq;
    if (l >= g.L) return;
    const int d = g.d, f = threadIdx.x, h = j / (batch.hq / g.H), lh = l * g.H + h;
    const int stride = 2 + g.rtpv + d;
    __shared__ float a[256], b[128], ac[128];
    __shared__ float s_m, s_l;
    if (f == 0) {
        float m = -FLT_MAX;
        for (int sp = 0; sp < g.splits; ++sp)
            m = fmaxf(m, g.ws_part[(((size_t)sp * g.L + l) * batch.hq + j) * stride]);
        float lsum = 0.f;
        for (int sp = 0; sp < g.splits; ++sp) {
            const float *p = g.ws_part + (((size_t)sp * g.L + l) * batch.hq + j) * stride;
            lsum += __expf(p[0] - m) * p[1];
        }
        s_m = m;
        s_l = lsum;
    }
    __syncthreads();
    const float m = s_m;
    for (int r = f; r < g.rtpv; r += blockDim.x) {
        float acc = 0.f;
        for (int sp = 0; sp < g.splits; ++sp) {
            const float *p = g.ws_part + (((size_t)sp * g.L + l) * batch.hq + j) * stride;
            acc = fmaf(__expf(p[0] - m), p[2 + r], acc);
        }
        a[r] = acc;
    }
    if (f < d) {
        float acc = 0.f;
        for (int sp = 0; sp < g.splits; ++sp) {
            const float *p = g.ws_part + (((size_t)sp * g.L + l) * batch.hq + j) * stride;
            acc = fmaf(__expf(p[0] - m), p[2 + g.rtpv + f], acc);
        }
        b[f] = acc;
    }
    __syncthreads();
    const T *uf = reinterpret_cast<const T *>(g.uf_v), *core = reinterpret_cast<const T *>(g.core_v);
    if (f < g.rfv) {
        float acc = 0.f;
        for (int r = 0; r < g.rtv; ++r) acc = fmaf(a[r], ld_param(core, ((size_t)lh * g.rtv + r) * g.rfv + f), acc);
        ac[f] = acc;
    }
    __syncthreads();
    if (f < d) {
        float o = 0.f;
        for (int c = 0; c < g.rfv; ++c) o = fmaf(ac[c], ld_param(uf, (size_t)f * g.rfv + c), o);
        if (g.bv > 0) {
            const float rv = g.isd * hadamard_row(b, d, f);
            o += sign_neg(g.sv, f) ? -rv : rv;
        }
        const float inv = 1.f / s_l;
        g.out[((size_t)l * batch.hq + j) * d + f] = o * inv;
        if (f == 0) g.lse[(size_t)l * batch.hq + j] = m + __logf(s_l);
    }
}

// ---------------------------------------------------------------- launchers
template <typename T, int G>
static hipError_t split_g(const AttnBatch &b, int maxLH, int maxSplits, size_t lds, hipStream_t s) {
    hipLaunchKernelGGL((k_att_split<T, G>), dim3(maxSplits, maxLH, b.n), dim3(kSplitThreads), lds, s, b);
    return hipGetLastError();
}

template <typename T>
static hipError_t attn_t(const AttnBatch &b, int maxL, int maxLH, int maxSplits, int maxRtpk, int maxD,
                         hipStream_t s) {
    {
        KTimeScope kts("k_att_prep", s);
        hipLaunchKernelGGL(k_att_prep<T>, dim3(maxL * b.hq, b.n), dim3(128), 0, s, b);
        if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    }
    const int G = b.hq / b.it[0].H;
    const size_t lds = ((size_t)G * (maxRtpk + maxD) + (size_t)G * kChunk) * sizeof(float);
    {
        KTimeScope kts("k_att_split", s);
        hipError_t e;
        switch (G) {
            case 1: e = split_g<T, 1>(b, maxLH, maxSplits, lds, s); break;
            case 2: e = split_g<T, 2>(b, maxLH, maxSplits, lds, s); break;
            case 4: e = split_g<T, 4>(b, maxLH, maxSplits, lds, s); break;
            case 8: e = split_g<T, 8>(b, maxLH, maxSplits, lds, s); break;
            default: return hipErrorInvalidValue;
        }
        if (e != hipSuccess) return e;
    }
    KTimeScope kts("k_att_combine", s);
    hipLaunchKernelGGL(k_att_combine<T>, dim3(maxL * b.hq, b.n), dim3(128), 0, s, b);
    return hipGetLastError();
}

hipError_t launch_attention(const AttnBatch &b, int dtype, hipStream_t s) {
    if (b.n <= 0) return hipSuccess;
    int maxL = 0, maxLH = 0, maxSplits = 0, maxRtpk = 0, maxD = 0;
    for (int i = 0; i < b.n; ++i) {
        maxL = std::max(maxL, b.it[i].L);
        maxLH = std::max(maxLH, b.it[i].L * b.it[i].H);
        maxSplits = std::max(maxSplits, b.it[i].splits);
        maxRtpk = std::max(maxRtpk, b.it[i].rtpk);
        maxD = std::max(maxD, b.it[i].d);
    }
    return dtype == JOLT_BF16 ? attn_t<uint16_t>(b, maxL, maxLH, maxSplits, maxRtpk, maxD, s)
                              : attn_t<float>(b, maxL, maxLH, maxSplits, maxRtpk, maxD, s);
}

}  // namespace jolt
