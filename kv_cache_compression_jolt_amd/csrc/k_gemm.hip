// Batched fp32 GEMMs of the planner on fp32 MFMA: a generic one (core
// projection, U_t = Q U~, block-Jacobi rotations) and the symmetric Gram of the
// rows of a panel (CholeskyQR Grams, B B^T).
//
// One workgroup computes a 64 x 64 tile of C (4 waves, 2 x 2 tiles of 32 x 32 on
// v_mfma_f32_32x32x2f32), or a 128 x 128 tile when both M and N exceed 64.  K is staged through LDS 32 deep; the next slice is
// loaded into registers while the current one is multiplied.  Operands are
// addressed by element strides, so transposed views need no copies; loads are
// coalesced along whichever index has stride 1.
#include "bf16_split.h"
#include "dev_common.h"
#include "plan_kernels.h"
#include "ktimer.h"

namespace jolt {

namespace {

constexpr int kKS = 32;        // K slice
constexpr int kPad = 68;       // LDS row stride (64 + 4)

struct Slice {
    float a[8], b[8];
};

__device__ __forceinline__ void load_slice(const GemmItem &it, int i0, int j0, int k0, int ke, int tid, Slice &s) {
    const bool a_kfast = it.a_k == 1, b_jfast = it.b_j == 1;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int e = tid + 256 * q;
        int ii, kk;
        if (a_kfast) { ii = e >> 5; kk = e & 31; } else { ii = e & 63; kk = e >> 6; }
        const int gi = i0 + ii, gk = k0 + kk;
        s.a[q] = (gi < it.M && gk < ke) ? it.a[(int64_t)gi * it.a_i + (int64_t)gk * it.a_k] : 0.f;
        int kb, jj;
        if (b_jfast) { kb = e >> 6; jj = e & 63; } else { kb = e & 31; jj = e >> 5; }
        const int gj = j0 + jj, gk2 = k0 + kb;
        s.b[q] = (gj < it.N && gk2 < ke) ? it.b[(int64_t)gk2 * it.b_k + (int64_t)gj * it.b_j] : 0.f;
    }
}

__device__ __forceinline__ void store_slice(const GemmItem &it, int tid, const Slice &s, float (*As)[kPad],
                                            float (*Bs)[kPad]) {
    const bool a_kfast = it.a_k == 1, b_jfast = it.b_j == 1;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int e = tid + 256 * q;
        int ii, kk;
        if (a_kfast) { ii = e >> 5; kk = e & 31; } else { ii = e & 63; kk = e >> 6; }
        As[kk][ii] = s.a[q];
        int kb, jj;
        if (b_jfast) { kb = e >> 6; jj = e & 63; } else { kb = e & 31; jj = e >> 5; }
        Bs[kb][jj] = s.b[q];
    }
}

}  // namespace

__global__ __launch_bounds__(256) void k_gemm(GemmBatch batch, int maxSplit) {
    __shared__ float As[kKS][kPad];    // As[k][i]
    __shared__ float Bs[kKS][kPad];    // Bs[k][j]
    const int z = blockIdx.z;
    const GemmItem &it0 = batch.it[z % batch.n];
    const int sp = (z / batch.n) % maxSplit, bi = (z / batch.n) / maxSplit;
    const int i0 = blockIdx.y * 64, j0 = blockIdx.x * 64;
    if (sp >= it0.nsplit || bi >= it0.nb || i0 >= it0.M || j0 >= it0.N) return;
    GemmItem it = it0;
    it.a += bi * it0.a_z;
    it.b += bi * it0.b_z;
    it.c += bi * it0.c_z;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wm = wid >> 1, wn = wid & 1;
    const int kb = sp * it.kchunk, ke = min(it.K, kb + it.kchunk);
    f32x16 acc = {};
    Slice cur;
    load_slice(it, i0, j0, kb, ke, tid, cur);
    for (int k0 = kb; k0 < ke; k0 += kKS) {
        __syncthreads();
        store_slice(it, tid, cur, As, Bs);
        __syncthreads();
        if (k0 + kKS < ke) load_slice(it, i0, j0, k0 + kKS, ke, tid, cur);
        const int kh = lane >> 5, mi = wm * 32 + (lane & 31), nj = wn * 32 + (lane & 31);
#pragma unroll
        for (int s = 0; s < kKS / 2; ++s)
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(As[2 * s + kh][mi], Bs[2 * s + kh][nj], acc, 0, 0, 0);
    }
    float *c = it.c + (int64_t)sp * it.c_split;
    const int gj = j0 + wn * 32 + (lane & 31);
    if (gj < it.N)
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
            const int gi = i0 + wm * 32 + frag_row(lane, jj);
            if (gi < it.M) c[(int64_t)gi * it.c_i + (int64_t)gj * it.c_j] = acc[jj];
        }
}

// ---------------------------------------------------------------- 128 x 128 tiles
// The same product for launches whose M and N both exceed 64: a workgroup of 4
// waves computes a 128 x 128 tile of C, each wave a 64 x 64 quarter as 2 x 2
// MFMA tiles, so that every 32-deep K slice staged in LDS feeds 64 MFMAs per
// wave between two barriers (16 for the 64 x 64 tiles), and every operand
// element staged serves twice as many products.
constexpr int kBT = 128, kBPad = 132;

// A thread's 16 elements of each operand's slice, walked with a fixed step so
// that one base pointer and one stride cover them: element q of operand A is
// (i, k) = (i0 + r + q dr, k0 + c + q dc) with (r, c, dr, dc) = (tid / 32,
// tid % 32, 8, 0) when k has unit stride (threads run along k), else (tid %
// 128, tid / 128, 0, 2) (threads run along i); B's (j, k) likewise.
struct Walk {
    int r, c, dr, dc;         // first (row, column) in the slice and the step per element
};
__device__ __forceinline__ Walk walk128(bool cfast, int tid) {
    return cfast ? Walk{tid >> 5, tid & 31, 8, 0} : Walk{tid & 127, tid >> 7, 0, 2};
}

__global__ __launch_bounds__(256) void k_gemm128(GemmBatch batch, int maxSplit) {
    __shared__ float As[kKS][kBPad];    // As[k][i]
    __shared__ float Bs[kKS][kBPad];    // Bs[k][j]
    const int z = blockIdx.z;
    const GemmItem &it0 = batch.it[z % batch.n];
    const int sp = (z / batch.n) % maxSplit, bi = (z / batch.n) / maxSplit;
    const int i0 = blockIdx.y * kBT, j0 = blockIdx.x * kBT;
    if (sp >= it0.nsplit || bi >= it0.nb || i0 >= it0.M || j0 >= it0.N) return;
    const float *A = it0.a + bi * it0.a_z;
    const float *B = it0.b + bi * it0.b_z;
    float *C = it0.c + bi * it0.c_z + (int64_t)sp * it0.c_split;
    const int M = it0.M, N = it0.N;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wm = wid >> 1, wn = wid & 1, kh = lane >> 5, l32 = lane & 31;
    const int kb = sp * it0.kchunk, ke = min(it0.K, kb + it0.kchunk);
    // A walks (r, c) = (i, k) and B walks (r, c) = (j, k); threads run along
    // whichever index has unit stride
    const Walk wa = walk128(it0.a_k == 1, tid), vb = walk128(it0.b_j != 1, tid);
    const int64_t a_step = (int64_t)wa.dr * it0.a_i + (int64_t)wa.dc * it0.a_k;
    const int64_t b_step = (int64_t)vb.dr * it0.b_j + (int64_t)vb.dc * it0.b_k;
    float va[16], vbv[16];
    auto load = [&](int k0) {
        const float *pa = A + (int64_t)(i0 + wa.r) * it0.a_i + (int64_t)(k0 + wa.c) * it0.a_k;
        const float *pb = B + (int64_t)(j0 + vb.r) * it0.b_j + (int64_t)(k0 + vb.c) * it0.b_k;
        if (i0 + kBT <= M && j0 + kBT <= N && k0 + kKS <= ke) {      // an interior slice: no masks
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                va[q] = pa[q * a_step];
                vbv[q] = pb[q * b_step];
            }
            return;
        }
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const bool oka = i0 + wa.r + q * wa.dr < M && k0 + wa.c + q * wa.dc < ke;
            const bool okb = j0 + vb.r + q * vb.dr < N && k0 + vb.c + q * vb.dc < ke;
            const float x = *(oka ? pa + q * a_step : A);
            const float y = *(okb ? pb + q * b_step : B);
            va[q] = oka ? x : 0.f;
            vbv[q] = okb ? y : 0.f;
        }
    };
    f32x16 acc[2][2];
#pragma unroll
    for (int tm = 0; tm < 2; ++tm)
#pragma unroll
        for (int tn = 0; tn < 2; ++tn) acc[tm][tn] = f32x16{};
    load(kb);
    for (int k0 = kb; k0 < ke; k0 += kKS) {
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            As[wa.c + q * wa.dc][wa.r + q * wa.dr] = va[q];
            Bs[vb.c + q * vb.dc][vb.r + q * vb.dr] = vbv[q];
        }
        __syncthreads();
        if (k0 + kKS < ke) load(k0 + kKS);
#pragma unroll
        for (int s = 0; s < kKS / 2; ++s) {
            float a[2], b[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                a[t] = As[2 * s + kh][64 * wm + 32 * t + l32];
                b[t] = Bs[2 * s + kh][64 * wn + 32 * t + l32];
            }
#pragma unroll
            for (int tm = 0; tm < 2; ++tm)
#pragma unroll
                for (int tn = 0; tn < 2; ++tn)
                    acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[tm], b[tn], acc[tm][tn], 0, 0, 0);
        }
    }
#pragma unroll
    for (int tn = 0; tn < 2; ++tn) {
        const int gj = j0 + 64 * wn + 32 * tn + l32;
        if (gj >= N) continue;
#pragma unroll
        for (int tm = 0; tm < 2; ++tm)
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) {
                const int gi = i0 + 64 * wm + 32 * tm + frag_row(lane, jj);
                if (gi < M) C[(int64_t)gi * it0.c_i + (int64_t)gj * it0.c_j] = acc[tm][tn][jj];
            }
    }
}

// ---------------------------------------------------------------- split-operand GEMM
// C = A B as k_gemm128 (128 x 128 tiles, 4 waves of 2 x 2 MFMA tiles, slices of
// kKS), on the bf16 MFMA: every operand value v is split into hi = bf16(v) and
// lo = bf16(v - hi) on its way into LDS, and a tile accumulates hi_a hi_b +
// hi_a lo_b + lo_a hi_b (exact products, fp32 accumulation; the omitted lo lo
// and the split are below 2^-16 of |a b|).  Each operand must have unit stride
// along its row index or along K; its values go to K-contiguous LDS rows.
__global__ __launch_bounds__(256) void k_gemm128_bx3(GemmBatch batch, int maxSplit) {
    constexpr int XP = kKS + 8;                       // bf16 pitch of a tile row (80 B)
    __shared__ __attribute__((aligned(16))) uint16_t Ah[kBT * XP], Al[kBT * XP], Bh[kBT * XP], Bl[kBT * XP];
    const int z = blockIdx.z;
    const GemmItem &it0 = batch.it[z % batch.n];
    const int sp = (z / batch.n) % maxSplit, bi = (z / batch.n) / maxSplit;
    const int i0 = blockIdx.y * kBT, j0 = blockIdx.x * kBT;
    if (sp >= it0.nsplit || bi >= it0.nb || i0 >= it0.M || j0 >= it0.N) return;
    const float *A = it0.a + bi * it0.a_z;
    const float *B = it0.b + bi * it0.b_z;
    float *C = it0.c + bi * it0.c_z + (int64_t)sp * it0.c_split;
    const int M = it0.M, N = it0.N;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wm = wid >> 1, wn = wid & 1, kh = lane >> 5, l32 = lane & 31;
    const int kb = sp * it0.kchunk, ke = min(it0.K, kb + it0.kchunk);
    // An operand with unit stride along K: a thread takes two runs of 8
    // consecutive K of one row (4 lanes per 32 K of a row), each loaded as two
    // 16-byte loads where whole and aligned.  Unit stride along its rows: a
    // thread takes 4 consecutive rows x 4 consecutive K (rows 4 (tid % 32) ..,
    // K 4 (tid / 32) ..), one 16-byte load per K.  Either way the thread
    // stores 16 values, split into hi and lo, as row pieces of the LDS tiles.
    const bool akf = it0.a_k == 1, bkf = it0.b_k == 1;
    float va[16], vb[16];
    auto load_op = [&](const float *X, int64_t s_r, int64_t s_k, bool kf, int r0, int R, int k0, float *v) {
        if (kf) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int gr = r0 + (tid >> 2) + 64 * u, gk0 = k0 + 8 * (tid & 3);
                const float *p = X + (int64_t)(gr < R ? gr : 0) * s_r + gk0;
                if (gr < R && gk0 + 8 <= ke && (reinterpret_cast<uintptr_t>(p) & 15) == 0) {
                    const float4 a = *reinterpret_cast<const float4 *>(p), b = *reinterpret_cast<const float4 *>(p + 4);
                    v[8 * u + 0] = a.x; v[8 * u + 1] = a.y; v[8 * u + 2] = a.z; v[8 * u + 3] = a.w;
                    v[8 * u + 4] = b.x; v[8 * u + 5] = b.y; v[8 * u + 6] = b.z; v[8 * u + 7] = b.w;
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const bool ok = gr < R && gk0 + e < ke;
                        const float x = *(ok ? p + e : X);
                        v[8 * u + e] = ok ? x : 0.f;
                    }
                }
            }
        } else {
            const int gr0 = r0 + 4 * (tid & 31), gk0 = k0 + 4 * (tid >> 5);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int gk = gk0 + c;
                const float *p = X + (int64_t)(gk < ke ? gk : 0) * s_k + gr0;
                if (gk < ke && gr0 + 4 <= R && (reinterpret_cast<uintptr_t>(p) & 15) == 0) {
                    const float4 a = *reinterpret_cast<const float4 *>(p);
                    v[4 * c + 0] = a.x; v[4 * c + 1] = a.y; v[4 * c + 2] = a.z; v[4 * c + 3] = a.w;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const bool ok = gk < ke && gr0 + e < R;
                        const float x = *(ok ? p + e : X);
                        v[4 * c + e] = ok ? x : 0.f;
                    }
                }
            }
        }
    };
    auto store_op = [&](const float *v, uint16_t *H, uint16_t *L, bool kf) {
        if (kf) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int r = (tid >> 2) + 64 * u, kk = 8 * (tid & 3);
                uint32_t h[4], l[4];
#pragma unroll
                for (int p = 0; p < 4; ++p) split_bf16x2(v[8 * u + 2 * p], v[8 * u + 2 * p + 1], h[p], l[p]);
                *reinterpret_cast<uint4 *>(H + r * XP + kk) = make_uint4(h[0], h[1], h[2], h[3]);
                *reinterpret_cast<uint4 *>(L + r * XP + kk) = make_uint4(l[0], l[1], l[2], l[3]);
            }
        } else {
            const int r0l = 4 * (tid & 31), kk = 4 * (tid >> 5);
#pragma unroll
            for (int e = 0; e < 4; ++e) {             // row r0l + e: K kk .. kk + 3 are v[4 c + e]
                uint32_t h0, l0, h1, l1;
                split_bf16x2(v[e], v[4 + e], h0, l0);
                split_bf16x2(v[8 + e], v[12 + e], h1, l1);
                *reinterpret_cast<uint2 *>(H + (r0l + e) * XP + kk) = make_uint2(h0, h1);
                *reinterpret_cast<uint2 *>(L + (r0l + e) * XP + kk) = make_uint2(l0, l1);
            }
        }
    };
    auto load = [&](int k0) {
        load_op(A, it0.a_i, it0.a_k, akf, i0, M, k0, va);
        load_op(B, it0.b_j, it0.b_k, bkf, j0, N, k0, vb);
    };
    f32x16 acc[2][2];
#pragma unroll
    for (int tm = 0; tm < 2; ++tm)
#pragma unroll
        for (int tn = 0; tn < 2; ++tn) acc[tm][tn] = f32x16{};
    load(kb);
    for (int k0 = kb; k0 < ke; k0 += kKS) {
        __syncthreads();
        store_op(va, Ah, Al, akf);
        store_op(vb, Bh, Bl, bkf);
        __syncthreads();
        if (k0 + kKS < ke) load(k0 + kKS);
#pragma unroll
        for (int ks = 0; ks < kKS / 16; ++ks) {
            FragBF16 ah[2], al[2], bh[2], bl[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int ra = (64 * wm + 32 * t + l32) * XP + 16 * ks + 8 * kh;
                const int rb = (64 * wn + 32 * t + l32) * XP + 16 * ks + 8 * kh;
                ah[t] = load_frag(Ah + ra); al[t] = load_frag(Al + ra);
                bh[t] = load_frag(Bh + rb); bl[t] = load_frag(Bl + rb);
            }
#pragma unroll
            for (int tm = 0; tm < 2; ++tm)
#pragma unroll
                for (int tn = 0; tn < 2; ++tn) {
                    mfma(ah[tm], bh[tn], acc[tm][tn]);
                    mfma(ah[tm], bl[tn], acc[tm][tn]);
                    mfma(al[tm], bh[tn], acc[tm][tn]);
                }
        }
    }
#pragma unroll
    for (int tn = 0; tn < 2; ++tn) {
        const int gj = j0 + 64 * wn + 32 * tn + l32;
        if (gj >= N) continue;
#pragma unroll
        for (int tm = 0; tm < 2; ++tm)
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) {
                const int gi = i0 + 64 * wm + 32 * tm + frag_row(lane, jj);
                if (gi < M) C[(int64_t)gi * it0.c_i + (int64_t)gj * it0.c_j] = acc[tm][tn][jj];
            }
    }
}

// ---------------------------------------------------------------- symmetric Gram
// WG (8 waves) per (split, item): the split's columns of Y go through LDS in
// chunks of 64 (P rows, zero past k and len; the next chunk is loaded into
// registers meanwhile); wave w owns upper tiles (tm <= tn) w, w + 8, w + 16 of
// the 32 x 32 tile grid, whose MFMA operands are both rows of the staged chunk.
//
// The products run on the bf16 MFMA: each staged value y is split once into
// hi = bf16(y) and lo = bf16(y - hi) (|y - hi - lo| <= 2^-18 |y|), and a tile
// accumulates hi_a hi_b + hi_a lo_b + lo_a hi_b (each product exact in fp32;
// the omitted lo_a lo_b is below 2^-16 of |y_a y_b|), three 32x32x16 MFMAs
// per 16 columns where fp32 operands take eight 32x32x2 ones at twice the
// cycles each.  Per product that is about 2^-16 relative, random in sign, so
// a Gram entry over a few thousand columns is as close to the exact sum as
// its fp32 accumulation already is.
constexpr int kSgKC = 64, kSgXP = kSgKC + 8;   // chunk columns; bf16 pitch of a staged row (144 B)

// KMAX: the largest order of the launch (192, or kSymGramWideK: then up to 6
// tiles per wave).
template <int KMAX, class B>
__global__ __launch_bounds__(512) void k_sym_gram(B batch) {
    constexpr int TPW = ((KMAX / 32) * (KMAX / 32 + 1) / 2 + 7) / 8;     // tiles per wave
    extern __shared__ __attribute__((aligned(16))) uint8_t sg_lds[];
    const SymGramItem &it = batch.it[blockIdx.y];
    const int sp = blockIdx.x;
    if (sp >= it.nsplit) return;
    const int k = it.k, ntm = (k + 31) >> 5, P = 32 * ntm, ntiles = ntm * (ntm + 1) / 2;
    uint16_t *yh = reinterpret_cast<uint16_t *>(sg_lds);    // [P][kSgXP] hi planes of the chunk
    uint16_t *yl = yh + (size_t)P * kSgXP;                  // [P][kSgXP] lo planes
    const int tb = sp * it.chunk, te = min(it.len, tb + it.chunk);
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, m32 = lane & 31, kh = lane >> 5;
    int tmv[TPW], tnv[TPW];
    bool tv[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        int t = wid + 8 * u, tm = 0;
        tv[u] = t < ntiles;
        if (!tv[u]) t = 0;
        while (t >= ntm - tm) {
            t -= ntm - tm;
            ++tm;
        }
        tmv[u] = tm;
        tnv[u] = tm + t;
    }
    constexpr int kPieces = (KMAX * kSgKC / 4 + 511) / 512;     // float4 per thread
    float4 stg[kPieces];
    auto load = [&](int t0) {
#pragma unroll
        for (int q = 0; q < kPieces; ++q) {
            const int p = tid + 512 * q;
            const int r = p >> 4, c = t0 + 4 * (p & 15);
            const bool ok = r < k && c < te;                 // te is a multiple of 4
            const float4 v = *reinterpret_cast<const float4 *>(it.y + (size_t)(ok ? r : 0) * it.ldy + (ok ? c : 0));
            stg[q] = ok ? v : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };
    auto store = [&]() {
#pragma unroll
        for (int q = 0; q < kPieces; ++q) {
            const int p = tid + 512 * q;
            if (p < P * (kSgKC / 4)) {
                uint32_t h01, h23, l01, l23;
                split_bf16x2(stg[q].x, stg[q].y, h01, l01);
                split_bf16x2(stg[q].z, stg[q].w, h23, l23);
                const size_t o = (size_t)(p >> 4) * kSgXP + 4 * (p & 15);
                *reinterpret_cast<uint2 *>(yh + o) = make_uint2(h01, h23);
                *reinterpret_cast<uint2 *>(yl + o) = make_uint2(l01, l23);
            }
        }
    };
    f32x16 acc[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u) acc[u] = f32x16{};
    if (tb < te) load(tb);
    for (int t0 = tb; t0 < te; t0 += kSgKC) {
        __syncthreads();
        store();
        __syncthreads();
        if (t0 + kSgKC < te) load(t0 + kSgKC);
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            if (!tv[u]) continue;
            const size_t ra = (size_t)(32 * tmv[u] + m32) * kSgXP + 8 * kh;
            const size_t rb = (size_t)(32 * tnv[u] + m32) * kSgXP + 8 * kh;
#pragma unroll
            for (int k0 = 0; k0 < kSgKC; k0 += 16) {
                const FragBF16 ah = load_frag(yh + ra + k0), bh = load_frag(yh + rb + k0);
                const FragBF16 al = load_frag(yl + ra + k0), bl = load_frag(yl + rb + k0);
                mfma(ah, bh, acc[u]);
                mfma(ah, bl, acc[u]);
                mfma(al, bh, acc[u]);
            }
        }
    }
    // each tile in place, and off-diagonal tiles mirrored through a 32 x 33
    // LDS transpose per wave, so both stores run along rows of the partial
    float *out = it.part + (size_t)sp * it.kp * it.kp;
    __syncthreads();                            // every wave is done with the staged chunk
    float *tr = reinterpret_cast<float *>(sg_lds) + wid * (32 * 33);
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        if (!tv[u]) continue;
        const int r0 = 32 * tmv[u], c0 = 32 * tnv[u];
#pragma unroll
        for (int q = 0; q < 16; ++q) out[(size_t)(r0 + frag_row(lane, q)) * it.kp + c0 + m32] = acc[u][q];
        if (r0 == c0) continue;
#pragma unroll
        for (int q = 0; q < 16; ++q) tr[frag_row(lane, q) * 33 + m32] = acc[u][q];
        wave_lds_sync();
#pragma unroll
        for (int b = 0; b < 32; b += 2)             // mirror row c0 + b + kh: tile column b + kh
            out[(size_t)(c0 + b + kh) * it.kp + r0 + m32] = tr[m32 * 33 + b + kh];
        wave_lds_sync();
    }
}

// items: the host copy of the launch's items (checks and sizes); b: what the
// kernel reads them from (a by-value batch or a device table)
template <class B>
static hipError_t sym_gram_go(const SymGramItem *items, int n, const B &b, int maxK, int maxSplit, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    if (maxK > kSymGramWideK) return hipErrorInvalidValue;
    for (int i = 0; i < n; ++i) {
        const SymGramItem &it = items[i];
        if (it.len % 4 || it.ldy % 4 || it.chunk % kSgKC || it.kp < 32 * ((it.k + 31) / 32)) return hipErrorInvalidValue;
    }
    KTimeScope kts("k_sym_gram", s);
    // the staged chunk (hi and lo planes), or 8 waves' 32 x 33 transpose tiles, whichever is larger
    const size_t lds = std::max<size_t>((size_t)2 * 32 * ((maxK + 31) / 32) * kSgXP * sizeof(uint16_t),
                                        (size_t)8 * 32 * 33 * sizeof(float));
    if (maxK > kSymGramMaxK) {
        static hipError_t state = hipErrorNotReady;     // one per instantiation
        if (state == hipErrorNotReady) {
            hipFuncAttributes fa;
            state = hipFuncGetAttributes(&fa, reinterpret_cast<const void *>(k_sym_gram<kSymGramWideK, B>));
            if (state == hipSuccess)
                state = hipFuncSetAttribute(reinterpret_cast<const void *>(k_sym_gram<kSymGramWideK, B>),
                                            hipFuncAttributeMaxDynamicSharedMemorySize,
                                            160 * 1024 - (int)fa.sharedSizeBytes);
        }
        if (state != hipSuccess) return state;
        hipLaunchKernelGGL((k_sym_gram<kSymGramWideK, B>), dim3(maxSplit, n), dim3(512), lds, s, b);
    } else {
        hipLaunchKernelGGL((k_sym_gram<kSymGramMaxK, B>), dim3(maxSplit, n), dim3(512), lds, s, b);
    }
    return hipGetLastError();
}
hipError_t launch_sym_gram(const SymGramBatch &b, int maxK, int maxSplit, hipStream_t s) {
    return sym_gram_go(b.it, b.n, b, maxK, maxSplit, s);
}
hipError_t launch_sym_gram(const SymGramItem *host, const SymGramTable &dev, int maxK, int maxSplit, hipStream_t s) {
    return sym_gram_go(host, dev.n, dev, maxK, maxSplit, s);
}

hipError_t launch_gemm_split(const GemmBatch &b, int maxM, int maxN, int maxSplit, int maxNb, hipStream_t s) {
    if (b.n <= 0) return hipSuccess;
    for (int i = 0; i < b.n; ++i) {
        const GemmItem &g = b.it[i];
        if ((g.a_i != 1 && g.a_k != 1) || (g.b_j != 1 && g.b_k != 1))
            return launch_gemm(b, maxM, maxN, maxSplit, maxNb, s);     // operands of other strides: fp32
    }
    KTimeScope kts("k_gemm", s);
    dim3 g((maxN + kBT - 1) / kBT, (maxM + kBT - 1) / kBT, b.n * maxSplit * maxNb);
    hipLaunchKernelGGL(k_gemm128_bx3, g, dim3(256), 0, s, b, maxSplit);
    return hipGetLastError();
}

hipError_t launch_gemm(const GemmBatch &b, int maxM, int maxN, int maxSplit, int maxNb, hipStream_t s) {
    if (b.n <= 0) return hipSuccess;
    KTimeScope kts("k_gemm", s);
    if (maxM > 64 && maxN > 64) {
        dim3 g((maxN + kBT - 1) / kBT, (maxM + kBT - 1) / kBT, b.n * maxSplit * maxNb);
        hipLaunchKernelGGL(k_gemm128, g, dim3(256), 0, s, b, maxSplit);
    } else {
        dim3 g((maxN + 63) / 64, (maxM + 63) / 64, b.n * maxSplit * maxNb);
        hipLaunchKernelGGL(k_gemm, g, dim3(256), 0, s, b, maxSplit);
    }
    return hipGetLastError();
}

}  // namespace jolt
