// Batched fp32 GEMMs of the planner on fp32 MFMA: a generic one (core
// projection, U_t = Q U~, block-Jacobi rotations) and the symmetric Gram of the
// rows of a panel (CholeskyQR Grams, B B^T).
//
// One workgroup computes a 64 x 64 tile of C (4 waves, 2 x 2 tiles of 32 x 32 on
// v_mfma_f32_32x32x2f32).  K is staged through LDS 32 deep; the next slice is
// loaded into registers while the current one is multiplied.  Operands are
// addressed by element strides, so transposed views need no copies; loads are
// coalesced along whichever index has stride 1.
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

// ---------------------------------------------------------------- symmetric Gram
// WG (8 waves) per (split, item): the split's columns of Y go through LDS in
// chunks of 64 (P rows, zero past k and len; the next chunk is loaded into
// registers meanwhile); wave w owns upper tiles (tm <= tn) w, w + 8, w + 16 of
// the 32 x 32 tile grid, whose MFMA operands are both rows of the staged chunk.
constexpr int kSgKC = 64, kSgPitch = kSgKC + 1;

__global__ __launch_bounds__(512) void k_sym_gram(SymGramBatch batch) {
    extern __shared__ float ysg[];          // [P][kSgPitch]
    const SymGramItem &it = batch.it[blockIdx.y];
    const int sp = blockIdx.x;
    if (sp >= it.nsplit) return;
    const int k = it.k, ntm = (k + 31) >> 5, P = 32 * ntm, ntiles = ntm * (ntm + 1) / 2;
    const int tb = sp * it.chunk, te = min(it.len, tb + it.chunk);
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, m32 = lane & 31, kh = lane >> 5;
    int tmv[3], tnv[3];
    bool tv[3];
#pragma unroll
    for (int u = 0; u < 3; ++u) {
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
    constexpr int kPieces = (kSymGramMaxK * kSgKC / 4 + 511) / 512;     // float4 per thread
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
                float *d = ysg + (p >> 4) * kSgPitch + 4 * (p & 15);
                d[0] = stg[q].x;
                d[1] = stg[q].y;
                d[2] = stg[q].z;
                d[3] = stg[q].w;
            }
        }
    };
    f32x16 acc[3];
#pragma unroll
    for (int u = 0; u < 3; ++u) acc[u] = f32x16{};
    if (tb < te) load(tb);
    for (int t0 = tb; t0 < te; t0 += kSgKC) {
        __syncthreads();
        store();
        __syncthreads();
        if (t0 + kSgKC < te) load(t0 + kSgKC);
#pragma unroll
        for (int u = 0; u < 3; ++u) {
            if (!tv[u]) continue;
            const float *ra = ysg + (32 * tmv[u] + m32) * kSgPitch + kh;
            const float *rb = ysg + (32 * tnv[u] + m32) * kSgPitch + kh;
#pragma unroll 8
            for (int k0 = 0; k0 < kSgKC; k0 += 2)
                acc[u] = __builtin_amdgcn_mfma_f32_32x32x2f32(ra[k0], rb[k0], acc[u], 0, 0, 0);
        }
    }
    // each tile in place, and off-diagonal tiles mirrored through a 32 x 33
    // LDS transpose per wave, so both stores run along rows of the partial
    float *out = it.part + (size_t)sp * it.kp * it.kp;
    __syncthreads();                            // every wave is done with the staged chunk
    float *tr = ysg + wid * (32 * 33);
#pragma unroll
    for (int u = 0; u < 3; ++u) {
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

hipError_t launch_sym_gram(const SymGramBatch &b, int maxK, int maxSplit, hipStream_t s) {
    if (b.n <= 0) return hipSuccess;
    if (maxK > kSymGramMaxK) return hipErrorInvalidValue;
    for (int i = 0; i < b.n; ++i) {
        const SymGramItem &it = b.it[i];
        if (it.len % 4 || it.ldy % 4 || it.chunk % kSgKC || it.kp < 32 * ((it.k + 31) / 32)) return hipErrorInvalidValue;
    }
    KTimeScope kts("k_sym_gram", s);
    // the staged chunk, or 8 waves' 32 x 33 transpose tiles, whichever is larger
    const size_t lds = std::max<size_t>((size_t)32 * ((maxK + 31) / 32) * kSgPitch, 8 * 32 * 33) * sizeof(float);
    hipLaunchKernelGGL(k_sym_gram, dim3(maxSplit, b.n), dim3(512), lds, s, b);
    return hipGetLastError();
}

hipError_t launch_gemm(const GemmBatch &b, int maxM, int maxN, int maxSplit, int maxNb, hipStream_t s) {
    if (b.n <= 0) return hipSuccess;
    KTimeScope kts("k_gemm", s);
    dim3 g((maxN + 63) / 64, (maxM + 63) / 64, b.n * maxSplit * maxNb);
    hipLaunchKernelGGL(k_gemm, g, dim3(256), 0, s, b, maxSplit);
    return hipGetLastError();
}

}  // namespace jolt
