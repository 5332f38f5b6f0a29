// Generic batched fp32 GEMM of the planner (Gram of sketch panels, B B^T,
// core projection, U_t = Q U~, block-Jacobi rotations) on fp32 MFMA.
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

hipError_t launch_gemm(const GemmBatch &b, int maxM, int maxN, int maxSplit, int maxNb, hipStream_t s) {
    if (b.n <= 0) return hipSuccess;
    KTimeScope kts("k_gemm", s);
    dim3 g((maxN + 63) / 64, (maxM + 63) / 64, b.n * maxSplit * maxNb);
    hipLaunchKernelGGL(k_gemm, g, dim3(256), 0, s, b, maxSplit);
    return hipGetLastError();
}

}  // namespace jolt
