// Plan-stage kernels for gfx950: the passes over the cache tensor (MFMA), the
// small dense fp32 linear algebra (GEMM, Cholesky, triangular solve, Jacobi
// eigensolver) and the parameter store.
//
// Method ("A JoLT for the KV cache", landing page abstract): partial Tucker
// decomposition of the grouped cache tensor along the token and feature modes;
// the token factor by an exact token-mode SVD (eigenvectors of A A^T, A the
// token unfolding) or by FlashJoLT's randomized approximation (range finder of
// Halko, Martinsson & Tropp: sketch, orthonormalise, power iteration, small SVD
// of B = Q^T A); the feature factor from the d x d feature Gram.
//
// MFMA fragment convention (v_mfma_f32_32x32x16_bf16 / 32x32x2f32): lane l
// supplies row l % 32 of A and column l % 32 of B with the 8 consecutive K
// indices k0 + 8 (l / 32) + i; the 32x32 fp32 result sits at
// D[8 (j / 4) + 4 (l / 32) + j % 4][l % 32], j = 0..15.
#include <float.h>
#include <stdlib.h>

#include <algorithm>
#include <cstring>

#include "dev_common.h"
#include "plan_kernels.h"
#include "ktimer.h"

namespace jolt {

// ====================================================================== X-pass A M
// out[s][c][t] = sum over the split's features k of x[t][k] m[k][c] (x the token
// unfolding, m the sketch operand stored as m[c][k]).
//
// WG: 256 tokens, as NWV waves of R 32-token row fragments (4 x 2, or 8 x 1
// for the widest column tiles, whose NF accumulators per row fragment leave no
// registers for a second one), and NF column fragments of 32.  The K range
// (lh_split whole (layer, head) blocks) runs in chunks of 64 features.  A chunk
// of m (NF*32 columns x 64) is staged once per WG in LDS, double buffered, and
// read by all the waves; x fragments come straight from global memory, each
// element once, one chunk ahead.
template <typename T, int KC_>
struct XmTile {
    static constexpr int PER = 16 / sizeof(T);     // elements per 16-byte piece
    static constexpr int KC = KC_;                 // K chunk
    static constexpr int KP = KC + PER;            // LDS row pitch (elements)
    static constexpr int U = KC / 16;              // MFMA K steps per chunk
};

template <typename T, int NF, int KC_, int R, int NWV>
__global__ __launch_bounds__(64 * NWV) void k_xm(XmBatch batch, int d, int ncol_tiles) {
    static_assert(32 * R * NWV == 256, "256 tokens per workgroup");
    constexpr int NT = 64 * NWV;
    using Frag = typename Elem<T>::Frag;
    using Tile = XmTile<T, KC_>;
    constexpr int PER = Tile::PER, KC = Tile::KC, KP = Tile::KP, U = Tile::U;
    constexpr int ROWS = 32 * NF;
    constexpr int PIECES = ROWS * KC / PER;                 // 16-byte pieces per m chunk
    constexpr int PPT = (PIECES + NT - 1) / NT;             // per thread
    extern __shared__ __attribute__((aligned(16))) unsigned char xm_lds[];
    T *ms = reinterpret_cast<T *>(xm_lds);                  // [2][ROWS][KP]
    const Block3 blk = xcd_block();
    const XmItem it = batch.it[blk.z];      // a copy: its fields stay in registers
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, ln = lane & 31, h = lane >> 5;
    const int tw = blk.x * 256 + wave * 32 * R;             // this wave's first token
    const int c0 = (blk.y % ncol_tiles) * ROWS;
    const int sp = blk.y / ncol_tiles;
    if (blk.x * 256 >= it.T || c0 >= it.ncols || sp >= it.nsplit) return;
    const bool wv = tw < it.T;                              // T is a multiple of 64 (of 32 R)
    const T *x = reinterpret_cast<const T *>(it.x);
    const T *m = reinterpret_cast<const T *>(it.m);
    const int n = it.LH * d;
    const int kb = sp * it.lh_split * d, ke = min(n, kb + it.lh_split * d);
    const int nck = (ke - kb) / KC;

    // m chunk staging: piece p -> row p / (KC / PER), 16 bytes at column (p % (KC / PER)) * PER
    uint4 stg[PPT];
    auto load_m = [&](int k0) {
        const int lh = k0 / d, fb = k0 - lh * d;
#pragma unroll
        for (int q = 0; q < PPT; ++q) {
            const int p = threadIdx.x + NT * q;
            const int r = p / (KC / PER), kk = (p % (KC / PER)) * PER;
            const int c = c0 + r;
            const bool ok = p < PIECES && c < it.ncols;
            const T *src = m + (size_t)(ok ? c : 0) * it.m_c + (size_t)lh * it.m_blk + fb + (ok ? kk : 0);
            const uint4 v = *reinterpret_cast<const uint4 *>(src);
            stg[q] = ok ? v : make_uint4(0u, 0u, 0u, 0u);
        }
    };
    auto store_m = [&](int buf) {
#pragma unroll
        for (int q = 0; q < PPT; ++q) {
            const int p = threadIdx.x + NT * q;
            if (p < PIECES) {
                const int r = p / (KC / PER), kk = (p % (KC / PER)) * PER;
                *reinterpret_cast<uint4 *>(ms + ((size_t)buf * ROWS + r) * KP + kk) = stg[q];
            }
        }
    };
    // x fragments of a chunk: rows tw + 32 r + ln, K = 16 u + 8 h + (0..7)
    Frag an[R][U], a[R][U];
    auto load_x = [&](int k0) {
        const int lh = k0 / d, fb = k0 - lh * d;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int tok = wv ? tw + 32 * r + ln : 0;
            const T *xa = x + ((size_t)lh * it.T + tok) * d + fb + 8 * h;
#pragma unroll
            for (int u = 0; u < U; ++u) an[r][u] = load_frag(xa + 16 * u);
        }
    };

    f32x16 acc[R][NF];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int f = 0; f < NF; ++f) acc[r][f] = f32x16{};
    if (nck > 0) {
        load_m(kb);
        load_x(kb);
        store_m(0);
    }
    for (int ci = 0; ci < nck; ++ci) {
        __syncthreads();
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int u = 0; u < U; ++u) a[r][u] = an[r][u];
        const bool more = ci + 1 < nck;
        if (more) {
            load_m(kb + (ci + 1) * KC);
            load_x(kb + (ci + 1) * KC);
        }
        const T *mb = ms + (size_t)(ci & 1) * ROWS * KP;
        if (wv) {
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int f = 0; f < NF; ++f) {
                    const Frag b = load_frag(mb + (32 * f + ln) * KP + 16 * u + 8 * h);
#pragma unroll
                    for (int r = 0; r < R; ++r) mfma(a[r][u], b, acc[r][f]);
                }
            // LDS reads kept 4 ahead of the MFMAs that use them
            sched_reads_ahead<U * NF, R, 4>();
        }
        if (more) store_m((ci + 1) & 1);
    }
    if (!wv) return;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
        const int c = c0 + 32 * f + ln;
        if (c < it.ncols) {
            float *o = it.out + (size_t)sp * it.ncols * it.ldo + (size_t)c * it.ldo + tw;
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int row = 32 * r + 8 * q + 4 * h;
                    *reinterpret_cast<float4 *>(o + row) = make_float4(acc[r][f][4 * q], acc[r][f][4 * q + 1],
                                                                       acc[r][f][4 * q + 2], acc[r][f][4 * q + 3]);
                }
        }
    }
}

// ====================================================================== staging helper
// 64 rows x d features (row stride d) -> LDS transposed xs[f][r] with row pitch XP.
template <typename T>
__device__ __forceinline__ void stage_transposed(const T *src, int d, T *xs, int XP) {
    constexpr int PER = 16 / sizeof(T);
    const int chunks = 64 * d / PER;
    for (int c = threadIdx.x; c < chunks; c += blockDim.x) {
        const int r = c / (d / PER), f = (c % (d / PER)) * PER;
        const uint4 v = *reinterpret_cast<const uint4 *>(src + (size_t)r * d + f);
        const T *e = reinterpret_cast<const T *>(&v);
#pragma unroll
        for (int i = 0; i < PER; ++i) xs[(f + i) * XP + r] = e[i];
    }
}

// ====================================================================== X-pass Q^T A
// out[s][c][F] = sum over the split's tokens t of q[c][t] x[t][F], F = lh d + f
// the global feature index (the token unfolding's column).
//
// WG: a tile of 256 features (NWV waves x R row fragments of 32: 4 x 2, or
// 8 x 1 for the widest column tiles) and NF column fragments of 32.  Per chunk
// of TC tokens the WG stages, once, x's tile transposed to xs[F][t] (token
// pairs packed in 32-bit words for bf16) and the chunk of q (hi and lo parts
// when LO) as qs[c][t].  Two LDS buffers: while the waves run the MFMAs of one
// chunk out of one buffer, the next chunk (already in registers) is stored
// into the other and the chunk after it is loaded from global memory, with one
// barrier per chunk.  TC is 64 tokens when two such buffers fit the 160 KB of
// LDS, else 32.  Each wave reads R x fragments and NF (2 NF) q fragments per
// 16 tokens from LDS.
template <typename T, int NF, bool LO, int NT>
struct XtqTile {
    static constexpr int PER = 16 / sizeof(T);
    static constexpr int FT = 256;                       // features per WG
    static constexpr int QR = 32 * NF * (LO ? 2 : 1);    // q rows staged (hi rows, then lo rows)
    static constexpr size_t buf_for(int tc) { return (size_t)(FT + QR) * (tc + PER) * sizeof(T); }
    static constexpr int TC = 2 * buf_for(64) <= 160 * 1024 ? 64 : 32;   // tokens per chunk
    static constexpr int XP = TC + PER;                  // LDS pitch of xs and qs rows
    static constexpr int BUF = (FT + QR) * XP;           // elements per buffer
    static constexpr int XPIECES = FT * TC / PER / (sizeof(T) == 2 ? 2 : 1);  // loads of x per chunk
    static constexpr int XPT = XPIECES / NT;
    static constexpr int QPIECES = QR * TC / PER;
    static constexpr int QPT = (QPIECES + NT - 1) / NT;
    static constexpr size_t lds_bytes = 2 * buf_for(TC);
    static_assert(XPIECES % NT == 0, "x pieces spread evenly over the threads");
    static_assert(lds_bytes <= 160 * 1024, "two chunk buffers in LDS");
};

template <typename T, int NF, bool LO, int R, int NWV>
__global__ __launch_bounds__(64 * NWV) void k_xtq(XtqBatch batch, int d, int maxSplit) {
    static_assert(32 * R * NWV == 256, "256 features per workgroup");
    constexpr int NT = 64 * NWV;
    using Tile = XtqTile<T, NF, LO, NT>;
    using Frag = typename Elem<T>::Frag;
    constexpr int PER = Tile::PER, FT = Tile::FT, TC = Tile::TC, XP = Tile::XP, QR = Tile::QR;
    constexpr int XPT = Tile::XPT, QPT = Tile::QPT, QPIECES = Tile::QPIECES;
    constexpr bool BF = sizeof(T) == 2;
    extern __shared__ __attribute__((aligned(16))) unsigned char xtq_lds[];
    T *const lds = reinterpret_cast<T *>(xtq_lds);       // 2 x ([FT][XP] x rows, then [QR][XP] q rows)
    const Block3 blk = xcd_block();
    const XtqItem it = batch.it[blk.z];     // a copy: its fields stay in registers
    const int n = it.LH * d;
    const int F0 = blk.y * FT, sp = blk.x % maxSplit, c0 = (blk.x / maxSplit) * 32 * NF;
    if (F0 >= n || sp >= it.nsplit || c0 >= it.ncols) return;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, ln = lane & 31, h = lane >> 5;
    const T *x = reinterpret_cast<const T *>(it.x);
    const T *qh = reinterpret_cast<const T *>(it.qh);
    const T *ql = reinterpret_cast<const T *>(it.ql);
    const int tb = sp * it.tsplit, te = min(it.T, tb + it.tsplit);
    const int nck = (te - tb) / TC;                       // T and the split are multiples of 64

    // x staging.  bf16: piece = 2 consecutive tokens x 8 features (two 16-byte
    // loads), lanes: 8 token pairs x 8 feature groups; fp32: piece = 1 token x 4
    // features, lanes: 16 tokens x 4 feature groups.
    constexpr int TPL = BF ? 8 : 16;                      // token slots per wave pass
    constexpr int FGL = 64 / TPL;                         // feature groups per wave pass
    uint4 xr[XPT][BF ? 2 : 1];
    auto load_x = [&](int t0) {
#pragma unroll
        for (int q = 0; q < XPT; ++q) {
            const int pass = wave + NWV * q;              // 0 .. NWV XPT - 1
            const int tl = lane % TPL, fg = lane / TPL;
            const int tpass = pass % (TC / (BF ? 2 : 1) / TPL), fpass = pass / (TC / (BF ? 2 : 1) / TPL);
            const int t = t0 + (tpass * TPL + tl) * (BF ? 2 : 1);
            const int F = F0 + (fpass * FGL + fg) * PER;
            const bool ok = F < n;
            const int Fc = ok ? F : 0;
            const int lh = Fc / d, f = Fc - lh * d;
            const T *src = x + ((size_t)lh * it.T + t) * d + f;
            const uint4 v0 = *reinterpret_cast<const uint4 *>(src);
            xr[q][0] = ok ? v0 : make_uint4(0u, 0u, 0u, 0u);
            if constexpr (BF) {
                const uint4 v1 = *reinterpret_cast<const uint4 *>(src + d);
                xr[q][1] = ok ? v1 : make_uint4(0u, 0u, 0u, 0u);
            }
        }
    };
    auto store_x = [&](T *xs) {
#pragma unroll
        for (int q = 0; q < XPT; ++q) {
            const int pass = wave + NWV * q;
            const int tl = lane % TPL, fg = lane / TPL;
            const int tpass = pass % (TC / (BF ? 2 : 1) / TPL), fpass = pass / (TC / (BF ? 2 : 1) / TPL);
            const int tt = (tpass * TPL + tl) * (BF ? 2 : 1);
            const int fr = (fpass * FGL + fg) * PER;
            if constexpr (BF) {
                const uint32_t *a0 = reinterpret_cast<const uint32_t *>(&xr[q][0]);
                const uint32_t *a1 = reinterpret_cast<const uint32_t *>(&xr[q][1]);
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    // features 2w, 2w+1 of tokens tt, tt+1 -> (t, t+1) word in rows fr+2w, fr+2w+1
                    const uint32_t lo = __builtin_amdgcn_perm(a1[w], a0[w], 0x05040100u);
                    const uint32_t hi = __builtin_amdgcn_perm(a1[w], a0[w], 0x07060302u);
                    *reinterpret_cast<uint32_t *>(xs + (fr + 2 * w) * XP + tt) = lo;
                    *reinterpret_cast<uint32_t *>(xs + (fr + 2 * w + 1) * XP + tt) = hi;
                }
            } else {
                const float *a0 = reinterpret_cast<const float *>(&xr[q][0]);
#pragma unroll
                for (int w = 0; w < 4; ++w) xs[(fr + w) * XP + tt] = a0[w];
            }
        }
    };
    // q staging: row r < 32 NF is hi column c0 + r, else lo column r - 32 NF
    uint4 qr[QPT];
    auto load_q = [&](int t0) {
#pragma unroll
        for (int q = 0; q < QPT; ++q) {
            const int p = threadIdx.x + NT * q;
            const int r = p / (TC / PER), tt = (p % (TC / PER)) * PER;
            const int c = c0 + (r < 32 * NF ? r : r - 32 * NF);
            const bool ok = p < QPIECES && c < it.ncols;
            const T *base = (LO && r >= 32 * NF) ? ql : qh;
            const uint4 v = *reinterpret_cast<const uint4 *>(base + (size_t)(ok ? c : 0) * it.ldq + t0 + (ok ? tt : 0));
            qr[q] = ok ? v : make_uint4(0u, 0u, 0u, 0u);
        }
    };
    auto store_q = [&](T *qs) {
#pragma unroll
        for (int q = 0; q < QPT; ++q) {
            const int p = threadIdx.x + NT * q;
            if (p < QPIECES) {
                const int r = p / (TC / PER), tt = (p % (TC / PER)) * PER;
                *reinterpret_cast<uint4 *>(qs + r * XP + tt) = qr[q];
            }
        }
    };

    f32x16 acc[R][NF];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int f = 0; f < NF; ++f) acc[r][f] = f32x16{};
    const int fw = 32 * R * wave;                         // this wave's first feature in the tile
    if (nck > 0) {
        load_x(tb);
        load_q(tb);
        store_x(lds);
        store_q(lds + FT * XP);
        if (nck > 1) {
            load_x(tb + TC);
            load_q(tb + TC);
        }
    }
    __syncthreads();
    for (int ci = 0; ci < nck; ++ci) {
        const T *xs = lds + (ci & 1) * Tile::BUF;
        const T *qs = xs + FT * XP;
#pragma unroll
        for (int kk = 0; kk < TC; kk += 16) {
            Frag a[R];
#pragma unroll
            for (int r = 0; r < R; ++r) a[r] = load_frag(xs + (fw + 32 * r + ln) * XP + kk + 8 * h);
#pragma unroll
            for (int f = 0; f < NF; ++f) {
                const Frag b = load_frag(qs + (32 * f + ln) * XP + kk + 8 * h);
#pragma unroll
                for (int r = 0; r < R; ++r) mfma(a[r], b, acc[r][f]);
                if constexpr (LO) {
                    const Frag bl = load_frag(qs + (32 * NF + 32 * f + ln) * XP + kk + 8 * h);
#pragma unroll
                    for (int r = 0; r < R; ++r) mfma(a[r], bl, acc[r][f]);
                }
            }
        }
        // LDS reads kept ahead of the MFMAs (per 16 tokens: R x fragments, then
        // one q fragment per R MFMAs)
        if constexpr (BF) sched_reads_ahead<(TC / 16) * (R + NF * (LO ? 2 : 1)), R, 8>();
        if (ci + 1 < nck) {
            // the other buffer was last read before the previous barrier
            T *nx = lds + ((ci + 1) & 1) * Tile::BUF;
            store_x(nx);
            store_q(nx + FT * XP);
            if (ci + 2 < nck) {
                load_x(tb + (ci + 2) * TC);
                load_q(tb + (ci + 2) * TC);
            }
        }
        __syncthreads();
    }
    float *out = it.out + (size_t)sp * it.ncols * n;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
        const int c = c0 + 32 * f + ln;
        if (c < it.ncols) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int Fr = F0 + fw + 32 * r;
                if (Fr < n) {
                    float *o = out + (size_t)c * n + Fr;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int row = 8 * q + 4 * h;
                        *reinterpret_cast<float4 *>(o + row) = make_float4(acc[r][f][4 * q], acc[r][f][4 * q + 1],
                                                                           acc[r][f][4 * q + 2], acc[r][f][4 * q + 3]);
                    }
                }
            }
        }
    }
}

// ====================================================================== feature Gram
// Partial Grams of 64-row chunks (rows of the (l, h, t) x d unfolding; plans
// keep T, and so every chunk, a multiple of 64).  Per chunk the rows go to LDS
// transposed, xs[f][r] (bf16 row pairs packed in 32-bit words); the next
// chunk's rows are in flight in registers while the MFMAs run on the current
// one, and each fragment is one 16-byte LDS read.  Only the upper fragment
// pairs (mf <= nf) are formed, dealt to the waves in row order (pair t to wave
// t mod 4); a lower tile is the transpose of its upper one, whose every entry
// is the same sum of the same exact products in the same order, and is stored
// from it.
template <typename T>
__global__ __launch_bounds__(256) void k_gram_rows(GramBatch batch, int d) {
    constexpr int PER = 16 / sizeof(T);            // features per 16-byte piece
    constexpr int XP = 64 + PER;                   // pitch (elements) of a feature's row in xs
    __shared__ __attribute__((aligned(16))) T xs[128 * XP];
    const GramItem it = batch.it[blockIdx.z];   // a copy: its fields stay in registers
    const int p = blockIdx.x;
    if (p >= it.P) return;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, ln = lane & 31, h = lane >> 5;
    const int nmf = d / 32;                        // 4 or 2 fragments per side
    const T *x = reinterpret_cast<const T *>(it.x);
    const int64_t rb = (int64_t)p * it.chunk;
    const int64_t re = min(it.rows, rb + it.chunk);
    // staging tasks: row pair rp (32 per chunk) x 16-byte piece fc of the row
    const int nfc = d / PER, ntask = 32 * nfc / 256;   // 1, 2 or 4 per thread
    uint4 lo[4], hi[4];
    auto load = [&](int64_t r0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (j < ntask) {
                const int t = tid + 256 * j, rp = t / nfc, fc = t - rp * nfc;
                const T *src = x + (r0 + 2 * rp) * d + fc * PER;
                lo[j] = *reinterpret_cast<const uint4 *>(src);
                hi[j] = *reinterpret_cast<const uint4 *>(src + d);
            }
        }
    };
    auto store = [&]() {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (j < ntask) {
                const int t = tid + 256 * j, rp = t / nfc, fc = t - rp * nfc;
                if constexpr (sizeof(T) == 2) {
                    uint32_t *xw = reinterpret_cast<uint32_t *>(xs);
                    const uint32_t a[4] = {lo[j].x, lo[j].y, lo[j].z, lo[j].w}, b[4] = {hi[j].x, hi[j].y, hi[j].z, hi[j].w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        xw[(fc * PER + 2 * i) * (XP / 2) + rp] = (a[i] & 0xFFFFu) | (b[i] << 16);
                        xw[(fc * PER + 2 * i + 1) * (XP / 2) + rp] = (a[i] >> 16) | (b[i] & 0xFFFF0000u);
                    }
                } else {
                    const float a[4] = {__uint_as_float(lo[j].x), __uint_as_float(lo[j].y), __uint_as_float(lo[j].z),
                                        __uint_as_float(lo[j].w)};
                    const float b[4] = {__uint_as_float(hi[j].x), __uint_as_float(hi[j].y), __uint_as_float(hi[j].z),
                                        __uint_as_float(hi[j].w)};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        reinterpret_cast<float *>(xs)[(fc * PER + i) * XP + 2 * rp] = a[i];
                        reinterpret_cast<float *>(xs)[(fc * PER + i) * XP + 2 * rp + 1] = b[i];
                    }
                }
            }
        }
    };
    // upper fragment pairs owned by this wave: t = wave + 4 i, t -> (mf, nf) in
    // row order of the upper triangle
    f32x16 acc[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) acc[i] = f32x16{};
    const int nq = nmf * (nmf + 1) / 2;
    int pm[3], pn[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        int t = wave + 4 * i, mf = 0;
        while (t >= nmf - mf && mf < nmf - 1) {
            t -= nmf - mf;
            ++mf;
        }
        pm[i] = mf;
        pn[i] = mf + t;
    }
    if (rb < re) load(rb);
    for (int64_t r0 = rb; r0 < re; r0 += 64) {
        __syncthreads();                           // the previous chunk's reads of xs are done
        store();
        __syncthreads();
        if (r0 + 64 < re) load(r0 + 64);
#pragma unroll
        for (int kk = 0; kk < 64; kk += 16) {
#pragma unroll
            for (int i = 0; i < 3; ++i) {
                if (wave + 4 * i < nq) {
                    const typename Elem<T>::Frag a = load_frag(xs + (32 * pm[i] + ln) * XP + kk + 8 * h);
                    const typename Elem<T>::Frag b = load_frag(xs + (32 * pn[i] + ln) * XP + kk + 8 * h);
                    mfma(a, b, acc[i]);
                }
            }
        }
    }
    float *out = it.out + (size_t)p * d * d;
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        if (wave + 4 * i < nq) {
            const int mf = pm[i], nf = pn[i];
#pragma unroll
            for (int j = 0; j < 16; ++j) out[(size_t)(32 * mf + frag_row(lane, j)) * d + 32 * nf + ln] = acc[i][j];
            if (mf != nf)
                // the mirror: row 32 nf + ln, columns 32 mf + frag_row(lane, 4 c .. 4 c + 3)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    *reinterpret_cast<float4 *>(out + (size_t)(32 * nf + ln) * d + 32 * mf + frag_row(lane, 4 * c)) =
                        make_float4(acc[i][4 * c], acc[i][4 * c + 1], acc[i][4 * c + 2], acc[i][4 * c + 3]);
        }
    }
}

// ====================================================================== split reduction
// Sums of split partials in split order (the same order every run): four
// consecutive entries per thread, with float4 accesses when the item's
// pointers and stride allow them.
__global__ void k_reduce(ReduceBatch batch) {
    const ReduceItem &it = batch.it[blockIdx.y];
    const int64_t i = 4 * ((int64_t)blockIdx.x * blockDim.x + threadIdx.x);
    if (i >= it.count) return;
    const bool vec = i + 4 <= it.count && it.stride % 4 == 0 &&
                     ((reinterpret_cast<uintptr_t>(it.part) | reinterpret_cast<uintptr_t>(it.out)) & 15) == 0;
    if (vec) {
        float4 s = *reinterpret_cast<const float4 *>(it.part + i);
#pragma unroll 4
        for (int p = 1; p < it.nsplit; ++p) {
            const float4 v = *reinterpret_cast<const float4 *>(it.part + (int64_t)p * it.stride + i);
            s.x += v.x;
            s.y += v.y;
            s.z += v.z;
            s.w += v.w;
        }
        *reinterpret_cast<float4 *>(it.out + i) = s;
    } else {
        for (int64_t e = i; e < i + 4 && e < it.count; ++e) {
            float s = 0.f;
            for (int p = 0; p < it.nsplit; ++p) s += it.part[(int64_t)p * it.stride + e];
            it.out[e] = s;
        }
    }
}

// ====================================================================== Cholesky
// One WG per matrix; the lower triangle is held packed in LDS:
// L(i, j) at i (i + 1) / 2 + j.  Right-looking: pivot, scale the column, rank-1
// update of the trailing triangle.  Pivots at or below the shift floor are
// clamped so rank-deficient sketches still give a usable basis.
__global__ __launch_bounds__(1024) void k_cholesky(CholBatch batch) {
    extern __shared__ float lp[];
    __shared__ float s_red[32];
    __shared__ float s_shift;
    const CholItem &it = batch.it[blockIdx.x];
    const int k = it.k, tid = threadIdx.x, nt = blockDim.x;
    // trace for the shift
    float tr = 0.f;
    for (int i = tid; i < k; i += nt) tr += it.g[(size_t)i * it.ld + i];
    for (int o = 32; o > 0; o >>= 1) tr += __shfl_xor(tr, o);
    if ((tid & 63) == 0) s_red[tid >> 6] = tr;
    __syncthreads();
    if (tid == 0) {
        float t = 0.f;
        for (int w = 0; w < (nt + 63) / 64; ++w) t += s_red[w];
        s_shift = it.rel_shift * t / (float)k;
        if (!(s_shift > 0.f)) s_shift = FLT_MIN;
    }
    __syncthreads();
    const float shift = s_shift;
    for (int e = tid; e < k * (k + 1) / 2; e += nt) {
        int i = (int)((sqrtf(8.f * e + 1.f) - 1.f) * 0.5f);
        while (i * (i + 1) / 2 > e) --i;
        while ((i + 1) * (i + 2) / 2 <= e) ++i;
        const int j = e - i * (i + 1) / 2;
        float v = 0.5f * (it.g[(size_t)i * it.ld + j] + it.g[(size_t)j * it.ld + i]);
        if (i == j) v += shift;
        lp[e] = v;
    }
    __syncthreads();
    // Column j is left unscaled while it updates the trailing triangle
    // (L(i,c) -= L(i,j) L(c,j) / d_j with d_j the pivot before the square root);
    // every column is scaled by 1 / sqrt(d_j) at the end.  One barrier per column.
    const int ti = tid >> 5, tj = tid & 31, nti = nt >> 5;
    for (int j = 0; j < k; ++j) {
        const int jj = j * (j + 1) / 2 + j;
        const float dj = fmaxf(lp[jj], shift);
        const float rdj = 1.f / dj;
        for (int i = j + 1 + ti; i < k; i += nti) {
            const float lij = lp[i * (i + 1) / 2 + j] * rdj;
            float *row = lp + i * (i + 1) / 2;
            for (int c = j + 1 + tj; c <= i; c += 32) row[c] -= lij * lp[c * (c + 1) / 2 + j];
        }
        __syncthreads();
    }
    // scale the columns: L(i, j) = lp(i, j) / sqrt(d_j), L(j, j) = sqrt(d_j)
    for (int e = tid; e < k * (k + 1) / 2; e += nt) {
        int i = (int)((sqrtf(8.f * e + 1.f) - 1.f) * 0.5f);
        while (i * (i + 1) / 2 > e) --i;
        while ((i + 1) * (i + 2) / 2 <= e) ++i;
        const int j = e - i * (i + 1) / 2;
        const float dj = fmaxf(lp[j * (j + 1) / 2 + j], shift);
        const float v = (i == j) ? sqrtf(dj) : lp[e] / sqrtf(dj);
        it.l[(size_t)i * it.ld + j] = v;
    }
    for (int e = tid; e < k * k; e += nt) {
        const int i = e / k, j = e % k;
        if (j > i) it.l[(size_t)i * it.ld + j] = 0.f;
    }
}

// ====================================================================== triangular solve
// WG: 32 columns of y; 1024 threads = 32 columns x 32 partial-sum lanes.
// Row i of the result: q[i] = (y[i] - sum_{c<i} L[i][c] q[c]) / L[i][i].
__global__ __launch_bounds__(1024) void k_trsm(TrsmBatch batch, int l_in_lds) {
    extern __shared__ float sh[];
    const TrsmItem &it = batch.it[blockIdx.y];
    const int t0 = blockIdx.x * 32;
    if (t0 >= it.len) return;
    const int tid = threadIdx.x, col = tid >> 5, cl = tid & 31;
    const int k = it.k;
    float *qs = sh;                        // [k][33]
    float *ls = sh + k * 33;               // packed lower triangle of L (when it fits)
    for (int e = tid; e < k * 32; e += 1024) {
        const int r = e / 32, c = e % 32;
        qs[r * 33 + c] = (t0 + c < it.len) ? it.y[(size_t)r * it.ldy + t0 + c] : 0.f;
    }
    if (l_in_lds)
        for (int i = tid >> 5; i < k; i += 32)
            for (int c = tid & 31; c <= i; c += 32) ls[i * (i + 1) / 2 + c] = it.l[(size_t)i * it.ld + c];
    __syncthreads();
    for (int i = 0; i < k; ++i) {
        const float *li = l_in_lds ? ls + i * (i + 1) / 2 : it.l + (size_t)i * it.ld;
        float s = 0.f;
        for (int c = cl; c < i; c += 32) s = fmaf(li[c], qs[c * 33 + col], s);
        for (int o = 16; o > 0; o >>= 1) s += __shfl_xor(s, o, 32);
        if (cl == 0) qs[i * 33 + col] = (qs[i * 33 + col] - s) / li[i];
        __syncthreads();
    }
    for (int e = tid; e < k * 32; e += 1024) {
        const int r = e / 32, c = e % 32;
        if (t0 + c < it.len) it.q[(size_t)r * it.ldy + t0 + c] = qs[r * 33 + c];
    }
}

// ====================================================================== Jacobi (LDS)
// Two-sided Jacobi, parallel (round-robin) ordering: each of the m - 1 rounds of a
// sweep pairs all indices disjointly; the round's rotations zero a[p][q] by the
// symmetric 2x2 Schur decomposition and are applied together block by block,
// A <- J^T A J, V <- V J (Golub & Van Loan, Matrix Computations, sec. 8.5).
// A rotation is skipped when |a_pq| <= tol sqrt(|a_pp a_qq|); a sweep with no
// rotation ends the iteration.
__device__ __forceinline__ int rr_pos(int i, int round, int m) {
    if (i == 0) return 0;
    return 1 + ((i - 1 - round) % (m - 1) + (m - 1)) % (m - 1);
}

template <int NT, class B>
__global__ __launch_bounds__(NT) void k_jacobi_lds(B batch, int max_sweeps, int retry_only) {
    extern __shared__ float sm[];
    __shared__ int sP[kJacobiMaxN / 2 + 1], sQ[kJacobiMaxN / 2 + 1];
    __shared__ float sC[kJacobiMaxN / 2 + 1], sS[kJacobiMaxN / 2 + 1];
    __shared__ int s_rot;
    const JacItem &it = batch.it[blockIdx.x];
    if (retry_only && (!it.sweeps_out || *it.sweeps_out != kEigRetry)) return;
    const int n = it.n, m = n + (n & 1), half = m / 2;
    const int tid = threadIdx.x;
    constexpr int nt = NT;
    __shared__ float s_fro[32];
    float *A = sm, *Vt = sm + m * m;           // Vt[c][r] = component r of vector c
    float fro = 0.f;
    for (int e = tid; e < m * m; e += nt) {
        const int r = e / m, c = e % m;
        const float v = (r < n && c < n) ? 0.5f * (it.a[(size_t)r * it.lda + c] + it.a[(size_t)c * it.lda + r]) : 0.f;
        A[e] = v;
        fro += v * v;
        Vt[e] = (r == c) ? 1.f : 0.f;
    }
    for (int o = 32; o > 0; o >>= 1) fro += __shfl_xor(fro, o);
    if ((tid & 63) == 0) s_fro[tid >> 6] = fro;
    __syncthreads();
    if (tid == 0) {
        float t = 0.f;
        for (int w = 0; w < (nt >> 6); ++w) t += s_fro[w];
        s_fro[0] = sqrtf(t);
    }
    __syncthreads();
    const float tol = 1.0e-6f;
    // below this an off-diagonal entry is at the fp32 rounding level of the whole matrix
    const float abs_floor = 2.0e-7f * s_fro[0];
    int sweeps = 0;
    bool done = false;
    for (; sweeps < max_sweeps && !done; ++sweeps) {
        if (tid == 0) s_rot = 0;
        __syncthreads();
        for (int round = 0; round < m - 1; ++round) {
            for (int pr = tid; pr < half; pr += nt) {
                int p = rr_pos(pr, round, m), q = rr_pos(m - 1 - pr, round, m);
                if (p > q) { const int t = p; p = q; q = t; }
                const float apq = A[p * m + q], app = A[p * m + p], aqq = A[q * m + q];
                float c = 1.f, s = 0.f;
                if (fabsf(apq) > tol * sqrtf(fabsf(app) * fabsf(aqq)) && fabsf(apq) > abs_floor &&
                    fabsf(apq) > 1e-30f) {
                    const float tau = (aqq - app) / (2.f * apq);
                    const float t = (tau >= 0.f) ? 1.f / (tau + sqrtf(1.f + tau * tau))
                                                 : -1.f / (-tau + sqrtf(1.f + tau * tau));
                    c = 1.f / sqrtf(1.f + t * t);
                    s = t * c;
                    s_rot = 1;
                }
                sP[pr] = p; sQ[pr] = q; sC[pr] = c; sS[pr] = s;
            }
            __syncthreads();
            // 32 x 32 thread grid: rows of pair blocks by ti, columns by tj
            const int ti = tid >> 5, tj = tid & 31;
            for (int i = ti; i < half; i += nt >> 5) {
                const int pi = sP[i], qi = sQ[i];
                const float ci = sC[i], si = sS[i];
                float *rp = A + pi * m, *rq = A + qi * m;
                for (int j = tj; j < half; j += 32) {
                    const int pj = sP[j], qj = sQ[j];
                    const float cj = sC[j], sj = sS[j];
                    if (si == 0.f && sj == 0.f) continue;
                    const float b00 = rp[pj], b01 = rp[qj], b10 = rq[pj], b11 = rq[qj];
                    const float m00 = cj * b00 - sj * b01, m01 = sj * b00 + cj * b01;
                    const float m10 = cj * b10 - sj * b11, m11 = sj * b10 + cj * b11;
                    float n01 = ci * m01 - si * m11, n10 = si * m00 + ci * m10;
                    if (i == j) { n01 = 0.f; n10 = 0.f; }
                    rp[pj] = ci * m00 - si * m10; rp[qj] = n01;
                    rq[pj] = n10; rq[qj] = si * m01 + ci * m11;
                }
            }
            // V <- V J on the transposed copy: two contiguous rows per pair
            for (int j = ti; j < half; j += nt >> 5) {
                const float cj = sC[j], sj = sS[j];
                if (sj == 0.f) continue;
                float *vp = Vt + sP[j] * m, *vq = Vt + sQ[j] * m;
                for (int r = tj; r < m; r += 32) {
                    const float a = vp[r], b = vq[r];
                    vp[r] = cj * a - sj * b;
                    vq[r] = sj * a + cj * b;
                }
            }
            __syncthreads();
        }
        done = (s_rot == 0);
        __syncthreads();
    }
    if (tid == 0 && it.sweeps_out) *it.sweeps_out = done ? sweeps : -1;
    // The accumulated rotations are orthogonal only to rounding, and over
    // ~10^3 rotations per index the rounding drifts their scale: with
    // V = U S (U orthogonal, S = diag |v_i|) the diagonal of V^T A V is
    // |v_i|^2 lambda_i.  Take lambda_i = a_ii / |v_i|^2 and unit vectors.
    for (int i = tid; i < n; i += nt) {
        float s2 = 0.f;
        for (int r = 0; r < n; ++r) s2 = fmaf(Vt[i * m + r], Vt[i * m + r], s2);
        const float inv = 1.f / sqrtf(s2);
        A[i * m + i] = A[i * m + i] / s2;
        for (int r = 0; r < n; ++r) Vt[i * m + r] *= inv;
    }
    __syncthreads();
    if (it.raw) {
        // rotation close to the identity for a nearly diagonal input (block Jacobi inner solve)
        for (int e = tid; e < n * n; e += nt) {
            const int r = e / n, c = e % n;
            it.vec[(size_t)r * it.ldv + c] = Vt[c * m + r];
        }
        for (int i = tid; i < n; i += nt) it.lam[i] = A[i * m + i];
        return;
    }
    // sort descending (ties by index), sign-normalise, write out
    for (int i = tid; i < n; i += nt) {
        const float li = A[i * m + i];
        int rank = 0;
        for (int j = 0; j < n; ++j) {
            const float lj = A[j * m + j];
            rank += (lj > li) || (lj == li && j < i);
        }
        int best = 0;
        float bm = -1.f;
        for (int r = 0; r < n; ++r) {
            const float v = fabsf(Vt[i * m + r]);
            if (v > bm) { bm = v; best = r; }
        }
        const float sg = Vt[i * m + best] < 0.f ? -1.f : 1.f;
        it.lam[rank] = li;
        for (int r = 0; r < n; ++r) it.vec[(size_t)r * it.ldv + rank] = sg * Vt[i * m + r];
    }
}

// ====================================================================== block Jacobi helpers
// Large symmetric problems (n > 142) run block Jacobi: the padded N x N matrix
// (N = 64 NB) is kept with the block pairs of the current round adjacent, each
// 128 x 128 pair sub-matrix is diagonalised by k_jacobi_lds, and the block
// rotations are applied with the fp32 GEMM.  These kernels set up, permute,
// measure and finish that iteration.

// a[N][N] = g (n x n, ld) padded with zeros, v = I
__global__ void k_eig_init(EigBatch batch) {
    const EigItem &it = batch.it[blockIdx.y];
    const int64_t NN = (int64_t)it.N * it.N;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < NN; e += (int64_t)gridDim.x * blockDim.x) {
        const int r = (int)(e / it.N), c = (int)(e % it.N);
        it.a[e] = (r < it.n && c < it.n) ? 0.5f * (it.g[(size_t)r * it.ldg + c] + it.g[(size_t)c * it.ldg + r]) : 0.f;
        it.v[e] = (r == c) ? 1.f : 0.f;
    }
}

// 64-wide blocks: a_out[B'][C'] = a_in[src[B']][src[C']], v_out[:, B'] = v_in[:, src[B']]
__global__ void k_block_permute(EigBatch batch, BlockPerm perm) {
    const EigItem &it = batch.it[blockIdx.y];
    const int64_t NN = (int64_t)it.N * it.N;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < NN; e += (int64_t)gridDim.x * blockDim.x) {
        const int r = (int)(e / it.N), c = (int)(e % it.N);
        const int sr = perm.src[r >> 6] * 64 + (r & 63), sc = perm.src[c >> 6] * 64 + (c & 63);
        it.t[e] = it.a[(size_t)sr * it.N + sc];
        it.vt[e] = it.v[(size_t)r * it.N + sc];
    }
}

// out[0] = sum of squares off the diagonal, out[1] = total
__global__ void k_offnorm(EigBatch batch) {
    const EigItem &it = batch.it[blockIdx.x];
    __shared__ float s0[32], s1[32];
    float off = 0.f, tot = 0.f;
    const int64_t NN = (int64_t)it.N * it.N;
    for (int64_t e = threadIdx.x; e < NN; e += blockDim.x) {
        const float v = it.a[e];
        const float q = v * v;
        tot += q;
        if (e / it.N != e % it.N) off += q;
    }
    for (int o = 32; o > 0; o >>= 1) { off += __shfl_xor(off, o); tot += __shfl_xor(tot, o); }
    if ((threadIdx.x & 63) == 0) { s0[threadIdx.x >> 6] = off; s1[threadIdx.x >> 6] = tot; }
    __syncthreads();
    if (threadIdx.x == 0) {
        float a = 0.f, b = 0.f;
        for (int w = 0; w < (int)(blockDim.x >> 6); ++w) { a += s0[w]; b += s1[w]; }
        it.norms[0] = a;
        it.norms[1] = b;
    }
}

// eigenpairs (diag(a), v columns) sorted descending, padding vectors last,
// columns sign-normalised; vec[r][c] (ld ldv) for r, c < n, lam[c]
__global__ void k_eig_finish(EigBatch batch) {
    const EigItem &it = batch.it[blockIdx.y];
    const int N = it.N, n = it.n;
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < N; i += gridDim.x * blockDim.x) {
        // a padding vector has its weight on rows >= n
        float wpad = 0.f;
        for (int r = n; r < N; ++r) wpad += it.v[(size_t)r * N + i] * it.v[(size_t)r * N + i];
        const bool pad = wpad > 0.5f;
        const float li = it.a[(size_t)i * N + i];
        int rank = 0;
        for (int j = 0; j < N; ++j) {
            float wj = 0.f;
            for (int r = n; r < N; ++r) wj += it.v[(size_t)r * N + j] * it.v[(size_t)r * N + j];
            const bool pj = wj > 0.5f;
            const float lj = it.a[(size_t)j * N + j];
            bool before;
            if (pad != pj) before = !pj;                // real vectors first
            else before = (lj > li) || (lj == li && j < i);
            rank += before;
        }
        if (pad || rank >= n) continue;
        int best = 0;
        float bm = -1.f;
        for (int r = 0; r < n; ++r) {
            const float v = fabsf(it.v[(size_t)r * N + i]);
            if (v > bm) { bm = v; best = r; }
        }
        const float sg = it.v[(size_t)best * N + i] < 0.f ? -1.f : 1.f;
        it.lam[rank] = li;
        for (int r = 0; r < n; ++r) it.vec[(size_t)r * it.ldv + rank] = sg * it.v[(size_t)r * N + i];
    }
}

// ====================================================================== batched small kernels
__global__ void k_trace_batch(SmallBatch batch) {
    const SmallItem &it = batch.it[blockIdx.x];
    __shared__ double red[256];
    double s = 0.0;
    for (int i = threadIdx.x; i < it.a; i += blockDim.x) s += (double)it.in[(size_t)i * it.a + i];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int o = blockDim.x / 2; o > 0; o >>= 1) {
        if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
        __syncthreads();
    }
    if (threadIdx.x == 0) *it.out64 = red[0];
}

__global__ void k_energy_batch(SmallBatch batch) {
    const SmallItem &it = batch.it[blockIdx.y];
    const int LH = it.a, rt_max = it.b, d = it.c;
    const int e = blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= rt_max * d) return;
    float s = 0.f;
    for (int lh = 0; lh < LH; ++lh) {
        const float v = it.in[(size_t)lh * rt_max * d + e];
        s = fmaf(v, v, s);
    }
    it.out32[e] = s;
}

// One workgroup per item: step x step block sums, then prefix sums along the
// rows and down the columns of the grid (fp64), then the fixed-rank sum.  The
// grid lives in LDS while it is built when it has at most lds_cells cells
// (the prefix sums are chains of dependent read-modify-writes), else in place
// in global memory; either way the same additions in the same order.
__global__ __launch_bounds__(256) void k_energy_grid(GridBatch batch, int lds_cells) {
    extern __shared__ double sgrid[];
    __shared__ double red[4];
    const GridItem &it = batch.it[blockIdx.x];
    const int tid = threadIdx.x, nr = it.nr, nf = it.nf, st = it.step, d = it.d;
    const bool in_lds = nr * nf <= lds_cells;
    double *S = in_lds ? sgrid : it.S;
    for (int c = tid; c < nr * nf; c += 256) {
        const int bi = c / nf, bj = c - bi * nf;
        double s = 0.0;
        for (int r = bi * st; r < (bi + 1) * st; ++r) {
            const float *row = it.E + (size_t)r * d + bj * st;
#pragma unroll 8
            for (int f = 0; f < st; ++f) s += (double)row[f];
        }
        S[c] = s;
    }
    __syncthreads();
    for (int bi = tid; bi < nr; bi += 256)
        for (int bj = 1; bj < nf; ++bj) S[bi * nf + bj] += S[bi * nf + bj - 1];
    __syncthreads();
    for (int bj = tid; bj < nf; bj += 256)
        for (int bi = 1; bi < nr; ++bi) S[bi * nf + bj] += S[(bi - 1) * nf + bj];
    __syncthreads();
    if (in_lds)
        for (int c = tid; c < nr * nf; c += 256) it.S[c] = S[c];
    if (it.frt > 0 && it.frf > 0) {
        double s = 0.0;
        for (int e = tid; e < it.frt * it.frf; e += 256) {
            const int r = e / it.frf, f = e - r * it.frf;
            s += (double)it.E[(size_t)r * d + f];
        }
        for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
        if ((tid & 63) == 0) red[tid >> 6] = s;
        __syncthreads();
        if (tid == 0) *it.s_fixed = (red[0] + red[1]) + (red[2] + red[3]);
    } else if (tid == 0) {
        *it.s_fixed = 0.0;
    }
}

__global__ void k_to_bf16_batch(SmallBatch batch) {
    const SmallItem &it = batch.it[blockIdx.y];
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < it.count; i += (int64_t)gridDim.x * blockDim.x) {
        const float v = it.in[i];
        const uint16_t h = f32_to_bf16(v);
        it.hi[i] = h;
        if (it.lo) it.lo[i] = f32_to_bf16(v - bf16_to_f32(h));
    }
}

// omt[c][r] = Omega[r][c] (+-1, counter r k + c of stream 1), zero rows c >= k;
// each thread takes 8 consecutive r of one row c (n is a multiple of 8), one
// 16-byte store of bf16 or two of fp32
__global__ void k_gen_omega_batch(SmallBatch batch) {
    const SmallItem &it = batch.it[blockIdx.y];
    const int k = it.a, kp = it.b;
    const uint32_t n8 = (uint32_t)(it.count / kp / 8), total = (uint32_t)kp * n8;
    for (uint32_t g = blockIdx.x * blockDim.x + threadIdx.x; g < total; g += gridDim.x * blockDim.x) {
        const int c = (int)(g / n8);
        const uint64_t r0 = (uint64_t)(g - (uint32_t)c * n8) * 8;
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = (c < k) ? rademacher(it.key, 1, (r0 + u) * (uint64_t)k + c) : 0.f;
        const size_t e = (size_t)c * n8 * 8 + r0;
        if (it.hi) {
            uint32_t w[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) w[u] = (uint32_t)f32_to_bf16(v[2 * u]) | ((uint32_t)f32_to_bf16(v[2 * u + 1]) << 16);
            *reinterpret_cast<uint4 *>(it.hi + e) = make_uint4(w[0], w[1], w[2], w[3]);
        }
        if (it.out32) {
            *reinterpret_cast<float4 *>(it.out32 + e) = make_float4(v[0], v[1], v[2], v[3]);
            *reinterpret_cast<float4 *>(it.out32 + e + 4) = make_float4(v[4], v[5], v[6], v[7]);
        }
    }
}

// ====================================================================== small helpers
__global__ void k_to_bf16(const float *in, uint16_t *hi, uint16_t *lo, int64_t count) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= count) return;
    const float v = in[i];
    const uint16_t h = f32_to_bf16(v);
    hi[i] = h;
    if (lo) lo[i] = f32_to_bf16(v - bf16_to_f32(h));
}

__global__ void k_transpose(const float *in, float *out, int rows, int cols, int ldi, int ldo) {
    __shared__ float tile[32][33];
    const int r0 = blockIdx.y * 32, c0 = blockIdx.x * 32;
    for (int i = threadIdx.y; i < 32; i += blockDim.y) {
        const int r = r0 + i, c = c0 + threadIdx.x;
        if (r < rows && c < cols) tile[i][threadIdx.x] = in[(size_t)r * ldi + c];
    }
    __syncthreads();
    for (int i = threadIdx.y; i < 32; i += blockDim.y) {
        const int c = c0 + i, r = r0 + threadIdx.x;
        if (r < rows && c < cols) out[(size_t)c * ldo + r] = tile[threadIdx.x][i];
    }
}

__global__ void k_zero(uint32_t *p, size_t words) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < words) p[i] = 0;
}

// ====================================================================== parameter store
template <typename T>
__device__ __forceinline__ void put_param(uint8_t *base, size_t idx, float v) {
    if (sizeof(T) == 2) reinterpret_cast<uint16_t *>(base)[idx] = f32_to_bf16(v);
    else reinterpret_cast<float *>(base)[idx] = v;
}

// Workgroups [0, tiles) transpose U~_t ([rt_max][T] in the plan, [T][rt]
// in the payload) through a 64 x 65 LDS tile, so that both the reads and the
// writes run along rows; the rest write U~_f, C~ and the header element by
// element (32-bit index math: the launcher checks the sizes).
template <typename T>
__global__ __launch_bounds__(256) void k_store(StoreBatch batch, int tiles) {
    __shared__ float tile[64][65];
    const StoreItem &it = batch.it[blockIdx.y];
    const int tid = threadIdx.x;
    if ((int)blockIdx.x < tiles) {
        const int ntt = (it.T + 63) / 64, ntr = (it.rt + 63) / 64;
        for (int tb = blockIdx.x; tb < ntt * ntr; tb += tiles) {
            const int t0 = 64 * (tb % ntt), r0 = 64 * (tb / ntt);
            __syncthreads();
            for (int e = tid; e < 64 * 64; e += 256) {
                const int r = e >> 6, t = e & 63;
                if (r0 + r < it.rt && t0 + t < it.T) tile[r][t] = it.ut[(size_t)(r0 + r) * it.T + t0 + t];
            }
            __syncthreads();
            for (int e = tid; e < 64 * 64; e += 256) {
                const int t = e >> 6, r = e & 63;
                if (r0 + r < it.rt && t0 + t < it.T)
                    put_param<T>(it.pay + it.off_ut, (size_t)(t0 + t) * it.rt + r0 + r, tile[r][t]);
            }
        }
        return;
    }
    const uint32_t n_uf = (uint32_t)it.d * it.rf, rr = (uint32_t)it.rt * it.rf, n_c = (uint32_t)it.LH * rr;
    const uint32_t total = n_uf + n_c + 16;
    for (uint32_t e = (blockIdx.x - tiles) * 256 + tid; e < total; e += (gridDim.x - tiles) * 256) {
        if (e < n_uf) {
            const uint32_t f = e / it.rf, j = e - f * it.rf;
            put_param<T>(it.pay + it.off_uf, e, it.uf[(size_t)f * it.d + j]);
        } else if (e < n_uf + n_c) {
            const uint32_t q = e - n_uf, lh = q / rr, rem = q - lh * rr, r = rem / it.rf, j = rem - r * it.rf;
            put_param<T>(it.pay + it.off_core, q, it.core[((size_t)lh * it.rt_max + r) * it.d + j]);
        } else {
            const uint32_t w = e - n_uf - n_c;
            reinterpret_cast<uint32_t *>(it.pay)[w] = it.header[w];
        }
    }
}

// ====================================================================== launchers
// Dynamic LDS above the default cap needs the per-kernel attribute; the cap
// plus the kernel's static LDS must stay within the 160 KB of a workgroup.
static hipError_t allow_dynamic_lds(const void *fn) {
    hipFuncAttributes fa;
    hipError_t e = hipFuncGetAttributes(&fa, fn);
    if (e != hipSuccess) return e;
    const int cap = 160 * 1024 - (int)fa.sharedSizeBytes;
    return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, cap);
}
static hipError_t ensure_lds_attrs() {
    static hipError_t state = hipErrorNotReady;
    if (state == hipErrorNotReady) {
        hipError_t e = allow_dynamic_lds(reinterpret_cast<const void *>(k_jacobi_lds<1024, JacBatch>));
        if (e == hipSuccess) e = allow_dynamic_lds(reinterpret_cast<const void *>(k_jacobi_lds<1024, JacTable>));
        if (e == hipSuccess) e = allow_dynamic_lds(reinterpret_cast<const void *>(k_cholesky));
        if (e == hipSuccess) e = allow_dynamic_lds(reinterpret_cast<const void *>(k_trsm));
        state = e;
    }
    return state;
}

template <typename T, int NF, int KC, int R = 2, int NWV = 4>
static hipError_t xm_launch(const XmBatch &b, int d, dim3 g, int tiles, hipStream_t s) {
    const size_t lds = (size_t)2 * 32 * NF * XmTile<T, KC>::KP * sizeof(T);
    const auto k = k_xm<T, NF, KC, R, NWV>;
    static hipError_t attr = hipErrorNotReady;
    if (attr == hipErrorNotReady) attr = allow_dynamic_lds(reinterpret_cast<const void *>(k));
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(k, g, dim3(64 * NWV), lds, s, b, d, tiles);
    return hipGetLastError();
}

// chunks of 64 features (128 measured slower: the wider tile spills)
template <typename T>
static hipError_t xm_nf(const XmBatch &b, int d, dim3 g, int nf, int tiles, hipStream_t s) {
    switch (nf) {
        case 1: return xm_launch<T, 1, 64>(b, d, g, tiles, s);
        case 2: return xm_launch<T, 2, 64>(b, d, g, tiles, s);
        case 3: return xm_launch<T, 3, 64>(b, d, g, tiles, s);
        case 4: return xm_launch<T, 4, 64>(b, d, g, tiles, s);
        default: break;
    }
    if constexpr (sizeof(T) == 2) {      // wider tiles fit the registers in bf16 only
        if (nf == 5) return xm_launch<T, 5, 64>(b, d, g, tiles, s);
        if (nf == 6) return xm_launch<T, 6, 64>(b, d, g, tiles, s);
        if (nf == 9) return xm_launch<T, 9, 64, 1, 8>(b, d, g, tiles, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_xm(const XmBatch &b, int dtype, int d, int maxT, int maxCols, int maxSplit, hipStream_t s) {
    if (b.n <= 0) return hipSuccess;
    if (d % 64) return hipErrorInvalidValue;
    KTimeScope kts("k_xm", s);
    int nf = (maxCols + 31) / 32;
    int tiles = 1;
    // bf16: up to 6 fragments in one tile, and 7 to 9 as one tile of 9 (the
    // whole sketch of an r_t = 256 plan in one pass over x); otherwise tiles of 4
    if (dtype == JOLT_BF16 && nf >= 7 && nf <= 9) nf = 9;
    else if (nf > (dtype == JOLT_BF16 ? 6 : 4)) { tiles = (nf + 3) / 4; nf = 4; }
    dim3 g((maxT + 255) / 256, tiles * maxSplit, b.n);
    return dtype == JOLT_BF16 ? xm_nf<uint16_t>(b, d, g, nf, tiles, s) : xm_nf<float>(b, d, g, nf, tiles, s);
}

template <typename T, int NF, bool LO, int R = 2, int NWV = 4>
static hipError_t xtq_launch(const XtqBatch &b, int d, dim3 g, int maxSplit, hipStream_t s) {
    const auto k = k_xtq<T, NF, LO, R, NWV>;
    static hipError_t attr = hipErrorNotReady;
    if (attr == hipErrorNotReady) attr = allow_dynamic_lds(reinterpret_cast<const void *>(k));
    if (attr != hipSuccess) return attr;
    const size_t lds = XtqTile<T, NF, LO, 64 * NWV>::lds_bytes;
    hipLaunchKernelGGL(k, g, dim3(64 * NWV), lds, s, b, d, maxSplit);
    return hipGetLastError();
}

template <typename T, bool LO>
static hipError_t xtq_nf(const XtqBatch &b, int d, dim3 g, int nf, int maxSplit, hipStream_t s) {
    switch (nf) {
        case 1: return xtq_launch<T, 1, LO>(b, d, g, maxSplit, s);
        case 2: return xtq_launch<T, 2, LO>(b, d, g, maxSplit, s);
        case 3: return xtq_launch<T, 3, LO>(b, d, g, maxSplit, s);
        case 4: return xtq_launch<T, 4, LO>(b, d, g, maxSplit, s);
        case 5: return xtq_launch<T, 5, LO>(b, d, g, maxSplit, s);
        default: break;
    }
    if constexpr (sizeof(T) == 2)
        if (nf == 9) return xtq_launch<T, 9, LO, 1, 8>(b, d, g, maxSplit, s);
    return hipErrorInvalidValue;
}

hipError_t launch_xtq(const XtqBatch &b, int dtype, int d, int maxLH, int maxSplit, int maxCols, hipStream_t s) {
    if (b.n <= 0) return hipSuccess;
    if (d % 32) return hipErrorInvalidValue;
    for (int i = 0; i < b.n; ++i)
        if (b.it[i].T % 64 || b.it[i].tsplit % 64) return hipErrorInvalidValue;
    KTimeScope kts("k_xtq", s);
    // column tiles of at most 5 fragments (160 columns); bf16 sketches of 7 to 9
    // fragments as one tile of 9 (x read once)
    const int frags = (maxCols + 31) / 32;
    int ctiles = (frags + 4) / 5, nf = (frags + ctiles - 1) / ctiles;
    if (dtype == JOLT_BF16 && frags >= 7 && frags <= 9) { ctiles = 1; nf = 9; }
    dim3 g(maxSplit * ctiles, (maxLH * d + 255) / 256, b.n);
    const bool lo = b.it[0].ql != nullptr;
    if (dtype == JOLT_BF16)
        return lo ? xtq_nf<uint16_t, true>(b, d, g, nf, maxSplit, s) : xtq_nf<uint16_t, false>(b, d, g, nf, maxSplit, s);
    return xtq_nf<float, false>(b, d, g, nf, maxSplit, s);
}

hipError_t launch_gram_rows(const GramBatch &b, int dtype, int d, int maxP, hipStream_t s) {
    if (b.n <= 0) return hipSuccess;
    KTimeScope kts("k_gram_rows", s);
    dim3 g(maxP, 1, b.n);
    if (dtype == JOLT_BF16) hipLaunchKernelGGL(k_gram_rows<uint16_t>, g, dim3(256), 0, s, b, d);
    else hipLaunchKernelGGL(k_gram_rows<float>, g, dim3(256), 0, s, b, d);
    return hipGetLastError();
}

hipError_t launch_reduce(const ReduceBatch &b, int64_t maxCount, hipStream_t s) {
    if (b.n <= 0 || maxCount <= 0) return hipSuccess;
    KTimeScope kts("k_reduce", s);
    dim3 g((unsigned)((maxCount + 1023) / 1024), b.n);        // 4 entries per thread
    hipLaunchKernelGGL(k_reduce, g, dim3(256), 0, s, b);
    return hipGetLastError();
}

hipError_t launch_cholesky(const CholBatch &b, int maxK, hipStream_t s) {
    if (b.n <= 0) return hipSuccess;
    // items with inverse != 0 go to the fused elimination, the rest to the factor
    CholBatch inv{}, fac{};
    int maxInv = 0, maxFac = 0;
    for (int i = 0; i < b.n; ++i) {
        if (b.it[i].inverse) { inv.it[inv.n++] = b.it[i]; maxInv = std::max(maxInv, b.it[i].k); }
        else { fac.it[fac.n++] = b.it[i]; maxFac = std::max(maxFac, b.it[i].k); }
    }
    if (hipError_t e = launch_chol_inv(inv, maxInv, s); e != hipSuccess) return e;
    if (fac.n == 0) return hipSuccess;
    if (hipError_t e = ensure_lds_attrs(); e != hipSuccess) return e;
    const size_t lds = (size_t)maxFac * (maxFac + 1) / 2 * sizeof(float);
    hipLaunchKernelGGL(k_cholesky, dim3(fac.n), dim3(1024), lds, s, fac);
    return hipGetLastError();
}

hipError_t launch_trsm(const TrsmBatch &b, int maxK, int maxLen, hipStream_t s) {
    if (b.n <= 0) return hipSuccess;
    if (hipError_t e = ensure_lds_attrs(); e != hipSuccess) return e;
    size_t lds = ((size_t)maxK * 33 + (size_t)maxK * (maxK + 1) / 2) * sizeof(float);
    const int l_in_lds = lds <= 150 * 1024;
    if (!l_in_lds) lds = (size_t)maxK * 33 * sizeof(float);
    hipLaunchKernelGGL(k_trsm, dim3((maxLen + 31) / 32, b.n), dim3(1024), lds, s, b, l_in_lds);
    return hipGetLastError();
}

template <class B>
static hipError_t jacobi_lds(int count, const B &b, int maxN, int max_sweeps, hipStream_t s, int retry_only) {
    if (count <= 0) return hipSuccess;
    if (hipError_t e = ensure_lds_attrs(); e != hipSuccess) return e;
    KTimeScope kts("k_jacobi_lds", s);
    const int m = maxN + (maxN & 1);
    const size_t lds = (size_t)2 * m * m * sizeof(float);
    hipLaunchKernelGGL((k_jacobi_lds<1024, B>), dim3(count), dim3(1024), lds, s, b, max_sweeps, retry_only);
    return hipGetLastError();
}
hipError_t launch_jacobi_lds(const JacBatch &b, int maxN, int max_sweeps, hipStream_t s, int retry_only) {
    return jacobi_lds(b.n, b, maxN, max_sweeps, s, retry_only);
}
hipError_t launch_jacobi_lds(const JacItem *, const JacTable &dev, int maxN, int max_sweeps, hipStream_t s,
                             int retry_only) {
    return jacobi_lds(dev.n, dev, maxN, max_sweeps, s, retry_only);
}

// ---------------------------------------------------------------- item tables
// A table chunk travels as the kernel's argument (under the 4 KB argument
// limit) and is written to device memory by one workgroup.
constexpr int kTableWords = 992;
struct TableChunk {
    uint32_t w[kTableWords];
    uint32_t *dst;
    int n;
};
__global__ __launch_bounds__(256) void k_put_table(TableChunk c) {
    for (int i = threadIdx.x; i < c.n; i += 256) c.dst[i] = c.w[i];
}
hipError_t launch_put_table(const void *host, size_t bytes, void *dev, hipStream_t s) {
    if (bytes % 4 || reinterpret_cast<uintptr_t>(dev) % 4) return hipErrorInvalidValue;
    const uint32_t *src = static_cast<const uint32_t *>(host);
    uint32_t *dst = static_cast<uint32_t *>(dev);
    for (size_t w0 = 0; w0 < bytes / 4; w0 += kTableWords) {
        TableChunk c;
        c.n = (int)std::min<size_t>(kTableWords, bytes / 4 - w0);
        c.dst = dst + w0;
        std::memcpy(c.w, src + w0, (size_t)c.n * 4);
        hipLaunchKernelGGL(k_put_table, dim3(1), dim3(256), 0, s, c);
        if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_eig_init(const EigBatch &b, int maxN, hipStream_t s) {
    if (b.n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_eig_init, dim3(std::min(1024, (maxN * maxN + 255) / 256), b.n), dim3(256), 0, s, b);
    return hipGetLastError();
}
hipError_t launch_block_permute(const EigBatch &b, const BlockPerm &p, int maxN, hipStream_t s) {
    if (b.n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_block_permute, dim3(std::min(2048, (maxN * maxN + 255) / 256), b.n), dim3(256), 0, s, b, p);
    return hipGetLastError();
}
hipError_t launch_offnorm(const EigBatch &b, hipStream_t s) {
    if (b.n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_offnorm, dim3(b.n), dim3(1024), 0, s, b);
    return hipGetLastError();
}
hipError_t launch_eig_finish(const EigBatch &b, int maxN, hipStream_t s) {
    if (b.n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_eig_finish, dim3((maxN + 63) / 64, b.n), dim3(64), 0, s, b);
    return hipGetLastError();
}

hipError_t launch_trace_batch(const SmallBatch &b, hipStream_t s) {
    if (b.n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_trace_batch, dim3(b.n), dim3(256), 0, s, b);
    return hipGetLastError();
}
hipError_t launch_energy_batch(const SmallBatch &b, int64_t maxCount, hipStream_t s) {
    if (b.n <= 0 || maxCount <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_energy_batch, dim3((unsigned)((maxCount + 255) / 256), b.n), dim3(256), 0, s, b);
    return hipGetLastError();
}
hipError_t launch_energy_grid(const GridBatch &b, hipStream_t s) {
    if (b.n <= 0) return hipSuccess;
    int cells = 0;
    for (int i = 0; i < b.n; ++i) cells = std::max(cells, b.it[i].nr * b.it[i].nf);
    const int lds_cells = cells <= 8000 ? cells : 0;        // within the default 64 KiB of LDS
    hipLaunchKernelGGL(k_energy_grid, dim3(b.n), dim3(256), (size_t)lds_cells * sizeof(double), s, b, lds_cells);
    return hipGetLastError();
}
hipError_t launch_to_bf16_batch(const SmallBatch &b, int64_t maxCount, hipStream_t s) {
    if (b.n <= 0 || maxCount <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_to_bf16_batch, dim3((unsigned)std::min<int64_t>(2048, (maxCount + 255) / 256), b.n), dim3(256),
                       0, s, b);
    return hipGetLastError();
}
hipError_t launch_gen_omega_batch(const SmallBatch &b, int64_t maxCount, hipStream_t s) {
    if (b.n <= 0 || maxCount <= 0) return hipSuccess;
    for (int i = 0; i < b.n; ++i) {
        const SmallItem &it = b.it[i];
        const int64_t n = it.b > 0 ? it.count / it.b : 0;
        if (it.b <= 0 || it.count % it.b || n % 8 || it.count / 8 > 0xFFFFFFFFll) return hipErrorInvalidValue;
    }
    hipLaunchKernelGGL(k_gen_omega_batch, dim3((unsigned)std::min<int64_t>(2048, (maxCount / 8 + 255) / 256), b.n),
                       dim3(256), 0, s, b);
    return hipGetLastError();
}

hipError_t launch_to_bf16(const float *in, uint16_t *hi, uint16_t *lo, int64_t count, hipStream_t s) {
    if (count <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_to_bf16, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, s, in, hi, lo, count);
    return hipGetLastError();
}

hipError_t launch_transpose(const float *in, float *out, int rows, int cols, int ldi, int ldo, hipStream_t s) {
    if (rows <= 0 || cols <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_transpose, dim3((cols + 31) / 32, (rows + 31) / 32), dim3(32, 8), 0, s, in, out, rows, cols,
                       ldi, ldo);
    return hipGetLastError();
}

hipError_t launch_zero(void *p, size_t bytes, hipStream_t s) {
    const size_t words = bytes / 4;
    if (words == 0) return hipSuccess;
    hipLaunchKernelGGL(k_zero, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, s, static_cast<uint32_t *>(p), words);
    return hipGetLastError();
}

hipError_t launch_store(const StoreBatch &b, int dtype, hipStream_t s) {
    if (b.n <= 0) return hipSuccess;
    uint64_t maxElem = 0;
    int tiles = 1;
    for (int i = 0; i < b.n; ++i) {
        const StoreItem &it = b.it[i];
        const uint64_t e = (uint64_t)it.d * it.rf + (uint64_t)it.LH * it.rt * it.rf + 16;
        if (e > 0xFFFFFFFFull) return hipErrorInvalidValue;
        maxElem = std::max(maxElem, e);
        tiles = std::max(tiles, std::min(512, ((it.T + 63) / 64) * ((it.rt + 63) / 64)));
    }
    dim3 g(tiles + (unsigned)std::min<uint64_t>(512, (maxElem + 255) / 256), b.n);
    if (dtype == JOLT_BF16) hipLaunchKernelGGL(k_store<uint16_t>, g, dim3(256), 0, s, b, tiles);
    else hipLaunchKernelGGL(k_store<float>, g, dim3(256), 0, s, b, tiles);
    return hipGetLastError();
}

}  // namespace jolt
