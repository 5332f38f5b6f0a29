// libjolt C ABI: handle, validation, sizes, payload header, compress / decompress
// orchestration and the test hooks.  The factorisation half of jolt_plan lives
// in plan.cpp.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "api_internal.h"
#include "attn.h"
#include "jolt_internal.h"
#include "payload.h"
#include "ktimer.h"
#include "plan_kernels.h"
#include "planner.h"

using namespace jolt;

struct jolt_handle_s {
    int device = 0;
    std::string err;
    hipStream_t side = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
    jolt::DualTables dual;
    uint8_t *readback = nullptr;    // pinned host memory for the plan's one readback
    size_t readback_cap = 0;
    float *sweep = nullptr;         // pinned host memory for block Jacobi's per-sweep norms
    void *scratch = nullptr;        // this device's address of the fixed scratch array
};

namespace jolt {

// ---------------------------------------------------------------- fixed device scratch
// The W~ workspace of jolt_decompress_noalloc: a file-scope device array, one
// copy per GPU for the life of the process.  Host code never uses the array's
// name as an address: jolt_create takes each device's address of it once, with
// that device current, and kernels get that address.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];
constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void *g_scratch_ptr[kMaxDevices];

static hipError_t scratch_address(int device, void **out) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    if (!g_scratch_ptr[device]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[device] = p;
    }
    *out = g_scratch_ptr[device];
    return hipSuccess;
}

jolt_status fail(jolt_handle h, jolt_status s, const char *fmt, ...) {
    if (h) {
        char buf[512];
        va_list ap;
        va_start(ap, fmt);
        vsnprintf(buf, sizeof buf, fmt, ap);
        va_end(ap);
        h->err = buf;
    }
    return s;
}

jolt_status hip_fail(jolt_handle h, hipError_t e, const char *where) {
    return fail(h, JOLT_E_DEVICE, "%s: %s", where, hipGetErrorString(e));
}

void clear_err(jolt_handle h) {
    if (h) h->err.clear();
}

DualTables &dual_tables(jolt_handle h) { return h->dual; }

hipError_t readback_buffer(jolt_handle h, size_t bytes, uint8_t **buf) {
    if (bytes > h->readback_cap) {
        // every earlier use ended with its stream synchronised, so the old
        // buffer is idle
        if (h->readback) (void)hipHostFree(h->readback);
        h->readback = nullptr;
        h->readback_cap = 0;
        const size_t cap = std::max<size_t>(bytes, 64 * 1024);
        if (hipError_t e = hipHostMalloc(reinterpret_cast<void **>(&h->readback), cap, hipHostMallocDefault);
            e != hipSuccess)
            return e;
        h->readback_cap = cap;
    }
    *buf = h->readback;
    return hipSuccess;
}

hipError_t sweep_buffer(jolt_handle h, float **buf) {
    if (!h->sweep)
        if (hipError_t e = hipHostMalloc(reinterpret_cast<void **>(&h->sweep), 2 * kMaxBatch * sizeof(float),
                                         hipHostMallocDefault);
            e != hipSuccess) {
            h->sweep = nullptr;
            return e;
        }
    *buf = h->sweep;
    return hipSuccess;
}

hipError_t side_stream(jolt_handle h, hipStream_t *st, hipEvent_t *fork, hipEvent_t *join) {
    if (!h->side) {
        hipStream_t s = nullptr;
        hipEvent_t f = nullptr, j = nullptr;
        hipError_t e = hipStreamCreateWithFlags(&s, hipStreamNonBlocking);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&f, hipEventDisableTiming);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&j, hipEventDisableTiming);
        if (e != hipSuccess) {
            if (j) (void)hipEventDestroy(j);
            if (f) (void)hipEventDestroy(f);
            if (s) (void)hipStreamDestroy(s);
            return e;
        }
        h->side = s;
        h->fork = f;
        h->join = j;
    }
    *st = h->side;
    *fork = h->fork;
    *join = h->join;
    return hipSuccess;
}

void drain_streams(jolt_handle h) {
    if (h->side) (void)hipStreamSynchronize(h->side);
}

void sign_bits_for(uint64_t seed, uint32_t item_id, int d, uint32_t out[4]) {
    const uint64_t key = item_key(seed, item_id);
    out[0] = out[1] = out[2] = out[3] = 0;
    for (int f = 0; f < d; ++f)
        if (rademacher(key, 0, (uint64_t)f) < 0.f) out[f >> 5] |= 1u << (f & 31);
}

jolt_status check_item(jolt_handle h, const jolt_item &it) {
    if (it.L < 1 || it.H < 1 || it.T < 1) return fail(h, JOLT_E_INVALID, "item: L, H, T must be >= 1");
    if (it.d != 64 && it.d != 128) return fail(h, JOLT_E_UNSUPPORTED, "item: d must be 64 or 128 (got %d)", it.d);
    if (it.dtype != JOLT_BF16 && it.dtype != JOLT_F32) return fail(h, JOLT_E_INVALID, "item: unknown dtype");
    const double N = (double)it.L * it.H * it.T * it.d;
    if (N > 2147483647.0 || (double)it.L * it.H * it.T > 268435455.0)
        return fail(h, JOLT_E_UNSUPPORTED, "item: more than 2^31 elements");
    return JOLT_OK;
}

jolt_status check_alloc(jolt_handle h, const jolt_item &it, const jolt_alloc &a) {
    if (a.rt < 0 || a.rf < 0 || a.rt > it.T || a.rf > it.d || a.rt > 256)
        return fail(h, JOLT_E_INVALID, "alloc: ranks must satisfy 0 <= rt <= min(T, 256), 0 <= rf <= d");
    if (a.bits < 0 || a.bits == 1 || a.bits > 8) return fail(h, JOLT_E_INVALID, "alloc: bits must be 0 or 2..8");
    return JOLT_OK;
}

jolt_status check_items_uniform(jolt_handle h, const jolt_item *items, int n) {
    if (n < 0) return fail(h, JOLT_E_INVALID, "n < 0");
    if (n > 0 && !items) return fail(h, JOLT_E_INVALID, "items is NULL");
    for (int i = 0; i < n; ++i) {
        jolt_status s = check_item(h, items[i]);
        if (s) return s;
        if (items[i].dtype != items[0].dtype || items[i].d != items[0].d)
            return fail(h, JOLT_E_UNSUPPORTED, "all items of one call must share dtype and d");
    }
    return JOLT_OK;
}

}  // namespace jolt

// --------------------------------------------------------------------------- lifetime
extern "C" jolt_status jolt_create(int hip_device, jolt_handle *out) {
    if (!out) return JOLT_E_INVALID;
    *out = nullptr;
    int count = 0;
    hipError_t e = hipGetDeviceCount(&count);
    if (e != hipSuccess || hip_device < 0 || hip_device >= count) return JOLT_E_DEVICE;
    e = hipSetDevice(hip_device);
    if (e != hipSuccess) return JOLT_E_DEVICE;
    void *sp = nullptr;
    e = scratch_address(hip_device, &sp);      // the fixed scratch's address on this device
    if (e != hipSuccess) return JOLT_E_DEVICE;
    jolt_handle h = new jolt_handle_s();
    h->device = hip_device;
    h->scratch = sp;
    *out = h;
    return JOLT_OK;
}

extern "C" void jolt_destroy(jolt_handle h) {
    if (!h) return;
    if (h->side) {
        (void)hipSetDevice(h->device);
        (void)hipStreamSynchronize(h->side);
        (void)hipEventDestroy(h->join);
        (void)hipEventDestroy(h->fork);
        (void)hipStreamDestroy(h->side);
    }
    if (h->readback) (void)hipHostFree(h->readback);
    if (h->sweep) (void)hipHostFree(h->sweep);
    delete h;
}

extern "C" const char *jolt_status_str(jolt_status s) {
    switch (s) {
        case JOLT_OK: return "ok";
        case JOLT_E_INVALID: return "invalid argument";
        case JOLT_E_UNSUPPORTED: return "unsupported";
        case JOLT_E_WORKSPACE: return "workspace too small";
        case JOLT_E_INFEASIBLE: return "budget infeasible";
        case JOLT_E_NOCONV: return "eigensolver did not converge";
        case JOLT_E_DEVICE: return "device error";
        case JOLT_E_CORRUPT: return "corrupt payload";
    }
    return "unknown status";
}

extern "C" const char *jolt_last_error(jolt_handle h) { return h ? h->err.c_str() : ""; }

// --------------------------------------------------------------------------- sizes
extern "C" int64_t jolt_item_bytes(const jolt_item *it, int32_t rt, int32_t rf, int32_t bits) {
    if (!it) return -1;
    return item_bytes_impl(it->L, it->H, it->T, it->d, elem_bytes(it->dtype), rt, rf, bits);
}

extern "C" jolt_status jolt_payload_layout(const jolt_item *it, const jolt_alloc *a, size_t offsets[5],
                                           size_t *total) {
    if (!it || !a) return JOLT_E_INVALID;
    jolt_status s = check_item(nullptr, *it);
    if (s) return s;
    s = check_alloc(nullptr, *it, *a);
    if (s) return s;
    PayloadLayout p = payload_layout(*it, a->rt, a->rf, a->bits);
    if (offsets) {
        offsets[0] = p.ut; offsets[1] = p.uf; offsets[2] = p.core; offsets[3] = p.scales; offsets[4] = p.codes;
    }
    if (total) *total = p.total;
    return JOLT_OK;
}

extern "C" jolt_status jolt_payload_size(const jolt_item *it, const jolt_alloc *a, size_t *bytes) {
    return jolt_payload_layout(it, a, nullptr, bytes);
}

extern "C" jolt_status jolt_payload_header(const jolt_item *it, const jolt_alloc *a, void *header64) {
    if (!it || !a || !header64) return JOLT_E_INVALID;
    jolt_status s = check_item(nullptr, *it);
    if (s) return s;
    s = check_alloc(nullptr, *it, *a);
    if (s) return s;
    make_header(*it, *a, static_cast<uint8_t *>(header64));
    return JOLT_OK;
}

extern "C" jolt_status jolt_payload_validate(const void *header64, const jolt_item *it, const jolt_alloc *a) {
    if (!header64 || !it || !a) return JOLT_E_INVALID;
    jolt_status s = check_item(nullptr, *it);
    if (s) return s;
    s = check_alloc(nullptr, *it, *a);
    if (s) return s;
    uint8_t want[64];
    make_header(*it, *a, want);
    return std::memcmp(want, header64, 64) == 0 ? JOLT_OK : JOLT_E_CORRUPT;
}

extern "C" jolt_status jolt_workspace_size(const jolt_config *cfg, const jolt_item *items, int32_t n,
                                           size_t *plan_ws_bytes, size_t *codec_ws_bytes) {
    if (!cfg) return JOLT_E_INVALID;
    jolt_status s = check_items_uniform(nullptr, items, n);
    if (s) return s;
    PlanLayout pl;
    s = plan_layout(*cfg, items, n, &pl);
    if (s) return s;
    if (plan_ws_bytes) *plan_ws_bytes = pl.total;
    std::vector<int> rt(n, pl.rt_max);
    if (codec_ws_bytes) *codec_ws_bytes = std::max<size_t>(256, codec_ws_bytes_for(items, n, rt.data()));
    return JOLT_OK;
}

extern "C" jolt_status jolt_plan_factors(const jolt_config *cfg, const jolt_item *items, int32_t n,
                                         const void *plan_ws, int32_t i, jolt_factor_view *out) {
    if (!cfg || !out || !plan_ws || i < 0 || i >= n) return JOLT_E_INVALID;
    PlanLayout pl;
    jolt_status s = plan_layout(*cfg, items, n, &pl);
    if (s) return s;
    const uint8_t *b = static_cast<const uint8_t *>(plan_ws);
    const FactorOffsets &o = pl.item[i];
    out->ut = reinterpret_cast<const float *>(b + o.ut);
    out->uf = reinterpret_cast<const float *>(b + o.uf);
    out->lam_t = reinterpret_cast<const float *>(b + o.lam_t);
    out->lam_f = reinterpret_cast<const float *>(b + o.lam_f);
    out->core = reinterpret_cast<const float *>(b + o.core);
    out->energy = reinterpret_cast<const float *>(b + o.energy);
    out->normx2 = reinterpret_cast<const double *>(b + o.normx2);
    out->rt_max = pl.rt_max;
    out->rf_max = pl.rf_max;
    return JOLT_OK;
}

// --------------------------------------------------------------------------- allocation hook
extern "C" jolt_status jolt_plan_from_tables(int32_t n, const int32_t *n_cand, const int32_t *const *cand,
                                             const double *const *D, const int64_t *const *B, int64_t budget,
                                             jolt_alloc *out, double *lambda_out) {
    if (n <= 0 || !n_cand || !cand || !D || !B || !out) return JOLT_E_INVALID;
    std::vector<const Cand *> cp(n);
    for (int i = 0; i < n; ++i) cp[i] = reinterpret_cast<const Cand *>(cand[i]);
    std::vector<int> choice(n);
    jolt_status s = allocate(n, n_cand, cp.data(), D, B, budget, choice.data(), lambda_out);
    for (int i = 0; i < n; ++i) {
        const Cand &c = cp[i][choice[i]];
        out[i].rt = c.rt; out[i].rf = c.rf; out[i].bits = c.bits; out[i].reserved = 0;
        out[i].bytes = B[i][choice[i]];
        out[i].distortion = D[i][choice[i]];
    }
    return s;
}

// --------------------------------------------------------------------------- codec orchestration
namespace jolt {

// W~ for every item from its payload parameters, into codec_ws (rot: the
// encoder's rotated W~ for bf16 caches)
static jolt_status build_wt_all(jolt_handle h, const jolt_item *items, int n, const jolt_alloc *alloc,
                                const void *const *payload, uint8_t *ws, std::vector<void *> &wt_ptr,
                                bool rot, hipStream_t st) {
    const int D = items[0].d, dtype = items[0].dtype;
    size_t off = 0;
    wt_ptr.assign(n, nullptr);
    WtBatch b{};
    b.n = 0;
    int maxLH = 0, maxRtp = 0;
    auto flush = [&]() -> jolt_status {
        hipError_t e = (rot && dtype == JOLT_BF16) ? launch_build_wt_rot(b, D, maxLH, maxRtp, st)
                                                  : launch_build_wt(b, dtype, D, maxLH, maxRtp, st);
        if (e != hipSuccess) return hip_fail(h, e, "build_wt");
        b.n = 0; maxLH = 0; maxRtp = 0;
        return JOLT_OK;
    };
    for (int i = 0; i < n; ++i) {
        const jolt_item &it = items[i];
        PayloadLayout p = payload_layout(it, alloc[i].rt, alloc[i].rf, alloc[i].bits);
        const int rtp = round_up(p.rt, 16);
        wt_ptr[i] = ws + off;
        off += align_up((size_t)it.L * it.H * it.d * rtp * 4, 256);      // fp32, or bf16 hi + lo
        if (p.rt == 0) continue;
        const uint8_t *pay = static_cast<const uint8_t *>(payload[i]);
        WtItem &w = b.it[b.n++];
        w.uf = pay + p.uf;
        w.core = pay + p.core;
        w.wt = wt_ptr[i];
        w.LH = it.L * it.H; w.rt = p.rt; w.rf = p.rf; w.rtp = rtp;
        sign_bits_for(it.seed, it.item_id, it.d, w.sign_bits);
        maxLH = std::max(maxLH, w.LH);
        maxRtp = std::max(maxRtp, rtp);
        if (b.n == kMaxBatch) {
            jolt_status s = flush();
            if (s) return s;
        }
    }
    return flush();
}

static jolt_status run_codec(jolt_handle h, bool encode, const jolt_item *items, int n, const void *const *x_dev,
                             const jolt_alloc *alloc, void *codec_ws, size_t codec_ws_bytes,
                             void *const *payload_dev, void *const *out_dev, hipStream_t st) {
    jolt_status s = check_items_uniform(h, items, n);
    if (s) return s;
    if (n == 0) return JOLT_OK;
    if (!alloc || !payload_dev || (encode ? !x_dev : !out_dev)) return fail(h, JOLT_E_INVALID, "NULL array");
    std::vector<int> rts(n);
    for (int i = 0; i < n; ++i) {
        s = check_alloc(h, items[i], alloc[i]);
        if (s) return s;
        if (!payload_dev[i] || (encode ? !x_dev[i] : !out_dev[i])) return fail(h, JOLT_E_INVALID, "NULL pointer");
        rts[i] = (alloc[i].rt == 0 || alloc[i].rf == 0) ? 0 : alloc[i].rt;
    }
    const size_t need = codec_ws_bytes_for(items, n, rts.data());
    if (need > 0 && (!codec_ws || codec_ws_bytes < need))
        return fail(h, JOLT_E_WORKSPACE, "codec workspace: need %zu bytes, have %zu", need, codec_ws_bytes);
    std::vector<void *> wt;
    s = build_wt_all(h, items, n, alloc, reinterpret_cast<const void *const *>(payload_dev),
                     static_cast<uint8_t *>(codec_ws), wt, encode, st);
    if (s) return s;
    const int D = items[0].d, dtype = items[0].dtype;
    for (int bits = 0; bits <= 8; ++bits) {
        if (encode && bits == 0) continue;
        CodecBatch b{};
        b.n = 0;
        int maxT = 0, maxLH = 0;
        auto flush = [&]() -> jolt_status {
            if (b.n == 0) return JOLT_OK;
            hipError_t e = encode ? launch_encode(b, dtype, D, bits, maxT, maxLH, st)
                                  : launch_decode(b, dtype, D, bits, maxT, maxLH, st);
            if (e != hipSuccess) return hip_fail(h, e, encode ? "encode" : "decode");
            b.n = 0; maxT = 0; maxLH = 0;
            return JOLT_OK;
        };
        for (int i = 0; i < n; ++i) {
            if (alloc[i].bits != bits) continue;
            const jolt_item &it = items[i];
            PayloadLayout p = payload_layout(it, alloc[i].rt, alloc[i].rf, bits);
            uint8_t *pay = static_cast<uint8_t *>(payload_dev[i]);
            CodecItem &c = b.it[b.n++];
            c.x = encode ? x_dev[i] : nullptr;
            c.out = encode ? nullptr : out_dev[i];
            c.ut = pay + p.ut;
            c.wt = wt[i];
            c.scales = reinterpret_cast<uint16_t *>(pay + p.scales);
            c.codes = pay + p.codes;
            c.T = it.T; c.LH = it.L * it.H; c.rt = p.rt; c.rtp = round_up(p.rt, 16);
            sign_bits_for(it.seed, it.item_id, it.d, c.sign_bits);
            maxT = std::max(maxT, it.T);
            maxLH = std::max(maxLH, c.LH);
            if (b.n == kMaxBatch) {
                s = flush();
                if (s) return s;
            }
        }
        s = flush();
        if (s) return s;
    }
    return JOLT_OK;
}

}  // namespace jolt

extern "C" jolt_status jolt_encode_residual(jolt_handle h, const jolt_item *items, int32_t n,
                                            const void *const *x_dev, const jolt_alloc *alloc, void *codec_ws,
                                            size_t codec_ws_bytes, void *const *payload_dev, void *stream) {
    if (!h) return JOLT_E_INVALID;
    clear_err(h);
    return run_codec(h, true, items, n, x_dev, alloc, codec_ws, codec_ws_bytes, payload_dev, nullptr,
                     static_cast<hipStream_t>(stream));
}

extern "C" jolt_status jolt_decompress(jolt_handle h, const jolt_item *items, int32_t n, const jolt_alloc *alloc,
                                       const void *const *payload_dev, void *codec_ws, size_t codec_ws_bytes,
                                       void *const *out_dev, void *stream) {
    if (!h) return JOLT_E_INVALID;
    clear_err(h);
    return run_codec(h, false, items, n, nullptr, alloc, codec_ws, codec_ws_bytes,
                     const_cast<void *const *>(payload_dev), out_dev, static_cast<hipStream_t>(stream));
}

extern "C" jolt_status jolt_decompress_noalloc(jolt_handle h, const jolt_item *items, int32_t n,
                                               const jolt_alloc *alloc, const void *const *payload_dev,
                                               void *const *out_dev, void *stream) {
    if (!h) return JOLT_E_INVALID;
    clear_err(h);
    jolt_status s = check_items_uniform(h, items, n);
    if (s) return s;
    if (n == 0) return JOLT_OK;
    if (!alloc) return fail(h, JOLT_E_INVALID, "NULL array");
    std::vector<int> rts(n);
    for (int i = 0; i < n; ++i) {
        s = check_alloc(h, items[i], alloc[i]);
        if (s) return s;
        rts[i] = (alloc[i].rt == 0 || alloc[i].rf == 0) ? 0 : alloc[i].rt;
    }
    const size_t need = codec_ws_bytes_for(items, n, rts.data());
    if (need > kNoAllocScratchBytes)
        return fail(h, JOLT_E_WORKSPACE,
                    "decompress_noalloc: these items need %zu bytes of scratch, above the fixed %zu (split the call "
                    "or use jolt_decompress)", need, kNoAllocScratchBytes);
    return run_codec(h, false, items, n, nullptr, alloc, h->scratch, kNoAllocScratchBytes,
                     const_cast<void *const *>(payload_dev), out_dev, static_cast<hipStream_t>(stream));
}

extern "C" jolt_status jolt_compress(jolt_handle h, const jolt_config *cfg, const jolt_item *items, int32_t n,
                                     const void *const *x_dev, const jolt_alloc *alloc, const void *plan_ws,
                                     size_t plan_ws_bytes, void *codec_ws, size_t codec_ws_bytes,
                                     void *const *payload_dev, void *stream) {
    if (!h || !cfg) return JOLT_E_INVALID;
    clear_err(h);
    jolt_status s = check_items_uniform(h, items, n);
    if (s) return s;
    if (n == 0) return JOLT_OK;
    if (!alloc || !payload_dev || !x_dev || !plan_ws) return fail(h, JOLT_E_INVALID, "NULL array");
    PlanLayout pl;
    s = plan_layout(*cfg, items, n, &pl);
    if (s) return fail(h, s, "bad config");
    if (plan_ws_bytes < pl.total) return fail(h, JOLT_E_WORKSPACE, "plan workspace too small");
    for (int i = 0; i < n; ++i) {
        s = check_alloc(h, items[i], alloc[i]);
        if (s) return s;
        if (alloc[i].rt > pl.rt_max || alloc[i].rf > pl.rf_max)
            return fail(h, JOLT_E_INVALID, "alloc ranks exceed the planned maxima");
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    s = store_params(h, pl, items, n, alloc, plan_ws, payload_dev, st);
    if (s) return s;
    return run_codec(h, true, items, n, x_dev, alloc, codec_ws, codec_ws_bytes, payload_dev, nullptr, st);
}

// --------------------------------------------------------------------------- hooks
extern "C" jolt_status jolt_rotate(jolt_handle h, const float *in, float *out, int64_t rows, int32_t d,
                                   uint64_t seed, uint32_t item_id, int32_t inverse, void *stream) {
    if (!h) return JOLT_E_INVALID;
    clear_err(h);
    if (rows < 0 || (rows > 0 && (!in || !out))) return fail(h, JOLT_E_INVALID, "rotate: bad arguments");
    if (d != 64 && d != 128) return fail(h, JOLT_E_UNSUPPORTED, "rotate: d must be 64 or 128");
    uint32_t sb[4];
    sign_bits_for(seed, item_id, d, sb);
    hipError_t e = launch_rotate(in, out, rows, d, sb, inverse, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? JOLT_OK : hip_fail(h, e, "rotate");
}

extern "C" jolt_status jolt_quantize_pack(jolt_handle h, const float *rot, int64_t rows, int32_t d, int32_t bits,
                                          uint64_t *codes, uint16_t *scales, void *stream) {
    if (!h) return JOLT_E_INVALID;
    clear_err(h);
    if (rows < 0 || bits < 2 || bits > 8 || (rows > 0 && (!rot || !codes || !scales)))
        return fail(h, JOLT_E_INVALID, "quantize_pack: bad arguments");
    if (d != 64 && d != 128) return fail(h, JOLT_E_UNSUPPORTED, "quantize_pack: d must be 64 or 128");
    hipError_t e = launch_quantize_pack(rot, rows, d, bits, reinterpret_cast<uint8_t *>(codes), scales,
                                        static_cast<hipStream_t>(stream));
    return e == hipSuccess ? JOLT_OK : hip_fail(h, e, "quantize_pack");
}

extern "C" jolt_status jolt_unpack_dequant(jolt_handle h, const uint64_t *codes, const uint16_t *scales,
                                           int64_t rows, int32_t d, int32_t bits, float *out, void *stream) {
    if (!h) return JOLT_E_INVALID;
    clear_err(h);
    if (rows < 0 || bits < 2 || bits > 8 || (rows > 0 && (!out || !codes || !scales)))
        return fail(h, JOLT_E_INVALID, "unpack_dequant: bad arguments");
    if (d != 64 && d != 128) return fail(h, JOLT_E_UNSUPPORTED, "unpack_dequant: d must be 64 or 128");
    hipError_t e = launch_unpack_dequant(reinterpret_cast<const uint8_t *>(codes), scales, rows, d, bits, out,
                                         static_cast<hipStream_t>(stream));
    return e == hipSuccess ? JOLT_OK : hip_fail(h, e, "unpack_dequant");
}

extern "C" jolt_status jolt_rademacher(jolt_handle h, uint64_t seed, uint32_t item_id, uint32_t stream_id,
                                       uint64_t first, int64_t count, float *out, void *stream) {
    if (!h) return JOLT_E_INVALID;
    clear_err(h);
    if (count < 0 || (count > 0 && !out) || stream_id > 255) return fail(h, JOLT_E_INVALID, "rademacher: bad arguments");
    hipError_t e = launch_rademacher(item_key(seed, item_id), stream_id, first, count, out,
                                     static_cast<hipStream_t>(stream));
    return e == hipSuccess ? JOLT_OK : hip_fail(h, e, "rademacher");
}

extern "C" size_t jolt_eigh_workspace_size(int32_t n, int32_t count, int32_t force_jacobi) {
    if (n < 1 || n > kWideMaxN || count < 1 || (force_jacobi && n <= kJacobiMaxN)) return 0;
    return eig_tri_ws_bytes(n) * (size_t)std::min(count, 64);
}

extern "C" jolt_status jolt_eigh(jolt_handle h, int32_t n, int32_t count, const float *a, int32_t lda,
                                 int64_t mat_stride, float *vec, float *lam, int32_t *info, int32_t force_jacobi,
                                 void *workspace, size_t workspace_bytes, void *stream) {
    if (!h) return JOLT_E_INVALID;
    clear_err(h);
    if (n < 1 || n > kWideMaxN || count < 0 || lda < n || mat_stride < (int64_t)(n - 1) * lda + n)
        return fail(h, JOLT_E_INVALID, "eigh: bad sizes (n=%d count=%d lda=%d)", n, count, lda);
    if (force_jacobi && n > kJacobiMaxN) return fail(h, JOLT_E_INVALID, "eigh: the Jacobi solver takes n <= 142");
    if (count > 0 && (!a || !vec || !lam || !info)) return fail(h, JOLT_E_INVALID, "eigh: null pointer");
    const size_t need = jolt_eigh_workspace_size(n, count, force_jacobi);
    if (workspace_bytes < need || (need && (!workspace || reinterpret_cast<uintptr_t>(workspace) % 16)))
        return fail(h, JOLT_E_WORKSPACE, "eigh workspace: need %zu bytes (16-byte aligned), have %zu", need,
                    workspace_bytes);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const bool tri = need > 0;
    // one workspace region per matrix of a batch of up to 64; batches run in
    // stream order, so they reuse the regions
    const size_t wsb = tri ? eig_tri_ws_bytes(n) : 0;
    uint8_t *tws = static_cast<uint8_t *>(workspace);
    for (int i0 = 0; i0 < count; i0 += 64) {
        JacBatch b{};
        for (int i = i0; i < count && b.n < 64; ++i) {
            JacItem &j = b.it[b.n];
            j.a = a + (size_t)i * mat_stride;
            j.lda = lda;
            j.vec = vec + (size_t)i * n * n;
            j.ldv = n;
            j.lam = lam + (size_t)i * n;
            j.n = n;
            j.raw = 0;
            j.sweeps_out = info + i;
            j.tw = tri ? reinterpret_cast<float *>(tws + (size_t)b.n * wsb) : nullptr;
            ++b.n;
        }
        hipError_t e = tri ? launch_eig_tridiag(b, n, st) : launch_jacobi_lds(b, n, 30, st);
        if (e == hipSuccess && tri && n <= kTriMaxN) e = launch_jacobi_lds(b, n, 30, st, 1);
        if (e != hipSuccess) return hip_fail(h, e, "eigh");
    }
    return JOLT_OK;
}

extern "C" jolt_status jolt_kernel_timer(jolt_handle h, const char *kernel, int32_t enable) {
    if (!h) return JOLT_E_INVALID;
    clear_err(h);
    if (!kernel || !*kernel) return fail(h, JOLT_E_INVALID, "kernel_timer: no kernel name");
    hipError_t e = ktimer_enable(kernel, enable != 0);
    return e == hipSuccess ? JOLT_OK : hip_fail(h, e, "kernel_timer");
}

extern "C" jolt_status jolt_kernel_time(jolt_handle h, const char *kernel, double *total_ms, int64_t *launches) {
    if (!h) return JOLT_E_INVALID;
    clear_err(h);
    if (!kernel || !total_ms || !launches) return fail(h, JOLT_E_INVALID, "kernel_time: null argument");
    hipError_t e = ktimer_read(kernel, total_ms, launches);
    return e == hipSuccess ? JOLT_OK : hip_fail(h, e, "kernel_time");
}

// --------------------------------------------------------------------------- decode attention
namespace jolt {

// Token ranges of one group: about two workgroups per CU over the call, ranges
// a multiple of 256 tokens, none empty.
static void attn_splits(int T, int LH, int n, int *splits, int *per) {
    const int chunks = (T + 255) / 256;
    const int want = std::max(1, std::min(chunks, (512 + LH * n - 1) / std::max(1, LH * n)));
    *per = 256 * ((chunks + want - 1) / want);
    *splits = (T + *per - 1) / *per;
}

static jolt_status attn_check(jolt_handle h, const jolt_attn_group *g, int32_t n, int32_t q_heads) {
    if (n < 0 || (n > 0 && !g)) return fail(h, JOLT_E_INVALID, "attention: bad group array");
    for (int i = 0; i < n; ++i) {
        const jolt_item &k = g[i].k_item, &v = g[i].v_item;
        jolt_status s = check_item(h, k);
        if (s) return s;
        if ((s = check_item(h, v))) return s;
        if (k.L != v.L || k.H != v.H || k.T != v.T || k.d != v.d || k.dtype != v.dtype)
            return fail(h, JOLT_E_INVALID, "attention: K and V items of group %d differ in shape or dtype", i);
        if (k.dtype != g[0].k_item.dtype || k.d != g[0].k_item.d || k.H != g[0].k_item.H)
            return fail(h, JOLT_E_UNSUPPORTED, "attention: all groups of one call must share dtype, d and H");
        if ((s = check_alloc(h, k, g[i].k_alloc))) return s;
        if ((s = check_alloc(h, v, g[i].v_alloc))) return s;
        if (!g[i].k_payload || !g[i].v_payload || !g[i].q || !g[i].out || !g[i].lse)
            return fail(h, JOLT_E_INVALID, "attention: NULL pointer in group %d", i);
    }
    if (n > 0) {
        const int H = g[0].k_item.H;
        if (q_heads < H || q_heads % H) return fail(h, JOLT_E_INVALID, "attention: q_heads must be a multiple of H");
        const int G = q_heads / H;
        if (G != 1 && G != 2 && G != 4 && G != 8)
            return fail(h, JOLT_E_UNSUPPORTED, "attention: q_heads / H must be 1, 2, 4 or 8");
    }
    return JOLT_OK;
}

static size_t attn_ws_for(const jolt_attn_group &g, int q_heads, size_t *prep, size_t *part) {
    const jolt_item &k = g.k_item;
    const int rtk = (g.k_alloc.rt == 0 || g.k_alloc.rf == 0) ? 0 : g.k_alloc.rt;
    const int rtv = (g.v_alloc.rt == 0 || g.v_alloc.rf == 0) ? 0 : g.v_alloc.rt;
    int splits, per;
    attn_splits(k.T, k.L * k.H, 1, &splits, &per);
    *prep = align_up((size_t)k.L * q_heads * (round_up(rtk, 16) + k.d) * 4, 256);
    *part = align_up((size_t)splits * k.L * q_heads * (2 + round_up(rtv, 16) + k.d) * 4, 256);
    return *prep + *part;
}

}  // namespace jolt

extern "C" jolt_status jolt_attention_workspace_size(const jolt_attn_group *groups, int32_t n, int32_t q_heads,
                                                     size_t *bytes) {
    if (!bytes) return JOLT_E_INVALID;
    jolt_status s = attn_check(nullptr, groups, n, q_heads);
    if (s) return s;
    size_t tot = 0;
    for (int i = 0; i < n; ++i) {
        size_t a, b;
        tot += attn_ws_for(groups[i], q_heads, &a, &b);
    }
    *bytes = std::max<size_t>(tot, 256);
    return JOLT_OK;
}

extern "C" jolt_status jolt_decode_attention(jolt_handle h, const jolt_attn_group *groups, int32_t n,
                                             int32_t q_heads, float scale, void *workspace, size_t workspace_bytes,
                                             void *stream) {
    if (!h) return JOLT_E_INVALID;
    clear_err(h);
    jolt_status s = attn_check(h, groups, n, q_heads);
    if (s) return s;
    if (n == 0) return JOLT_OK;
    size_t need = 0;
    for (int i = 0; i < n; ++i) {
        size_t a, b;
        need += attn_ws_for(groups[i], q_heads, &a, &b);
    }
    if (!workspace || workspace_bytes < need)
        return fail(h, JOLT_E_WORKSPACE, "attention workspace: need %zu bytes, have %zu", need, workspace_bytes);
    if (!(scale > 0.f) || !std::isfinite(scale)) return fail(h, JOLT_E_INVALID, "attention: scale must be > 0");
    hipStream_t st = static_cast<hipStream_t>(stream);
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    const int nall = n;
    int cursor = 0;
    size_t off = 0;
    while (cursor < nall) {
        AttnBatch b{};
        b.n = 0;
        b.hq = q_heads;
        b.scale = scale;
        const int nb = std::min(kMaxBatch, nall - cursor);
        for (int i = cursor; i < cursor + nb; ++i) {
            const jolt_attn_group &g = groups[i];
            const jolt_item &k = g.k_item, &v = g.v_item;
            AttnGroup &a = b.it[b.n++];
            a.L = k.L; a.H = k.H; a.T = k.T; a.d = k.d;
            PayloadLayout pk = payload_layout(k, g.k_alloc.rt, g.k_alloc.rf, g.k_alloc.bits);
            PayloadLayout pv = payload_layout(v, g.v_alloc.rt, g.v_alloc.rf, g.v_alloc.bits);
            a.rtk = pk.rt; a.rfk = pk.rf; a.bk = g.k_alloc.bits; a.rtpk = round_up(pk.rt, 16);
            a.rtv = pv.rt; a.rfv = pv.rf; a.bv = g.v_alloc.bits; a.rtpv = round_up(pv.rt, 16);
            attn_splits(k.T, k.L * k.H, nb, &a.splits, &a.per_split);
            sign_bits_for(k.seed, k.item_id, k.d, a.sk);
            sign_bits_for(v.seed, v.item_id, v.d, a.sv);
            a.isd = 1.0f / std::sqrt((float)k.d);
            const uint8_t *kp = static_cast<const uint8_t *>(g.k_payload), *vp = static_cast<const uint8_t *>(g.v_payload);
            a.ut_k = kp + pk.ut; a.uf_k = kp + pk.uf; a.core_k = kp + pk.core;
            a.scales_k = reinterpret_cast<const uint16_t *>(kp + pk.scales); a.codes_k = kp + pk.codes;
            a.ut_v = vp + pv.ut; a.uf_v = vp + pv.uf; a.core_v = vp + pv.core;
            a.scales_v = reinterpret_cast<const uint16_t *>(vp + pv.scales); a.codes_v = vp + pv.codes;
            a.q = g.q; a.out = g.out; a.lse = g.lse;
            const size_t prep = align_up((size_t)k.L * q_heads * (a.rtpk + k.d) * 4, 256);
            const size_t part = align_up((size_t)a.splits * k.L * q_heads * (2 + a.rtpv + k.d) * 4, 256);
            a.ws_prep = reinterpret_cast<float *>(ws + off);
            a.ws_part = reinterpret_cast<float *>(ws + off + prep);
            off += prep + part;
        }
        hipError_t e = launch_attention(b, groups[0].k_item.dtype, st);
        if (e != hipSuccess) return hip_fail(h, e, "attention");
        cursor += nb;
    }
    return JOLT_OK;
}
