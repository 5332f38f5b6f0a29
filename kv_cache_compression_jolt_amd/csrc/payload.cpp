// Payload sections and header.
//
// Per item: [header 64 B | U~_t T x r_t | U~_f d x r_f | C~ L H r_t r_f | scales | codes],
// each section 256-byte aligned; parameter sections in the item dtype, scales
// bf16 (one per 64 rotated residual values), codes 8 b bytes per group.  The
// byte accounting of the allocator (jolt_item_bytes) counts the sections'
// payload bytes, not the header or the alignment padding.
#include <cstring>

#include "jolt_internal.h"
#include "payload.h"

namespace jolt {

PayloadLayout payload_layout(const jolt_item &it, int rt, int rf, int bits) {
    PayloadLayout p;
    if (rt == 0 || rf == 0) rt = rf = 0;
    const size_t e = elem_bytes(it.dtype);
    const size_t N = (size_t)it.L * it.H * it.T * it.d;
    const size_t groups = N / kGroup;
    p.rt = rt; p.rf = rf; p.bits = bits;
    p.ut_bytes = (size_t)it.T * rt * e;
    p.uf_bytes = (size_t)it.d * rf * e;
    p.core_bytes = (size_t)it.L * it.H * rt * rf * e;
    p.scales_bytes = bits ? groups * 2 : 0;
    p.codes_bytes = bits ? groups * 8 * (size_t)bits : 0;
    p.ut = 256;
    p.uf = align_up(p.ut + p.ut_bytes, 256);
    p.core = align_up(p.uf + p.uf_bytes, 256);
    p.scales = align_up(p.core + p.core_bytes, 256);
    p.codes = align_up(p.scales + p.scales_bytes, 256);
    p.total = align_up(p.codes + p.codes_bytes, 256);
    return p;
}

static uint32_t fnv1a(const uint8_t *p, size_t n) {
    uint32_t h = 2166136261u;
    for (size_t i = 0; i < n; ++i) { h ^= p[i]; h *= 16777619u; }
    return h;
}

// little-endian header:
//  0 magic u32 | 4 version u16 | 6 dtype u8 | 7 bits u8 | 8 L H T d i32 x4 | 24 rt rf i32 x2 |
// 32 group i32 | 36 item_id u32 | 40 seed u64 | 48 total bytes u64 | 56 reserved u32 | 60 fnv1a(0..60) u32
void make_header(const jolt_item &it, const jolt_alloc &a, uint8_t out[64]) {
    PayloadLayout p = payload_layout(it, a.rt, a.rf, a.bits);
    std::memset(out, 0, 64);
    auto put32 = [&](int off, uint32_t v) { std::memcpy(out + off, &v, 4); };
    auto put64 = [&](int off, uint64_t v) { std::memcpy(out + off, &v, 8); };
    put32(0, kMagic);
    uint16_t ver = kVersion;
    std::memcpy(out + 4, &ver, 2);
    out[6] = (uint8_t)it.dtype;
    out[7] = (uint8_t)a.bits;
    put32(8, (uint32_t)it.L); put32(12, (uint32_t)it.H); put32(16, (uint32_t)it.T); put32(20, (uint32_t)it.d);
    put32(24, (uint32_t)p.rt); put32(28, (uint32_t)p.rf);
    put32(32, (uint32_t)kGroup);
    put32(36, it.item_id);
    put64(40, it.seed);
    put64(48, (uint64_t)p.total);
    put32(60, fnv1a(out, 60));
}

size_t codec_ws_bytes_for(const jolt_item *items, int n, const int *rt) {
    size_t s = 0;
    for (int i = 0; i < n; ++i) {
        const int rtp = round_up(rt[i], 16);
        s += align_up((size_t)items[i].L * items[i].H * items[i].d * rtp * 4, 256);   // fp32, or bf16 hi + lo
    }
    return s;
}

}  // namespace jolt
