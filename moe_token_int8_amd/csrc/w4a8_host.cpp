// Host side of the W4A8 library: descriptor checks, blob layout, offline RTN
// quantization + packing, unpacking, status strings.  No HIP calls here.
//
// Sources (cited as P1..P5 with the page's own section names):
//   P2 "Kimi 2.7 MoE W4A8: 4-bit storage to INT8, deployment notes"   (xdnf.cn)
//   P3 "Quantization: formats, error and the real execution path"     (wineandchord.com)
//   P5 "Inference quantization, chapter 1: the Linear layer"          (sgdbs.github.io)
#include "w4a8_internal.h"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <thread>
#include <vector>

namespace w4a8 {

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool desc_valid(const w4a8_wdesc* d) {
    if (!d) return false;
    if (d->K <= 0 || d->N <= 0) return false;
    if (d->asymmetric != 0 && d->asymmetric != 1) return false;
    if (d->weight_bits != 0 && d->weight_bits != 4 && d->weight_bits != 8) return false;
    if (d->weight_bits == 8 && d->asymmetric) return false;   // 8-bit codes are symmetric
    if (d->scale_bits != 0 && d->scale_bits != 16 && d->scale_bits != 32) return false;
    const int g = d->group_size;
    if (g != 32 && g != 64 && g != 128 && g != 256 && g != d->K) return false;   // g = K: per channel
    if (d->K % g) return false;            // groups cannot cross rows (P3 reference)
    return true;
}

bool log_on() {
    static const bool on = [] {
        const char* e = std::getenv("W4A8_LOG");
        return e && *e && std::strcmp(e, "0") != 0;
    }();
    return on;
}

int desc_status(const w4a8_wdesc* d) {
    if (!desc_valid(d)) return W4A8_EINVAL;
    if (d->K % SB_K) return W4A8_EUNSUPPORTED;   // layout works in 128-deep superblocks
    return W4A8_OK;
}

Layout layout_of(const w4a8_wdesc* d) {
    Layout L;
    L.K = d->K;
    L.N = d->N;
    L.Np = (d->N + 15) / 16 * 16;
    L.g = d->group_size;
    L.G = d->K / d->group_size;
    L.asym = d->asymmetric;
    L.bits = d->weight_bits == 8 ? 8 : 4;
    L.sbytes = d->scale_bits == 16 ? 2 : 4;
    L.codes_off = W4A8_HEADER_BYTES;
    L.codes_bytes = size_t(L.Np) * size_t(L.K) * size_t(L.bits) / 8;
    L.scales_off = align256(L.codes_off + L.codes_bytes);
    L.scales_bytes = size_t(L.Np) * size_t(L.G) * size_t(L.sbytes);
    L.zeros_off = align256(L.scales_off + L.scales_bytes);
    L.zeros_bytes = L.asym ? size_t(L.Np) * size_t(L.G) : 0;
    L.total = align256(L.zeros_off + L.zeros_bytes);
    return L;
}

// Byte offset (from the start of the codes section) and nibble of code (k, n).
static inline void code_pos(const Layout& L, int k, int n, size_t* byte, int* nib) {
    const int sb = k / SB_K, kk = k % SB_K, c = n % 16;
    const int half = kk / 64, r = kk % 64;
    const int lane = (r / 16) * 16 + c, j = r % 16;
    const size_t sbi = size_t(n / 16) * size_t(L.K / SB_K) + size_t(sb);
    *byte = sbi * 1024 + size_t(lane) * 16 + size_t(half) * 8 + size_t(j / 8) * 4 + size_t(j % 4);
    *nib = (j % 8) / 4;
}

// 8-bit codes: superblock (16 columns x 128 k) = 2 KiB, 32 bytes per layout lane: byte
// 16 * half + j of lane (r / 16) * 16 + c holds k = 128 sb + 64 half + r with r % 16 = j, i.e.
// the 16 values the 4-bit form unpacks for that lane and half, in the same order.
static inline size_t code_pos8(const Layout& L, int k, int n) {
    const int sb = k / SB_K, kk = k % SB_K, c = n % 16;
    const int half = kk / 64, r = kk % 64;
    const int lane = (r / 16) * 16 + c, j = r % 16;
    const size_t sbi = size_t(n / 16) * size_t(L.K / SB_K) + size_t(sb);
    return sbi * 2048 + size_t(lane) * 32 + size_t(half) * 16 + size_t(j);
}

static inline size_t meta_index(const Layout& L, int i, int n) {
    return (size_t(n / 16) * size_t(L.G) + size_t(i)) * 16 + size_t(n % 16);
}

struct Header {
    char magic[8];
    uint32_t version, layout;
    int32_t K, N, group_size, asymmetric;
    uint32_t scale_dtype, zero_dtype;
    uint64_t codes_off, codes_bytes, scales_off, scales_bytes, zeros_off, zeros_bytes, total;
    uint32_t weight_bits;   // 4 or 8
};
static_assert(sizeof(Header) <= W4A8_HEADER_BYTES, "header too large");

static void write_header(const w4a8_wdesc* d, const Layout& L, uint8_t* blob) {
    Header h;
    std::memset(&h, 0, sizeof(h));
    std::memcpy(h.magic, "W4A8BLB1", 8);
    h.version = 1;
    h.layout = 1;
    h.K = d->K;
    h.N = d->N;
    h.group_size = d->group_size;
    h.asymmetric = d->asymmetric;
    h.codes_off = L.codes_off;
    h.codes_bytes = L.codes_bytes;
    h.scales_off = L.scales_off;
    h.scales_bytes = L.scales_bytes;
    h.zeros_off = L.zeros_off;
    h.zeros_bytes = L.zeros_bytes;
    h.total = L.total;
    h.weight_bits = uint32_t(L.bits);
    h.scale_dtype = L.sbytes == 2 ? 1u : 0u;
    std::memset(blob, 0, W4A8_HEADER_BYTES);
    std::memcpy(blob, &h, sizeof(h));
}

static int read_header(const void* blob, size_t bytes, w4a8_wdesc* d, Layout* L) {
    if (!blob || bytes < W4A8_HEADER_BYTES) return W4A8_EINVAL;
    Header h;
    std::memcpy(&h, blob, sizeof(h));
    if (std::memcmp(h.magic, "W4A8BLB1", 8) || h.version != 1 || h.layout != 1) return W4A8_EINVAL;
    if (h.weight_bits == 0) h.weight_bits = 4;          // headers written before the field existed
    if (h.weight_bits != 4 && h.weight_bits != 8) return W4A8_EINVAL;
    if (h.scale_dtype > 1) return W4A8_EINVAL;
    w4a8_wdesc dd{h.K, h.N, h.group_size, h.asymmetric, int32_t(h.weight_bits), h.scale_dtype ? 16 : 32};
    int st = desc_status(&dd);
    if (st) return st == W4A8_EUNSUPPORTED ? W4A8_EINVAL : st;
    Layout l = layout_of(&dd);
    if (h.total != l.total || h.codes_off != l.codes_off || h.scales_off != l.scales_off ||
        h.zeros_off != l.zeros_off || h.codes_bytes != l.codes_bytes ||
        h.scales_bytes != l.scales_bytes || h.zeros_bytes != l.zeros_bytes)
        return W4A8_EINVAL;
    if (bytes < l.total) return W4A8_ESIZE;
    *d = dd;
    *L = l;
    return W4A8_OK;
}

// Run f(n0, n1) over 16-column tiles split across host threads.
template <class F>
static void parallel_tiles(int Np, F f) {
    const int tiles = Np / 16;
    unsigned hw = std::thread::hardware_concurrency();
    int nt = int(std::min<unsigned>(hw ? hw : 1, 16u));
    nt = std::max(1, std::min(nt, tiles));
    if (nt == 1 || size_t(tiles) < 4) {
        f(0, tiles);
        return;
    }
    std::vector<std::thread> th;
    const int per = (tiles + nt - 1) / nt;
    for (int t = 0; t < nt; ++t) {
        int a = t * per, b = std::min(tiles, a + per);
        if (a >= b) break;
        th.emplace_back([=] { f(a, b); });
    }
    for (auto& x : th) x.join();
}

// Nearest binary16 value of a finite float (ties to even), returned as a float; +-infinity
// past the binary16 range.  Binary16 has 11 significant bits down to 2^-14 and a fixed
// spacing of 2^-24 below it (subnormals).
static float round_f16(float f) {
    const double v = std::fabs(double(f));
    if (v == 0.0 || !std::isfinite(v)) return f;
    int e;
    std::frexp(v, &e);                                   // v in [2^(e-1), 2^e)
    const int qe = std::max(e - 11, -24);                // spacing of the binary16 grid at v
    double r = std::ldexp(std::nearbyint(std::ldexp(v, -qe)), qe);
    if (r > 65504.0) r = HUGE_VAL;
    return float(std::copysign(r, double(f)));
}

// Bit pattern of a binary16 value held exactly in a float (an output of round_f16).
static uint16_t f16_bits(float h) {
    const uint16_t sign = std::signbit(h) ? 0x8000u : 0u;
    const double v = std::fabs(double(h));
    if (std::isnan(v)) return sign | 0x7e00u;
    if (std::isinf(v)) return sign | 0x7c00u;
    if (v < std::ldexp(1.0, -14)) return uint16_t(sign | uint16_t(std::ldexp(v, 24)));   // subnormal or 0
    int e;
    const double m = std::frexp(v, &e);                  // v = (1 + f / 1024) 2^(e - 1)
    return uint16_t(sign | uint16_t((e - 1 + 15) << 10) | uint16_t(std::ldexp(m, 11) - 1024.0));
}

static float f16_value(uint16_t b) {
    const int ex = (b >> 10) & 31, fr = b & 1023;
    double v;
    if (ex == 31) v = fr ? NAN : HUGE_VAL;
    else if (ex == 0) v = std::ldexp(double(fr), -24);
    else v = std::ldexp(double(1024 + fr), ex - 25);
    return float((b & 0x8000u) ? -v : v);
}

static void store_scale(const Layout& L, uint8_t* scales, size_t idx, float s) {
    if (L.sbytes == 2) reinterpret_cast<uint16_t*>(scales)[idx] = f16_bits(s);
    else reinterpret_cast<float*>(scales)[idx] = s;
}

static float load_scale(const Layout& L, const uint8_t* scales, size_t idx) {
    return L.sbytes == 2 ? f16_value(reinterpret_cast<const uint16_t*>(scales)[idx])
                         : reinterpret_cast<const float*>(scales)[idx];
}

// Quantize one group (g values of column n, stride N) -- P3 "Basic mapping" and the P3
// symmetric group-wise reference; IEEE float32 division and round-half-to-even (rint under
// the default rounding mode), matching the per-group rule stated in w4a8.h.
// h16: the float32 scale is first rounded to binary16, and the codes use the rounded value.
static void rtn_group(const float* w, size_t stride, int g, int asym, int bits, bool h16, int8_t* q, float* s_out,
                      uint8_t* z_out) {
    if (!asym) {
        const float qmax = bits == 8 ? 127.0f : 7.0f;    // 2^(bits-1) - 1
        float amax = 0.0f;
        for (int t = 0; t < g; ++t) amax = std::max(amax, std::fabs(w[size_t(t) * stride]));
        float s = amax / qmax;
        if (h16) s = round_f16(s);
        const float d = s > 0.0f ? s : 1.0f;
        for (int t = 0; t < g; ++t) {
            float r = std::rint(w[size_t(t) * stride] / d);
            r = std::min(qmax, std::max(-qmax, r));
            q[t] = int8_t(r);
        }
        *s_out = s;
        *z_out = 0;
        return;
    }
    float lo = 0.0f, hi = 0.0f;
    for (int t = 0; t < g; ++t) {
        const float v = w[size_t(t) * stride];
        lo = std::min(lo, v);
        hi = std::max(hi, v);
    }
    const float range = hi - lo;
    float s = range / 15.0f;
    if (h16) s = round_f16(s);
    if (!(s > 0.0f)) {
        for (int t = 0; t < g; ++t) q[t] = 0;
        *s_out = s;
        *z_out = 0;
        return;
    }
    float z = std::rint(-lo / s);
    z = std::min(15.0f, std::max(0.0f, z));
    for (int t = 0; t < g; ++t) {
        float r = std::rint(w[size_t(t) * stride] / s) + z;
        r = std::min(15.0f, std::max(0.0f, r));
        q[t] = int8_t(r);
    }
    *s_out = s;
    *z_out = uint8_t(z);
}

static void store_code(const Layout& L, uint8_t* codes, int k, int n, int q) {
    if (L.bits == 8) {
        codes[code_pos8(L, k, n)] = uint8_t(int8_t(q));
        return;
    }
    size_t byte;
    int nib;
    code_pos(L, k, n, &byte, &nib);
    const uint8_t v = uint8_t(q) & 0xF;
    codes[byte] = nib ? uint8_t((codes[byte] & 0x0F) | (v << 4)) : uint8_t((codes[byte] & 0xF0) | v);
}

}  // namespace w4a8

using namespace w4a8;

extern "C" {

size_t w4a8_packed_size(const w4a8_wdesc* d) {
    if (desc_status(d) != W4A8_OK) return 0;
    return layout_of(d).total;
}

int w4a8_pack(const w4a8_wdesc* d, const float* W, void* blob_host, size_t blob_bytes) {
    int st = desc_status(d);
    if (st) return st;
    if (!W || !blob_host) return W4A8_EINVAL;
    const Layout L = layout_of(d);
    if (blob_bytes < L.total) return W4A8_ESIZE;
    const size_t KN = size_t(d->K) * size_t(d->N);
    for (size_t i = 0; i < KN; ++i)
        if (!std::isfinite(W[i])) return W4A8_EINVAL;
    uint8_t* blob = static_cast<uint8_t*>(blob_host);
    std::memset(blob, 0, L.total);
    write_header(d, L, blob);
    uint8_t* codes = blob + L.codes_off;
    uint8_t* scales = blob + L.scales_off;
    uint8_t* zeros = blob + L.zeros_off;
    const int g = L.g, N = L.N;
    std::atomic<bool> overflow(false);
    parallel_tiles(L.Np, [&](int t0, int t1) {
        std::vector<int8_t> q(static_cast<size_t>(g));
        for (int n = t0 * 16; n < std::min(N, t1 * 16); ++n) {
            for (int i = 0; i < L.G; ++i) {
                float s;
                uint8_t z;
                rtn_group(W + size_t(i) * g * N + n, size_t(N), g, L.asym, L.bits, L.sbytes == 2, q.data(), &s, &z);
                if (!std::isfinite(s)) overflow = true;
                store_scale(L, scales, meta_index(L, i, n), s);
                if (L.asym) zeros[meta_index(L, i, n)] = z;
                for (int t = 0; t < g; ++t) store_code(L, codes, i * g + t, n, q[size_t(t)]);
            }
        }
    });
    return overflow ? W4A8_EINVAL : W4A8_OK;     // a scale past the binary16 range
}

int w4a8_pack_codes(const w4a8_wdesc* d, const int8_t* codesIn, const float* scalesIn,
                    const uint8_t* zerosIn, void* blob_host, size_t blob_bytes) {
    int st = desc_status(d);
    if (st) return st;
    if (!codesIn || !scalesIn || !blob_host) return W4A8_EINVAL;
    if (d->asymmetric && !zerosIn) return W4A8_EINVAL;
    const Layout L = layout_of(d);
    if (blob_bytes < L.total) return W4A8_ESIZE;
    const size_t KN = size_t(d->K) * size_t(d->N);
    const int qmax = L.bits == 8 ? 127 : 7;
    const int lo = d->asymmetric ? 0 : -qmax, hi = d->asymmetric ? 15 : qmax;
    for (size_t i = 0; i < KN; ++i)
        if (codesIn[i] < lo || codesIn[i] > hi) return W4A8_EINVAL;
    if (d->asymmetric)
        for (size_t i = 0; i < size_t(L.G) * size_t(L.N); ++i)
            if (zerosIn[i] > 15) return W4A8_EINVAL;
    uint8_t* blob = static_cast<uint8_t*>(blob_host);
    std::memset(blob, 0, L.total);
    write_header(d, L, blob);
    uint8_t* codes = blob + L.codes_off;
    uint8_t* scales = blob + L.scales_off;
    uint8_t* zeros = blob + L.zeros_off;
    const int N = L.N;
    if (L.sbytes == 2)
        for (size_t i = 0; i < size_t(L.G) * size_t(N); ++i)
            if (std::isfinite(scalesIn[i]) && !std::isfinite(round_f16(scalesIn[i]))) return W4A8_EINVAL;
    parallel_tiles(L.Np, [&](int t0, int t1) {
        for (int n = t0 * 16; n < std::min(N, t1 * 16); ++n) {
            for (int i = 0; i < L.G; ++i) {
                const float sv = scalesIn[size_t(i) * N + n];
                store_scale(L, scales, meta_index(L, i, n), L.sbytes == 2 ? round_f16(sv) : sv);
                if (L.asym) zeros[meta_index(L, i, n)] = zerosIn[size_t(i) * N + n];
            }
            for (int k = 0; k < L.K; ++k) store_code(L, codes, k, n, codesIn[size_t(k) * N + n]);
        }
    });
    return W4A8_OK;
}

int w4a8_unpack_codes(const void* blob_host, size_t blob_bytes, w4a8_wdesc* d_out, int8_t* codesOut,
                      float* scalesOut, uint8_t* zerosOut) {
    w4a8_wdesc d;
    Layout L;
    int st = read_header(blob_host, blob_bytes, &d, &L);
    if (st) return st;
    if (d_out) *d_out = d;
    const uint8_t* blob = static_cast<const uint8_t*>(blob_host);
    const uint8_t* codes = blob + L.codes_off;
    const uint8_t* scales = blob + L.scales_off;
    const uint8_t* zeros = blob + L.zeros_off;
    for (int n = 0; n < L.N; ++n) {
        for (int i = 0; i < L.G; ++i) {
            if (scalesOut) scalesOut[size_t(i) * L.N + n] = load_scale(L, scales, meta_index(L, i, n));
            if (zerosOut && L.asym) zerosOut[size_t(i) * L.N + n] = zeros[meta_index(L, i, n)];
        }
        if (codesOut && L.bits == 8)
            for (int k = 0; k < L.K; ++k) codesOut[size_t(k) * L.N + n] = int8_t(codes[code_pos8(L, k, n)]);
        else if (codesOut)
            for (int k = 0; k < L.K; ++k) {
                size_t byte;
                int nib;
                code_pos(L, k, n, &byte, &nib);
                int v = (codes[byte] >> (nib * 4)) & 0xF;
                if (!L.asym && v >= 8) v -= 16;
                codesOut[size_t(k) * L.N + n] = int8_t(v);
            }
    }
    return W4A8_OK;
}

int w4a8_blob_check(const void* blob_host, size_t blob_bytes, const w4a8_wdesc* d) {
    int st = desc_status(d);
    if (st) return st;
    w4a8_wdesc h;
    Layout L;
    st = read_header(blob_host, blob_bytes, &h, &L);
    if (st) return st;
    if (h.K != d->K || h.N != d->N || h.group_size != d->group_size || h.asymmetric != d->asymmetric ||
        layout_of(&h).bits != layout_of(d).bits || layout_of(&h).sbytes != layout_of(d).sbytes)
        return W4A8_EINVAL;
    return W4A8_OK;
}

const char* w4a8_status_string(int s) {
    switch (s) {
        case W4A8_OK: return "ok";
        case W4A8_EINVAL: return "invalid argument";
        case W4A8_ESIZE: return "buffer too small";
        case W4A8_EUNSUPPORTED: return "unsupported shape or format (no fallback)";
        case W4A8_EHIP: return "HIP launch error";
        default: return "unknown status";
    }
}

int w4a8_version(void) { return 1; }

}  // extern "C"
