// Host-side packing code under AddressSanitizer and UndefinedBehaviorSanitizer: every entry point
// of the packer (sizes, RTN pack, code pack, unpack, blob check) on a spread of formats, the
// round trip pack -> unpack -> pack_codes (byte-identical blob), and the error paths (short
// buffers, truncated and corrupted blobs, invalid descriptors, out-of-range codes).  Built and
// run by tests/test_host_sanitize.py with the host compiler; exits non-zero on a failed check,
// and the sanitizers abort on any memory or undefined-behaviour error.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "../include/w4a8.h"

static int fails = 0;
#define CHECK(c)                                                             \
    do {                                                                     \
        if (!(c)) {                                                          \
            std::printf("FAIL line %d: %s\n", __LINE__, #c);                 \
            ++fails;                                                         \
        }                                                                    \
    } while (0)

struct Case {
    int K, N, g, asym, bits, sbits;
};

int main() {
    std::mt19937 rng(7);
    std::normal_distribution<float> nd(0.0f, 0.02f);
    const Case cases[] = {
        {128, 16, 128, 0, 4, 32}, {256, 40, 64, 1, 4, 32},  {512, 33, 32, 0, 4, 32},   {512, 48, 256, 1, 4, 32},
        {384, 24, 384, 1, 4, 32}, {256, 16, 128, 0, 8, 32}, {256, 50, 64, 1, 4, 16},   {1024, 100, 128, 0, 4, 16},
        {640, 7, 128, 1, 4, 32},  {128, 1, 32, 0, 8, 32},   {2048, 64, 2048, 0, 8, 32},
    };
    for (const Case& c : cases) {
        w4a8_wdesc d;
        std::memset(&d, 0, sizeof(d));
        d.K = c.K; d.N = c.N; d.group_size = c.g; d.asymmetric = c.asym; d.weight_bits = c.bits; d.scale_bits = c.sbits;
        const size_t n = w4a8_packed_size(&d);
        CHECK(n > W4A8_HEADER_BYTES);
        std::vector<float> W(size_t(c.K) * c.N);
        for (auto& w : W) w = nd(rng);
        // an all-zero group in the first column and a lone large value
        for (int k = 0; k < c.g && k < c.K; ++k) W[size_t(k) * c.N] = 0.0f;
        W[W.size() / 2] = 0.5f;
        std::vector<uint8_t> blob(n, 0xCD), blob2(n, 0xCD);
        CHECK(w4a8_pack(&d, W.data(), blob.data(), n) == W4A8_OK);
        CHECK(w4a8_blob_check(blob.data(), n, &d) == W4A8_OK);
        const size_t G = size_t(c.K / c.g) * c.N;
        std::vector<int8_t> codes(size_t(c.K) * c.N);
        std::vector<float> scales(G);
        std::vector<uint8_t> zeros(G);
        w4a8_wdesc d2;
        CHECK(w4a8_unpack_codes(blob.data(), n, &d2, codes.data(), scales.data(), c.asym ? zeros.data() : nullptr) ==
              W4A8_OK);
        CHECK(d2.K == c.K && d2.N == c.N && d2.group_size == c.g && d2.asymmetric == c.asym);
        CHECK(w4a8_pack_codes(&d, codes.data(), scales.data(), c.asym ? zeros.data() : nullptr, blob2.data(), n) ==
              W4A8_OK);
        CHECK(std::memcmp(blob.data(), blob2.data(), n) == 0);
        // outputs may be skipped
        CHECK(w4a8_unpack_codes(blob.data(), n, nullptr, nullptr, nullptr, nullptr) == W4A8_OK);
        // short buffers and truncated blobs
        CHECK(w4a8_pack(&d, W.data(), blob2.data(), n - 1) == W4A8_ESIZE);
        CHECK(w4a8_blob_check(blob.data(), n - 1, &d) != W4A8_OK);
        CHECK(w4a8_blob_check(blob.data(), 16, &d) != W4A8_OK);
        CHECK(w4a8_unpack_codes(blob.data(), 100, nullptr, codes.data(), nullptr, nullptr) != W4A8_OK);
        // a corrupted header
        std::vector<uint8_t> bad(blob);
        bad[0] ^= 0xFF;
        CHECK(w4a8_blob_check(bad.data(), n, &d) != W4A8_OK);
        CHECK(w4a8_unpack_codes(bad.data(), n, nullptr, codes.data(), nullptr, nullptr) != W4A8_OK);
        // a blob of another shape
        w4a8_wdesc d3 = d;
        d3.N = c.N + 16;
        CHECK(w4a8_blob_check(blob.data(), n, &d3) != W4A8_OK);
        // out-of-range codes and zero points; a non-finite weight
        std::vector<int8_t> oob(codes);
        oob[oob.size() - 1] = c.bits == 8 ? -128 : (c.asym ? 16 : 8);
        CHECK(w4a8_pack_codes(&d, oob.data(), scales.data(), c.asym ? zeros.data() : nullptr, blob2.data(), n) ==
              W4A8_EINVAL);
        if (c.asym) {
            std::vector<uint8_t> zb(zeros);
            zb[0] = 16;
            CHECK(w4a8_pack_codes(&d, codes.data(), scales.data(), zb.data(), blob2.data(), n) == W4A8_EINVAL);
        }
        std::vector<float> Wn(W);
        Wn[1] = std::nanf("");
        CHECK(w4a8_pack(&d, Wn.data(), blob2.data(), n) == W4A8_EINVAL);
        CHECK(w4a8_pack(&d, nullptr, blob2.data(), n) == W4A8_EINVAL);
        CHECK(w4a8_pack(&d, W.data(), nullptr, n) == W4A8_EINVAL);
    }
    // invalid descriptors
    const Case bad[] = {{100, 16, 100, 0, 4, 32}, {256, 16, 96, 0, 4, 32}, {256, 0, 128, 0, 4, 32},
                        {-128, 16, 128, 0, 4, 32}, {256, 16, 128, 0, 5, 32}, {256, 16, 128, 0, 4, 24}};
    for (const Case& c : bad) {
        w4a8_wdesc d;
        std::memset(&d, 0, sizeof(d));
        d.K = c.K; d.N = c.N; d.group_size = c.g; d.asymmetric = c.asym; d.weight_bits = c.bits; d.scale_bits = c.sbits;
        CHECK(w4a8_packed_size(&d) == 0);
        float w[4] = {0, 0, 0, 0};
        uint8_t b[512];
        CHECK(w4a8_pack(&d, w, b, sizeof(b)) != W4A8_OK);
    }
    CHECK(w4a8_packed_size(nullptr) == 0);
    CHECK(std::strlen(w4a8_status_string(W4A8_EINVAL)) > 0);
    std::printf("%d failed checks\n", fails);
    return fails ? 1 : 0;
}
