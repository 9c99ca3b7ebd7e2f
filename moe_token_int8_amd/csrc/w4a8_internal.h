// Internal declarations shared by the host and device translation units of the library.
#pragma once

#include <cstddef>
#include <cstdint>

#include "../../include/w4a8.h"

namespace w4a8 {

constexpr int SB_K = 128;   // superblock depth: 16 columns x 128 k = 1 KiB of packed codes
                            // (2 KiB with 8-bit codes)

struct Layout {
    int K, N, Np, g, G, asym;
    int bits;               // 4 or 8 (desc weight_bits, 0 read as 4)
    int sbytes;             // bytes per scale: 4 (float32) or 2 (binary16, desc scale_bits 16)
    size_t codes_off, codes_bytes, scales_off, scales_bytes, zeros_off, zeros_bytes, total;
};

bool desc_valid(const w4a8_wdesc* d);
int desc_status(const w4a8_wdesc* d);   // OK, EINVAL (bad desc) or EUNSUPPORTED (layout)
Layout layout_of(const w4a8_wdesc* d);

// W4A8_LOG set in the environment (to anything but "0"): the GEMM and MoE entry points print one
// line each to stderr, naming the call, its shape and the kernel variant it resolved to.
bool log_on();

}  // namespace w4a8
