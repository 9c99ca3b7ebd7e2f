// INT8 MFMA throughput of one gfx950 device with nothing but MFMAs in the loop: the ceiling the
// prefill GEMM's tensor work is measured against (its dense INT8 peak).
//
// Every wave runs ITERS rounds of NACC independent MFMAs (independent accumulators, so the
// matrix core never waits on a previous result), on operands held in registers, and stores its
// accumulators once at the end so that nothing is optimised away.  One launch covers every
// compute unit several times over.  Printed: ops per launch (2 * m * n * k per MFMA), the
// median launch time over REPS launches (HIP events) and TOP/s, for v_mfma_i32_32x32x32_i8
// (the prefill kernel's instruction) and v_mfma_i32_16x16x64_i8 (the decode kernels').
//
// Build and run:  hipcc --offload-arch=gfx950 -O3 -o mfma_peak mfma_peak.hip && ./mfma_peak
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <vector>

#define CK(x)                                                                              \
    do {                                                                                   \
        hipError_t e_ = (x);                                                               \
        if (e_ != hipSuccess) {                                                            \
            std::fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            std::exit(1);                                                                  \
        }                                                                                  \
    } while (0)

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int ITERS = 2048;
constexpr int REPS = 9;

// 32x32x32: 4 independent 16-register accumulators per wave
__global__ __launch_bounds__(256) void mfma32_loop(const int* in, int* out) {
    const int lane = threadIdx.x & 63;
    v4i a = {in[lane & 7], in[(lane + 1) & 7], in[(lane + 2) & 7], in[(lane + 3) & 7]};
    v4i b = {in[(lane + 4) & 7], in[(lane + 5) & 7], in[(lane + 6) & 7], in[(lane + 7) & 7]};
    v16i c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int i = 0; i < ITERS; ++i) {
        c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c3, 0, 0, 0);
    }
    int s = 0;
    for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// 16x16x64: 8 independent 4-register accumulators per wave
__global__ __launch_bounds__(256) void mfma16_loop(const int* in, int* out) {
    const int lane = threadIdx.x & 63;
    v4i a = {in[lane & 7], in[(lane + 1) & 7], in[(lane + 2) & 7], in[(lane + 3) & 7]};
    v4i b = {in[(lane + 4) & 7], in[(lane + 5) & 7], in[(lane + 6) & 7], in[(lane + 7) & 7]};
    v4i c[8];
    for (int j = 0; j < 8; ++j) c[j] = v4i{0, 0, 0, 0};
    for (int i = 0; i < ITERS; ++i) {
#pragma unroll
        for (int j = 0; j < 8; ++j) c[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c[j], 0, 0, 0);
    }
    int s = 0;
    for (int j = 0; j < 8; ++j) s += c[j][0] + c[j][1] + c[j][2] + c[j][3];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

template <typename K>
static double time_launch(K kern, int blocks, const int* in, int* out) {
    hipEvent_t e0, e1;
    CK(hipEventCreate(&e0));
    CK(hipEventCreate(&e1));
    kern<<<blocks, 256>>>(in, out);                      // warm-up (clocks, code load)
    CK(hipDeviceSynchronize());
    std::vector<float> t;
    for (int r = 0; r < REPS; ++r) {
        CK(hipEventRecord(e0));
        kern<<<blocks, 256>>>(in, out);
        CK(hipEventRecord(e1));
        CK(hipEventSynchronize(e1));
        float ms = 0;
        CK(hipEventElapsedTime(&ms, e0, e1));
        t.push_back(ms);
    }
    std::sort(t.begin(), t.end());
    CK(hipEventDestroy(e0));
    CK(hipEventDestroy(e1));
    return t[REPS / 2];
}

int main() {
    hipDeviceProp_t p;
    CK(hipGetDeviceProperties(&p, 0));
    const int cus = p.multiProcessorCount;
    const int blocks = cus * 8;                          // 8 workgroups of 4 waves per compute unit
    int *in = nullptr, *out = nullptr;
    CK(hipMalloc(&in, 8 * sizeof(int)));
    CK(hipMalloc(&out, size_t(blocks) * 256 * sizeof(int)));
    const int h[8] = {0x01020304, 0x05060708, 0x7f7f7f7f, 0x11223344, 0x01010101, 0x02020202, 0x03030303, 0x04040404};
    CK(hipMemcpy(in, h, sizeof(h), hipMemcpyHostToDevice));
    std::printf("device %s, %d compute units, %d workgroups x 4 waves, %d rounds per wave\n", p.gcnArchName, cus,
                blocks, ITERS);
    const double waves = double(blocks) * 4;
    const double ops32 = waves * ITERS * 4 * 2.0 * 32 * 32 * 32;
    const double ops16 = waves * ITERS * 8 * 2.0 * 16 * 16 * 64;
    const double ms32 = time_launch(mfma32_loop, blocks, in, out);
    const double ms16 = time_launch(mfma16_loop, blocks, in, out);
    std::printf("v_mfma_i32_32x32x32_i8: %.4e ops in %.3f ms (median of %d) = %.1f TOP/s\n", ops32, ms32, REPS,
                ops32 / (ms32 * 1e-3) / 1e12);
    std::printf("v_mfma_i32_16x16x64_i8: %.4e ops in %.3f ms (median of %d) = %.1f TOP/s\n", ops16, ms16, REPS,
                ops16 / (ms16 * 1e-3) / 1e12);
    CK(hipFree(in));
    CK(hipFree(out));
    return 0;
}
