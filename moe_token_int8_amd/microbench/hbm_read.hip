// HBM streaming-read ceiling of one gfx950 device in the launch shape of the decode GEMMs: the
// floor the weight-streaming kernels are measured against (P5 section 11: at decode sizes the
// GEMM is bound by the bytes it moves).
//
// Each workgroup (1024 threads) reads its contiguous share of a buffer with 16-byte non-temporal
// loads, all of a thread's loads issued before any use (as the decode kernels issue a wave's
// weight superblocks), and folds them into one word that is stored only if it equals a value no
// input holds, so nothing is optimised away.  The launches rotate over COPIES copies of the
// buffer (more than the 256 MB Infinity Cache holds, so every launch reads HBM) and are replayed
// from a HIP graph, so the host's launch rate does not pace them.  Printed per configuration:
// bytes per launch, the mean launch-to-launch time over 64 launches (median of REPS graph
// replays, HIP events) and the read rate; an empty kernel of the same grid gives the fixed cost
// of a launch.
//
// Build and run:  hipcc --offload-arch=gfx950 -O3 -o hbm_read hbm_read.hip && ./hbm_read
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
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

constexpr int NTHR = 1024;
constexpr int PER = 8;                      // 16-byte loads per thread: 128 KiB per workgroup
constexpr size_t WG_BYTES = size_t(NTHR) * PER * 16;
constexpr int LAUNCHES = 64;
constexpr int REPS = 7;
constexpr int COPIES = 16;

// workgroup b reads bytes [b * WG_BYTES, (b + 1) * WG_BYTES) of its copy; load j of thread t is
// 16 bytes at t * 16 + j * NTHR * 16 (each load instruction of a wave covers 1 KiB contiguously)
__global__ __launch_bounds__(NTHR) void stream_read(const uint8_t* __restrict__ base, uint32_t* sink) {
    const v4i* p = reinterpret_cast<const v4i*>(base + size_t(blockIdx.x) * WG_BYTES) + threadIdx.x;
    v4i v[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) v[j] = __builtin_nontemporal_load(p + j * NTHR);
    __builtin_amdgcn_sched_barrier(0);                  // every load is issued before the first use
    uint32_t x = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) x ^= uint32_t(v[j].x ^ v[j].y ^ v[j].z ^ v[j].w);
    if (x == 0x9e3779b9u) sink[threadIdx.x] = x;     // the buffers hold zeros: never taken
}

__global__ __launch_bounds__(NTHR) void empty_kernel(uint32_t* sink) {
    if (threadIdx.x == NTHR && sink) sink[0] = 1u;      // never taken
}

static float median(std::vector<float> v) {
    std::sort(v.begin(), v.end());
    return v[v.size() / 2];
}

// mean launch-to-launch time (us) of LAUNCHES graph-replayed launches, median of REPS replays
template <class F>
static float time_graph(hipStream_t s, F enqueue) {
    hipGraph_t g;
    hipGraphExec_t ge;
    CK(hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal));
    for (int i = 0; i < LAUNCHES; ++i) enqueue(i);
    CK(hipStreamEndCapture(s, &g));
    CK(hipGraphInstantiate(&ge, g, nullptr, nullptr, 0));
    CK(hipGraphLaunch(ge, s));
    CK(hipStreamSynchronize(s));
    hipEvent_t a, b;
    CK(hipEventCreate(&a));
    CK(hipEventCreate(&b));
    std::vector<float> t;
    for (int r = 0; r < REPS; ++r) {
        CK(hipEventRecord(a, s));
        CK(hipGraphLaunch(ge, s));
        CK(hipEventRecord(b, s));
        CK(hipEventSynchronize(b));
        float ms = 0.0f;
        CK(hipEventElapsedTime(&ms, a, b));
        t.push_back(ms * 1e3f / LAUNCHES);
    }
    CK(hipEventDestroy(a));
    CK(hipEventDestroy(b));
    CK(hipGraphExecDestroy(ge));
    CK(hipGraphDestroy(g));
    return median(t);
}

int main() {
    hipDeviceProp_t prop;
    CK(hipGetDeviceProperties(&prop, 0));
    std::printf("device %s, %d compute units; %d launches per graph, median of %d replays, %d rotating copies\n",
                prop.gcnArchName, prop.multiProcessorCount, LAUNCHES, REPS, COPIES);
    const int grids[] = {224, 256, 896, 1792};
    const size_t max_bytes = size_t(1792) * WG_BYTES;
    uint8_t* buf = nullptr;
    uint32_t* sink = nullptr;
    CK(hipMalloc(&buf, max_bytes * COPIES));
    CK(hipMemset(buf, 0, max_bytes * COPIES));
    CK(hipMalloc(&sink, NTHR * sizeof(uint32_t)));
    hipStream_t s;
    CK(hipStreamCreate(&s));
    for (int G : grids) {
        const size_t bytes = size_t(G) * WG_BYTES;
        const float te = time_graph(s, [&](int) { empty_kernel<<<G, NTHR, 0, s>>>(sink); });
        const float tr = time_graph(s, [&](int i) {
            stream_read<<<G, NTHR, 0, s>>>(buf + size_t(i % COPIES) * max_bytes, sink);
        });
        std::printf("grid %5d x %d threads: read %10zu B per launch in %7.3f us = %7.1f GB/s; empty kernel %6.3f us\n",
                    G, NTHR, bytes, tr, double(bytes) / (tr * 1e-6) / 1e9, te);
    }
    CK(hipGetLastError());
    CK(hipStreamDestroy(s));
    CK(hipFree(buf));
    CK(hipFree(sink));
    return 0;
}
