// Grouped (MoE) W4A8 GEMM for K <= 4096: every expert, hot or cold, in one streaming launch.
//
// Sources (cited with the page's own section names):
//   P1 "Kimi 2.7 MoE: from 4-bit storage to INT8 (W4A8)" (pwwt.cn), section 4.4 step 4: the grouped
//      expert GEMM over router-sorted tokens, "the performance key"; section 5.2: the 4-bit layout
//      matches the MFMA operand layout.
//   P2 "Kimi 2.7 MoE W4A8 ... deployment notes" (xdnf.cn), section 4.2: MoE layers are bound by
//      weight movement, not arithmetic.
//
// A workgroup owns one row tile of one expert (up to 32 sorted rows, gathered from the token rows
// when `gather` is set) and 16 column tiles (256 columns; 32 tiles on large launches of 16-row
// tiles).  It stages the tile's activation rows in LDS once, with coalesced 16-byte loads, and
// then streams its columns in CG groups of NT tiles: wave (t, q) owns tile t of the group over the
// K-slice q (SBN superblocks), the weights, scales and zero points of two groups are in flight at
// a time (double-buffered registers, fully unrolled so every wait is per register), and each
// group's KW slice sums are added in slice order through LDS before the row scale and the store.
// An expert's weights are therefore read once per row tile and its activations once per 256 (or
// 512) columns; experts with no rows launch nothing that reads their weights.
#include <hip/hip_runtime.h>

#include "w4a8_device.h"
#include "w4a8_internal.h"

namespace w4a8 {

// Column tiles per workgroup: 16, or 32 for 16-row tiles on launches of many workgroups.  Measured
// on the 256-expert down GEMM (K = 2048, 7168 columns, about 215 one-tile experts): 32 tiles per
// workgroup halve the activation staging per column and the workgroup count, layer 0.964-0.967 ->
// 0.953-0.958 ms; on the 64-expert layer's cold experts (61 row tiles) 32 tiles leave 1.4 rounds
// of workgroups, and that layer went from 0.25 to 0.39 ms.
constexpr int MST_TILES = 16;
constexpr int MST_TILES_WIDE = 32;
constexpr long long MST_WIDE_MIN_WG = 4096;   // 16-tile workgroups (upper bound) from which 32 are used

template <int MS, int NT, int KW, int TILES = MST_TILES>
struct MoeStreamShape {
    static constexpr int MT = 16 * MS;
    static constexpr int NTHR = 64 * NT * KW;                  // 512
    static constexpr int CG = TILES / NT;                      // column groups
    static constexpr size_t LDS_RED = size_t(KW - 1) * NT * MS * 4 * 64 * 4;
    static constexpr size_t LDS_PAIR = size_t(NT) * MS * 4 * 64 * 4;   // paired form: a group's final sums
    // activation rows padded by 32 bytes (a multiple of 128 plus 32: the 16 rows x 4 k-chunks of
    // a 16x16x64 operand read fall in distinct LDS banks)
    static size_t lds(int K) { return size_t(MT) * size_t(K + 32) + LDS_RED + LDS_PAIR; }
    static_assert(NTHR == 512, "8 waves: two per SIMD, so each has 256 registers");
};

// One workgroup's row tile tr of one expert, whose blob is `blob` (the format is the template's).
template <int MS, int NT, int KW, int SBN, int GPS, bool ASYM, bool H16, int TILES>
__device__ __forceinline__ void moe_stream_body(const GemmArgs& a, const TileRows tr, const uint8_t* blob) {
    using S = MoeStreamShape<MS, NT, KW, TILES>;
    constexpr int MT = S::MT, NTHR = S::NTHR, CG = S::CG, NV = MS * 4;
    // activation pieces (16 bytes) per thread: the K <= KW * SBN * 128 rows of a full tile
    constexpr int APT = (MT * KW * SBN * 8 + NTHR - 1) / NTHR;
    extern __shared__ __align__(16) uint8_t smem[];
    const int K = a.K, ROWB = K + 32;
    float* red = reinterpret_cast<float*>(smem + size_t(MT) * ROWB);
    float* pbuf = reinterpret_cast<float*>(smem + size_t(MT) * ROWB + S::LDS_RED);
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int t = wave % NT, q = wave / NT;
    const int ntiles = (a.N + 15) / 16;
    const int nsb = K / SB_K;

    const int rbeg = tr.rbeg, nrows = tr.rend - tr.rbeg;
    const uint8_t* codes = blob + a.codes_off;
    const float* scales = reinterpret_cast<const float*>(blob + a.scales_off);
    const uint16_t* scales16 = reinterpret_cast<const uint16_t*>(blob + a.scales_off);
    const uint8_t* zeros = blob + a.zeros_off;
    // paired form (static SiLU-requant epilogue): group g holds gate tile bx * CG + g (t = 0) and
    // its up tile (t = 1)
    const bool pair = a.Hq != nullptr;
    static_assert(NT == 2 && NT * KW >= NV, "paired form: one gate and one up tile per group");

    // source row (of Xq and sx) of tile row r, held by lane r: one gather load per lane, shared
    // by cross-lane reads, so no activation piece waits on a dependent load of its own
    int srcl = -1;
    if (lane < nrows) srcl = a.gather ? gather_src(a, rbeg + lane) : rbeg + lane;

    // 1. the tile's activation rows, requested first (they gate the first MFMA)
    const int ppr = nsb * 8;                                     // pieces per row
    uint4 xv[APT];
#pragma unroll
    for (int i = 0; i < APT; ++i) {
        const int p = tid + i * NTHR, row = p / ppr, c = p - row * ppr;
        const int src = __shfl(srcl, row & 63, 64);
        xv[i] = make_uint4(0, 0, 0, 0);
        if (row < nrows && src >= 0) xv[i] = *reinterpret_cast<const uint4*>(a.Xq + size_t(src) * K + c * 16);
    }
    // row scales of the rows this lane stores (slice-0 waves store)
    float sxr[MS][4];
#pragma unroll
    for (int ms = 0; ms < MS; ++ms)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = ms * 16 + 4 * (lane >> 4) + i;
            const int src = __shfl(srcl, row, 64);
            sxr[ms][i] = 0.0f;
            if (q == 0 && row < nrows && src >= 0) sxr[ms][i] = a.sx[src];
        }

    // paired form: the expert's static scale of h (first needed in the first group's epilogue)
    const float s_e = pair ? a.s_dn[tr.expert] : 0.0f;

    // 2. per column group g (register set g % 2): scales, zero points and weight superblocks
    const int s0 = q * SBN;
    float sc[2][SBN][GPS];
    uint32_t zq[2][SBN][GPS];
    uint4 bq[2][SBN];
    auto tile_of = [&](int g) { return pair_tile(a, (int(blockIdx.x) * CG + g) * NT, t, NT); };
    auto load_group = [&](const int g, const int set) __attribute__((always_inline)) {
        const uint32_t tc = uint32_t(min(tile_of(g), ntiles - 1));
#pragma unroll
        for (int s = 0; s < SBN; ++s) {
            const uint32_t sb = uint32_t(min(s0 + s, nsb - 1));
#pragma unroll
            for (int gi = 0; gi < GPS; ++gi) {
                const uint32_t mi = (tc * uint32_t(a.G) + sb * GPS + gi) * 16u + uint32_t(lane & 15);
                sc[set][s][gi] = H16 ? f16_to_f32(scales16[mi]) : scales[mi];
                zq[set][s][gi] = ASYM ? uint32_t(zeros[mi]) : 0u;
            }
        }
#pragma unroll
        for (int s = 0; s < SBN; ++s) {
            const uint32_t sb = uint32_t(min(s0 + s, nsb - 1));
            bq[set][s] = stream_load(codes + ((tc * uint32_t(nsb) + sb) * 1024u + uint32_t(lane) * 16u));
        }
    };
    load_group(0, 0);
    asm volatile("" ::: "memory");                               // keep the stream issued here

    // 3. activations to LDS (rows past the tile are not written; their outputs are never stored);
    //    the second group is requested once the activation registers are free
#pragma unroll
    for (int i = 0; i < APT; ++i) {
        const int p = tid + i * NTHR, row = p / ppr, c = p - row * ppr;
        if (row < nrows) *reinterpret_cast<uint4*>(smem + row * ROWB + c * 16) = xv[i];
    }
    if (CG > 1) load_group(1, 1);
    asm volatile("" ::: "memory");
    lds_barrier();

    // 4. column groups in order, alternating register sets 0 and 1
    const v4i zero4 = {0, 0, 0, 0};
    auto group = [&](const int g, const int set) __attribute__((always_inline)) {
        float accf[MS][4];
#pragma unroll
        for (int ms = 0; ms < MS; ++ms)
#pragma unroll
            for (int i = 0; i < 4; ++i) accf[ms][i] = 0.0f;
#pragma unroll
        for (int s = 0; s < SBN; ++s) {
            const int sb = s0 + s;
            if (sb >= nsb) break;                                // uniform per wave
            v4i acc[MS];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int gi = GPS == 2 ? h : 0;
                const uint32_t zc = ASYM ? (128u - zq[set][s][gi]) * 0x01010101u : 0u;
                const v4i b = unpack_b<ASYM>(h ? bq[set][s].z : bq[set][s].x, h ? bq[set][s].w : bq[set][s].y, zc);
                const bool first = GPS == 2 || h == 0;
#pragma unroll
                for (int ms = 0; ms < MS; ++ms) {
                    const uint4 av = *reinterpret_cast<const uint4*>(
                        smem + (ms * 16 + (lane & 15)) * ROWB + sb * SB_K + h * 64 + 16 * (lane >> 4));
                    const v4i A = v4i{int(av.x), int(av.y), int(av.z), int(av.w)};
                    acc[ms] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, b, first ? zero4 : acc[ms], 0, 0, 0);
                }
                if (GPS == 2 || h == 1) {
                    const float scl = ASYM ? sc[set][s][gi] : sc[set][s][gi] * 0.0625f;
#pragma unroll
                    for (int ms = 0; ms < MS; ++ms)
#pragma unroll
                        for (int i = 0; i < 4; ++i) accf[ms][i] = fmaf(float(acc[ms][i]), scl, accf[ms][i]);
                }
            }
        }
        // the register set of this group is free: request group g + 2 into it
        if (g + 2 < CG) {
            load_group(g + 2, set);
            asm volatile("" ::: "memory");
        }
        // slice-ordered reduction through LDS, row scale, store
        if (q > 0) {
#pragma unroll
            for (int ms = 0; ms < MS; ++ms)
#pragma unroll
                for (int i = 0; i < 4; ++i) red[(((q - 1) * NT + t) * NV + ms * 4 + i) * 64 + lane] = accf[ms][i];
        }
        lds_barrier();
        if (q == 0) {
#pragma unroll
            for (int w = 1; w < KW; ++w)
#pragma unroll
                for (int ms = 0; ms < MS; ++ms)
#pragma unroll
                    for (int i = 0; i < 4; ++i) accf[ms][i] += red[(((w - 1) * NT + t) * NV + ms * 4 + i) * 64 + lane];
            const int tile = tile_of(g);
            const int col = tile * 16 + (lane & 15);
            if (!pair && tile < ntiles && col < a.N) {
#pragma unroll
                for (int ms = 0; ms < MS; ++ms)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int row = ms * 16 + 4 * (lane >> 4) + i;
                        if (row >= nrows) continue;
                        const float y = accf[ms][i] * sxr[ms][i];
                        const size_t yi = size_t(rbeg + row) * a.ldy + col;
                        if (a.out_f32)
                            reinterpret_cast<float*>(a.Y)[yi] = y;
                        else
                            reinterpret_cast<uint16_t*>(a.Y)[yi] = uint16_t(f32_to_bf16_rne(y));
                    }
            }
        }
        if (pair) {
            // the two slice-0 waves put the group's final gate and up outputs in LDS; then wave w
            // forms the codes of accumulator slot w (one value per lane), so the SiLU-requant
            // is spread over the workgroup instead of lengthening one wave's path
            if (q == 0) {
#pragma unroll
                for (int ms = 0; ms < MS; ++ms)
#pragma unroll
                    for (int i = 0; i < 4; ++i) pbuf[(t * NV + ms * 4 + i) * 64 + lane] = accf[ms][i] * sxr[ms][i];
            }
            lds_barrier();
            const int gt = int(blockIdx.x) * CG + g;
            const int row = (wave / 4) * 16 + 4 * (lane >> 4) + (wave & 3);
            if (wave < NV && gt < a.pair_n / 16 && row < nrows) {
                const float yg = pbuf[wave * 64 + lane], yu = pbuf[(NV + wave) * 64 + lane];
                a.Hq[size_t(rbeg + row) * a.pair_n + gt * 16 + (lane & 15)] =
                    int8_t(silu_static_code(yg, yu, static_row_scale(s_e)));
            }
        }
        if (g + 1 < CG) lds_barrier();                           // the reduction area is reused
    };
    // Fully unrolled, except for 16-row tiles at 32 tiles per workgroup with 8 superblocks per
    // slice, g = 64 and zero points: unrolled, that instance keeps part of its double-buffered
    // registers in scratch (272 bytes per lane), and a loop over pairs of groups (register sets
    // fixed at 0 and 1 inside it) took a 64-token, 256-expert layer at H = 4096 from 1.456 to
    // 0.632 ms.  The other instances are faster unrolled (the 256-expert C5 layer 0.94 ms
    // against 1.00 ms with the pair loop).
    if constexpr (CG > 8 && SBN == 8 && GPS == 2 && ASYM) {
        static_assert(CG % 2 == 0, "groups come in pairs");
#pragma unroll 1
        for (int g = 0; g < CG; g += 2) {
            group(g, 0);
            group(g + 1, 1);
        }
    } else {
#pragma unroll
        for (int g = 0; g < CG; ++g) group(g, g & 1);
    }
    // paired form: the workgroup of the first column block writes the row scales of h
    if (pair && blockIdx.x == 0 && tid < nrows) a.sh[rbeg + tid] = s_e;
}

template <int MS, int NT, int KW, int SBN, int GPS, bool ASYM, bool H16, int TILES = MST_TILES>
__global__ __launch_bounds__(512) void gemm_moe_stream_kernel(GemmArgs a) {
    const TileRows tr = moe_tile<16 * MS>(a, blockIdx.y, int(threadIdx.x) & 63);
    if (tr.expert < 0) return;                                   // uniform over the workgroup
    moe_stream_body<MS, NT, KW, SBN, GPS, ASYM, H16, TILES>(a, tr, a.blob + size_t(tr.expert) * a.expert_stride);
}

// Format classes in one launch: the workgroup resolves its expert's class, then runs the code of
// that class's format (every branch is uniform over the workgroup; only one is taken).
template <int MS, int NT, int KW, int SBN, int TILES>
__global__ __launch_bounds__(512) void gemm_moe_stream_classes_kernel(GemmArgs a, MoeClasses mc) {
    const TileRows tr = moe_tile<16 * MS>(a, blockIdx.y, int(threadIdx.x) & 63);
    if (tr.expert < 0) return;
    const uint8_t* blob;
    const int fmt = __builtin_amdgcn_readfirstlane(moe_class_resolve(mc, __builtin_amdgcn_readfirstlane(tr.expert), a, blob));
#define W4A8_MSC(F_, GPS_, ASYM_, H16_) \
    case F_: moe_stream_body<MS, NT, KW, SBN, GPS_, ASYM_, H16_, TILES>(a, tr, blob); break;
    switch (fmt) {
        W4A8_MSC(0, 1, false, false)
        W4A8_MSC(1, 2, false, false)
        W4A8_MSC(2, 1, true, false)
        W4A8_MSC(3, 2, true, false)
        W4A8_MSC(4, 1, false, true)
        W4A8_MSC(5, 2, false, true)
        W4A8_MSC(6, 1, true, true)
        W4A8_MSC(7, 2, true, true)
        default: break;
    }
#undef W4A8_MSC
}

template <int MS, int NT, int KW, int SBN, int GPS, bool ASYM, bool H16, int TILES>
static void launch_moe_stream_t(const GemmArgs& a, int slots, hipStream_t s) {
    using S = MoeStreamShape<MS, NT, KW, TILES>;
    auto kern = gemm_moe_stream_kernel<MS, NT, KW, SBN, GPS, ASYM, H16, TILES>;
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                                       int(S::lds(KW * SBN * SB_K)));
    (void)attr;
    const int ntiles = (a.N + 15) / 16;
    kern<<<dim3((ntiles + TILES - 1) / TILES, slots), dim3(S::NTHR), S::lds(a.K), s>>>(a);
}

template <int MS, int GPS, bool ASYM, bool H16, int TILES = MST_TILES>
static void launch_moe_stream_k(const GemmArgs& a, int slots, hipStream_t s) {
    const int nsb = a.K / SB_K;
    // 4 slices of SBN superblocks cover K (up to 32 superblocks)
    if (nsb <= 8) launch_moe_stream_t<MS, 2, 4, 2, GPS, ASYM, H16, TILES>(a, slots, s);
    else if (nsb <= 12) launch_moe_stream_t<MS, 2, 4, 3, GPS, ASYM, H16, TILES>(a, slots, s);
    else if (nsb <= 16) launch_moe_stream_t<MS, 2, 4, 4, GPS, ASYM, H16, TILES>(a, slots, s);
    else if (nsb <= 24) launch_moe_stream_t<MS, 2, 4, 6, GPS, ASYM, H16, TILES>(a, slots, s);
    else launch_moe_stream_t<MS, 2, 4, 8, GPS, ASYM, H16, TILES>(a, slots, s);
}

bool moe_stream_fits(int K, int gps) { return K <= 32 * SB_K && (gps == 1 || gps == 2); }

void launch_moe_stream(const GemmArgs& a, int mt, int gps, bool asym, int slots, hipStream_t s) {
#define W4A8_MST(MS_, GPS_, ASYM_)                                                     \
    do {                                                                               \
        if (a.h16) launch_moe_stream_k<MS_, GPS_, ASYM_, true>(a, slots, s);           \
        else launch_moe_stream_k<MS_, GPS_, ASYM_, false>(a, slots, s);                \
    } while (0)
    const long long ntiles = (a.N + 15) / 16;
    const bool wide = (long long)slots * ((ntiles + MST_TILES - 1) / MST_TILES) >= MST_WIDE_MIN_WG;
    if (mt == 16 && wide) {
#define W4A8_MSTW(GPS_, ASYM_)                                                              \
    do {                                                                                    \
        if (a.h16) launch_moe_stream_k<1, GPS_, ASYM_, true, MST_TILES_WIDE>(a, slots, s);  \
        else launch_moe_stream_k<1, GPS_, ASYM_, false, MST_TILES_WIDE>(a, slots, s);       \
    } while (0)
        if (gps == 1) { if (asym) W4A8_MSTW(1, true); else W4A8_MSTW(1, false); }
        else { if (asym) W4A8_MSTW(2, true); else W4A8_MSTW(2, false); }
#undef W4A8_MSTW
    } else if (mt == 16) {
        if (gps == 1) { if (asym) W4A8_MST(1, 1, true); else W4A8_MST(1, 1, false); }
        else { if (asym) W4A8_MST(1, 2, true); else W4A8_MST(1, 2, false); }
    } else {
        if (gps == 1) { if (asym) W4A8_MST(2, 1, true); else W4A8_MST(2, 1, false); }
        else { if (asym) W4A8_MST(2, 2, true); else W4A8_MST(2, 2, false); }
    }
#undef W4A8_MST
}

template <int MS, int NT, int KW, int SBN, int TILES>
static void launch_moe_stream_classes_t(const GemmArgs& a, const MoeClasses& mc, int slots, hipStream_t s) {
    using S = MoeStreamShape<MS, NT, KW, TILES>;
    auto kern = gemm_moe_stream_classes_kernel<MS, NT, KW, SBN, TILES>;
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                                       int(S::lds(KW * SBN * SB_K)));
    (void)attr;
    const int ntiles = (a.N + 15) / 16;
    kern<<<dim3((ntiles + TILES - 1) / TILES, slots), dim3(S::NTHR), S::lds(a.K), s>>>(a, mc);
}

template <int MS, int TILES = MST_TILES>
static void launch_moe_stream_classes_k(const GemmArgs& a, const MoeClasses& mc, int slots, hipStream_t s) {
    const int nsb = a.K / SB_K;
    if (nsb <= 8) launch_moe_stream_classes_t<MS, 2, 4, 2, TILES>(a, mc, slots, s);
    else if (nsb <= 12) launch_moe_stream_classes_t<MS, 2, 4, 3, TILES>(a, mc, slots, s);
    else if (nsb <= 16) launch_moe_stream_classes_t<MS, 2, 4, 4, TILES>(a, mc, slots, s);
    else if (nsb <= 24) launch_moe_stream_classes_t<MS, 2, 4, 6, TILES>(a, mc, slots, s);
    else launch_moe_stream_classes_t<MS, 2, 4, 8, TILES>(a, mc, slots, s);
}

void launch_moe_stream_classes(const GemmArgs& a, const MoeClasses& mc, int mt, int slots, hipStream_t s) {
    const long long ntiles = (a.N + 15) / 16;
    const bool wide = (long long)slots * ((ntiles + MST_TILES - 1) / MST_TILES) >= MST_WIDE_MIN_WG;
    if (mt == 16 && wide) launch_moe_stream_classes_k<1, MST_TILES_WIDE>(a, mc, slots, s);
    else if (mt == 16) launch_moe_stream_classes_k<1>(a, mc, slots, s);
    else launch_moe_stream_classes_k<2>(a, mc, slots, s);
}

}  // namespace w4a8
