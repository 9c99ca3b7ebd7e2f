// Dense W4A8 decode GEMM with one K-slice per wave (up to 32 rows, 2048 < K <= 4096).
//
// Sources (cited with the page's own section names):
//   P1 "Kimi 2.7 MoE: from 4-bit storage to INT8 (W4A8)" (pwwt.cn), section 5.1-5.2: the INT8
//      matrix instruction with the 4-bit layout matched to its operand layout; section 3.3: the
//      per-token activation scale; section 4.2: group-wise 4-bit weights with a float32 scale.
//   P5 "Inference quantization, chapter 1: the Linear layer" (sgdbs.github.io), section 7: INT32
//      accumulation per group, the float32 epilogue with act_scale x w_scale; section 11: at
//      decode sizes the GEMM is bound by the weight bytes it moves.
//
// A workgroup (16 waves) covers 4 column tiles (64 columns) over all of K.  Wave q owns the
// K-slice of superblocks [q * SW, q * SW + SW) for all four tiles:
//   1. it copies its slice of the tile's activation rows into an LDS region that only it uses
//      (coalesced 16-byte loads; rows padded by 32 bytes so the operand reads are free of bank
//      conflicts), so no workgroup barrier stands between its loads and its first MFMA;
//   2. it issues the weight superblocks of its slice (16 bytes per lane each, non-temporal) and
//      their group scales / zero points, all waits per register;
//   3. it reads every activation operand once and uses it for the four tiles;
//   4. after one barrier, the 16 slice sums of every output are added in slice order through
//      LDS (a fixed order: the result does not depend on scheduling), then the row scale and
//      the store.
// Against the chunked decode kernel (four waves per K-slice sharing one staged activation tile
// behind a workgroup barrier), each wave starts computing as soon as its own 8 KiB of
// activations land, and the LDS operand reads drop fourfold (one read per operand instead of one
// per tile).
//
// The kernel serves 16-row tiles (1-16 rows) and 32-row tiles (17-32 rows).  Measured against the
// chunked kernel on the 4096 x 14336 projection: 32 rows 9.4-9.6 -> 8.9-9.0 us, 16 rows 8.0 ->
// 7.7-7.8 us, 8 rows 7.9-8.1 -> 7.8 us.  Folding the per-token quantization into it (every wave
// quantizing its slice of the bfloat16 rows after a workgroup abs-max) was measured and dropped:
// 8 rows 10.7 -> 14.4 us, since every workgroup repeats the whole quantization.
#include <hip/hip_runtime.h>

#include "w4a8_device.h"
#include "w4a8_internal.h"

namespace w4a8 {

template <int MS, int SW>
struct DecodeSplitShape {
    static constexpr int NT = 4, KW = 16, MT = 16 * MS, NTHR = 64 * KW;
    static constexpr int ROWB = SW * SB_K + 32;                 // padded row of a wave's slice
    static constexpr int ACT = MT * ROWB;                       // activation bytes of a wave region
    static constexpr int PART = NT * MS * 64 * 16;              // slice partials: 4 floats per lane and tile row block
    static constexpr int REG = ACT > PART ? ACT : PART;
    static constexpr size_t LDS = size_t(KW) * REG;
};

// Weight superblocks per wave requested before the wave's activation slice is copied to LDS;
// the rest follow right after the copy.  All of them (8 at K = 4096): measured against 4 on the
// 4096 x 14336 projection, 9.08-9.16 against 9.14-9.43 us.
constexpr int DSPLIT_EARLY = 8;

template <int MS, int SW, int GPS, bool ASYM, bool H16>
__global__ __launch_bounds__(1024) void gemm_decode_split_kernel(GemmArgs a) {
    using S = DecodeSplitShape<MS, SW>;
    constexpr int NT = S::NT, KW = S::KW, MT = S::MT, ROWB = S::ROWB;
    constexpr int PPR = SW * 8;                                 // 16-byte pieces per slice row
    constexpr int APL = MT * PPR / 64;                          // pieces per lane
    constexpr int NB = NT * SW;                                 // weight superblocks per wave
    constexpr int BE = DSPLIT_EARLY < NB ? DSPLIT_EARLY : NB;
    static_assert(GPS == 1 || GPS == 2, "g = 128 or g = 64");
    static_assert((MT * PPR) % 64 == 0, "whole pieces per lane");
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63, q = __builtin_amdgcn_readfirstlane(tid >> 6);
    uint8_t* reg = smem + q * S::REG;
    const int ntiles = (a.N + 15) / 16;
    const int nsb = a.K / SB_K;
    const int rbeg = blockIdx.y * MT;
    const int nrows = min(a.M - rbeg, MT);
    const int sb0 = q * SW;
    const int nsw = max(0, min(SW, nsb - sb0));                 // superblocks in this slice (uniform)
    const uint8_t* codes = a.blob + a.codes_off;
    const float* scales = reinterpret_cast<const float*>(a.blob + a.scales_off);
    const uint16_t* scales16 = reinterpret_cast<const uint16_t*>(a.blob + a.scales_off);
    const uint8_t* zeros = a.blob + a.zeros_off;

    // reduction role of this thread (after the barrier): MS outputs of tile rt, row block rms,
    // rows ri0 .. ri0 + MS - 1 of the 4-row group of lane; its row scales are fetched first so
    // the epilogue never waits on a load
    const int w = tid >> 6;
    const int rt = w >> 2;
    const int rms = MS == 2 ? (w >> 1) & 1 : 0;
    const int ri0 = MS == 2 ? (w & 1) * 2 : (w & 3);
    // (the loads are unconditional, from a clamped row: a load under a data-dependent branch
    // would make the compiler wait for every load in flight at the join)
    float sxr[MS];
#pragma unroll
    for (int j = 0; j < MS; ++j) {
        const int row = rms * 16 + 4 * (lane >> 4) + ri0 + j;
        sxr[j] = a.sx[rbeg + min(row, nrows - 1)];
    }

    // 1. this wave's activation slice: piece p = lane + 64 j is row p / PPR, 16 bytes at
    //    column p % PPR of the slice.  Rows past the tile's end and superblocks past K are
    //    given an offset past the buffer's end, which a buffer load answers with zeros and no
    //    memory access (their MFMA outputs are never stored)
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t*>(a.Xq + size_t(rbeg) * a.K), 0, nrows * a.K, 0x00020000);
    uint4 xv[APL];
#pragma unroll
    for (int j = 0; j < APL; ++j) {
        const int p = lane + 64 * j, row = p / PPR, c = p - row * PPR;
        const bool ok = row < nrows && (c >> 3) < nsw;
        const uint32_t off = ok ? uint32_t(row * a.K + sb0 * SB_K + c * 16) : 0x80000000u;
        const v4i v = __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0);
        xv[j] = make_uint4(uint32_t(v.x), uint32_t(v.y), uint32_t(v.z), uint32_t(v.w));
    }
    // 2. group scales and zero points of the slice's 4 x SW superblocks
    float sc[NT][SW][GPS];
    uint32_t zq[NT][SW][GPS];
    uint32_t boff[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int tile = min(int(blockIdx.x) * NT + t, ntiles - 1);
        boff[t] = uint32_t(tile) * uint32_t(nsb) * 1024u + uint32_t(lane) * 16u;
        const uint32_t moff = uint32_t(tile) * uint32_t(a.G) * 16u + uint32_t(lane & 15);
#pragma unroll
        for (int s = 0; s < SW; ++s) {
            const uint32_t sb = uint32_t(min(sb0 + s, nsb - 1));
#pragma unroll
            for (int gi = 0; gi < GPS; ++gi) {
                const uint32_t mi = moff + (sb * GPS + gi) * 16u;
                sc[t][s][gi] = H16 ? f16_to_f32(scales16[mi]) : scales[mi];
                zq[t][s][gi] = ASYM ? uint32_t(zeros[mi]) : 0u;
            }
        }
    }
    // 3. weight superblocks in the order they are consumed (slice superblock major, tile minor)
    uint4 bq[NB];
    auto wload = [&](int u) __attribute__((always_inline)) {
        const int s = u / NT, t = u - s * NT;
        const uint32_t sb = uint32_t(min(sb0 + s, nsb - 1));
        bq[u] = stream_load(codes + (boff[t] + sb * 1024u));
    };
#pragma unroll
    for (int u = 0; u < BE; ++u) wload(u);
    // 4. the slice into this wave's LDS region (the waits are per register, so the weight loads
    //    stay in flight); the same wave reads it back, and a wave's LDS operations complete in
    //    issue order, so no barrier is needed
#pragma unroll
    for (int j = 0; j < APL; ++j) {
        const int p = lane + 64 * j, row = p / PPR, c = p - row * PPR;
        *reinterpret_cast<uint4*>(reg + row * ROWB + c * 16) = xv[j];
    }
#pragma unroll
    for (int u = BE; u < NB; ++u) wload(u);
    // keep these requests issued here: otherwise each is sunk next to its first use behind a
    // full wait
    asm volatile("" ::: "memory");

    // 5. MFMAs: every activation operand is read once and used for the four tiles
    float accf[NT][MS][4];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int ms = 0; ms < MS; ++ms)
#pragma unroll
            for (int i = 0; i < 4; ++i) accf[t][ms][i] = 0.0f;
    const v4i zero4 = {0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < SW; ++s) {
        if (s >= nsw) continue;                          // uniform; the loop stays unrolled
        v4i A[2][MS];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int ms = 0; ms < MS; ++ms) {
                const uint4 av = *reinterpret_cast<const uint4*>(reg + (ms * 16 + (lane & 15)) * ROWB + s * SB_K +
                                                                 h * 64 + 16 * (lane >> 4));
                A[h][ms] = v4i{int(av.x), int(av.y), int(av.z), int(av.w)};
            }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const uint4 wq = bq[s * NT + t];
            v4i acc[MS];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t zl = zq[t][s][GPS == 2 ? h : 0];
                const uint32_t zc = ASYM ? (128u - zl) * 0x01010101u : 0u;
                const v4i b = unpack_b<ASYM>(h ? wq.z : wq.x, h ? wq.w : wq.y, zc);
                const bool first = GPS == 2 || h == 0;
#pragma unroll
                for (int ms = 0; ms < MS; ++ms)
                    acc[ms] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[h][ms], b, first ? zero4 : acc[ms], 0, 0, 0);
                if (GPS == 2 || h == 1) {
                    const float g = sc[t][s][GPS == 2 ? h : 0];
                    const float scl = ASYM ? g : g * 0.0625f;
#pragma unroll
                    for (int ms = 0; ms < MS; ++ms)
#pragma unroll
                        for (int i = 0; i < 4; ++i) accf[t][ms][i] = fmaf((float)acc[ms][i], scl, accf[t][ms][i]);
                }
            }
        }
    }

    // 6. slice partials into this wave's region (its activations are no longer read), then the
    //    fixed-order sum over the 16 slices
    //    Layout: each tile row block's 4 accumulators per lane are split into 4 / MS planes of MS
    //    consecutive values, lane-contiguous, so that both the writes and the reducers' reads (MS
    //    values per lane) cover contiguous bytes across a wave: no LDS bank conflicts (a float4 per
    //    lane, read 8 bytes at a time, conflicted two ways).
    constexpr int NPL = 4 / MS;                                  // planes per tile row block
    asm volatile("" ::: "memory");
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int ms = 0; ms < MS; ++ms)
#pragma unroll
            for (int pl = 0; pl < NPL; ++pl) {
                float* dst = reinterpret_cast<float*>(reg + (((t * MS + ms) * NPL + pl) * 64 + lane) * (4 * MS));
#pragma unroll
                for (int j = 0; j < MS; ++j) dst[j] = accf[t][ms][pl * MS + j];
            }
    __syncthreads();
    float y[MS];
#pragma unroll
    for (int j = 0; j < MS; ++j) y[j] = 0.0f;
#pragma unroll
    for (int w2 = 0; w2 < KW; ++w2) {
        const float* p = reinterpret_cast<const float*>(
            smem + w2 * S::REG + (((rt * MS + rms) * NPL + ri0 / MS) * 64 + lane) * (4 * MS));
#pragma unroll
        for (int j = 0; j < MS; ++j) y[j] += p[j];
    }
    const int tile = int(blockIdx.x) * NT + rt;
    const int col = tile * 16 + (lane & 15);
    if (tile >= ntiles || col >= a.N) return;
#pragma unroll
    for (int j = 0; j < MS; ++j) {
        const int row = rms * 16 + 4 * (lane >> 4) + ri0 + j;
        if (row >= nrows) continue;
        const float v = y[j] * sxr[j];      // row < nrows: sxr[j] is this row's scale
        if (a.out_f32)
            reinterpret_cast<float*>(a.Y)[size_t(rbeg + row) * a.ldy + col] = v;
        else
            reinterpret_cast<uint16_t*>(a.Y)[size_t(rbeg + row) * a.ldy + col] = (uint16_t)f32_to_bf16_rne(v);
    }
}

bool decode_split_fits(int K, int M, int gps, int bits) {
    const int nsb = K / SB_K;
    return bits == 4 && (gps == 1 || gps == 2) && M >= 1 && M <= 32 && nsb > 16 && nsb <= 32;
}

template <int MS, int GPS, bool ASYM, bool H16>
static void launch_split_t(const GemmArgs& a, hipStream_t s) {
    using S = DecodeSplitShape<MS, 2>;
    auto kern = gemm_decode_split_kernel<MS, 2, GPS, ASYM, H16>;
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(S::LDS));
    (void)attr;
    const int ntiles = (a.N + 15) / 16;
    const dim3 grid((ntiles + S::NT - 1) / S::NT, (a.M + S::MT - 1) / S::MT);
    kern<<<grid, dim3(S::NTHR), S::LDS, s>>>(a);
}

template <int MS>
static void launch_split_ms(const GemmArgs& a, int gps, bool asym, hipStream_t s) {
    if (gps == 1) {
        if (a.h16) { if (asym) launch_split_t<MS, 1, true, true>(a, s); else launch_split_t<MS, 1, false, true>(a, s); }
        else if (asym) launch_split_t<MS, 1, true, false>(a, s); else launch_split_t<MS, 1, false, false>(a, s);
    } else {
        if (a.h16) { if (asym) launch_split_t<MS, 2, true, true>(a, s); else launch_split_t<MS, 2, false, true>(a, s); }
        else if (asym) launch_split_t<MS, 2, true, false>(a, s); else launch_split_t<MS, 2, false, false>(a, s);
    }
}

void launch_decode_split(const GemmArgs& a, int gps, bool asym, hipStream_t s) {
    if (a.M <= 16) launch_split_ms<1>(a, gps, asym, s);
    else launch_split_ms<2>(a, gps, asym, s);
}

}  // namespace w4a8
