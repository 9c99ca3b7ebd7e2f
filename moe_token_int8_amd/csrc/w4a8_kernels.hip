// gfx950 (CDNA4) kernels and GPU entry points of the W4A8 library.
//
// Sources (cited as P1..P5 with the page's own section names):
//   P1 "Kimi 2.7 MoE: from 4-bit storage to INT8 (W4A8)"              (pwwt.cn)
//   P3 "Quantization: formats, error and the real execution path"     (wineandchord.com)
//   P5 "Inference quantization, chapter 1: the Linear layer"          (sgdbs.github.io)
//
// Data path of the GEMM (P5 section 4 "ideal path", P1 sections 4.4 and 5.2):
//   packed INT4 codes --128-bit load--> registers --shift/mask--> INT8 MFMA operand
//   INT8 x INT8 -> INT32 per K-group (v_mfma_i32_16x16x64_i8)
//   per group: acc_f32 = fma(float(P_group), s_w[group, n], acc_f32)
//   end: y = acc_f32 * s_x[m] -> bfloat16 (round to nearest even) or float32.
// Dequantized weights never leave registers.
//
// MFMA 16x16x64 i8 operand convention used throughout: lane l supplies 16 bytes of
// A row (l % 16) and of B column (l % 16), both for k in [16*(l/16), 16*(l/16)+16) of
// the 64-deep step, in the same byte order, so every product pairs the same k on both
// sides.  The INT32 result of lane l is C[4*(l/16) + i][l % 16], i = 0..3.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <type_traits>

#include "w4a8_device.h"
#include "w4a8_internal.h"

namespace w4a8 {

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
    return v;
}

// Block-wide max of |x| bit patterns (non-negative floats order like unsigned integers;
// NaN patterns sort above +Inf).  nwaves <= 16.
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* red, int nwaves) {
    v = wave_max_u32(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = v;
    __syncthreads();
    uint32_t r = 0;
    for (int w = 0; w < nwaves; ++w) r = max(r, red[w]);
    return r;
}

// ------------------------------------------------------------------------------------
// per-token INT8 activation quantization (P1 section 3.3, P5 section 8.3)
// One 256-thread workgroup per row; each thread holds IT x 8 bf16 values in registers
// so the row is read from HBM once.
// SMOOTH: every value is first multiplied by inv_alpha[k] (one float32 product), the
// activation side of the equivalent rescaling Y = (X diag(alpha)^-1)(diag(alpha) W) (P3
// "Weight-Activation"), fused here so that it adds no kernel; the product is recomputed,
// identically, in the quantization pass instead of being held in registers.
// ------------------------------------------------------------------------------------
template <int IT, bool SMOOTH = false>
__global__ __launch_bounds__(256) void quant_act_kernel(const uint16_t* __restrict__ X, int K, int ldx,
                                                        int8_t* __restrict__ Xq, float* __restrict__ sx,
                                                        const float* __restrict__ inv_alpha = nullptr) {
    __shared__ uint32_t red[4];
    const int row = blockIdx.x, tid = threadIdx.x;
    const uint16_t* xr = X + size_t(row) * size_t(ldx);
    uint4 v[IT];
    uint32_t amax = 0;
    // the 8 factors of the values at k (SMOOTH)
    auto factors = [&](int k, float (&f)[8]) {
        const float4 a = *reinterpret_cast<const float4*>(inv_alpha + k);
        const float4 b = *reinterpret_cast<const float4*>(inv_alpha + k + 4);
        f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
    };
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int k = (it * 256 + tid) * 8;
        v[it] = make_uint4(0, 0, 0, 0);
        if (k < K) v[it] = *reinterpret_cast<const uint4*>(xr + k);
        const uint32_t w[4] = {v[it].x, v[it].y, v[it].z, v[it].w};
        if constexpr (SMOOTH) {
            if (k < K) {
                float f[8];
                factors(k, f);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    amax = max(amax, __float_as_uint(bf16_to_f32(w[j] & 0xffffu) * f[2 * j]) & 0x7fffffffu);
                    amax = max(amax, __float_as_uint(bf16_to_f32(w[j] >> 16) * f[2 * j + 1]) & 0x7fffffffu);
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                amax = max(amax, (w[j] & 0x7fffu) << 16);
                amax = max(amax, w[j] & 0x7fff0000u);
            }
        }
    }
    amax = block_max_u32(amax, red, 4);
    const RowScale rs = row_scale(amax);
    int8_t* qr = Xq + size_t(row) * size_t(K);
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int k = (it * 256 + tid) * 8;
        if (k >= K) continue;
        const uint32_t w[4] = {v[it].x, v[it].y, v[it].z, v[it].w};
        uint32_t out[2] = {0, 0};
        if (rs.finite) {
            float f[8] = {1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f};
            if constexpr (SMOOTH) factors(k, f);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float x0 = bf16_to_f32(w[j] & 0xffffu), x1 = bf16_to_f32(w[j] >> 16);
                if constexpr (SMOOTH) {
                    x0 *= f[2 * j];
                    x1 *= f[2 * j + 1];
                }
                const int q0 = quant_one(x0, rs.d, rs.inv, rs.fast);
                const int q1 = quant_one(x1, rs.d, rs.inv, rs.fast);
                const uint32_t pair = (uint32_t(q0) & 0xffu) | ((uint32_t(q1) & 0xffu) << 8);
                out[j >> 1] |= pair << ((j & 1) * 16);
            }
        }
        *reinterpret_cast<uint2*>(qr + k) = make_uint2(out[0], out[1]);
    }
    if (tid == 0) sx[row] = rs.s;
}

// ------------------------------------------------------------------------------------
// SiLU-gated activation + per-row requantization (P1 section 1 and section 3.1)
// ------------------------------------------------------------------------------------
// Static (calibrated) activation scales (P1 section 3.2: the scale is measured on a
// calibration set ahead of time, so serving needs no row reduction; section 3.1: each expert
// keeps its own scale).  The rule is the per-token one with the scale given.

// Expert that owns sorted row r: the e with offs[e] <= r < offs[e + 1], for offs
// non-decreasing with offs[0] = 0 and r < offs[E] (binary search; uniform per workgroup).
__device__ __forceinline__ int expert_of_row(const int32_t* __restrict__ offs, int E, int r) {
    int lo = 0, hi = E;                        // offs[lo] <= r < offs[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (offs[mid] <= r) lo = mid;
        else hi = mid;
    }
    return lo;
}

// Row r of Xq quantizes source row src of X with the scale s[e]: src = r (gather == NULL) or
// gather[r] / k; e = 0 (offs == NULL) or the expert that owns sorted row r.  Rows no expert
// owns (r >= offs[E]: routing ids outside [0, E)) and gathered rows outside [0, T) get zero
// codes and scale 0.  One 256-thread workgroup per row, one pass: each thread issues the loads
// of its IT pieces of 8 values at once, then quantizes and stores them (rows longer than
// IT * 2048 values take several such passes).
template <int IT>
__global__ __launch_bounds__(256) void quant_static_kernel(const uint16_t* __restrict__ X, int K, int ldx, int T,
                                                           const float* __restrict__ s,
                                                           const int32_t* __restrict__ gather, int k,
                                                           const int32_t* __restrict__ offs, int E,
                                                           int8_t* __restrict__ Xq, float* __restrict__ sx) {
    const int row = blockIdx.x, tid = threadIdx.x;
    int e = 0, src = row;
    bool live = true;
    if (offs) {
        live = row < offs[E];
        if (live) e = expert_of_row(offs, E, row);
    }
    if (gather && live) {
        const int gr = gather[row];
        src = gr >= 0 ? gr / k : -1;
        live = src >= 0 && src < T;
    }
    const float sv = live ? s[e] : 0.0f;
    const uint16_t* xr = X + size_t(live ? src : 0) * size_t(ldx);
    int8_t* qr = Xq + size_t(row) * size_t(K);
    for (int base = 0; base < K; base += IT * 256 * 8) {
        uint4 v[IT];
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int kk = base + (it * 256 + tid) * 8;
            v[it] = make_uint4(0, 0, 0, 0);
            if (live && kk < K) v[it] = *reinterpret_cast<const uint4*>(xr + kk);
        }
        const RowScale rs = static_row_scale(sv);
        // the scale is uniform per row: the d > 2^120 handling is one branch, not a select per value
        auto quantize = [&](auto huge) __attribute__((always_inline)) {
#pragma unroll
            for (int it = 0; it < IT; ++it) {
                const int kk = base + (it * 256 + tid) * 8;
                if (kk >= K) continue;
                uint32_t out[2] = {0, 0};
                if (rs.finite) {
                    const uint32_t w[4] = {v[it].x, v[it].y, v[it].z, v[it].w};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int q0 = quant_static_one<decltype(huge)::value>(bf16_to_f32(w[j] & 0xffffu), rs);
                        const int q1 = quant_static_one<decltype(huge)::value>(bf16_to_f32(w[j] >> 16), rs);
                        const uint32_t pair = (uint32_t(q0) & 0xffu) | ((uint32_t(q1) & 0xffu) << 8);
                        out[j >> 1] |= pair << ((j & 1) * 16);
                    }
                }
                *reinterpret_cast<uint2*>(qr + kk) = make_uint2(out[0], out[1]);
            }
        };
        if (__builtin_amdgcn_readfirstlane(int(rs.huge))) quantize(std::true_type{});
        else quantize(std::false_type{});
    }
    if (tid == 0) sx[row] = sv;
}

// STATIC: row r (in expert-sorted order) takes the scale s[e] of the expert that owns it
// (zero codes and scale 0 past offs[E]) instead of its own abs-max.
template <int IT, bool STATIC = false>
__global__ __launch_bounds__(256) void silu_quant_kernel(const uint16_t* __restrict__ GU, int I,
                                                         int8_t* __restrict__ Hq, float* __restrict__ sh,
                                                         const float* __restrict__ s = nullptr,
                                                         const int32_t* __restrict__ offs = nullptr, int E = 0) {
    __shared__ uint32_t red[4];
    const int row = blockIdx.x, tid = threadIdx.x;
    const uint16_t* gp = GU + size_t(row) * size_t(2 * I);
    const uint16_t* up = gp + I;
    float h[IT][8];
    uint32_t amax = 0;
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int k = (it * 256 + tid) * 8;
        uint4 gv = make_uint4(0, 0, 0, 0), uv = make_uint4(0, 0, 0, 0);
        if (k < I) {
            gv = *reinterpret_cast<const uint4*>(gp + k);
            uv = *reinterpret_cast<const uint4*>(up + k);
        }
        const uint32_t g4[4] = {gv.x, gv.y, gv.z, gv.w}, u4[4] = {uv.x, uv.y, uv.z, uv.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t gb = (j & 1) ? (g4[j >> 1] >> 16) : (g4[j >> 1] & 0xffffu);
            const uint32_t ub = (j & 1) ? (u4[j >> 1] >> 16) : (u4[j >> 1] & 0xffffu);
            h[it][j] = silu_mul(bf16_to_f32(gb), bf16_to_f32(ub));
            amax = max(amax, __float_as_uint(h[it][j]) & 0x7fffffffu);
        }
    }
    RowScale rs;
    if constexpr (STATIC) {
        rs = static_row_scale(row < offs[E] ? s[expert_of_row(offs, E, row)] : 0.0f);
    } else {
        amax = block_max_u32(amax, red, 4);
        rs = row_scale(amax);
    }
    int8_t* qr = Hq + size_t(row) * size_t(I);
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int k = (it * 256 + tid) * 8;
        if (k >= I) continue;
        uint32_t out[2] = {0, 0};
        if (rs.finite) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int q = STATIC ? quant_static_one(h[it][j], rs) : quant_one(h[it][j], rs.d, rs.inv, rs.fast);
                out[j >> 2] |= (uint32_t(q) & 0xffu) << ((j & 3) * 8);
            }
        }
        *reinterpret_cast<uint2*>(qr + k) = make_uint2(out[0], out[1]);
    }
    if (tid == 0) sh[row] = rs.s;
}

// ------------------------------------------------------------------------------------
// W4A8 GEMM, decode variant (M-tiles of 16 or 32 rows; dense decode and per-expert tiles)
//
// Workgroup = NT column tiles (16 columns each) x KW K-slices, one wave per (tile, slice).
// Each chunk of CS = KW*SBN superblocks (128 k each) is processed in one shot:
//   1. the workgroup loads the chunk's activation rows [MT x 128*CS] into LDS (these loads
//      are issued first, so waiting for them never waits on the weight stream);
//   2. every wave issues the loads of all SBN of its weight superblocks (16 bytes per lane
//      per superblock) and of their group scales / zero points, then consumes them in
//      issue order while later ones are still in flight;
//   3. activation fragments come from LDS (ds_read, counted separately from the weight
//      loads).
// So every weight byte of a chunk is requested from HBM at once, activations are read
// from L2 once per workgroup, and the dequantized weights exist only in registers.
// The KW slices' float32 accumulators are summed in slice order through LDS (the result
// does not depend on scheduling), then the row scale is applied and the tile stored.
// ------------------------------------------------------------------------------------
template <int MS, int NT, int KW, int SBN>
struct DecodeShape {
    static constexpr int MT = 16 * MS;
    static constexpr int NTHR = 64 * NT * KW;
    static constexpr int CS = KW * SBN;                        // superblocks per chunk
    // padded LDS row stride: 32 bytes past a multiple of 128, so the 16 rows x 4 k-chunks that a
    // 16x16x64 operand read spreads over lanes land in distinct banks (with 16 bytes of padding,
    // chunk c + 1 of row r and chunk c of row r + 1 shared banks: SQ_LDS_BANK_CONFLICT counted
    // about 2.8 conflict cycles per LDS instruction)
    static constexpr int ROWB = CS * SB_K + 32;
    static constexpr int APT = (MT * CS * 8 + NTHR - 1) / NTHR;  // 16-byte A pieces / thread
    static constexpr size_t LDS_A = size_t(MT) * ROWB;
    static constexpr size_t LDS_RED = size_t(KW > 1 ? KW - 1 : 1) * NT * MS * 4 * 64 * 4;
    static constexpr size_t LDS = LDS_A + LDS_RED;
};

// w4a8_linear fuses quantization into the GEMM up to this many activation values.  Every
// workgroup quantizes all of them, and that redundant work outgrows the launch it saves
// quickly (measured on the 4096 x 14336 projection: fused beats quantize-then-GEMM at
// M = 1 and 2, loses at M = 8).
constexpr size_t FUSED_MAX_ELEMS = 8192;

// FQ (w4a8_linear, M * K <= FUSED_MAX_ELEMS): every workgroup quantizes the bf16 rows itself
// (the per-token rule of quant_act_kernel, the same device routines) straight into its LDS
// activation tile; workgroup 0 also exports the codes and row scales.
// W8: 8-bit weight codes (2 KiB superblocks, 32 bytes per layout lane), used as MFMA operands
// as loaded; otherwise 4-bit codes unpacked in registers.
// H16: binary16 group scales (converted to float32 as loaded).
template <int MS, int NT, int KW, int SBN, int GPS, bool ASYM, int MODE, bool MOE, bool MULTI, bool FQ, bool W8,
          bool H16 = false>
__global__ __launch_bounds__(64 * NT * KW) void gemm_decode_kernel(GemmArgs a) {
    using S = DecodeShape<MS, NT, KW, SBN>;
    static_assert(!FQ || (MS == 1 && !MOE && MODE == MODE_OUT && !MULTI), "fused quantization: dense, one chunk");
    static_assert(!W8 || (!ASYM && !MOE), "8-bit codes: symmetric, dense");
    // GPS: groups per superblock, 4 (g = 32), 2 (g = 64) or 1 (g = 128); 0 is g = 256, one group per two
    // superblocks (a wave's superblocks come in aligned pairs, so a group never straddles waves)
    // GPS -1: per-channel scales (g = K): each wave converts its slice's int32 sum once, and
    // the slices add in the fixed float32 reduction below
    static_assert(GPS > 0 || !MOE, "g = 256 and per-channel: dense");
    static_assert(GPS != 4 || !MOE, "g = 32: dense");
    static_assert(GPS >= 0 || MODE == MODE_OUT, "per-channel partials: the prefill kernel only");
    constexpr int NG = GPS <= 0 ? 1 : GPS;              // scale entries per superblock
    auto gidx = [](int sb, int gi) { return GPS < 0 ? 0 : GPS == 0 ? sb / 2 : sb * GPS + gi; };
    constexpr uint32_t SBB = W8 ? 2048u : 1024u;         // bytes per superblock
    constexpr uint32_t LB = W8 ? 32u : 16u;              // bytes per layout lane
    constexpr int MT = S::MT, NTHR = S::NTHR, CS = S::CS, ROWB = S::ROWB, APT = S::APT;
    // weight superblocks requested before the activation hand-off (the rest right after it)
    constexpr int BE = MS == 2 ? (SBN < 3 ? SBN : 3) : (SBN < 4 ? SBN : 4);
    extern __shared__ __align__(16) uint8_t smem[];
    float* red = reinterpret_cast<float*>(smem + S::LDS_A);
    uint32_t* rowmax = reinterpret_cast<uint32_t*>(smem + S::LDS);   // FQ: row abs-maxima
    // wave-derived indices are made explicitly uniform so per-slice loops branch on scalars
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int t = wave % NT, q = wave / NT;
    const int ntiles = (a.N + 15) / 16;
    // paired form (grouped, static SiLU-requant epilogue): tiles t < NT / 2 are gate tiles, the
    // others their up tiles
    const int tile = MOE ? pair_tile(a, blockIdx.x * NT, t, NT) : blockIdx.x * NT + t;
    const bool tvalid = tile < ntiles;
    const int tile_c = tvalid ? tile : ntiles - 1;
    const int nsb = a.K / SB_K;

    int rbeg, rend, expert = 0;
    const uint8_t* blob = a.blob;
    if (!MOE) {
        rbeg = blockIdx.y * MT;
        rend = min(a.M, rbeg + MT);
    } else {
        const TileRows tr = moe_tile<MT>(a, blockIdx.y, lane);
        if (tr.expert < 0) return;                       // uniform over the workgroup
        rbeg = tr.rbeg;
        rend = tr.rend;
        expert = tr.expert;
        blob = a.blob + size_t(tr.expert) * a.expert_stride;
    }
    const int nrows = rend - rbeg;
    const uint8_t* codes = blob + a.codes_off;
    const float* scales = reinterpret_cast<const float*>(blob + a.scales_off);
    const uint16_t* scales16 = reinterpret_cast<const uint16_t*>(blob + a.scales_off);
    const uint8_t* zeros = blob + a.zeros_off;

    // grouped form: source row (of Xq and sx) of tile row r, held by lane r and shared by
    // cross-lane reads, so no activation piece waits on a dependent gather load of its own
    int srcl = -1;
    if constexpr (MOE) {
        if (lane < nrows) srcl = a.gather ? gather_src(a, rbeg + lane) : rbeg + lane;
    }
    auto src_of = [&](int r) { return MOE ? __shfl(srcl, r & 63, 64) : rbeg + r; };

    // row scales of the rows this lane stores, fetched before anything else so the
    // epilogue never waits on a load
    float sxr[MS][4];
#pragma unroll
    for (int ms = 0; ms < MS; ++ms)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sxr[ms][i] = 0.0f;
            const int r = ms * 16 + 4 * (lane >> 4) + i;
            const int srow = src_of(r);
            if (!FQ && MODE != MODE_PARTIALS && q == 0 && r < nrows) sxr[ms][i] = srow >= 0 ? a.sx[srow] : 0.0f;
        }

    float accf[MS][4];
#pragma unroll
    for (int ms = 0; ms < MS; ++ms)
#pragma unroll
        for (int i = 0; i < 4; ++i) accf[ms][i] = 0.0f;
    const v4i zero4 = {0, 0, 0, 0};

    // one chunk of the K loop.  A K that fits one chunk (MULTI = false) runs it as
    // straight-line code, so no loop-carried state forces conservative load waits.
    auto chunk = [&](const int cb) __attribute__((always_inline)) {
        const int clen = min(CS, nsb - cb);
        const int rowpieces = clen * 8;                  // 16-byte int8 pieces per row in this chunk
        // Load order matters: every wave of the workgroup first requests its activation
        // pieces and group scales, then a barrier, and only then the weight stream.  The
        // memory pipeline of a compute unit serves requests roughly in order, so the small
        // operands that gate the first MFMA never queue behind another wave's weights.
        // 1. activation pieces into registers: piece p = tid + i * NTHR is row p / (CS * 8),
        //    16 bytes at column p % (CS * 8); rows past the tile's end are neither loaded nor
        //    written (their MFMA outputs are never stored)
        //    (FQ: the piece's 16 bfloat16 values, 32 bytes; one piece per thread covers the
        //    M rows, which the launcher checks: (M - 1) * CS * 8 + nsb * 8 <= NTHR)
        constexpr int APX = FQ ? 1 : S::APT;
        uint4 xv[S::APT];
        uint4 xb[FQ ? 1 : 1][2];
#pragma unroll
        for (int i = 0; i < APX; ++i) {
            const int pc = tid + i * NTHR;
            const int row = pc / (CS * 8), c = pc - row * (CS * 8);
            xv[i] = make_uint4(0, 0, 0, 0);
            if (FQ) xb[0][0] = xb[0][1] = make_uint4(0, 0, 0, 0);
            const int srow = src_of(row);
            const int src = (row < nrows && c < rowpieces) ? srow : -1;
            if (src >= 0) {
                if (FQ) {
                    const uint4* xp = reinterpret_cast<const uint4*>(a.X + size_t(src) * a.ldx + c * 16);
                    xb[0][0] = xp[0];
                    xb[0][1] = xp[1];
                } else {
                    xv[i] = *reinterpret_cast<const uint4*>(a.Xq + size_t(src) * a.K + size_t(cb) * SB_K + c * 16);
                }
            }
        }
        // 2. this wave's group scales and zero points
        const int s0 = cb + q * SBN;
        const int s_end = min(cb + clen, s0 + SBN);
        uint4 bq[SBN];
        uint4 bq2[W8 ? SBN : 1];                         // W8: the lane's second 16 bytes
        float sc[SBN][NG];
        uint32_t zq[SBN][NG];
        // 32-bit offsets from wave-uniform bases (a blob is far below 4 GiB): saddr-form loads,
        // no 64-bit per-lane addresses to keep alive
        const uint32_t boff = (uint32_t(tile_c) * uint32_t(nsb)) * SBB + uint32_t(lane) * LB;
        const uint32_t moff = uint32_t(tile_c) * uint32_t(a.G) * 16u + uint32_t(lane & 15);
#pragma unroll
        for (int s = 0; s < SBN; ++s) {
            const uint32_t sb = uint32_t(min(s0 + s, nsb - 1));
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
                const uint32_t mi = moff + uint32_t(gidx(int(sb), gi)) * 16u;
                sc[s][gi] = H16 ? f16_to_f32(scales16[mi]) : scales[mi];
                if (ASYM) zq[s][gi] = zeros[mi];
            }
        }
        // 3. issue fence: all small requests of the workgroup are out before any weight request
        //    (FQ: it also publishes the cleared row maxima)
        if (FQ) {
            if (tid < MT) rowmax[tid] = 0u;
            lds_barrier();
        } else {
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        }
        // 4. this wave's first BE weight superblocks, in the order they are consumed; the rest
        //    follow once the activations are in LDS, which keeps the activation loads from
        //    queueing behind the whole weight stream
#pragma unroll
        for (int s = 0; s < BE; ++s) {
            const uint32_t sb = uint32_t(min(s0 + s, nsb - 1));
            bq[s] = stream_load(codes + (boff + sb * SBB));
            if constexpr (W8) bq2[s] = stream_load(codes + (boff + sb * SBB + 16u));
        }
        // 5. activations into LDS.  Waits are per register, so the weight loads stay in flight.
        if (FQ) {
            // row abs-max: a row holds CS * 8 pieces, a multiple of 64, so each wave's 64
            // pieces of one iteration lie in one row: a wave max and one LDS atomic
#pragma unroll
            for (int i = 0; i < APX; ++i) {
                const int pc = tid + i * NTHR;
                const int row = pc / (CS * 8);
                uint32_t amax = 0;
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const uint32_t wv[4] = {xb[0][hh].x, xb[0][hh].y, xb[0][hh].z, xb[0][hh].w};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        amax = max(amax, (wv[j] & 0x7fffu) << 16);
                        amax = max(amax, wv[j] & 0x7fff0000u);
                    }
                }
                amax = wave_max_u32(amax);
                if (lane == 0 && row < nrows) atomicMax(rowmax + row, amax);
            }
            lds_barrier();
#pragma unroll
            for (int i = 0; i < APX; ++i) {
                const int pc = tid + i * NTHR;
                const int row = pc / (CS * 8), c = pc - row * (CS * 8);
                if (row >= nrows || c >= rowpieces) continue;
                const RowScale rs = row_scale(rowmax[row]);
                uint32_t out[4] = {0, 0, 0, 0};
                if (rs.finite) {
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const uint32_t wv[4] = {xb[0][hh].x, xb[0][hh].y, xb[0][hh].z, xb[0][hh].w};
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const int q0 = quant_one(bf16_to_f32(wv[j] & 0xffffu), rs.d, rs.inv, rs.fast);
                            const int q1 = quant_one(bf16_to_f32(wv[j] >> 16), rs.d, rs.inv, rs.fast);
                            const uint32_t pair = (uint32_t(q0) & 0xffu) | ((uint32_t(q1) & 0xffu) << 8);
                            out[hh * 2 + (j >> 1)] |= pair << ((j & 1) * 16);
                        }
                    }
                }
                *reinterpret_cast<uint4*>(smem + row * ROWB + c * 16) = make_uint4(out[0], out[1], out[2], out[3]);
            }
#pragma unroll
            for (int ms = 0; ms < MS; ++ms)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = ms * 16 + 4 * (lane >> 4) + i;
                    sxr[ms][i] = (q == 0 && row < nrows) ? row_scale<false>(rowmax[row]).s : 0.0f;
                }
        } else {
#pragma unroll
            for (int i = 0; i < S::APT; ++i) {
                const int pc = tid + i * NTHR;
                const int row = pc / (CS * 8), c = pc - row * (CS * 8);
                if (row < nrows && c < rowpieces) *reinterpret_cast<uint4*>(smem + row * ROWB + c * 16) = xv[i];
            }
        }
        lds_barrier();
#pragma unroll
        for (int s = BE; s < SBN; ++s) {
            const uint32_t sb = uint32_t(min(s0 + s, nsb - 1));
            bq[s] = stream_load(codes + (boff + sb * SBB));
            if constexpr (W8) bq2[s] = stream_load(codes + (boff + sb * SBB + 16u));
        }
        // keep these requests issued here: otherwise each is sunk next to its first use
        // behind a full wait, leaving one weight load in flight per wave
        asm volatile("" ::: "memory");
        // 6. MFMA over this wave's superblocks
        v4i acc[MS];
#pragma unroll
        for (int s = 0; s < SBN; ++s) {
            const int sb = s0 + s;
            if (sb >= s_end) break;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                // GPS 4 (g = 32): the half's 64 k hold groups 2h (lanes 0-31) and 2h + 1
                // (lanes 32-63); each group runs its own MFMA with the other lanes' B zeroed
                v4i b;
                if constexpr (W8) {
                    const uint4 u = h ? bq2[s] : bq[s];
                    b = v4i{int(u.x), int(u.y), int(u.z), int(u.w)};
                } else {
                    const uint32_t w0 = h ? bq[s].z : bq[s].x;
                    const uint32_t w1 = h ? bq[s].w : bq[s].y;
                    const uint32_t zl = GPS == 4 ? ((lane >> 5) ? zq[s][NG > 1 ? 2 * h + 1 : 0] : zq[s][NG > 1 ? 2 * h : 0])
                                                 : zq[s][GPS == 2 ? h : 0];
                    const uint32_t zc = ASYM ? (128u - zl) * 0x01010101u : 0u;
                    b = unpack_b<ASYM>(w0, w1, zc);
                }
                v4i A[MS];
#pragma unroll
                for (int ms = 0; ms < MS; ++ms) {
                    const uint4 av = *reinterpret_cast<const uint4*>(
                        smem + (ms * 16 + (lane & 15)) * ROWB + (sb - cb) * SB_K + h * 64 + 16 * (lane >> 4));
                    A[ms] = v4i{int(av.x), int(av.y), int(av.z), int(av.w)};
                }
#pragma unroll
              for (int u = 0; u < (GPS == 4 ? 2 : 1); ++u) {
                const int gi = GPS == 4 ? 2 * h + u : (GPS == 2) ? h : 0;
                v4i bu = b;
                if constexpr (GPS == 4) {
                    if ((lane >> 5) != u) bu = zero4;
                }
                const bool first = GPS < 0    ? (h == 0 && s == 0)
                                   : GPS == 0 ? (h == 0 && s % 2 == 0)
                                              : ((GPS >= 2) || h == 0);
#pragma unroll
                for (int ms = 0; ms < MS; ++ms)
                    acc[ms] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[ms], bu, first ? zero4 : acc[ms], 0, 0, 0);
                if (GPS < 0    ? (h == 1 && sb == s_end - 1)
                    : GPS == 0 ? (h == 1 && s % 2 == 1)
                               : (GPS >= 2 || h == 1)) {
                    if (MODE == MODE_PARTIALS) {
                        const int col = tile * 16 + (lane & 15);
#pragma unroll
                        for (int ms = 0; ms < MS; ++ms)
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const int row = rbeg + ms * 16 + 4 * (lane >> 4) + i;
                                if (tvalid && row < rend && col < a.N) {
                                    const int v = (ASYM || W8) ? acc[ms][i] : (acc[ms][i] >> 4);
                                    a.P[(size_t(row) * a.N + col) * a.G + size_t(gidx(sb, gi))] = v;
                                }
                            }
                    } else {
                        const float scl = (ASYM || W8) ? sc[s][gi] : sc[s][gi] * 0.0625f;
#pragma unroll
                        for (int ms = 0; ms < MS; ++ms)
#pragma unroll
                            for (int i = 0; i < 4; ++i) accf[ms][i] = fmaf((float)acc[ms][i], scl, accf[ms][i]);
                    }
                }
              }
            }
        }
        if (cb + CS < nsb) lds_barrier();                // LDS is rewritten by the next chunk
    };
    if constexpr (!MULTI) {
        chunk(0);                                        // the launcher guarantees nsb <= CS
    } else {
        for (int cb = 0; cb < nsb; cb += CS) chunk(cb);
    }
    if (MODE == MODE_PARTIALS) return;

    // slice-ordered reduction through its own LDS region, row scale, store
    constexpr int NV = MS * 4;
    if (KW > 1) {
        if (q > 0) {
#pragma unroll
            for (int ms = 0; ms < MS; ++ms)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    red[(((q - 1) * NT + t) * NV + ms * 4 + i) * 64 + lane] = accf[ms][i];
        }
        __syncthreads();
        if (q != 0) return;
#pragma unroll
        for (int w = 1; w < KW; ++w)
#pragma unroll
            for (int ms = 0; ms < MS; ++ms)
#pragma unroll
                for (int i = 0; i < 4; ++i) accf[ms][i] += red[(((w - 1) * NT + t) * NV + ms * 4 + i) * 64 + lane];
    }
    if (FQ && blockIdx.x == 0) {
        // fused path: workgroup 0 exports the activation codes and row scales (after all of
        // its weight loads, so no store sits inside the load stream); the threads still
        // running here are 0 .. NT * 64 - 1 (KW > 1) or all of them
        const int rp = nsb * 8;                          // 16-byte pieces per row
        for (int pc = tid; pc < nrows * rp; pc += (KW > 1 ? NT * 64 : NTHR)) {
            const int row = pc / rp, c = pc - row * rp;
            *reinterpret_cast<uint4*>(const_cast<int8_t*>(a.Xq) + size_t(rbeg + row) * a.K + c * 16) =
                *reinterpret_cast<const uint4*>(smem + row * ROWB + c * 16);
        }
        if (tid < nrows) const_cast<float*>(a.sx)[rbeg + tid] = row_scale<false>(rowmax[tid]).s;
    }
    if constexpr (MOE && MODE == MODE_OUT) {
        if (a.Hq) {
            // paired form: the up waves hand their outputs to the gate waves through the
            // activation area of LDS (every wave's MFMAs are done); only the slice-0 waves are
            // still running (s_barrier waits for the waves that have not ended)
            static_assert(NT % 2 == 0, "paired form: gate and up tiles in equal numbers");
            float* pb = reinterpret_cast<float*>(smem);
            const RowScale prs = static_row_scale(a.s_dn[expert]);
            if (t >= NT / 2) {
#pragma unroll
                for (int ms = 0; ms < MS; ++ms)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        pb[((t - NT / 2) * NV + ms * 4 + i) * 64 + lane] = accf[ms][i] * sxr[ms][i];
            }
            lds_barrier();
            const int gt = int(blockIdx.x) * (NT / 2) + t;
            if (t < NT / 2 && gt < a.pair_n / 16) {
#pragma unroll
                for (int ms = 0; ms < MS; ++ms)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int row = ms * 16 + 4 * (lane >> 4) + i;
                        if (rbeg + row >= rend) continue;
                        const float yu = pb[(t * NV + ms * 4 + i) * 64 + lane];
                        a.Hq[size_t(rbeg + row) * a.pair_n + gt * 16 + (lane & 15)] =
                            int8_t(silu_static_code(accf[ms][i] * sxr[ms][i], yu, prs));
                    }
            }
            if (blockIdx.x == 0 && tid < nrows) a.sh[rbeg + tid] = prs.s;
            return;
        }
    }
    const int col = tile * 16 + (lane & 15);
    if (!tvalid || col >= a.N) return;
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = rbeg + ms * 16 + 4 * (lane >> 4) + i;
            if (row >= rend) continue;
            const float y = accf[ms][i] * sxr[ms][i];
            if (a.out_f32)
                reinterpret_cast<float*>(a.Y)[size_t(row) * a.ldy + col] = y;
            else
                reinterpret_cast<uint16_t*>(a.Y)[size_t(row) * a.ldy + col] = (uint16_t)f32_to_bf16_rne(y);
        }
    }
}

// ------------------------------------------------------------------------------------
// W4A8 GEMM, K-slice variant for the grouped (MoE) form: activations straight into registers
//
// A workgroup covers T column tiles (16 columns each) over all of K.  Wave w owns the
// K-slice of superblocks [w * SW, w * SW + SW): it loads its activation fragments once
// into registers (no LDS staging, no barrier before the first MFMA) and reuses them for
// all T tiles, then streams the T x SW weight superblocks of that slice.  Each tile's
// float32 partial goes to LDS as soon as the tile is done; after one barrier every
// thread sums the KW slice partials of its outputs in slice order (fixed, so the result
// does not depend on timing), applies the row scale and stores.
//
// Per workgroup: weights T * SW * KW KiB from HBM, activations MT x K from L2, LDS
// traffic only for the slice reduction (2 * KW * T * 64 * 4 * MS floats).
// ------------------------------------------------------------------------------------

// TG > 1: the workgroup streams TG groups of T tiles one after another, the loads of two
// groups in flight (double-buffered registers), so each workgroup's fixed costs (activation
// fragments, slice reduction, launch) are spread over TG times more weight bytes.
template <int MS, int T, int TG = 1>
struct KsliceShape {
    static constexpr int MT = 16 * MS;
    static constexpr int NV = 4 * MS;                          // accumulators per lane per tile
    static constexpr int TT = T * TG;                          // tiles per workgroup
    // slice partials, then 32 row scales (and 32 floats spare)
    static constexpr size_t lds(int kw) { return size_t(kw) * TT * 64 * NV * 4 + 64 * 4; }
};

// RL (grouped form): a workgroup takes up to MOE_KSLICE_ROWS rows of one expert and runs its
// MT-row tiles one after another on the weights it holds in registers, so an expert's
// weights are streamed once per column tile instead of once per row tile.
constexpr int MOE_KSLICE_ROWS = 128;

template <int MS, int T, int SW, int GPS, bool ASYM, int MODE, bool MOE, int TG, bool RL, bool H16 = false>
__global__ __launch_bounds__(1024) void gemm_kslice_kernel(GemmArgs a) {
    using S = KsliceShape<MS, T, TG>;
    static_assert(!RL || (MOE && MODE == MODE_OUT && TG == 1), "row loop: grouped form, one tile group");
    constexpr int NV = S::NV, TT = S::TT;
    extern __shared__ __align__(16) uint8_t smem[];
    float* red = reinterpret_cast<float*>(smem);              // [KW][TT][64][NV]
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int KW = blockDim.x >> 6;
    const int ntiles = (a.N + 15) / 16;
    const int tile0 = blockIdx.x * TT;
    const int nsb = a.K / SB_K;
    const int sb0 = w * SW;

    int rbeg, rend, rall;                                // rows of the current tile; of the workgroup
    int expert = 0;
    const uint8_t* blob = a.blob;
    if (!MOE) {
        rbeg = blockIdx.y * S::MT;
        rend = min(a.M, rbeg + S::MT);
        rall = rend;
    } else {
        const TileRows tr = moe_tile<RL ? MOE_KSLICE_ROWS : S::MT>(a, blockIdx.y, lane);
        if (tr.expert < 0) return;                       // uniform over the workgroup
        rbeg = tr.rbeg;
        rall = tr.rend;
        rend = min(rall, rbeg + S::MT);
        expert = tr.expert;
        blob = a.blob + size_t(tr.expert) * a.expert_stride;
    }
    int nrows = rend - rbeg;
    const uint8_t* codes = blob + a.codes_off;
    const float* scales = reinterpret_cast<const float*>(blob + a.scales_off);
    const uint16_t* scales16 = reinterpret_cast<const uint16_t*>(blob + a.scales_off);
    const uint8_t* zeros = blob + a.zeros_off;

    // row scales of the tile's rows: fetched first, parked in LDS after the MFMAs
    float* sxs = red + size_t(KW) * TT * 64 * NV;
    float sxv = 0.0f;
    auto load_sx = [&]() __attribute__((always_inline)) {
        sxv = 0.0f;
        if (MODE != MODE_PARTIALS && tid < S::MT && tid < nrows) {
            const int src = (MOE && a.gather) ? gather_src(a, rbeg + tid) : rbeg + tid;
            sxv = src >= 0 ? a.sx[src] : 0.0f;
        }
    };
    load_sx();

    // 1. activation fragments of this wave's K-slice: lane l holds row ms * 16 + l % 16 and
    //    the 16 K-values [16 * (l / 16), +16) of each 64-deep half (the MFMA A operand)
    v4i A[SW][2][MS];
    auto load_a = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int ms = 0; ms < MS; ++ms) {
            const int row = ms * 16 + (lane & 15);
            int src = -1;
            if (row < nrows) src = (MOE && a.gather) ? gather_src(a, rbeg + row) : rbeg + row;
            const bool rv = src >= 0;
            const int8_t* xrow = rv ? a.Xq + size_t(src) * a.K : a.Xq;
#pragma unroll
            for (int s = 0; s < SW; ++s)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    A[s][h][ms] = v4i{0, 0, 0, 0};
                    if (rv && sb0 + s < nsb)
                        A[s][h][ms] = *reinterpret_cast<const v4i*>(xrow + (sb0 + s) * SB_K + h * 64 + 16 * (lane >> 4));
                }
        }
    };
    load_a();
    // 2. per tile group (register set g % 2): group scales and zero points of its T tiles x
    //    SW superblocks, then its weight superblocks in the order they are consumed
    constexpr int NSET = TG > 1 ? 2 : 1;
    float sc[NSET][T][SW][GPS];
    uint32_t zq[NSET][T][SW][GPS];
    uint4 bq[NSET][T][SW];
    auto load_meta = [&](const int g) __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const uint32_t tc = uint32_t(min(MOE ? pair_tile(a, tile0, g * T + t, TT) : tile0 + g * T + t, ntiles - 1));
#pragma unroll
            for (int s = 0; s < SW; ++s) {
                const uint32_t sb = uint32_t(min(sb0 + s, nsb - 1));
#pragma unroll
                for (int gi = 0; gi < GPS; ++gi) {
                    const uint32_t mi = (tc * uint32_t(a.G) + sb * GPS + gi) * 16u + uint32_t(lane & 15);
                    sc[g % NSET][t][s][gi] = H16 ? f16_to_f32(scales16[mi]) : scales[mi];
                    if (ASYM) zq[g % NSET][t][s][gi] = zeros[mi];
                }
            }
        }
    };
    auto load_w = [&](const int g) __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const uint32_t tc = uint32_t(min(MOE ? pair_tile(a, tile0, g * T + t, TT) : tile0 + g * T + t, ntiles - 1));
#pragma unroll
            for (int s = 0; s < SW; ++s) {
                const uint32_t sb = uint32_t(min(sb0 + s, nsb - 1));
                bq[g % NSET][t][s] = stream_load(codes + ((tc * uint32_t(nsb) + sb) * 1024u + uint32_t(lane) * 16u));
            }
        }
    };
    load_meta(0);
    // issue fence: the small requests of every wave go out before any weight request
    lds_barrier();
    // 3. the weight stream: group 0, then group 1 (its scales first)
    load_w(0);
    if constexpr (TG > 1) {
        load_meta(1);
        load_w(1);
    }
    asm volatile("" ::: "memory");                      // keep the whole stream issued here
    // 4. per tile: MFMAs over the slice, per-group epilogue, partial to LDS; after each tile
    //    group, the group two ahead is requested into the registers it used
    const v4i zero4 = {0, 0, 0, 0};
    auto compute = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        const int g = tt / T, t = tt % T, set = g % NSET;
        float accf[MS][4];
#pragma unroll
        for (int ms = 0; ms < MS; ++ms)
#pragma unroll
            for (int i = 0; i < 4; ++i) accf[ms][i] = 0.0f;
        const int tile = tile0 + tt;
#pragma unroll
        for (int s = 0; s < SW; ++s) {
            if (sb0 + s >= nsb) break;
            v4i acc[MS];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int gi = (GPS == 2) ? h : 0;
                const uint32_t w0 = h ? bq[set][t][s].z : bq[set][t][s].x;
                const uint32_t w1 = h ? bq[set][t][s].w : bq[set][t][s].y;
                const uint32_t zc = ASYM ? (128u - zq[set][t][s][gi]) * 0x01010101u : 0u;
                const v4i b = unpack_b<ASYM>(w0, w1, zc);
                const bool first = (GPS == 2) || h == 0;
#pragma unroll
                for (int ms = 0; ms < MS; ++ms)
                    acc[ms] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[s][h][ms], b, first ? zero4 : acc[ms], 0, 0, 0);
                if (GPS == 2 || h == 1) {
                    if (MODE == MODE_PARTIALS) {
                        const int col = tile * 16 + (lane & 15);
#pragma unroll
                        for (int ms = 0; ms < MS; ++ms)
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const int row = ms * 16 + 4 * (lane >> 4) + i;
                                if (tile < ntiles && row < nrows && col < a.N) {
                                    const int v = ASYM ? acc[ms][i] : (acc[ms][i] >> 4);
                                    a.P[(size_t(rbeg + row) * a.N + col) * a.G + size_t(sb0 + s) * GPS + gi] = v;
                                }
                            }
                    } else {
                        const float scl = ASYM ? sc[set][t][s][gi] : sc[set][t][s][gi] * 0.0625f;
#pragma unroll
                        for (int ms = 0; ms < MS; ++ms)
#pragma unroll
                            for (int i = 0; i < 4; ++i) accf[ms][i] = fmaf((float)acc[ms][i], scl, accf[ms][i]);
                    }
                }
            }
        }
        if (MODE != MODE_PARTIALS) {
            float4* dst = reinterpret_cast<float4*>(red + ((size_t(w) * TT + tt) * 64 + lane) * NV);
#pragma unroll
            for (int ms = 0; ms < MS; ++ms) dst[ms] = make_float4(accf[ms][0], accf[ms][1], accf[ms][2], accf[ms][3]);
        }
        if constexpr (TG > 2) {
            if (t == T - 1 && g + 2 < TG) {
                load_meta(g + 2);
                load_w(g + 2);
                asm volatile("" ::: "memory");
            }
        }
    }
    };
    compute();
    if (MODE == MODE_PARTIALS) return;
    if (tid < S::MT) sxs[tid] = sxv;
    __syncthreads();
    // 5. slice-ordered sum, row scale, store.  Output o = (t * 64 + l) * NV + j holds
    //    C[row = (j / 4) * 16 + 4 * (l / 16) + j % 4][col = 16 * t + l % 16] of the tile grid.
    auto reduce_store = [&]() __attribute__((always_inline)) {
    if (MOE && MODE == MODE_OUT && a.Hq) {
        // paired form: tile slots [0, TT/2) are gate tiles, [TT/2, TT) their up tiles; output o
        // of a gate slot and output o + half of its up slot are the same row and h column
        static_assert(TT % 2 == 0, "paired form: gate and up tiles in equal numbers");
        constexpr int half = TT / 2 * 64 * NV;
        const RowScale prs = static_row_scale(a.s_dn[expert]);
        for (int o = tid; o < half; o += int(blockDim.x)) {
            const int j = o % NV, lo = (o / NV) % 64, t = o / (NV * 64);
            const int row = (j >> 2) * 16 + 4 * (lo >> 4) + (j & 3);
            const int gt = tile0 / 2 + t;
            if (row >= nrows || gt >= a.pair_n / 16) continue;
            float yg = red[o], yu = red[o + half];
            for (int k = 1; k < KW; ++k) {
                yg += red[size_t(k) * TT * 64 * NV + o];
                yu += red[size_t(k) * TT * 64 * NV + o + half];
            }
            const int code = silu_static_code(yg * sxs[row], yu * sxs[row], prs);
            a.Hq[size_t(rbeg + row) * a.pair_n + gt * 16 + (lo & 15)] = int8_t(code);
        }
        if (blockIdx.x == 0 && tid < nrows) a.sh[rbeg + tid] = prs.s;
        return;
    }
    for (int o = tid; o < TT * 64 * NV; o += int(blockDim.x)) {
        const int j = o % NV, lo = (o / NV) % 64, t = o / (NV * 64);
        const int row = (j >> 2) * 16 + 4 * (lo >> 4) + (j & 3);
        const int col = (tile0 + t) * 16 + (lo & 15);
        if (row >= nrows || tile0 + t >= ntiles || col >= a.N) continue;
        float y = red[o];
        for (int k = 1; k < KW; ++k) y += red[size_t(k) * TT * 64 * NV + o];
        y *= sxs[row];
        const size_t yi = size_t(rbeg + row) * a.ldy + col;
        if (a.out_f32)
            reinterpret_cast<float*>(a.Y)[yi] = y;
        else
            reinterpret_cast<uint16_t*>(a.Y)[yi] = (uint16_t)f32_to_bf16_rne(y);
    }
    };
    reduce_store();
    if constexpr (RL) {
        // the expert's further row tiles, on the weights, scales and zero points held in
        // registers (their loads have all completed by now)
        for (int r0 = rbeg + S::MT; r0 < rall; r0 += S::MT) {
            rbeg = r0;
            rend = min(rall, r0 + S::MT);
            nrows = rend - rbeg;
            load_sx();
            load_a();
            __syncthreads();                             // partials and row scales of the last tile are read
            compute();
            if (tid < S::MT) sxs[tid] = sxv;
            __syncthreads();
            reduce_store();
        }
    }
}

// ------------------------------------------------------------------------------------
// W4A8 GEMM, prefill variant (large M): v_mfma_i32_32x32x32_i8, 256 x 128 workgroup tile
//
// 8 waves in a 4 (M) x 2 (N) grid, each computing a 64 x 64 tile as 2 x 2 MFMA tiles of
// 32 x 32.  Per 128-deep superblock the workgroup stages through LDS (double buffered):
//   - the activation tile [256 x 128] int8, rows padded to 144 bytes (conflict-free
//     16-byte fragment reads);
//   - the weight tile [128 columns x 128 k] unpacked ONCE by the workgroup from its packed
//     nibbles into INT8 (q - z) MFMA operands, so the four waves that share a column block
//     do not repeat the unpack;
//   - the group scales of its 128 columns.
// Global loads run two superblocks ahead of the MFMAs through registers.
//
// 32x32x32 operand mapping: MFMA step j (0..3) of a superblock covers k in [32j, 32j+32);
// lane L supplies row/column L % 32 and k in [32j + 16*(L/32), +16).  The unpacked weight
// tile is stored as [j][L/32][column][16 bytes] so a fragment is one 16-byte LDS read per
// lane.  The INT32 result of lane L, register r, is C[8*(r/4) + 4*(L/32) + r%4][L % 32].
// ------------------------------------------------------------------------------------
typedef int v16i __attribute__((ext_vector_type(16)));

// Workgroup id -> (M tile, N tile).  Consecutive ids are dealt round robin to the 8 XCDs,
// so each XCD is given a contiguous range of tile indices; inside it, tiles are walked in
// groups of 4 M tiles so that workgroups running together on one XCD share activation and
// weight tiles in its L2.
__device__ __forceinline__ void prefill_tile(int b, int mtiles, int ntiles, int* mt, int* nt) {
    const int T = mtiles * ntiles;
    const int per = T / 8, rem = T % 8;
    const int x = b % 8, j = b / 8;
    const int t = x * per + min(x, rem) + j;
    constexpr int GM = 4;
    const int group = t / (GM * ntiles);
    const int first = group * GM;
    const int gsz = min(GM, mtiles - first);
    const int in = t - group * GM * ntiles;
    *mt = first + in % gsz;
    *nt = in / gsz;
}

constexpr int PF_BM = 256, PF_BN = 128, PF_THREADS = 512;
constexpr int PF_AROW = SB_K + 16;                       // padded activation row (bytes)
constexpr int PF_A_BYTES = PF_BM * PF_AROW;              // 36864
constexpr int PF_B_BYTES = PF_BN * SB_K;                 // unpacked int8 weights: 16384
constexpr int PF_S_BYTES = (PF_BN / 16) * 4 * 64;        // scales of up to 4 groups: 2048
constexpr int PF_STAGE = PF_A_BYTES + PF_B_BYTES + PF_S_BYTES;
constexpr int PF_LDS = 2 * PF_STAGE;

struct PfRegs {
    uint4 a[4];     // activation pieces
    uint4 b;        // 16 bytes of packed codes (one layout lane of one 16-column tile)
    uint4 b2;       // W8: the lane's second 16 bytes
    uint4 m;        // scales piece (threads that stage metadata)
    uint32_t z;     // zero points of this thread's column, one byte per group
};

// W8: 8-bit weight codes, copied to the LDS operand layout as loaded (no unpack).
// H16: binary16 group scales, converted to float32 before they are staged in LDS.
template <bool ASYM, int GPS, int MODE, bool W8, bool H16 = false>
__global__ __launch_bounds__(PF_THREADS, 1) void gemm_prefill_kernel(GemmArgs a) {
    static_assert(!W8 || !ASYM, "8-bit codes: symmetric");
    // GPS 0: g = 256, one group per superblock pair (even, odd), which the loop runs back to back
    // GPS -1: per-channel scales (g = K), one int32 sum over all of K and one epilogue
    constexpr int NG = GPS <= 0 ? 1 : GPS;              // scale entries per superblock
    auto gidx = [](int sb, int gi) { return GPS < 0 ? 0 : GPS == 0 ? sb / 2 : sb * GPS + gi; };
    constexpr int SBB = W8 ? 2048 : 1024;                // code bytes per superblock
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 3, wn = wave >> 2;
    const int ntl16 = (a.N + 15) / 16;                   // 16-column tiles in the blob
    const int ntiles = (ntl16 + 7) / 8;
    const int mtiles = (a.M + PF_BM - 1) / PF_BM;
    int mt, nt;
    prefill_tile(blockIdx.x, mtiles, ntiles, &mt, &nt);
    const int m0 = mt * PF_BM, mend = a.M;
    const int t0 = nt * 8;                               // first 16-column tile
    auto tile_l = [&](int l) { return t0 + l; };         // blob tile of the workgroup's l-th tile
    const int nsb = a.K / SB_K;
    const uint8_t* codes = a.blob + a.codes_off;
    const uint8_t* scales_b = a.blob + a.scales_off;
    const uint8_t* zeros_b = a.blob + a.zeros_off;

    // staging: thread tid owns layout lane (tid % 64) of 16-column tile (tid / 64)
    const int b_tile = min(tile_l(wave), ntl16 - 1);
    const int st_q4 = lane >> 4, st_c = lane & 15;
    const int nmeta_s = 8 * NG * 4;                      // 16-byte scale pieces
    // Activation and code loads go through buffer resources.  Each lane's offset is fixed for
    // the whole K loop and the superblock advances only the scalar offset, so the loop spends
    // no vector instructions on addresses, and the loads are unconditional, so the compiler
    // can count them and wait for one register set only.  Rows past the tile's end load the
    // tile's last row (their outputs are never stored).  Offsets are 32-bit: the activations'
    // base is the tile's first row and the codes' base is the wave's column tile (the launcher
    // checks that PF_BM rows fit).
    const int8_t* xbase = a.Xq + size_t(m0) * a.K;
    const __amdgpu_buffer_rsrc_t xr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(xbase), 0, 0x7fffffff, 0x00020000);
    const __amdgpu_buffer_rsrc_t cr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(codes + size_t(__builtin_amdgcn_readfirstlane(b_tile)) * nsb * SBB), 0, 0x7fffffff,
        0x00020000);
    const __amdgpu_buffer_rsrc_t sr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(scales_b), 0, 0x7fffffff, 0x00020000);
    int aoff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int p = tid + i * PF_THREADS;
        const int row = p >> 3, c = p & 7;
        aoff[i] = (min(m0 + row, mend - 1) - m0) * a.K + c * 16;
    }
    auto gload = [&](PfRegs& r, int sb) {
        sb = __builtin_amdgcn_readfirstlane(sb);         // uniform: the scalar offsets below
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const v4i t = __builtin_amdgcn_raw_buffer_load_b128(xr, aoff[i], sb * SB_K, 0);
            r.a[i] = make_uint4(uint32_t(t.x), uint32_t(t.y), uint32_t(t.z), uint32_t(t.w));
        }
        {
            const v4i t = __builtin_amdgcn_raw_buffer_load_b128(cr, lane * (SBB / 64), sb * SBB, 0);
            r.b = make_uint4(uint32_t(t.x), uint32_t(t.y), uint32_t(t.z), uint32_t(t.w));
        }
        if constexpr (W8) {
            const v4i t = __builtin_amdgcn_raw_buffer_load_b128(cr, lane * 32 + 16, sb * SBB, 0);
            r.b2 = make_uint4(uint32_t(t.x), uint32_t(t.y), uint32_t(t.z), uint32_t(t.w));
        }
        if (ASYM) {
            r.z = 0;
#pragma unroll
            for (int gi = 0; gi < NG; ++gi)
                r.z |= uint32_t(zeros_b[(size_t(b_tile) * a.G + size_t(gidx(sb, gi))) * 16 + st_c]) << (8 * gi);
        }
        {   // every thread loads a piece (threads past nmeta_s repeat one and never store it)
            const int mt = tid % nmeta_s;
            const int tl = mt / (NG * 4), gi = (mt / 4) % NG, q4 = mt % 4;
            const int tile = min(tile_l(tl), ntl16 - 1);
            const int mo = (tile * a.G + gidx(sb, gi)) * 16 + q4 * 4;
            if constexpr (H16) {
                const auto t = __builtin_amdgcn_raw_buffer_load_b64(sr, mo * 2, 0, 0);
                const uint32_t h0 = uint32_t(t[0]), h1 = uint32_t(t[1]);
                r.m = make_uint4(__float_as_uint(f16_to_f32(uint16_t(h0 & 0xffffu))),
                                 __float_as_uint(f16_to_f32(uint16_t(h0 >> 16))),
                                 __float_as_uint(f16_to_f32(uint16_t(h1 & 0xffffu))),
                                 __float_as_uint(f16_to_f32(uint16_t(h1 >> 16))));
            } else {
                const v4i t = __builtin_amdgcn_raw_buffer_load_b128(sr, mo * 4, 0, 0);
                r.m = make_uint4(uint32_t(t.x), uint32_t(t.y), uint32_t(t.z), uint32_t(t.w));
            }
        }
    };
    auto lstore = [&](const PfRegs& r, int stage) {
        uint8_t* st = smem + stage * PF_STAGE;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int p = tid + i * PF_THREADS;
            *reinterpret_cast<uint4*>(st + (p >> 3) * PF_AROW + (p & 7) * 16) = r.a[i];
        }
        // unpack the 32 codes: half h holds k = 64h + 16*q4 + [0, 16) -> MFMA step
        // j = 2h + q4/2, lane half q4 % 2
        const int col = wave * 16 + st_c;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            // g = 32: the staging thread's 16 k (q4) lie in group 2h + q4 / 2
            const int gi = GPS == 4 ? 2 * h + (st_q4 >> 1) : (GPS == 2) ? h : 0;
            v4i u;
            if constexpr (W8) {
                const uint4 v = h ? r.b2 : r.b;
                u = v4i{int(v.x), int(v.y), int(v.z), int(v.w)};
            } else {
                const uint32_t zc = ASYM ? (128u - ((r.z >> (8 * gi)) & 0xffu)) * 0x01010101u : 0u;
                u = unpack_b<ASYM>(h ? r.b.z : r.b.x, h ? r.b.w : r.b.y, zc);
            }
            const int j = 2 * h + (st_q4 >> 1), hl = st_q4 & 1;
            *reinterpret_cast<v4i*>(st + PF_A_BYTES + ((j * 2 + hl) * PF_BN + col) * 16) = u;
        }
        if (tid < nmeta_s) {
            const int tl = tid / (NG * 4), gi = (tid / 4) % NG, q4 = tid % 4;
            *reinterpret_cast<uint4*>(st + PF_A_BYTES + PF_B_BYTES + ((tl * NG + gi) * 16 + q4 * 4) * 4) = r.m;
        }
    };

    v16i acc[2][2];
    float accf[2][2][16];
#pragma unroll
    for (int ms = 0; ms < 2; ++ms)
#pragma unroll
        for (int ns = 0; ns < 2; ++ns)
#pragma unroll
            for (int r = 0; r < 16; ++r) accf[ms][ns][r] = 0.0f;
    const v16i zero16 = {};

    // per-lane constants of the fragment reads
    const int l32 = lane & 31, hi = lane >> 5;
    int a_off[2];
#pragma unroll
    for (int ms = 0; ms < 2; ++ms) a_off[ms] = (wm * 64 + ms * 32 + l32) * PF_AROW + hi * 16;
    int b_off[2], s_off[2], col_g[2];
#pragma unroll
    for (int ns = 0; ns < 2; ++ns) {
        const int colw = wn * 64 + ns * 32 + l32;       // column inside the workgroup tile
        b_off[ns] = PF_A_BYTES + (hi * PF_BN + colw) * 16;
        s_off[ns] = PF_A_BYTES + PF_B_BYTES + (((colw >> 4) * NG) * 16 + (colw & 15)) * 4;
        col_g[ns] = tile_l(colw >> 4) * 16 + (colw & 15);
    }

    auto compute = [&](int stage, int sb) {
        const uint8_t* st = smem + stage * PF_STAGE;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int gi = GPS == 4 ? j : (GPS == 2) ? (j >> 1) : 0;   // MFMA step j is k in [32j, 32j + 32)
            v4i A[2], B[2];
#pragma unroll
            for (int ms = 0; ms < 2; ++ms) {
                const uint4 v = *reinterpret_cast<const uint4*>(st + a_off[ms] + j * 32);
                A[ms] = v4i{int(v.x), int(v.y), int(v.z), int(v.w)};
            }
#pragma unroll
            for (int ns = 0; ns < 2; ++ns) B[ns] = *reinterpret_cast<const v4i*>(st + b_off[ns] + j * 2 * PF_BN * 16);
            const bool first = GPS < 0    ? (j == 0 && sb == 0)
                             : GPS == 0 ? (j == 0 && sb % 2 == 0)
                             : GPS == 4 ? true : GPS == 2 ? ((j & 1) == 0) : (j == 0);
#pragma unroll
            for (int ms = 0; ms < 2; ++ms)
#pragma unroll
                for (int ns = 0; ns < 2; ++ns)
                    acc[ms][ns] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[ms], B[ns], first ? zero16 : acc[ms][ns], 0, 0, 0);
            const bool last = GPS < 0    ? (j == 3 && sb == nsb - 1)
                            : GPS == 0 ? (j == 3 && sb % 2 == 1)
                            : GPS == 4 ? true : GPS == 2 ? ((j & 1) == 1) : (j == 3);
            if (last) {
                if (MODE == MODE_PARTIALS) {
#pragma unroll
                    for (int ms = 0; ms < 2; ++ms)
#pragma unroll
                        for (int ns = 0; ns < 2; ++ns) {
                            const int col = col_g[ns];
#pragma unroll
                            for (int r = 0; r < 16; ++r) {
                                const int row = m0 + wm * 64 + ms * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
                                if (row < mend && col < a.N) {
                                    const int v = (ASYM || W8) ? acc[ms][ns][r] : (acc[ms][ns][r] >> 4);
                                    a.P[(size_t(row) * a.N + col) * a.G + size_t(gidx(sb, gi))] = v;
                                }
                            }
                        }
                } else {
#pragma unroll
                    for (int ns = 0; ns < 2; ++ns) {
                        float scl = *reinterpret_cast<const float*>(st + s_off[ns] + gi * 64);
                        if (!ASYM && !W8) scl *= 0.0625f;
#pragma unroll
                        for (int ms = 0; ms < 2; ++ms)
#pragma unroll
                            for (int r = 0; r < 16; ++r)
                                accf[ms][ns][r] = fmaf((float)acc[ms][ns][r], scl, accf[ms][ns][r]);
                    }
                }
            }
        }
    };

    // pipeline: register set s%2 holds the loads of superblock s; stage s%2 of LDS holds
    // superblock s while it is computed (prefetches past the last superblock reload the last one
    // and are never stored).  A straight-line pair loop without the conditional stores and the
    // mid-loop exit gave per-register waits in the assembly but no measurable speed at g >= 128,
    // and with two or four group epilogues per superblock its register pressure spilled
    // (g = 32: 720 -> 140 TOPS), so the loop keeps this form.
    PfRegs R0, R1;
    gload(R0, 0);
    gload(R1, min(1, nsb - 1));
    lstore(R0, 0);
    gload(R0, min(2, nsb - 1));
    __syncthreads();
    for (int kb = 0; kb < nsb; kb += 2) {
        // even superblock kb: stage 0; R1 holds kb+1, R0 holds kb+2
        if (kb + 1 < nsb) lstore(R1, 1);
        gload(R1, min(kb + 3, nsb - 1));
        compute(0, kb);
        __syncthreads();
        if (kb + 1 >= nsb) break;
        // odd superblock kb+1: stage 1; R0 holds kb+2, R1 holds kb+3
        if (kb + 2 < nsb) lstore(R0, 0);
        gload(R0, min(kb + 4, nsb - 1));
        compute(1, kb + 1);
        __syncthreads();
    }
    if (MODE == MODE_PARTIALS) return;

    // row scale of tile row wm * 64 + lane, loaded once per lane; each output register takes its
    // row's by a cross-lane read
    const float sxl = m0 + wm * 64 + lane < mend ? a.sx[m0 + wm * 64 + lane] : 0.0f;
    auto row_sx = [&](int ms, int r) { return __shfl(sxl, ms * 32 + 8 * (r >> 2) + 4 * hi + (r & 3), 64); };

    // row scales, then store
#pragma unroll
    for (int ms = 0; ms < 2; ++ms) {
        float sxv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) sxv[r] = row_sx(ms, r);
#pragma unroll
        for (int ns = 0; ns < 2; ++ns) {
            const int col = col_g[ns];
            if (col >= a.N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm * 64 + ms * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
                if (row >= mend) continue;
                const float y = accf[ms][ns][r] * sxv[r];
                if (a.out_f32)
                    reinterpret_cast<float*>(a.Y)[size_t(row) * a.ldy + col] = y;
                else
                    reinterpret_cast<uint16_t*>(a.Y)[size_t(row) * a.ldy + col] = (uint16_t)f32_to_bf16_rne(y);
            }
        }
    }
}

// ------------------------------------------------------------------------------------
// MoE align: stable counting sort of routed rows by expert (P1 section 4.4 dispatch).
// One 1024-thread workgroup.  Rows are cut into B blocks of L consecutive rows; block b's
// per-expert counts live at cnt[e * (B + 1) + b] (padded stride: conflict-free in both
// passes).  Positions: off[e] + counts of earlier blocks + order inside the block.
// ------------------------------------------------------------------------------------
// STAGE: the R expert ids are first copied to LDS with coalesced loads, so both passes over
// them read LDS instead of issuing one dependent global load per row.
template <bool STAGE>
__global__ __launch_bounds__(1024) void moe_align_kernel(const int32_t* __restrict__ ids, int R, int E, int L,
                                                         int B, int32_t* __restrict__ sorted_rows,
                                                         int32_t* __restrict__ offsets, int32_t* __restrict__ inv) {
    extern __shared__ __align__(16) uint8_t smem[];
    int* cnt = reinterpret_cast<int*>(smem);   // E * (B + 1)
    int* wsum = cnt + E * (B + 1);             // 16 wave totals
    int* sid = wsum + 16;                      // STAGE: the R ids
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int stride = B + 1;
    for (int i = tid; i < E * stride; i += 1024) cnt[i] = 0;
    if (STAGE)
        for (int i = tid; i < R; i += 1024) sid[i] = ids[i];
    __syncthreads();
    auto id_of = [&](int r) { return STAGE ? sid[r] : ids[r]; };
    if (tid < B) {
        const int r1 = min(R, (tid + 1) * L);
        for (int r = tid * L; r < r1; ++r) {
            const int e = id_of(r);
            if (e >= 0 && e < E) cnt[e * stride + tid]++;
        }
    }
    __syncthreads();
    // Output position of chunk b's first row of expert e: the exclusive prefix sum of the count
    // matrix read in (expert, chunk) order, i.e. over experts first and over the chunks of one
    // expert second.  Thread tid scans the NS consecutive entries [tid * NS, tid * NS + NS) of
    // that order, the threads' totals are scanned across the block, and the entries are
    // replaced by their positions.
    // (the whole launch is one workgroup on one compute unit, so the walk steps through
    // (expert, chunk) without a division per entry)
    const int n = E * B;
    const int NS = (n + 1023) / 1024;
    const int i0 = min(n, tid * NS), cntn = min(n, i0 + NS) - i0;
    const int e0 = B > 0 ? i0 / B : 0, b0 = B > 0 ? i0 - e0 * B : 0;
    int tot = 0;
    for (int j = 0, e = e0, b = b0; j < cntn; ++j) {
        tot += cnt[e * stride + b];
        if (++b == B) { b = 0; ++e; }
    }
    int incl = tot;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int wbase = 0;
    for (int w = 0; w < wave; ++w) wbase += wsum[w];
    int run = wbase + incl - tot;
    for (int j = 0, e = e0, b = b0; j < cntn; ++j) {
        const int c = cnt[e * stride + b];
        cnt[e * stride + b] = run;
        run += c;
        if (++b == B) { b = 0; ++e; }
    }
    __syncthreads();
    // expert e's rows start at chunk 0's position; the last expert's end is the total
    if (tid < E) offsets[tid] = B > 0 ? cnt[tid * stride] : 0;
    if (tid == 0) {
        int total = 0;
        for (int w = 0; w < 16; ++w) total += wsum[w];
        offsets[E] = total;
    }
    if (tid < B) {
        const int r1 = min(R, (tid + 1) * L);
        for (int r = tid * L; r < r1; ++r) {
            const int e = id_of(r);
            if (e >= 0 && e < E) {
                const int pos = cnt[e * stride + tid]++;
                sorted_rows[pos] = r;
                inv[r] = pos;
            } else {
                inv[r] = -1;
            }
        }
    }
}

// ------------------------------------------------------------------------------------
// un-permute + top-k weighted combine (P1 section 4.3): float32, j ascending.
// ------------------------------------------------------------------------------------
// KM > 0: k <= KM, all k rows requested at once (their indices and weights first); KM = 0:
// any k, one row after another.  The sum runs over j ascending either way.
template <int KM>
__global__ __launch_bounds__(256) void moe_combine_kernel(const uint16_t* __restrict__ Yd,
                                                          const int32_t* __restrict__ inv,
                                                          const float* __restrict__ w, int k, int H,
                                                          uint16_t* __restrict__ out) {
    const int t = blockIdx.x;
    int rj[KM > 0 ? KM : 1];
    float wj[KM > 0 ? KM : 1];
#pragma unroll
    for (int j = 0; j < KM; ++j) {
        rj[j] = j < k ? inv[t * k + j] : -1;
        wj[j] = j < k ? w[t * k + j] : 0.0f;
    }
    auto add_row = [&](float* acc, const uint4 v, const float wgt) __attribute__((always_inline)) {
        const uint32_t x[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[2 * i] = fmaf(wgt, bf16_to_f32(x[i] & 0xffffu), acc[2 * i]);
            acc[2 * i + 1] = fmaf(wgt, bf16_to_f32(x[i] >> 16), acc[2 * i + 1]);
        }
    };
    for (int c = threadIdx.x * 8; c < H; c += 256 * 8) {
        float acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
        if constexpr (KM > 0) {
            uint4 v[KM];
#pragma unroll
            for (int j = 0; j < KM; ++j)
                v[j] = rj[j] >= 0 ? *reinterpret_cast<const uint4*>(Yd + size_t(rj[j]) * H + c) : make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int j = 0; j < KM; ++j)
                if (rj[j] >= 0) add_row(acc, v[j], wj[j]);
        } else {
            for (int j = 0; j < k; ++j) {
                const int r = inv[t * k + j];
                if (r < 0) continue;
                add_row(acc, *reinterpret_cast<const uint4*>(Yd + size_t(r) * H + c), w[t * k + j]);
            }
        }
        uint4 o;
        o.x = f32_to_bf16_rne(acc[0]) | (f32_to_bf16_rne(acc[1]) << 16);
        o.y = f32_to_bf16_rne(acc[2]) | (f32_to_bf16_rne(acc[3]) << 16);
        o.z = f32_to_bf16_rne(acc[4]) | (f32_to_bf16_rne(acc[5]) << 16);
        o.w = f32_to_bf16_rne(acc[6]) | (f32_to_bf16_rne(acc[7]) << 16);
        *reinterpret_cast<uint4*>(out + size_t(t) * H + c) = o;
    }
}

// ------------------------------------------------------------------------------------
// host-side launch helpers
// ------------------------------------------------------------------------------------
static inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

static int launch_status() {
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? W4A8_OK : W4A8_EHIP;
}

static int row_iters(int K) {
    int it = (K + 2047) / 2048;
    int p = 1;
    while (p < it) p <<= 1;
    return p;
}

template <int IT>
static void launch_quant(const uint16_t* X, int M, int K, int ldx, int8_t* Xq, float* sx, hipStream_t s,
                         const float* inv_alpha = nullptr) {
    if (inv_alpha) quant_act_kernel<IT, true><<<dim3(M), dim3(256), 0, s>>>(X, K, ldx, Xq, sx, inv_alpha);
    else quant_act_kernel<IT><<<dim3(M), dim3(256), 0, s>>>(X, K, ldx, Xq, sx);
}

template <int IT>
static void launch_silu(const uint16_t* GU, int R, int I, int8_t* Hq, float* sh, hipStream_t s,
                        const float* sstat = nullptr, const int32_t* offs = nullptr, int E = 0) {
    if (sstat) silu_quant_kernel<IT, true><<<dim3(R), dim3(256), 0, s>>>(GU, I, Hq, sh, sstat, offs, E);
    else silu_quant_kernel<IT><<<dim3(R), dim3(256), 0, s>>>(GU, I, Hq, sh);
}

// Variant table of the decode GEMM.  (NT, KW, SBN): column tiles per workgroup, K slices,
// superblocks per slice; chosen so that one chunk covers K whenever it fits.
struct DecodeCfg {
    int ms, nt, kw, sbn;
};

static DecodeCfg decode_cfg(int K, int mt) {
    const int nsb = K / SB_K;
    DecodeCfg c{mt / 16, 4, 4, 8};
    if (nsb > 32 && mt == 16) {     // long K: 8 slices of up to 8 superblocks, 2 tiles
        c.nt = 2;
        c.kw = 8;
        c.sbn = 8;
    } else {                        // one chunk of up to 32 superblocks (more chunks if longer)
        const int per = (nsb + 3) / 4;
        c.sbn = per <= 2 ? 2 : (per <= 4 ? 4 : 8);
    }
    return c;
}

template <int MS, int NT, int KW, int SBN, int GPS, bool ASYM, int MODE, bool MOE, bool MULTI = false, bool FQ = false,
          bool W8 = false, bool H16 = false>
static void launch_decode_t(const GemmArgs& a, dim3 grid, hipStream_t s) {
    using S = DecodeShape<MS, NT, KW, SBN>;
    auto kern = gemm_decode_kernel<MS, NT, KW, SBN, GPS, ASYM, MODE, MOE, MULTI, FQ, W8, H16>;
    constexpr size_t lds = S::LDS + (FQ ? 128 : 0);           // FQ: row abs-maxima
    static const hipError_t attr =
        hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    (void)attr;
    kern<<<grid, dim3(S::NTHR), lds, s>>>(a);
}

// Fused quantization + GEMM on the chunked kernel (dense, 16-row tile, K in one chunk).
template <int GPS, bool ASYM, bool W8 = false, bool H16 = false>
static void launch_decode_fused(const GemmArgs& a, const DecodeCfg& c, dim3 grid, hipStream_t s) {
    if (c.kw == 8) launch_decode_t<1, 2, 8, 8, GPS, ASYM, MODE_OUT, false, false, true, W8, H16>(a, grid, s);
    else if (c.sbn == 2) launch_decode_t<1, 4, 4, 2, GPS, ASYM, MODE_OUT, false, false, true, W8, H16>(a, grid, s);
    else if (c.sbn == 4) launch_decode_t<1, 4, 4, 4, GPS, ASYM, MODE_OUT, false, false, true, W8, H16>(a, grid, s);
    else launch_decode_t<1, 4, 4, 8, GPS, ASYM, MODE_OUT, false, false, true, W8, H16>(a, grid, s);
}

template <int MS, int GPS, bool ASYM, int MODE, bool MOE, bool W8 = false, bool H16 = false>
static void launch_decode_shape(const GemmArgs& a, const DecodeCfg& c, dim3 grid, hipStream_t s) {
    if (c.kw == 8) {
        if constexpr (MS == 1) {
            if (a.K > 64 * SB_K) launch_decode_t<MS, 2, 8, 8, GPS, ASYM, MODE, MOE, true, false, W8, H16>(a, grid, s);
            else launch_decode_t<MS, 2, 8, 8, GPS, ASYM, MODE, MOE, false, false, W8, H16>(a, grid, s);
        }
    } else if (c.sbn == 2) launch_decode_t<MS, 4, 4, 2, GPS, ASYM, MODE, MOE, false, false, W8, H16>(a, grid, s);
    else if (c.sbn == 4) launch_decode_t<MS, 4, 4, 4, GPS, ASYM, MODE, MOE, false, false, W8, H16>(a, grid, s);
    else if (a.K > 32 * SB_K) launch_decode_t<MS, 4, 4, 8, GPS, ASYM, MODE, MOE, true, false, W8, H16>(a, grid, s);
    else launch_decode_t<MS, 4, 4, 8, GPS, ASYM, MODE, MOE, false, false, W8, H16>(a, grid, s);
}

// gps: groups per superblock (2, 1, 0 for g = 256, -1 per-channel); w8: 8-bit codes.  g = 256,
// per-channel and 8-bit codes are dense-form only (the entry points check).
template <int MODE, bool MOE>
static void launch_decode(const GemmArgs& a, const DecodeCfg& c, int gps, bool asym, dim3 grid, hipStream_t s,
                          bool w8 = false) {
#define W4A8_DEC(MS_, GPS_, ASYM_) launch_decode_shape<MS_, GPS_, ASYM_, MODE, MOE>(a, c, grid, s)
    if constexpr (!MOE) {
        if (gps == 4) {                                   // g = 32 (dense form only)
            if (w8) { if (c.ms == 1) launch_decode_shape<1, 4, false, MODE, false, true>(a, c, grid, s);
                      else launch_decode_shape<2, 4, false, MODE, false, true>(a, c, grid, s); }
            else if (c.ms == 1) { if (asym) W4A8_DEC(1, 4, true); else W4A8_DEC(1, 4, false); }
            else { if (asym) W4A8_DEC(2, 4, true); else W4A8_DEC(2, 4, false); }
            return;
        }
        if (w8) {
            if (c.ms == 1) { if (gps == 1) launch_decode_shape<1, 1, false, MODE, false, true>(a, c, grid, s);
                             else if (gps == 2) launch_decode_shape<1, 2, false, MODE, false, true>(a, c, grid, s);
                             else if (gps == 0) launch_decode_shape<1, 0, false, MODE, false, true>(a, c, grid, s);
                             else if constexpr (MODE == MODE_OUT) launch_decode_shape<1, -1, false, MODE, false, true>(a, c, grid, s); }
            else { if (gps == 1) launch_decode_shape<2, 1, false, MODE, false, true>(a, c, grid, s);
                   else if (gps == 2) launch_decode_shape<2, 2, false, MODE, false, true>(a, c, grid, s);
                   else if (gps == 0) launch_decode_shape<2, 0, false, MODE, false, true>(a, c, grid, s);
                   else if constexpr (MODE == MODE_OUT) launch_decode_shape<2, -1, false, MODE, false, true>(a, c, grid, s); }
            return;
        }
        if (gps == 0) {                                   // g = 256 (dense form only)
            if (c.ms == 1) { if (asym) W4A8_DEC(1, 0, true); else W4A8_DEC(1, 0, false); }
            else { if (asym) W4A8_DEC(2, 0, true); else W4A8_DEC(2, 0, false); }
            return;
        }
        if constexpr (MODE == MODE_OUT) {
            if (gps < 0) {                                // per-channel (dense form, outputs only)
                if (c.ms == 1) { if (asym) W4A8_DEC(1, -1, true); else W4A8_DEC(1, -1, false); }
                else { if (asym) W4A8_DEC(2, -1, true); else W4A8_DEC(2, -1, false); }
                return;
            }
        }
    }
#undef W4A8_DEC
    // 4-bit codes, g in {64, 128}: float32 or binary16 scales
#define W4A8_DEC(MS_, GPS_, ASYM_)                                                              \
    do {                                                                                        \
        if (a.h16) launch_decode_shape<MS_, GPS_, ASYM_, MODE, MOE, false, true>(a, c, grid, s); \
        else launch_decode_shape<MS_, GPS_, ASYM_, MODE, MOE>(a, c, grid, s);                  \
    } while (0)
    if (c.ms == 1) {
        if (gps == 1) { if (asym) W4A8_DEC(1, 1, true); else W4A8_DEC(1, 1, false); }
        else { if (asym) W4A8_DEC(1, 2, true); else W4A8_DEC(1, 2, false); }
    } else {
        if (gps == 1) { if (asym) W4A8_DEC(2, 1, true); else W4A8_DEC(2, 1, false); }
        else { if (asym) W4A8_DEC(2, 2, true); else W4A8_DEC(2, 2, false); }
    }
#undef W4A8_DEC
}


// K-slice kernel (grouped form): T tiles per group, TG groups per workgroup, SW superblocks per
// wave, KW waves.
struct KsliceCfg {
    int t, sw, kw, tg;
    bool rl;        // grouped form: run the expert's row tiles in one workgroup
};

// Tile groups per workgroup for the grouped (MoE) form at 16-row tiles and K in (4096, 8192]:
// there one workgroup fills a compute unit (its registers), and with a single 32-column
// group it would spend most of its life on fixed costs between short weight streams.
constexpr int MOE_KSLICE_TG = 8;
// K <= 2048 at 16-row tiles: 8 waves of two superblocks, 4 groups of 2 tiles, so that two
// workgroups (registers, 64 KiB of slice partials each) share a compute unit
constexpr int MOE_KSLICE_TG_SHORT = 4;

static bool kslice_cfg(int K, int mt, KsliceCfg* c, bool moe = false) {
    const int nsb = K / SB_K;
    c->tg = 1;
    c->rl = false;
    if (nsb <= 16 && moe && mt == 16 && nsb > 2) {
        c->t = 2;
        c->sw = 2;
        c->tg = MOE_KSLICE_TG_SHORT;
    } else if (nsb <= 16) {
        c->t = 4;
        c->sw = 1;
        // measured: worth it at 32-row tiles (an expert's weights are read once instead of
        // once per tile); at 16-row tiles the extra registers cost the second resident
        // workgroup per compute unit, which matters more
        c->rl = moe && mt == 32;
    } else if (nsb <= 32) {
        c->t = 4;
        c->sw = 2;
        c->rl = moe && mt == 16;
    } else if (nsb <= 64 && mt == 16) {   // 32-row tiles at this depth would not fit in registers
        c->t = moe ? 1 : 2;
        c->sw = 4;
        if (moe) c->tg = MOE_KSLICE_TG;
    } else {
        return false;
    }
    c->kw = (nsb + c->sw - 1) / c->sw;
    return true;
}


template <int MS, int T, int SW, int GPS, bool ASYM, int MODE, bool MOE, int TG = 1, bool RL = false, bool H16 = false>
static void launch_kslice_t(const GemmArgs& a, int kw, int ytiles, hipStream_t s) {
    using S = KsliceShape<MS, T, TG>;
    static_assert(S::lds(16) <= 160 * 1024, "slice partials exceed LDS");
    auto kern = gemm_kslice_kernel<MS, T, SW, GPS, ASYM, MODE, MOE, TG, RL, H16>;
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                                       int(S::lds(16)));
    (void)attr;
    const int ntiles = (a.N + 15) / 16;
    const size_t lds = S::lds(kw);
    kern<<<dim3((ntiles + S::TT - 1) / S::TT, ytiles), dim3(64 * kw), lds, s>>>(a);
}

template <int MS, int GPS, bool ASYM, int MODE, bool MOE, bool H16 = false>
static void launch_kslice_shape(const GemmArgs& a, const KsliceCfg& c, int ytiles, hipStream_t s) {
    // shapes kslice_cfg can return for this form (others are not instantiated)
    if (c.sw == 1) {
        if constexpr (MOE && MS == 2 && MODE == MODE_OUT) {
            if (c.rl) {
                launch_kslice_t<MS, 4, 1, GPS, ASYM, MODE, MOE, 1, true, H16>(a, c.kw, ytiles, s);
                return;
            }
        }
        launch_kslice_t<MS, 4, 1, GPS, ASYM, MODE, MOE, 1, false, H16>(a, c.kw, ytiles, s);
    } else if (c.sw == 2) {
        if constexpr (MOE && MS == 1) {
            if (c.tg == MOE_KSLICE_TG_SHORT) {
                launch_kslice_t<MS, 2, 2, GPS, ASYM, MODE, MOE, MOE_KSLICE_TG_SHORT, false, H16>(a, c.kw, ytiles, s);
                return;
            }
        }
        if constexpr (MOE && MS == 1 && MODE == MODE_OUT) {
            if (c.rl) {
                launch_kslice_t<MS, 4, 2, GPS, ASYM, MODE, MOE, 1, true, H16>(a, c.kw, ytiles, s);
                return;
            }
        }
        launch_kslice_t<MS, 4, 2, GPS, ASYM, MODE, MOE, 1, false, H16>(a, c.kw, ytiles, s);
    } else if constexpr (MS == 1) {
        if constexpr (MOE) launch_kslice_t<MS, 1, 4, GPS, ASYM, MODE, MOE, MOE_KSLICE_TG, false, H16>(a, c.kw, ytiles, s);
        else launch_kslice_t<MS, 2, 4, GPS, ASYM, MODE, MOE, 1, false, H16>(a, c.kw, ytiles, s);
    }
}

template <int MODE, bool MOE>
static void launch_kslice(const GemmArgs& a, const KsliceCfg& c, int ms, int gps, bool asym, int ytiles,
                          hipStream_t s) {
#define W4A8_KS(MS_, GPS_, ASYM_)                                                           \
    do {                                                                                    \
        if (a.h16) launch_kslice_shape<MS_, GPS_, ASYM_, MODE, MOE, true>(a, c, ytiles, s); \
        else launch_kslice_shape<MS_, GPS_, ASYM_, MODE, MOE>(a, c, ytiles, s);            \
    } while (0)
    if (ms == 1) {
        if (gps == 1) { if (asym) W4A8_KS(1, 1, true); else W4A8_KS(1, 1, false); }
        else { if (asym) W4A8_KS(1, 2, true); else W4A8_KS(1, 2, false); }
    } else {
        if (gps == 1) { if (asym) W4A8_KS(2, 1, true); else W4A8_KS(2, 1, false); }
        else { if (asym) W4A8_KS(2, 2, true); else W4A8_KS(2, 2, false); }
    }
#undef W4A8_KS
}

template <bool ASYM, int GPS, int MODE, bool W8 = false, bool H16 = false>
static void launch_prefill_t(const GemmArgs& a, hipStream_t s) {
    auto kern = gemm_prefill_kernel<ASYM, GPS, MODE, W8, H16>;
    static const hipError_t attr =
        hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, PF_LDS);
    (void)attr;
    const int mtiles = (a.M + PF_BM - 1) / PF_BM;
    const int ntiles = ((a.N + 15) / 16 + 7) / 8;
    kern<<<dim3(mtiles * ntiles), dim3(PF_THREADS), PF_LDS, s>>>(a);
}

// gps: groups per superblock (4 for g = 32, 2, 1, 0 for g = 256, -1 per-channel); w8: 8-bit codes
template <int MODE>
static void launch_prefill(const GemmArgs& a, int gps, bool asym, hipStream_t s, bool w8 = false) {
    if (gps == 4) {                                       // g = 32
        if (w8) launch_prefill_t<false, 4, MODE, true>(a, s);
        else if (asym) launch_prefill_t<true, 4, MODE>(a, s);
        else launch_prefill_t<false, 4, MODE>(a, s);
        return;
    }
    if (w8) {
        if (gps == 1) launch_prefill_t<false, 1, MODE, true>(a, s);
        else if (gps == 2) launch_prefill_t<false, 2, MODE, true>(a, s);
        else if (gps == 0) launch_prefill_t<false, 0, MODE, true>(a, s);
        else launch_prefill_t<false, -1, MODE, true>(a, s);
        return;
    }
    if (gps == 0) {                                       // g = 256
        if (asym) launch_prefill_t<true, 0, MODE>(a, s); else launch_prefill_t<false, 0, MODE>(a, s);
        return;
    }
    if (gps < 0) {                                        // per-channel
        if (asym) launch_prefill_t<true, -1, MODE>(a, s); else launch_prefill_t<false, -1, MODE>(a, s);
        return;
    }
    // 4-bit codes, g in {64, 128}: float32 or binary16 scales
#define W4A8_PF(ASYM_, GPS_)                                                     \
    do {                                                                         \
        if (a.h16) launch_prefill_t<ASYM_, GPS_, MODE, false, true>(a, s);       \
        else launch_prefill_t<ASYM_, GPS_, MODE>(a, s);                          \
    } while (0)
    if (gps == 1) {
        if (asym) W4A8_PF(true, 1); else W4A8_PF(false, 1);
    } else {
        if (asym) W4A8_PF(true, 2); else W4A8_PF(false, 2);
    }
#undef W4A8_PF
}

// MoE experts with at least this many rows run on 128 x 128 MFMA tiles (gemm_moe_tile_kernel):
// each expert's weights are streamed once per 128 rows instead of once per 16 or 32, for at
// most a quarter of the tile's MFMA rows idle.  Measured on the 64-expert top-6 layer: 96
// beats 128 by 3-4 %; at 64 the tile launch no longer fits one round of workgroups and loses.
constexpr int MOE_TILE_MIN_ROWS = 96;

// Dense GEMMs with more rows than this use the prefill kernel.
constexpr int PREFILL_MIN_M = 33;

// The 256 x 128 prefill kernel reads activations through 32-bit buffer offsets from the row
// tile's first row (PF_BM rows).
static bool prefill_offsets_fit(int K, size_t rows) { return rows * size_t(K) < (size_t(1) << 31); }

static dim3 decode_grid(const Layout& L, const DecodeCfg& c, int ytiles) {
    const int ntiles = L.Np / 16;
    return dim3((ntiles + c.nt - 1) / c.nt, ytiles);
}

// g = 32, g = 256 and per-channel scales (g = K) run on the dense kernels only; the grouped
// (MoE) entry points reject them.  One group's sum stays in an int32 accumulator, so g * 127
// times the largest operand the kernels feed must stay below 2^31.  That operand is q - z <= 15
// for asymmetric codes, 16 q <= 112 for symmetric 4-bit codes (the nibble sits in the high half
// of the byte; the 1/16 is folded into the scale) and q <= 127 for 8-bit codes.  This bounds K for
// per-channel scales: K <= 150912 (symmetric 4-bit), K < 1127304 (asymmetric), K < 133144 (8-bit).
static bool kernel_format_ok(const w4a8_wdesc* d) {
    const int g = d->group_size;
    if (g != 32 && g != 64 && g != 128 && g != 256 && g != d->K) return false;
    // binary16 scales: 4-bit codes with g in {64, 128}
    if (d->scale_bits == 16 && (d->weight_bits == 8 || (g != 64 && g != 128))) return false;
    const int64_t qr = d->weight_bits == 8 ? 127 : (d->asymmetric ? 15 : 112);
    return int64_t(g) * 127 * qr < (int64_t(1) << 31);
}

// Groups per 128-deep superblock as the kernels' GPS: 4 (g = 32), 2 (g = 64), 1 (g = 128), 0
// (g = 256: one group per two superblocks), -1 (per-channel: g = K > 256, one group over all
// of K).
static int gps_of(const w4a8_wdesc* d) {
    if (d->group_size == d->K && d->K > 256) return -1;
    return SB_K / d->group_size;
}

// The grouped (MoE) kernels take 4-bit codes with g in {64, 128}.
static bool grouped_format_ok(const w4a8_wdesc* d) {
    return layout_of(d).bits == 4 && (gps_of(d) == 1 || gps_of(d) == 2);
}

static int dense_mt(int M) { return M <= 16 ? 16 : 32; }

static GemmArgs make_args(const Layout& L, const int8_t* Xq, const float* sx, int M, const void* blob) {
    GemmArgs a;
    std::memset(&a, 0, sizeof(a));
    a.Xq = Xq;
    a.sx = sx;
    a.M = M;
    a.K = L.K;
    a.N = L.N;
    a.G = L.G;
    a.blob = static_cast<const uint8_t*>(blob);
    a.codes_off = L.codes_off;
    a.scales_off = L.scales_off;
    a.zeros_off = L.zeros_off;
    a.h16 = L.sbytes == 2;
    return a;
}

static int check_gemm_desc(const w4a8_wdesc* d) {
    int st = desc_status(d);
    if (st) return st;
    if (!kernel_format_ok(d)) return W4A8_EUNSUPPORTED;
    // the kernels address one blob's codes and scales with 32-bit offsets
    const Layout L = layout_of(d);
    if (L.codes_bytes >= (size_t(1) << 31) || L.scales_bytes >= (size_t(1) << 31)) return W4A8_EUNSUPPORTED;
    return W4A8_OK;
}

// w4a8_linear quantizes these rows inside the GEMM (the chunked kernel's fused form: a 16-row
// tile, K in one chunk, one 16-value piece per thread)
static bool linear_fuses(const Layout& L, int M) {
    const DecodeCfg fc = decode_cfg(L.K, 16);
    const int fcs = fc.kw * fc.sbn;                      // superblocks per chunk
    return M <= 16 && size_t(M) * L.K <= FUSED_MAX_ELEMS && L.K / SB_K <= fcs &&
           (M - 1) * fcs * 8 + (L.K / SB_K) * 8 <= 64 * fc.nt * fc.kw;
}

}  // namespace w4a8

using namespace w4a8;

extern "C" {

static int quant_act_impl(const void* X, int M, int K, int ldx, const float* inv_alpha, int8_t* Xq, float* sx,
                          void* stream) {
    if (M < 0 || K <= 0 || ldx < K) return W4A8_EINVAL;
    if (M == 0) return W4A8_OK;
    if (!X || !Xq || !sx) return W4A8_EINVAL;
    if (K % 16 || ldx % 8 || !aligned16(X) || !aligned16(Xq) || !aligned16(inv_alpha)) return W4A8_EINVAL;
    if (K > 65536) return W4A8_EUNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint16_t* x = static_cast<const uint16_t*>(X);
    switch (row_iters(K)) {
        case 1: launch_quant<1>(x, M, K, ldx, Xq, sx, s, inv_alpha); break;
        case 2: launch_quant<2>(x, M, K, ldx, Xq, sx, s, inv_alpha); break;
        case 4: launch_quant<4>(x, M, K, ldx, Xq, sx, s, inv_alpha); break;
        case 8: launch_quant<8>(x, M, K, ldx, Xq, sx, s, inv_alpha); break;
        case 16: launch_quant<16>(x, M, K, ldx, Xq, sx, s, inv_alpha); break;
        case 32: launch_quant<32>(x, M, K, ldx, Xq, sx, s, inv_alpha); break;
        default: return W4A8_EUNSUPPORTED;
    }
    return launch_status();
}

int w4a8_quant_act(const void* X, int M, int K, int ldx, int8_t* Xq, float* sx, void* stream) {
    return quant_act_impl(X, M, K, ldx, nullptr, Xq, sx, stream);
}

int w4a8_quant_act_smooth(const void* X, int M, int K, int ldx, const float* inv_alpha, int8_t* Xq, float* sx,
                          void* stream) {
    if (M > 0 && !inv_alpha) return W4A8_EINVAL;
    return quant_act_impl(X, M, K, ldx, inv_alpha, Xq, sx, stream);
}

static int quant_static_impl(const void* X, int rows, int K, int ldx, int T, const float* s, const int32_t* gather,
                             int k, const int32_t* offs, int E, int8_t* Xq, float* sx, void* stream) {
    if (rows < 0 || K <= 0 || ldx < K) return W4A8_EINVAL;
    if (rows == 0) return W4A8_OK;
    if (!X || !s || !Xq || !sx) return W4A8_EINVAL;
    if (K % 16 || ldx % 8 || !aligned16(X) || !aligned16(Xq)) return W4A8_EINVAL;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const uint16_t* x = static_cast<const uint16_t*>(X);
    const dim3 grid(rows), block(256);
    switch (std::min(row_iters(K), 8)) {      // longer rows: several passes of 8 pieces per thread
        case 1: quant_static_kernel<1><<<grid, block, 0, st>>>(x, K, ldx, T, s, gather, k, offs, E, Xq, sx); break;
        case 2: quant_static_kernel<2><<<grid, block, 0, st>>>(x, K, ldx, T, s, gather, k, offs, E, Xq, sx); break;
        case 4: quant_static_kernel<4><<<grid, block, 0, st>>>(x, K, ldx, T, s, gather, k, offs, E, Xq, sx); break;
        default: quant_static_kernel<8><<<grid, block, 0, st>>>(x, K, ldx, T, s, gather, k, offs, E, Xq, sx); break;
    }
    return launch_status();
}

int w4a8_quant_act_static(const void* X, int M, int K, int ldx, const float* s, int8_t* Xq, float* sx,
                          void* stream) {
    return quant_static_impl(X, M, K, ldx, M, s, nullptr, 1, nullptr, 0, Xq, sx, stream);
}

int w4a8_moe_quant_static(const void* X, int T, int H, int ldx, const int32_t* sorted_rows, int k,
                          const int32_t* offsets, int E, const float* s, int8_t* Xq, float* sx, void* stream) {
    if (T < 0 || k <= 0 || E <= 0 || E > 1024) return W4A8_EINVAL;
    if ((long long)T * k > (1 << 24)) return W4A8_EUNSUPPORTED;
    if (T > 0 && (!sorted_rows || !offsets)) return W4A8_EINVAL;
    return quant_static_impl(X, T * k, H, ldx, T, s, sorted_rows, k, offsets, E, Xq, sx, stream);
}

int w4a8_gemm(const int8_t* Xq, const float* sx, int M, const void* blob, const w4a8_wdesc* d, void* Y,
              int ldy, int out_dtype, void* stream) {
    int st = check_gemm_desc(d);
    if (st) return st;
    if (M < 0 || (out_dtype != W4A8_OUT_BF16 && out_dtype != W4A8_OUT_F32)) return W4A8_EINVAL;
    if (M == 0) return W4A8_OK;
    if (!Xq || !sx || !blob || !Y || ldy < d->N) return W4A8_EINVAL;
    if (!aligned16(Xq) || !aligned16(blob)) return W4A8_EINVAL;
    const Layout L = layout_of(d);
    GemmArgs a = make_args(L, Xq, sx, M, blob);
    a.Y = Y;
    a.ldy = ldy;
    a.out_f32 = out_dtype == W4A8_OUT_F32;
    if (M >= PREFILL_MIN_M && !prefill_offsets_fit(L.K, PF_BM)) return W4A8_EINVAL;
    if (log_on()) std::fprintf(stderr, "w4a8: w4a8_gemm M=%d K=%d N=%d -> %s\n", M, L.K, L.N, w4a8_kernel_name(d, M));
    if (M >= PREFILL_MIN_M) {
        launch_prefill<MODE_OUT>(a, gps_of(d), d->asymmetric, static_cast<hipStream_t>(stream), L.bits == 8);
        return launch_status();
    }
    // the split kernel (one K-slice per wave) serves the decode rows, except those that
    // w4a8_linear quantizes inside the GEMM: they stay on the chunked kernel, whose fused form
    // shares its summation order (fused and unfused results are bit-identical)
    if (!linear_fuses(L, M) && decode_split_fits(L.K, M, gps_of(d), L.bits)) {
        launch_decode_split(a, gps_of(d), d->asymmetric, static_cast<hipStream_t>(stream));
        return launch_status();
    }
    const int mt = dense_mt(M);
    const DecodeCfg c = decode_cfg(L.K, mt);
    const dim3 grid = decode_grid(L, c, (M + mt - 1) / mt);
    launch_decode<MODE_OUT, false>(a, c, gps_of(d), d->asymmetric, grid, static_cast<hipStream_t>(stream),
                                   L.bits == 8);
    return launch_status();
}

int w4a8_linear(const void* X, int M, int K, int ldx, const void* blob, const w4a8_wdesc* d, void* Y, int ldy,
                int out_dtype, int8_t* Xq, float* sx, void* stream) {
    int st = check_gemm_desc(d);
    if (st) return st;
    if (M < 0 || K != d->K || (out_dtype != W4A8_OUT_BF16 && out_dtype != W4A8_OUT_F32)) return W4A8_EINVAL;
    if (M == 0) return W4A8_OK;
    if (!X || !blob || !Y || !Xq || !sx || ldy < d->N || ldx < K) return W4A8_EINVAL;
    if (ldx % 8 || !aligned16(X) || !aligned16(Xq) || !aligned16(blob)) return W4A8_EINVAL;
    const Layout L = layout_of(d);
    // Fused path: the unfused decode kernel's workgroup layout and summation order, so the
    // result is bit-identical.  Each workgroup quantizes all M x K activations itself, so
    // fusing pays off only while that redundant work is small next to the launch it saves.
    const DecodeCfg fc = decode_cfg(L.K, 16);
    if (linear_fuses(L, M)) {
        if (log_on())
            std::fprintf(stderr, "w4a8: w4a8_linear M=%d K=%d N=%d -> %s, quantization fused\n", M, L.K, L.N,
                         w4a8_kernel_name(d, M));
        GemmArgs a = make_args(L, Xq, sx, M, blob);
        a.X = static_cast<const uint16_t*>(X);
        a.ldx = ldx;
        a.Y = Y;
        a.ldy = ldy;
        a.out_f32 = out_dtype == W4A8_OUT_F32;
        hipStream_t s = static_cast<hipStream_t>(stream);
        const dim3 grid = decode_grid(L, fc, 1);
        const int gps = gps_of(d);
        if (L.bits == 8) {
            if (gps == 4) launch_decode_fused<4, false, true>(a, fc, grid, s);
            else if (gps == 1) launch_decode_fused<1, false, true>(a, fc, grid, s);
            else if (gps == 2) launch_decode_fused<2, false, true>(a, fc, grid, s);
            else if (gps == 0) launch_decode_fused<0, false, true>(a, fc, grid, s);
            else launch_decode_fused<-1, false, true>(a, fc, grid, s);
        } else if (gps == 0) {
            if (d->asymmetric) launch_decode_fused<0, true>(a, fc, grid, s); else launch_decode_fused<0, false>(a, fc, grid, s);
        } else if (gps < 0) {
            if (d->asymmetric) launch_decode_fused<-1, true>(a, fc, grid, s); else launch_decode_fused<-1, false>(a, fc, grid, s);
        } else if (gps == 4) {
            if (d->asymmetric) launch_decode_fused<4, true>(a, fc, grid, s); else launch_decode_fused<4, false>(a, fc, grid, s);
        } else if (gps == 1) {
            if (a.h16) { if (d->asymmetric) launch_decode_fused<1, true, false, true>(a, fc, grid, s); else launch_decode_fused<1, false, false, true>(a, fc, grid, s); }
            else if (d->asymmetric) launch_decode_fused<1, true>(a, fc, grid, s); else launch_decode_fused<1, false>(a, fc, grid, s);
        } else {
            if (a.h16) { if (d->asymmetric) launch_decode_fused<2, true, false, true>(a, fc, grid, s); else launch_decode_fused<2, false, false, true>(a, fc, grid, s); }
            else if (d->asymmetric) launch_decode_fused<2, true>(a, fc, grid, s); else launch_decode_fused<2, false>(a, fc, grid, s);
        }
        return launch_status();
    }
    if (log_on()) std::fprintf(stderr, "w4a8: w4a8_linear M=%d K=%d N=%d -> quant_act + w4a8_gemm\n", M, L.K, L.N);
    if ((st = w4a8_quant_act(X, M, K, ldx, Xq, sx, stream))) return st;
    return w4a8_gemm(Xq, sx, M, blob, d, Y, ldy, out_dtype, stream);
}

int w4a8_gemm_partials(const int8_t* Xq, int M, const void* blob, const w4a8_wdesc* d, int32_t* P, void* stream) {
    int st = check_gemm_desc(d);
    if (st) return st;
    if (M < 0) return W4A8_EINVAL;
    if (M == 0) return W4A8_OK;
    if (!Xq || !blob || !P) return W4A8_EINVAL;
    if (!aligned16(Xq) || !aligned16(blob)) return W4A8_EINVAL;
    const Layout L = layout_of(d);
    GemmArgs a = make_args(L, Xq, nullptr, M, blob);
    a.P = P;
    if (M >= PREFILL_MIN_M) {
        if (!prefill_offsets_fit(L.K, PF_BM)) return W4A8_EINVAL;
        launch_prefill<MODE_PARTIALS>(a, gps_of(d), d->asymmetric, static_cast<hipStream_t>(stream),
                                      L.bits == 8);
        return launch_status();
    }
    // per-channel partials span all of K, which the decode kernels split across waves
    if (gps_of(d) < 0) return W4A8_EUNSUPPORTED;
    const int mt = dense_mt(M);
    const DecodeCfg c = decode_cfg(L.K, mt);
    const dim3 grid = decode_grid(L, c, (M + mt - 1) / mt);
    launch_decode<MODE_PARTIALS, false>(a, c, gps_of(d), d->asymmetric, grid,
                                        static_cast<hipStream_t>(stream), L.bits == 8);
    return launch_status();
}

int w4a8_moe_align(const int32_t* ids, int T, int k, int E, int32_t* sorted_rows, int32_t* offsets, int32_t* inv,
                   void* stream) {
    if (T < 0 || k <= 0 || E <= 0 || E > 1024) return W4A8_EINVAL;
    if (!offsets) return W4A8_EINVAL;
    const long long R = (long long)T * k;
    if (R > (1 << 24)) return W4A8_EUNSUPPORTED;
    if (R > 0 && (!ids || !sorted_rows || !inv)) return W4A8_EINVAL;
    const int LDS_INTS = 12288;
    int Bmax = std::min(1024, LDS_INTS / E - 1);
    if (Bmax < 1) Bmax = 1;
    int L = R > 0 ? int((R + Bmax - 1) / Bmax) : 1;
    int B = R > 0 ? int((R + L - 1) / L) : 0;
    size_t lds = (size_t(E) * (B + 1) + 16) * sizeof(int);
    hipStream_t s = static_cast<hipStream_t>(stream);
    constexpr long long STAGE_MAX = 16384;          // 64 KiB of ids next to <= 48 KiB of counts
    if (R <= STAGE_MAX) {
        static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(moe_align_kernel<true>),
                                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                                           int((LDS_INTS + 16 + STAGE_MAX) * sizeof(int)));
        (void)attr;
        moe_align_kernel<true><<<dim3(1), dim3(1024), lds + size_t(R) * sizeof(int), s>>>(
            ids, int(R), E, L, B, sorted_rows, offsets, inv);
    } else {
        moe_align_kernel<false><<<dim3(1), dim3(1024), lds, s>>>(ids, int(R), E, L, B, sorted_rows, offsets, inv);
    }
    return launch_status();
}

// ------------------------------------------------------------------------------------
// Side-by-side grouped launches
// ------------------------------------------------------------------------------------
// The format classes of a layer (w4a8_moe_forward_sets) are grouped GEMMs over disjoint expert
// ranges, so they write disjoint rows and do not depend on each other.  One after another, each
// class's launches end on a partial round of workgroups in which most compute units idle, and
// a class's share of the experts fills few rounds.  They are put side by side on helper streams
// of the current device instead, forked from and joined back into the caller's stream with
// events, so a call still completes in the caller's stream order and captures into one graph.
// (Measured on the 64-expert top-6 layer with two classes: 0.39 -> 0.34 ms.  One grouped GEMM's
// experts with many rows and its other experts were measured side by side too: each of those
// launches fills the chip by itself, and the events' cost cancelled the overlap.)  The helpers are
// created on first use (default priority) and kept for the life of the process; where they
// cannot be created, the launches run one after another on the caller's stream.  The enqueue
// sequence of a call runs under fork_mu, so calls from several host threads do not interleave
// their event records.
constexpr int FORK_MAX_DEVICES = 64;
constexpr int FORK_STREAMS = 4;

struct ForkSet {
    hipStream_t st[FORK_STREAMS];
    hipEvent_t fork;
    hipEvent_t join[FORK_STREAMS];
    int state;                        // 0: not tried yet, 1: ready, -1: unavailable
};
static std::mutex fork_mu;
static ForkSet fork_sets[FORK_MAX_DEVICES];

// The current device's helpers, or nullptr.  Call with fork_mu held.  They are not created while
// the caller's stream s is being captured into a graph (creation is not a stream operation and
// may not be allowed then): such a call runs its launches one after another.
static ForkSet* fork_set(hipStream_t s) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= FORK_MAX_DEVICES) return nullptr;
    ForkSet& f = fork_sets[dev];
    if (f.state == 0) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) {
            (void)hipGetLastError();
            return nullptr;
        }
        bool ok = hipEventCreateWithFlags(&f.fork, hipEventDisableTiming) == hipSuccess;
        for (int i = 0; ok && i < FORK_STREAMS; ++i)
            ok = hipStreamCreateWithFlags(&f.st[i], hipStreamNonBlocking) == hipSuccess &&
                 hipEventCreateWithFlags(&f.join[i], hipEventDisableTiming) == hipSuccess;
        if (!ok) (void)hipGetLastError();           // the failure must not surface as a launch error
        f.state = ok ? 1 : -1;
    }
    return f.state == 1 ? &f : nullptr;
}

// Helpers [i0, i1) wait for the work enqueued so far on s.
static int fork_to(ForkSet* f, hipStream_t s, int i0, int i1) {
    if (hipEventRecord(f->fork, s) != hipSuccess) return W4A8_EHIP;
    for (int i = i0; i < i1; ++i)
        if (hipStreamWaitEvent(f->st[i], f->fork, 0) != hipSuccess) return W4A8_EHIP;
    return W4A8_OK;
}

// s waits for everything enqueued on helpers [i0, i1).
static int join_from(ForkSet* f, hipStream_t s, int i0, int i1) {
    for (int i = i0; i < i1; ++i) {
        if (hipEventRecord(f->join[i], f->st[i]) != hipSuccess) return W4A8_EHIP;
        if (hipStreamWaitEvent(s, f->join[i], 0) != hipSuccess) return W4A8_EHIP;
    }
    return W4A8_OK;
}

// Hq set: the paired form (gate/up blob, static SiLU-requant epilogue into Hq, sh with scales s_dn).
// rows_cap: a bound on any expert's row count that the caller expects (the layer entry points pass
// T: a token routes to k distinct experts).  Below the MFMA-tile cut the 128-row tile launch is
// left out and the streaming kernels serve every expert; they take any row count, so an expert
// with more rows than the bound (duplicate routing ids) is still computed, only not on the tiles.
static int moe_gemm_impl(const int8_t* Xq, const float* sx, const int32_t* gather, int k, const int32_t* offsets,
                         int E, int rows, int src_rows, const void* blobs, size_t stride, const w4a8_wdesc* d,
                         void* Y, int out_dtype, int mt, hipStream_t s, int8_t* Hq = nullptr, float* sh = nullptr,
                         const float* s_dn = nullptr, int rows_cap = 1 << 30, const MoeClasses* mc = nullptr) {
    const bool tiles = rows >= MOE_TILE_MIN_ROWS && rows_cap >= MOE_TILE_MIN_ROWS;
    const Layout L = layout_of(d);
    if (log_on()) {
        const int nsb = L.K / SB_K;
        const char* cold = moe_stream_fits(L.K, gps_of(d)) ? "gemm_moe_stream_kernel"
                           : (nsb <= 64 && (mt == 16 || (nsb > 16 && nsb <= 32))) ? "gemm_kslice_kernel"
                                                                                  : "gemm_decode_kernel (grouped)";
        std::fprintf(stderr, "w4a8: %s E=%d rows=%d K=%d N=%d g=%d %s -> %s%s, %d-row tiles\n",
                     Hq ? "w4a8_moe_gemm_silu_static" : "w4a8_moe_gemm", E, rows, L.K, L.N, L.g,
                     d->asymmetric ? "asym" : "sym",
                     tiles ? "gemm_moe_tile_kernel (experts with >= 96 rows) + " : "",
                     cold, mt);
    }
    GemmArgs a = make_args(L, Xq, sx, rows, blobs);
    a.Hq = Hq;
    a.sh = sh;
    a.s_dn = s_dn;
    a.pair_n = L.N / 2;
    a.Y = Y;
    a.ldy = L.N;
    a.out_f32 = out_dtype == W4A8_OUT_F32;
    a.gather = gather;
    a.topk = k;
    a.src_rows = src_rows;
    a.offsets = offsets;
    a.E = E;
    a.expert_stride = stride;
    a.moe_lo = 0;
    a.moe_hi = 1 << 30;
    if (tiles) {
        // experts with many rows: prefill tiles; slots bound sum_e ceil(rows_e / tile rows) over
        // experts with rows_e >= MOE_TILE_MIN_ROWS (surplus workgroups find no tile and exit)
        a.moe_lo = MOE_TILE_MIN_ROWS;
        const int tslots = rows / 128 + rows / MOE_TILE_MIN_ROWS + 1;
        if (mc) launch_moe_tile_classes(a, *mc, tslots, s);
        else launch_moe_tile(a, gps_of(d), d->asymmetric, tslots, s);
        a.moe_lo = 0;
        a.moe_hi = MOE_TILE_MIN_ROWS;
    }
    // slots bound sum_e ceil(rows_e / per) over the experts; surplus workgroups exit at once
    const int slots = rows / mt + std::min(E, rows) + 1;
    if (moe_stream_fits(L.K, gps_of(d))) {
        // the experts below the MFMA-tile cut in one streaming launch: each workgroup stages one
        // row tile of one expert and streams 256 of its columns
        if (mc) launch_moe_stream_classes(a, *mc, mt, slots, s);
        else launch_moe_stream(a, mt, gps_of(d), d->asymmetric, slots, s);
        return launch_status();
    }
    if (mc) return W4A8_EUNSUPPORTED;                // format classes: streaming kernels only
    // 2048 < K <= 4096: 16-row tiles run in a row loop (32-row tiles would not leave the
    // registers for it), so each expert's weights are read once per column tile
    const int nsb = L.K / SB_K;
    const int kmt = (nsb > 16 && nsb <= 32) ? 16 : mt;
    KsliceCfg kc;
    if (kslice_cfg(L.K, kmt, &kc, true)) {
        // row loop: a workgroup runs up to MOE_KSLICE_ROWS rows of its expert
        const int kslots = kc.rl ? rows / MOE_KSLICE_ROWS + std::min(E, rows) + 1 : rows / kmt + std::min(E, rows) + 1;
        launch_kslice<MODE_OUT, true>(a, kc, kmt / 16, gps_of(d), d->asymmetric, kslots, s);
        return launch_status();
    }
    const DecodeCfg c = decode_cfg(L.K, mt);
    launch_decode<MODE_OUT, true>(a, c, gps_of(d), d->asymmetric, decode_grid(L, c, slots), s);
    return launch_status();
}

// Argument checks of one grouped GEMM (everything the launch below relies on), so that the
// layer entry points can run them all before their first launch.
static int moe_gemm_check(const int8_t* Xq, const float* sx, const int32_t* gather, int k, const int32_t* offsets,
                          int E, int rows, int src_rows, const void* blobs, size_t stride, const w4a8_wdesc* d,
                          const void* Y, int out_dtype) {
    int st = check_gemm_desc(d);
    if (st) return st;
    if (!grouped_format_ok(d)) return W4A8_EUNSUPPORTED;
    if (rows < 0 || src_rows < 0 || E <= 0 || (out_dtype != W4A8_OUT_BF16 && out_dtype != W4A8_OUT_F32))
        return W4A8_EINVAL;
    if (rows == 0) return W4A8_OK;
    if (!Xq || !sx || !offsets || !blobs || !Y) return W4A8_EINVAL;
    if (gather ? (k <= 0 || src_rows == 0) : src_rows < rows) return W4A8_EINVAL;
    const Layout L = layout_of(d);
    if (E > 1 && stride < L.total) return W4A8_EINVAL;
    if (!aligned16(Xq) || !aligned16(blobs) || (stride & 15)) return W4A8_EINVAL;
    return W4A8_OK;
}

// w4a8_moe_gemm with a bound on the rows of any expert (see moe_gemm_impl)
static int moe_gemm_capped(const int8_t* Xq, const float* sx, const int32_t* gather, int k, const int32_t* offsets,
                           int E, int rows, int src_rows, const void* blobs, size_t stride, const w4a8_wdesc* d,
                           void* Y, int out_dtype, void* stream, int rows_cap) {
    const int st = moe_gemm_check(Xq, sx, gather, k, offsets, E, rows, src_rows, blobs, stride, d, Y, out_dtype);
    if (st || rows == 0) return st;
    const int mt = rows / E >= 16 ? 32 : 16;
    return moe_gemm_impl(Xq, sx, gather, k, offsets, E, rows, src_rows, blobs, stride, d, Y, out_dtype, mt,
                         static_cast<hipStream_t>(stream), nullptr, nullptr, nullptr, rows_cap);
}

int w4a8_moe_gemm(const int8_t* Xq, const float* sx, const int32_t* gather, int k, const int32_t* offsets, int E,
                  int rows, int src_rows, const void* blobs, size_t stride, const w4a8_wdesc* d, void* Y,
                  int out_dtype, void* stream) {
    return moe_gemm_capped(Xq, sx, gather, k, offsets, E, rows, src_rows, blobs, stride, d, Y, out_dtype, stream,
                           1 << 30);
}

// Checks of the paired form on top of moe_gemm_check: the blob holds gate and up columns in
// equal numbers that split into whole 16-column tiles, and the outputs are given.
static int moe_gemm_silu_check(const int8_t* Xq, const float* sx, const int32_t* gather, int k,
                               const int32_t* offsets, int E, int rows, int src_rows, const void* blobs, size_t stride,
                               const w4a8_wdesc* d, const float* s, const int8_t* Hq, const float* sh) {
    const int st = moe_gemm_check(Xq, sx, gather, k, offsets, E, rows, src_rows, blobs, stride, d, Hq, W4A8_OUT_BF16);
    if (st || rows == 0) return st;
    if (d->N % 32) return W4A8_EINVAL;
    if (!s || !sh) return W4A8_EINVAL;
    return W4A8_OK;
}

static int moe_gemm_silu_capped(const int8_t* Xq, const float* sx, const int32_t* gather, int k,
                                const int32_t* offsets, int E, int rows, int src_rows, const void* blobs,
                                size_t stride, const w4a8_wdesc* d, const float* s, int8_t* Hq, float* sh,
                                void* stream, int rows_cap) {
    const int st = moe_gemm_silu_check(Xq, sx, gather, k, offsets, E, rows, src_rows, blobs, stride, d, s, Hq, sh);
    if (st || rows == 0) return st;
    const int mt = rows / E >= 16 ? 32 : 16;
    return moe_gemm_impl(Xq, sx, gather, k, offsets, E, rows, src_rows, blobs, stride, d, nullptr, W4A8_OUT_BF16, mt,
                         static_cast<hipStream_t>(stream), Hq, sh, s, rows_cap);
}

int w4a8_moe_gemm_silu_static(const int8_t* Xq, const float* sx, const int32_t* gather, int k,
                              const int32_t* offsets, int E, int rows, int src_rows, const void* blobs, size_t stride,
                              const w4a8_wdesc* d, const float* s, int8_t* Hq, float* sh, void* stream) {
    return moe_gemm_silu_capped(Xq, sx, gather, k, offsets, E, rows, src_rows, blobs, stride, d, s, Hq, sh, stream,
                                1 << 30);
}

// Longest row of the SiLU step: 8 passes of 2048 values per 256-thread workgroup.
constexpr int SILU_MAX_I = 16384;

static int silu_impl(const void* GU, int R, int I, int8_t* Hq, float* sh, const float* sstat, const int32_t* offs,
                     int E, void* stream) {
    if (R < 0 || I <= 0) return W4A8_EINVAL;
    if (R == 0) return W4A8_OK;
    if (!GU || !Hq || !sh) return W4A8_EINVAL;
    if (I % 16 || !aligned16(GU) || !aligned16(Hq)) return W4A8_EINVAL;
    if (I > SILU_MAX_I) return W4A8_EUNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint16_t* g = static_cast<const uint16_t*>(GU);
    switch (row_iters(I)) {
        case 1: launch_silu<1>(g, R, I, Hq, sh, s, sstat, offs, E); break;
        case 2: launch_silu<2>(g, R, I, Hq, sh, s, sstat, offs, E); break;
        case 4: launch_silu<4>(g, R, I, Hq, sh, s, sstat, offs, E); break;
        case 8: launch_silu<8>(g, R, I, Hq, sh, s, sstat, offs, E); break;
        default: return W4A8_EUNSUPPORTED;
    }
    return launch_status();
}

int w4a8_silu_mul_quant(const void* GU, int R, int I, int8_t* Hq, float* sh, void* stream) {
    return silu_impl(GU, R, I, Hq, sh, nullptr, nullptr, 0, stream);
}

int w4a8_silu_mul_quant_static(const void* GU, int R, int I, const int32_t* offsets, int E, const float* s,
                               int8_t* Hq, float* sh, void* stream) {
    if (E <= 0 || E > 1024) return W4A8_EINVAL;
    if (R > 0 && (!offsets || !s)) return W4A8_EINVAL;
    return silu_impl(GU, R, I, Hq, sh, s, offsets, E, stream);
}

int w4a8_moe_combine(const void* Yd, const int32_t* inv, const float* w, int T, int k, int H, void* out,
                     void* stream) {
    if (T < 0 || k <= 0 || H <= 0) return W4A8_EINVAL;
    if (T == 0) return W4A8_OK;
    if (!Yd || !inv || !w || !out) return W4A8_EINVAL;
    if (H % 8 || !aligned16(Yd) || !aligned16(out)) return W4A8_EINVAL;
    const uint16_t* yd = static_cast<const uint16_t*>(Yd);
    uint16_t* o = static_cast<uint16_t*>(out);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (k <= 8)
        moe_combine_kernel<8><<<dim3(T), dim3(256), 0, s>>>(yd, inv, w, k, H, o);
    else
        moe_combine_kernel<0><<<dim3(T), dim3(256), 0, s>>>(yd, inv, w, k, H, o);
    return launch_status();
}

// Workspace carve-up of w4a8_moe_forward (each piece 256-byte aligned).
struct MoeWs {
    size_t xq, sx, rows, offs, inv, gu, hq, sh, yd, total;
};

// per_row: the static-scale form quantizes each routed row (T * k rows) instead of each token
static MoeWs moe_ws(int T, int k, int H, int I, int E, bool per_row = false) {
    auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
    const size_t R = size_t(T) * size_t(k);
    const size_t QR = per_row ? R : size_t(T);
    MoeWs w;
    size_t o = 0;
    w.xq = o; o = al(o + QR * H);
    w.sx = o; o = al(o + QR * 4);
    w.rows = o; o = al(o + R * 4);
    w.offs = o; o = al(o + size_t(E + 1) * 4);
    w.inv = o; o = al(o + R * 4);
    w.gu = o; o = al(o + (per_row ? 0 : R * size_t(2 * I) * 2));   // the static form needs no gate/up buffer
    w.hq = o; o = al(o + R * size_t(I));
    w.sh = o; o = al(o + R * 4);
    w.yd = o; o = al(o + R * size_t(H) * 2);
    w.total = o;
    return w;
}

size_t w4a8_moe_workspace_size(int T, int k, int H, int I, int E) {
    if (T < 0 || k <= 0 || H <= 0 || I <= 0 || E <= 0) return 0;
    return moe_ws(T, k, H, I, E).total;
}

// Checks of a MoE layer entry point that do not depend on the weights: routing sizes, the
// pointers, the workspace and the row shapes of the quantization (X [T, H]), SiLU (I) and
// combine (H) steps.  Together with moe_gemm_check on both grouped GEMMs, every argument
// check of the chained steps runs before the layer's first launch, so an error return means
// that nothing was enqueued.  dyn: the layer quantizes X per token (w4a8_quant_act: H <= 65536).
static int moe_layer_check(const void* X, const int32_t* ids, const float* w, int T, int k, int E, int H, int I,
                           const void* ws, size_t ws_bytes, size_t ws_need, const void* out, bool dyn) {
    if (T < 0 || k <= 0 || E <= 0 || E > 1024) return W4A8_EINVAL;
    if ((long long)T * k > (1 << 24)) return W4A8_EUNSUPPORTED;
    if (T == 0) return W4A8_OK;
    if (!X || !ids || !w || !ws || !out) return W4A8_EINVAL;
    if (H % 16 || I % 16 || !aligned16(X) || !aligned16(out)) return W4A8_EINVAL;
    if ((dyn && H > 65536) || I > SILU_MAX_I) return W4A8_EUNSUPPORTED;
    if (ws_bytes < ws_need) return W4A8_ESIZE;
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return W4A8_EINVAL;
    return W4A8_OK;
}

// Workspace pieces of a MoE layer call.
struct MoeBufs {
    int8_t* xq;
    float* sx;
    int32_t *rows, *offs, *inv;
    void* gu;
    int8_t* hq;
    float* sh;
    void* yd;
};

static MoeBufs moe_bufs(void* ws, const MoeWs& L) {
    uint8_t* b = static_cast<uint8_t*>(ws);
    return MoeBufs{reinterpret_cast<int8_t*>(b + L.xq), reinterpret_cast<float*>(b + L.sx),
                   reinterpret_cast<int32_t*>(b + L.rows), reinterpret_cast<int32_t*>(b + L.offs),
                   reinterpret_cast<int32_t*>(b + L.inv), b + L.gu, reinterpret_cast<int8_t*>(b + L.hq),
                   reinterpret_cast<float*>(b + L.sh), b + L.yd};
}

int w4a8_moe_forward(const void* X, const int32_t* ids, const float* w, int T, int k, int E, const void* gu_blobs,
                     size_t gu_stride, const w4a8_wdesc* gu_desc, const void* d_blobs, size_t d_stride,
                     const w4a8_wdesc* d_desc, void* ws, size_t ws_bytes, void* out, void* stream) {
    int st = check_gemm_desc(gu_desc);
    if (st) return st;
    st = check_gemm_desc(d_desc);
    if (st) return st;
    if (!grouped_format_ok(gu_desc) || !grouped_format_ok(d_desc)) return W4A8_EUNSUPPORTED;
    if (T < 0 || k <= 0 || E <= 0) return W4A8_EINVAL;
    const int H = gu_desc->K, I2 = gu_desc->N;
    if (I2 % 2 || d_desc->K != I2 / 2 || d_desc->N != H) return W4A8_EINVAL;
    const int I = I2 / 2;
    const MoeWs L = moe_ws(T, k, H, I, E);
    if ((st = moe_layer_check(X, ids, w, T, k, E, H, I, ws, ws_bytes, L.total, out, true)) || T == 0) return st;
    const MoeBufs B = moe_bufs(ws, L);
    const int R = T * k;
    if ((st = moe_gemm_check(B.xq, B.sx, B.rows, k, B.offs, E, R, T, gu_blobs, gu_stride, gu_desc, B.gu,
                             W4A8_OUT_BF16)))
        return st;
    if ((st = moe_gemm_check(B.hq, B.sh, nullptr, k, B.offs, E, R, R, d_blobs, d_stride, d_desc, B.yd,
                             W4A8_OUT_BF16)))
        return st;
    // every step's checks have passed: from here on only a launch error can stop the chain
    if ((st = w4a8_quant_act(X, T, H, H, B.xq, B.sx, stream))) return st;
    if ((st = w4a8_moe_align(ids, T, k, E, B.rows, B.offs, B.inv, stream))) return st;
    // a token's k rows go to k distinct experts, so no expert has more than T rows (T bounds
    // the tile launch; duplicate ids stay correct, see moe_gemm_impl)
    if ((st = moe_gemm_capped(B.xq, B.sx, B.rows, k, B.offs, E, R, T, gu_blobs, gu_stride, gu_desc, B.gu,
                              W4A8_OUT_BF16, stream, T)))
        return st;
    if ((st = w4a8_silu_mul_quant(B.gu, R, I, B.hq, B.sh, stream))) return st;
    if ((st = moe_gemm_capped(B.hq, B.sh, nullptr, k, B.offs, E, R, R, d_blobs, d_stride, d_desc, B.yd,
                              W4A8_OUT_BF16, stream, T)))
        return st;
    return w4a8_moe_combine(B.yd, B.inv, w, T, k, H, out, stream);
}

// Scratch of w4a8_moe_forward_noalloc: the workspace of w4a8_moe_forward, held in device memory
// for the life of the process (one copy on each GPU the library runs on).  Host code never
// uses the name `scratch` as an address: each device's copy is reached through the pointer
// that hipGetSymbolAddress returns with that device current.
constexpr size_t NOALLOC_SCRATCH_BYTES = size_t(64) << 20;
static __device__ __align__(256) uint8_t scratch[NOALLOC_SCRATCH_BYTES];

constexpr int NOALLOC_MAX_DEVICES = 64;
static std::mutex scratch_mu;
static void* scratch_dev[NOALLOC_MAX_DEVICES];

// Address of the current device's scratch, looked up once per device.
static int scratch_of_current_device(void** ptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return W4A8_EHIP;
    if (dev < 0 || dev >= NOALLOC_MAX_DEVICES) return W4A8_EUNSUPPORTED;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_dev[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return W4A8_EHIP;
        scratch_dev[dev] = p;
    }
    *ptr = scratch_dev[dev];
    return W4A8_OK;
}

int w4a8_moe_forward_noalloc(const void* X, const int32_t* ids, const float* w, int T, int k, int E,
                             const void* gu_blobs, size_t gu_stride, const w4a8_wdesc* gu_desc, const void* d_blobs,
                             size_t d_stride, const w4a8_wdesc* d_desc, void* out, void* stream) {
    int st = check_gemm_desc(gu_desc);
    if (st) return st;
    if ((st = check_gemm_desc(d_desc))) return st;
    if (T < 0 || k <= 0 || E <= 0) return W4A8_EINVAL;
    const int H = gu_desc->K, I2 = gu_desc->N;
    if (I2 % 2 || d_desc->K != I2 / 2 || d_desc->N != H) return W4A8_EINVAL;
    if (T == 0) return W4A8_OK;
    // the layer's workspace must fit the scratch (checked before the device is touched)
    if (moe_ws(T, k, H, I2 / 2, E).total > NOALLOC_SCRATCH_BYTES) return W4A8_ESIZE;
    void* ws = nullptr;
    if ((st = scratch_of_current_device(&ws))) return st;
    // the layer writes every workspace byte it reads before reading it, so nothing left by an
    // earlier call needs clearing
    return w4a8_moe_forward(X, ids, w, T, k, E, gu_blobs, gu_stride, gu_desc, d_blobs, d_stride, d_desc, ws,
                            NOALLOC_SCRATCH_BYTES, out, stream);
}

int w4a8_moe_forward_sets(const void* X, const int32_t* ids, const float* w, int T, int k, const w4a8_expert_set* sets,
                          int nsets, void* ws, size_t ws_bytes, void* out, void* stream) {
    if (!sets || nsets <= 0 || T < 0 || k <= 0) return W4A8_EINVAL;
    int E = 0;
    for (int i = 0; i < nsets; ++i) {
        const w4a8_expert_set& st = sets[i];
        if (st.n_experts <= 0 || !st.gu_desc || !st.d_desc) return W4A8_EINVAL;
        int c = check_gemm_desc(st.gu_desc);
        if (c) return c;
        if ((c = check_gemm_desc(st.d_desc))) return c;
        if (!grouped_format_ok(st.gu_desc) || !grouped_format_ok(st.d_desc)) return W4A8_EUNSUPPORTED;
        // every set has the layer's shapes: gate/up [H, 2I], down [I, H]
        if (st.gu_desc->K != sets[0].gu_desc->K || st.gu_desc->N != sets[0].gu_desc->N ||
            st.d_desc->K != sets[0].d_desc->K || st.d_desc->N != sets[0].d_desc->N)
            return W4A8_EINVAL;
        E += st.n_experts;
    }
    const int H = sets[0].gu_desc->K, I2 = sets[0].gu_desc->N;
    if (I2 % 2 || sets[0].d_desc->K != I2 / 2 || sets[0].d_desc->N != H) return W4A8_EINVAL;
    const int I = I2 / 2;
    const MoeWs L = moe_ws(T, k, H, I, E);
    int st;
    if ((st = moe_layer_check(X, ids, w, T, k, E, H, I, ws, ws_bytes, L.total, out, true)) || T == 0) return st;
    const MoeBufs B = moe_bufs(ws, L);
    const int R = T * k;
    for (int i = 0, e0 = 0; i < nsets; e0 += sets[i].n_experts, ++i) {
        if ((st = moe_gemm_check(B.xq, B.sx, B.rows, k, B.offs + e0, sets[i].n_experts, R, T, sets[i].gu_blobs,
                                 sets[i].gu_stride, sets[i].gu_desc, B.gu, W4A8_OUT_BF16)))
            return st;
        if ((st = moe_gemm_check(B.hq, B.sh, nullptr, k, B.offs + e0, sets[i].n_experts, R, R, sets[i].d_blobs,
                                 sets[i].d_stride, sets[i].d_desc, B.yd, W4A8_OUT_BF16)))
            return st;
    }
    if ((st = w4a8_quant_act(X, T, H, H, B.xq, B.sx, stream))) return st;
    if ((st = w4a8_moe_align(ids, T, k, E, B.rows, B.offs, B.inv, stream))) return st;
    // each set is one grouped GEMM over its expert range: offs + e0 holds the absolute row ranges
    // of those experts, so the sets write disjoint output rows.  Set 0 runs on the caller's stream,
    // set i > 0 on helper (i - 1) % FORK_STREAMS, side by side.
    hipStream_t s = static_cast<hipStream_t>(stream);
    // a GEMM whose K fits the streaming kernels runs every set in one launch pair (tiles, then
    // streaming), each workgroup taking the format of its expert's set
    const bool one_gu = nsets > 1 && nsets <= MOE_MAX_CLASSES && moe_stream_fits(H, 1);
    const bool one_dn = nsets > 1 && nsets <= MOE_MAX_CLASSES && moe_stream_fits(I, 1);
    const int mt = R / E >= 16 ? 32 : 16;
    auto classes = [&](bool gate_up) {
        MoeClasses mc{};
        mc.n = nsets;
        for (int i = 0, e0 = 0; i < nsets; ++i) {
            const w4a8_wdesc* d = gate_up ? sets[i].gu_desc : sets[i].d_desc;
            const Layout Lc = layout_of(d);
            e0 += sets[i].n_experts;
            mc.e_end[i] = e0;
            mc.fmt[i] = (gps_of(d) - 1) | (Lc.asym ? 2 : 0) | (Lc.sbytes == 2 ? 4 : 0);
            mc.G[i] = Lc.G;
            mc.blob[i] = static_cast<const uint8_t*>(gate_up ? sets[i].gu_blobs : sets[i].d_blobs);
            mc.stride[i] = gate_up ? sets[i].gu_stride : sets[i].d_stride;
            mc.codes_off[i] = Lc.codes_off;
            mc.scales_off[i] = Lc.scales_off;
            mc.zeros_off[i] = Lc.zeros_off;
        }
        return mc;
    };
    std::lock_guard<std::mutex> lock(fork_mu);
    ForkSet* f = nsets > 1 && !(one_gu && one_dn) ? fork_set(s) : nullptr;
    const int nh = f ? std::min(nsets - 1, FORK_STREAMS) : 0;
    auto stage = [&](bool gate_up) -> int {
        int r;
        if (gate_up ? one_gu : one_dn) {
            const MoeClasses mc = classes(gate_up);
            return gate_up ? moe_gemm_impl(B.xq, B.sx, B.rows, k, B.offs, E, R, T, sets[0].gu_blobs,
                                           sets[0].gu_stride, sets[0].gu_desc, B.gu, W4A8_OUT_BF16, mt, s,
                                           nullptr, nullptr, nullptr, T, &mc)
                           : moe_gemm_impl(B.hq, B.sh, nullptr, k, B.offs, E, R, R, sets[0].d_blobs,
                                           sets[0].d_stride, sets[0].d_desc, B.yd, W4A8_OUT_BF16, mt, s,
                                           nullptr, nullptr, nullptr, T, &mc);
        }
        if (nh && (r = fork_to(f, s, 0, nh))) return r;
        for (int i = 0, e0 = 0; i < nsets; e0 += sets[i].n_experts, ++i) {
            const w4a8_expert_set& c = sets[i];
            void* cs = (i == 0 || !nh) ? stream : static_cast<void*>(f->st[(i - 1) % nh]);
            r = gate_up ? moe_gemm_capped(B.xq, B.sx, B.rows, k, B.offs + e0, c.n_experts, R, T, c.gu_blobs,
                                          c.gu_stride, c.gu_desc, B.gu, W4A8_OUT_BF16, cs, T)
                        : moe_gemm_capped(B.hq, B.sh, nullptr, k, B.offs + e0, c.n_experts, R, R, c.d_blobs,
                                          c.d_stride, c.d_desc, B.yd, W4A8_OUT_BF16, cs, T);
            if (r) return r;
        }
        return nh ? join_from(f, s, 0, nh) : W4A8_OK;
    };
    if ((st = stage(true))) return st;
    if ((st = w4a8_silu_mul_quant(B.gu, R, I, B.hq, B.sh, stream))) return st;
    if ((st = stage(false))) return st;
    return w4a8_moe_combine(B.yd, B.inv, w, T, k, H, out, stream);
}

size_t w4a8_moe_static_workspace_size(int T, int k, int H, int I, int E) {
    if (T < 0 || k <= 0 || H <= 0 || I <= 0 || E <= 0) return 0;
    return moe_ws(T, k, H, I, E, true).total;
}

int w4a8_moe_forward_static(const void* X, const int32_t* ids, const float* w, int T, int k, int E,
                            const void* gu_blobs, size_t gu_stride, const w4a8_wdesc* gu_desc, const void* d_blobs,
                            size_t d_stride, const w4a8_wdesc* d_desc, const float* s_gu, const float* s_dn,
                            void* ws, size_t ws_bytes, void* out, void* stream) {
    int st = check_gemm_desc(gu_desc);
    if (st) return st;
    st = check_gemm_desc(d_desc);
    if (st) return st;
    if (!grouped_format_ok(gu_desc) || !grouped_format_ok(d_desc)) return W4A8_EUNSUPPORTED;
    if (T < 0 || k <= 0 || E <= 0) return W4A8_EINVAL;
    const int H = gu_desc->K, I2 = gu_desc->N;
    if (I2 % 2 || d_desc->K != I2 / 2 || d_desc->N != H) return W4A8_EINVAL;
    const int I = I2 / 2;
    const MoeWs L = moe_ws(T, k, H, I, E, true);
    if ((st = moe_layer_check(X, ids, w, T, k, E, H, I, ws, ws_bytes, L.total, out, false)) || T == 0) return st;
    if (!s_gu || !s_dn) return W4A8_EINVAL;
    const MoeBufs B = moe_bufs(ws, L);
    const int R = T * k;
    if ((st = moe_gemm_silu_check(B.xq, B.sx, nullptr, k, B.offs, E, R, R, gu_blobs, gu_stride, gu_desc, s_dn,
                                  B.hq, B.sh)))
        return st;
    if ((st = moe_gemm_check(B.hq, B.sh, nullptr, k, B.offs, E, R, R, d_blobs, d_stride, d_desc, B.yd,
                             W4A8_OUT_BF16)))
        return st;
    if ((st = w4a8_moe_align(ids, T, k, E, B.rows, B.offs, B.inv, stream))) return st;
    // each routed row quantizes its token with the scale of its expert, already in sorted order
    if ((st = w4a8_moe_quant_static(X, T, H, H, B.rows, k, B.offs, E, s_gu, B.xq, B.sx, stream))) return st;
    // gate/up GEMM with the SiLU-requant folded into its epilogue: h's codes, no gate/up buffer
    if ((st = moe_gemm_silu_capped(B.xq, B.sx, nullptr, k, B.offs, E, R, R, gu_blobs, gu_stride, gu_desc, s_dn,
                                   B.hq, B.sh, stream, T)))
        return st;
    if ((st = moe_gemm_capped(B.hq, B.sh, nullptr, k, B.offs, E, R, R, d_blobs, d_stride, d_desc, B.yd,
                              W4A8_OUT_BF16, stream, T)))
        return st;
    return w4a8_moe_combine(B.yd, B.inv, w, T, k, H, out, stream);
}

const char* w4a8_kernel_name(const w4a8_wdesc* d, int M) {
    if (check_gemm_desc(d) != W4A8_OK || M < 0) return "unsupported";
    // one name per (form, row tile, format): [w8][kind: decode m16, decode m32, prefill][asym][g]
#define W4A8_NAMES(P, K, S) {P K S "_g64", P K S "_g128", P K S "_g256", P K S "_gK", P K S "_g32"}
    static const char* const names[2][3][2][5] = {
        {{W4A8_NAMES("w4a8", "_decode_m16", "_sym"), W4A8_NAMES("w4a8", "_decode_m16", "_asym")},
         {W4A8_NAMES("w4a8", "_decode_m32", "_sym"), W4A8_NAMES("w4a8", "_decode_m32", "_asym")},
         {W4A8_NAMES("w4a8", "_prefill", "_sym"), W4A8_NAMES("w4a8", "_prefill", "_asym")}},
        {{W4A8_NAMES("w8a8", "_decode_m16", "_sym"), {}},
         {W4A8_NAMES("w8a8", "_decode_m32", "_sym"), {}},
         {W4A8_NAMES("w8a8", "_prefill", "_sym"), {}}}};
#undef W4A8_NAMES
    // binary16 scales (4-bit codes, g in {64, 128})
    static const char* const names16[3][2][2] = {
        {{"w4a8_decode_m16_sym_g64_h16", "w4a8_decode_m16_sym_g128_h16"},
         {"w4a8_decode_m16_asym_g64_h16", "w4a8_decode_m16_asym_g128_h16"}},
        {{"w4a8_decode_m32_sym_g64_h16", "w4a8_decode_m32_sym_g128_h16"},
         {"w4a8_decode_m32_asym_g64_h16", "w4a8_decode_m32_asym_g128_h16"}},
        {{"w4a8_prefill_sym_g64_h16", "w4a8_prefill_sym_g128_h16"},
         {"w4a8_prefill_asym_g64_h16", "w4a8_prefill_asym_g128_h16"}}};
    const int kind = M >= PREFILL_MIN_M ? 2 : (dense_mt(M) == 32 ? 1 : 0);
    const int gps = gps_of(d);
    const int gi = gps == 2 ? 0 : gps == 1 ? 1 : gps == 0 ? 2 : gps == 4 ? 4 : 3;
    // the decode GEMMs that w4a8_gemm routes to the split kernel (one K-slice per wave):
    // [row tile][asym][g128][binary16 scales]
    static const char* const split_names[2][2][2][2] = {
        {{{"w4a8_decode_split_m16_sym_g64", "w4a8_decode_split_m16_sym_g64_h16"},
          {"w4a8_decode_split_m16_sym_g128", "w4a8_decode_split_m16_sym_g128_h16"}},
         {{"w4a8_decode_split_m16_asym_g64", "w4a8_decode_split_m16_asym_g64_h16"},
          {"w4a8_decode_split_m16_asym_g128", "w4a8_decode_split_m16_asym_g128_h16"}}},
        {{{"w4a8_decode_split_m32_sym_g64", "w4a8_decode_split_m32_sym_g64_h16"},
          {"w4a8_decode_split_m32_sym_g128", "w4a8_decode_split_m32_sym_g128_h16"}},
         {{"w4a8_decode_split_m32_asym_g64", "w4a8_decode_split_m32_asym_g64_h16"},
          {"w4a8_decode_split_m32_asym_g128", "w4a8_decode_split_m32_asym_g128_h16"}}}};
    const Layout L = layout_of(d);
    if (kind < 2 && M > 0 && !linear_fuses(L, M) && decode_split_fits(L.K, M, gps, L.bits))
        return split_names[kind][d->asymmetric ? 1 : 0][gps == 1 ? 1 : 0][L.sbytes == 2 ? 1 : 0];
    if (layout_of(d).sbytes == 2) return names16[kind][d->asymmetric][gi];
    return names[layout_of(d).bits == 8][kind][d->asymmetric][gi];
}

}  // extern "C"
