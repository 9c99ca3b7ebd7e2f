// gfx950 kernels and entry points of the W4A16 sibling: 16-bit (bfloat16) activations, the
// 4-bit weights of the W4A8 blob dequantized inside the kernel, bfloat16 MFMA.
//
// Sources (cited with the page's own section names):
//   P1 "Kimi 2.7 MoE: from 4-bit storage to INT8 (W4A8)" (pwwt.cn), section 5.3: the W4A16 row of
//      the format comparison (weights 4-bit, activations 16-bit).
//   P5 "Inference quantization, chapter 1: the Linear layer" (sgdbs.github.io), section 3.2: the
//      weight-only path, where the dequantization is fused into the GEMM.
//   P3 "Quantization: formats, error and the real execution path" (wineandchord.com), "Basic
//      mapping": w ~ s (q - z).
//
// Y[m, n] = sum_i s[i, n] * sum_{k in group i} x[m, k] * (q[k, n] - z[i, n]), float32 accumulation,
// bfloat16 or float32 output.  No activation quantization; dequantized weights never leave
// registers.
//
// Nibbles to bfloat16 operands.  The bfloat16 bit pattern 0x4180 | (v << 3) (v < 16) is exactly
// 16 + v (16 times 1 + v/16: the code fills the top four mantissa bits), so a shift and one AND-OR
// (asymmetric) or AND-XOR (symmetric) turn two packed nibbles into two bfloat16 operands: 16 + n
// (asymmetric, n = the unsigned code) or 24 + q (symmetric, from the two's-complement nibble:
// n ^ 8 = q + 8).  The MFMA then sums x * (C + (q - z)) with C = 16 + z or 24, and the group
// epilogue removes C times the group's activation sum S:
//   P = P' - C S,  acc = fma(P, s, acc).
// The offset costs float32 accuracy in proportion to C / |q - z|; with the code in the top
// mantissa bits C is at most 31 (with it in the low bits, 0x4300 | v = 128 + v, C would be about
// 136 and the error on the 4096-deep outlier inputs about 1.4e-3 instead of about 2e-4).
// The mask pairs nibbles (j, j + 2) of a 32-bit word, so each 8-value operand holds k in the
// order [0, 2, 1, 3, 4, 6, 5, 7] of its 8-block; the activations are staged in LDS in the same
// order (the permutation is its own inverse), so every product pairs the same k on both sides.
//
// MFMA 16x16x32 bf16 operand convention: lane l supplies 8 bfloat16 of A row (l % 16) and of B
// column (l % 16) for the k-block 8 (l / 16) of the 32-deep step; the result of lane l is
// C[4 (l / 16) + i][l % 16], i = 0..3.  A lane's 16 codes of one 64-deep half of the W4A8 layout
// (k = 64 h + 16 (l / 16) + j) feed two such steps: j in [0, 8) and j in [8, 16).
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>

#include "w4a8_device.h"
#include "w4a8_internal.h"

namespace w4a8 {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

struct A16Args {
    const uint16_t* X;          // bfloat16 activations [M, ldx]
    int ldx;
    int M, K, N, G;
    const uint8_t* blob;
    size_t codes_off, scales_off, zeros_off;
    void* Y;
    int ldy;
    int out_f32;
};

// Two bfloat16 operands from the nibbles at bits [sh, sh + 4) and [sh + 16, sh + 20) of w (sh in
// {0, 4, 8, 12}), each moved to bits [3, 7) of its half: 16 + n (asymmetric) or 24 + q (symmetric).
template <bool ASYM>
__device__ __forceinline__ uint32_t nib_pair_bf16(uint32_t w, int sh) {
    const uint32_t t = (sh >= 3 ? (w >> (sh - 3)) : (w << (3 - sh))) & 0x00780078u;
    return ASYM ? (t | 0x41804180u) : (t ^ 0x41C041C0u);
}

// One 8-value B operand from the 8 codes of a 32-bit word (byte i: code i in the low nibble,
// code i + 4 in the high nibble), in k order [0, 2, 1, 3, 4, 6, 5, 7].
template <bool ASYM>
__device__ __forceinline__ v8bf b_operand(uint32_t w) {
    typedef uint32_t v4u __attribute__((ext_vector_type(4)));
    const v4u u = {nib_pair_bf16<ASYM>(w, 0), nib_pair_bf16<ASYM>(w, 8), nib_pair_bf16<ASYM>(w, 4),
                   nib_pair_bf16<ASYM>(w, 12)};
    return __builtin_bit_cast(v8bf, u);
}

// The same permutation on 8 bfloat16 activations (16 bytes): swap elements 1 <-> 2 and 5 <-> 6.
__device__ __forceinline__ uint4 permute_act(uint4 v) {
    uint4 o;
    o.x = (v.x & 0xFFFFu) | (v.y << 16);                 // e0, e2
    o.y = (v.x >> 16) | (v.y & 0xFFFF0000u);             // e1, e3
    o.z = (v.z & 0xFFFFu) | (v.w << 16);                 // e4, e6
    o.w = (v.z >> 16) | (v.w & 0xFFFF0000u);             // e5, e7
    return o;
}

// ------------------------------------------------------------------------------------
// Decode form (M <= 32).  Workgroup = 4 column tiles x 4 K-slices, one wave per (tile, slice),
// over chunks of CS superblocks: the chunk's activation rows are staged in LDS (bfloat16, in the
// operand order above) together with each row's per-group sums; every wave streams SBN = CS / 4
// of its tile's superblocks.  The 4 slices' float32 sums are added in slice order through LDS.
// ------------------------------------------------------------------------------------
constexpr int A16_NT = 4, A16_KW = 4;

template <int MS, int CS>
struct A16Shape {
    static constexpr int MT = 16 * MS;
    static constexpr int NTHR = 64 * A16_NT * A16_KW;           // 1024
    static constexpr int SBN = CS / A16_KW;                     // superblocks per wave per chunk
    static constexpr int ROWB = CS * SB_K * 2 + 16;             // LDS row stride in bytes
    static constexpr int PPR = CS * SB_K / 8;                   // 16-byte pieces per row and chunk
    static constexpr int APT = MT * PPR / NTHR;                 // pieces per thread
    static constexpr int GMAX = CS * 2;                         // groups per chunk at g = 64
    static constexpr size_t LDS_A = size_t(MT) * ROWB;
    static constexpr size_t LDS_S = size_t(GMAX) * MT * 4;      // group sums [group][row]
    static constexpr size_t LDS_RED = size_t(A16_KW - 1) * A16_NT * MS * 4 * 64 * 4;
    static constexpr size_t LDS = LDS_A + LDS_S + LDS_RED;
    static_assert(NTHR % PPR == 0, "a thread's pieces share their column in the chunk");
    static_assert(LDS <= 160 * 1024, "LDS");
};

template <int MS, int CS, int GPS, bool ASYM>
__global__ __launch_bounds__(1024) void gemm_a16_decode_kernel(A16Args a) {
    using S = A16Shape<MS, CS>;
    constexpr int MT = S::MT, NTHR = S::NTHR, SBN = S::SBN, ROWB = S::ROWB, PPR = S::PPR, APT = S::APT;
    constexpr int PPG = (GPS == 2 ? 64 : 128) / 8;     // 16-byte pieces per group
    extern __shared__ __align__(16) uint8_t smem[];
    float* gsum = reinterpret_cast<float*>(smem + S::LDS_A);
    float* red = reinterpret_cast<float*>(smem + S::LDS_A + S::LDS_S);
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int t = wave % A16_NT, q = wave / A16_NT;
    const int ntiles = (a.N + 15) / 16;
    const int tile = blockIdx.x * A16_NT + t;
    const bool tvalid = tile < ntiles;
    const int tile_c = tvalid ? tile : ntiles - 1;
    const int nsb = a.K / SB_K;
    const int rbeg = blockIdx.y * MT;
    const int nrows = min(a.M, rbeg + MT) - rbeg;
    const uint8_t* codes = a.blob + a.codes_off;
    const float* scales = reinterpret_cast<const float*>(a.blob + a.scales_off);
    const uint8_t* zeros = a.blob + a.zeros_off;
    const uint32_t boff = uint32_t(tile_c) * uint32_t(nsb) * 1024u + uint32_t(lane) * 16u;
    const uint32_t moff = uint32_t(tile_c) * uint32_t(a.G) * 16u + uint32_t(lane & 15);

    float accf[MS][4];
#pragma unroll
    for (int ms = 0; ms < MS; ++ms)
#pragma unroll
        for (int i = 0; i < 4; ++i) accf[ms][i] = 0.0f;

    for (int cb = 0; cb < nsb; cb += CS) {
        const int clen = min(CS, nsb - cb);
        // 1. the chunk's activation pieces (issued first: they gate the first MFMA)
        uint4 xv[APT];
#pragma unroll
        for (int i = 0; i < APT; ++i) {
            const int p = tid + i * NTHR, row = p / PPR, c = p % PPR;
            xv[i] = make_uint4(0, 0, 0, 0);
            if (row < nrows && c < clen * 16)
                xv[i] = *reinterpret_cast<const uint4*>(a.X + size_t(rbeg + row) * a.ldx + size_t(cb) * SB_K + c * 8);
        }
        // 2. this wave's group scales and zero points, then its weight superblocks
        const int s0 = cb + q * SBN;
        float sc[SBN][GPS];
        uint32_t zq[SBN][GPS];
        uint4 bq[SBN];
#pragma unroll
        for (int s = 0; s < SBN; ++s) {
            const uint32_t sb = uint32_t(min(s0 + s, nsb - 1));
#pragma unroll
            for (int gi = 0; gi < GPS; ++gi) {
                const uint32_t mi = moff + (sb * GPS + gi) * 16u;
                sc[s][gi] = scales[mi];
                zq[s][gi] = ASYM ? uint32_t(zeros[mi]) : 0u;
            }
        }
#pragma unroll
        for (int s = 0; s < SBN; ++s) {
            const uint32_t sb = uint32_t(min(s0 + s, nsb - 1));
            bq[s] = stream_load(codes + (boff + sb * 1024u));
        }
        asm volatile("" ::: "memory");
        // 3. activations to LDS in operand order, and each row's sum over every group (float32,
        //    a fixed order: 8 values in k order, then the pieces pairwise); the PPG pieces of one
        //    group sit in PPG consecutive lanes
#pragma unroll
        for (int i = 0; i < APT; ++i) {
            const int p = tid + i * NTHR, row = p / PPR, c = p % PPR;
            const uint4 v = xv[i];
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
            float sum = 0.0f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                sum += bf16_to_f32(w[j] & 0xFFFFu);
                sum += bf16_to_f32(w[j] >> 16);
            }
#pragma unroll
            for (int o = 1; o < PPG; o <<= 1) sum += __shfl_xor(sum, o, 64);
            if (row < nrows && c < clen * 16) {
                *reinterpret_cast<uint4*>(smem + row * ROWB + c * 16) = permute_act(v);
                if (c % PPG == 0) gsum[(c / PPG) * MT + row] = sum;
            }
        }
        lds_barrier();
        // 4. MFMAs over this wave's superblocks, group epilogue
#pragma unroll
        for (int s = 0; s < SBN; ++s) {
            const int sb = s0 + s;
            if (sb >= cb + clen) continue;              // uniform per wave
            v4f acc[MS];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t w0 = h ? bq[s].z : bq[s].x, w1 = h ? bq[s].w : bq[s].y;
                const v8bf b0 = b_operand<ASYM>(w0), b1 = b_operand<ASYM>(w1);
                const bool first = GPS == 2 || h == 0;
#pragma unroll
                for (int ms = 0; ms < MS; ++ms) {
                    const uint8_t* ap = smem + (ms * 16 + (lane & 15)) * ROWB + ((sb - cb) * SB_K + h * 64 + 16 * (lane >> 4)) * 2;
                    const v8bf a0 = __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4*>(ap));
                    const v8bf a1 = __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4*>(ap + 16));
                    const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
                    acc[ms] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b0, first ? zero : acc[ms], 0, 0, 0);
                    acc[ms] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b1, acc[ms], 0, 0, 0);
                }
                if (GPS == 2 || h == 1) {
                    const int gi = GPS == 2 ? h : 0;
                    const int gc = (sb - cb) * GPS + gi;               // group index inside the chunk
                    const float C = ASYM ? float(16u + zq[s][gi]) : 24.0f;
#pragma unroll
                    for (int ms = 0; ms < MS; ++ms) {
                        const float4 g4 = *reinterpret_cast<const float4*>(gsum + gc * MT + ms * 16 + 4 * (lane >> 4));
                        const float gs[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            accf[ms][i] = fmaf(fmaf(-C, gs[i], acc[ms][i]), sc[s][gi], accf[ms][i]);
                    }
                }
            }
        }
        if (cb + CS < nsb) lds_barrier();               // the next chunk rewrites LDS
    }

    // slice-ordered reduction, store
    constexpr int NV = MS * 4;
    if (q > 0) {
#pragma unroll
        for (int ms = 0; ms < MS; ++ms)
#pragma unroll
            for (int i = 0; i < 4; ++i) red[(((q - 1) * A16_NT + t) * NV + ms * 4 + i) * 64 + lane] = accf[ms][i];
    }
    __syncthreads();
    if (q != 0) return;
#pragma unroll
    for (int w = 1; w < A16_KW; ++w)
#pragma unroll
        for (int ms = 0; ms < MS; ++ms)
#pragma unroll
            for (int i = 0; i < 4; ++i) accf[ms][i] += red[(((w - 1) * A16_NT + t) * NV + ms * 4 + i) * 64 + lane];
    const int col = tile * 16 + (lane & 15);
    if (!tvalid || col >= a.N) return;
#pragma unroll
    for (int ms = 0; ms < MS; ++ms)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = rbeg + ms * 16 + 4 * (lane >> 4) + i;
            if (row >= rbeg + nrows) continue;
            if (a.out_f32)
                reinterpret_cast<float*>(a.Y)[size_t(row) * a.ldy + col] = accf[ms][i];
            else
                reinterpret_cast<uint16_t*>(a.Y)[size_t(row) * a.ldy + col] = uint16_t(f32_to_bf16_rne(accf[ms][i]));
        }
}

template <int MS, int CS, int GPS, bool ASYM>
static void launch_a16_decode(const A16Args& a, int Np, hipStream_t s) {
    using S = A16Shape<MS, CS>;
    auto kern = gemm_a16_decode_kernel<MS, CS, GPS, ASYM>;
    static const hipError_t attr =
        hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, int(S::LDS));
    (void)attr;
    const dim3 grid((Np / 16 + A16_NT - 1) / A16_NT, (a.M + S::MT - 1) / S::MT);
    kern<<<grid, dim3(S::NTHR), S::LDS, s>>>(a);
}

// ------------------------------------------------------------------------------------
// Prefill form (M > 32).  Workgroup tile 128 rows x 128 columns, 8 waves (2 x 4) of 64 x 32 (4 x 2
// MFMA tiles of 16 x 16).  Per 128-deep superblock the workgroup stages the activation tile in LDS
// (bfloat16, operand order, double buffered, loads one superblock ahead) with each row's group
// sums; each wave loads the packed codes of its 2 column tiles itself (16 bytes per lane each, the
// two waves of a column block share them through L1) and turns them into operands in registers.
// ------------------------------------------------------------------------------------
constexpr int A16P_BM = 128, A16P_BN = 128, A16P_THREADS = 512;
constexpr int A16P_ROWB = SB_K * 2 + 16;                       // LDS row stride in bytes
constexpr int A16P_ABYTES = A16P_BM * A16P_ROWB;               // 34816
constexpr int A16P_SBYTES = 2 * A16P_BM * 4;                   // group sums, up to 2 groups
constexpr int A16P_STAGE = A16P_ABYTES + A16P_SBYTES;
constexpr int A16P_LDS = 2 * A16P_STAGE;
constexpr int A16P_APT = A16P_BM * 16 / A16P_THREADS;          // 16-byte pieces per thread: 4
constexpr int A16P_WC = 2;                                     // column tiles per wave

template <int GPS, bool ASYM>
__global__ __launch_bounds__(A16P_THREADS) void gemm_a16_prefill_kernel(A16Args a) {
    constexpr int PPG = (GPS == 2 ? 64 : 128) / 8;
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;
    const int mtiles = (a.M + A16P_BM - 1) / A16P_BM;
    const int mt = blockIdx.x % mtiles, nt = blockIdx.x / mtiles;   // consecutive workgroups share weights
    const int m0 = mt * A16P_BM;
    const int ntl16 = (a.N + 15) / 16;
    const int nsb = a.K / SB_K;
    const uint8_t* codes = a.blob + a.codes_off;
    const float* scales = reinterpret_cast<const float*>(a.blob + a.scales_off);
    const uint8_t* zeros = a.blob + a.zeros_off;
    // this wave's column tiles (clamped to the last one; their outputs are not stored)
    uint32_t boff[A16P_WC], moff[A16P_WC];
#pragma unroll
    for (int c = 0; c < A16P_WC; ++c) {
        const uint32_t tl = uint32_t(min(nt * 8 + wn * A16P_WC + c, ntl16 - 1));
        boff[c] = tl * uint32_t(nsb) * 1024u + uint32_t(lane) * 16u;
        moff[c] = tl * uint32_t(a.G) * 16u + uint32_t(lane & 15);
    }
    auto load_a = [&](uint4 (&xv)[A16P_APT], int sb) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < A16P_APT; ++i) {
            const int p = tid + i * A16P_THREADS, row = p >> 4, c = p & 15;
            const int r = min(m0 + row, a.M - 1);              // rows past M repeat the last row
            xv[i] = *reinterpret_cast<const uint4*>(a.X + size_t(r) * a.ldx + size_t(sb) * SB_K + c * 8);
        }
    };
    auto store_a = [&](const uint4 (&xv)[A16P_APT], int stage) __attribute__((always_inline)) {
        uint8_t* st = smem + stage * A16P_STAGE;
        float* gs = reinterpret_cast<float*>(st + A16P_ABYTES);
#pragma unroll
        for (int i = 0; i < A16P_APT; ++i) {
            const int p = tid + i * A16P_THREADS, row = p >> 4, c = p & 15;
            const uint4 v = xv[i];
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
            float sum = 0.0f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                sum += bf16_to_f32(w[j] & 0xFFFFu);
                sum += bf16_to_f32(w[j] >> 16);
            }
#pragma unroll
            for (int o = 1; o < PPG; o <<= 1) sum += __shfl_xor(sum, o, 64);
            *reinterpret_cast<uint4*>(st + row * A16P_ROWB + c * 16) = permute_act(v);
            if (c % PPG == 0) gs[(c / PPG) * A16P_BM + row] = sum;
        }
    };
    struct Meta {
        uint4 b[A16P_WC];
        float s[A16P_WC][GPS];
        uint32_t z[A16P_WC][GPS];
    };
    auto load_w = [&](Meta& m, int sb) __attribute__((always_inline)) {
#pragma unroll
        for (int c = 0; c < A16P_WC; ++c) {
            m.b[c] = *reinterpret_cast<const uint4*>(codes + (boff[c] + uint32_t(sb) * 1024u));
#pragma unroll
            for (int gi = 0; gi < GPS; ++gi) {
                const uint32_t mi = moff[c] + (uint32_t(sb) * GPS + gi) * 16u;
                m.s[c][gi] = scales[mi];
                m.z[c][gi] = ASYM ? uint32_t(zeros[mi]) : 0u;
            }
        }
    };

    float accf[4][A16P_WC][4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < A16P_WC; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) accf[r][c][i] = 0.0f;

    uint4 xv[A16P_APT];
    Meta cur, nxt;
    load_a(xv, 0);
    load_w(cur, 0);
    store_a(xv, 0);
    __syncthreads();
    for (int sb = 0; sb < nsb; ++sb) {
        const int stage = sb & 1;
        if (sb + 1 < nsb) {                              // next superblock: activations, codes, scales
            load_a(xv, sb + 1);
            load_w(nxt, sb + 1);
        }
        const uint8_t* st = smem + stage * A16P_STAGE;
        const float* gs = reinterpret_cast<const float*>(st + A16P_ABYTES);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            v4f acc[4][A16P_WC];
#pragma unroll
            for (int set = 0; set < 2; ++set) {
                v8bf b[A16P_WC];
#pragma unroll
                for (int c = 0; c < A16P_WC; ++c) {
                    const uint32_t w = set ? (h ? cur.b[c].w : cur.b[c].y) : (h ? cur.b[c].z : cur.b[c].x);
                    b[c] = b_operand<ASYM>(w);
                }
                const bool first = (GPS == 2 || h == 0) && set == 0;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const uint8_t* ap = st + (wm * 64 + r * 16 + (lane & 15)) * A16P_ROWB + (h * 64 + 16 * (lane >> 4)) * 2 + set * 16;
                    const v8bf av = __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4*>(ap));
                    const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int c = 0; c < A16P_WC; ++c)
                        acc[r][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, b[c], first ? zero : acc[r][c], 0, 0, 0);
                }
            }
            if (GPS == 2 || h == 1) {
                const int gi = GPS == 2 ? h : 0;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float4 g4 = *reinterpret_cast<const float4*>(gs + gi * A16P_BM + wm * 64 + r * 16 + 4 * (lane >> 4));
                    const float gv[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
                    for (int c = 0; c < A16P_WC; ++c) {
                        const float C = ASYM ? float(16u + cur.z[c][gi]) : 24.0f;
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            accf[r][c][i] = fmaf(fmaf(-C, gv[i], acc[r][c][i]), cur.s[c][gi], accf[r][c][i]);
                    }
                }
            }
        }
        if (sb + 1 < nsb) {
            store_a(xv, stage ^ 1);                      // the other stage was last read before the barrier below
            cur = nxt;
        }
        lds_barrier();                                   // LDS hand-off only: global loads may stay in flight
    }
#pragma unroll
    for (int c = 0; c < A16P_WC; ++c) {
        const int col = (nt * 8 + wn * A16P_WC + c) * 16 + (lane & 15);
        if (col >= a.N) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = m0 + wm * 64 + r * 16 + 4 * (lane >> 4) + i;
                if (row >= a.M) continue;
                if (a.out_f32)
                    reinterpret_cast<float*>(a.Y)[size_t(row) * a.ldy + col] = accf[r][c][i];
                else
                    reinterpret_cast<uint16_t*>(a.Y)[size_t(row) * a.ldy + col] = uint16_t(f32_to_bf16_rne(accf[r][c][i]));
            }
    }
}

template <int GPS, bool ASYM>
static void launch_a16_prefill(const A16Args& a, hipStream_t s) {
    auto kern = gemm_a16_prefill_kernel<GPS, ASYM>;
    static const hipError_t attr =
        hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, A16P_LDS);
    (void)attr;
    const int mtiles = (a.M + A16P_BM - 1) / A16P_BM, ntiles = (a.N + A16P_BN - 1) / A16P_BN;
    kern<<<dim3(mtiles * ntiles), dim3(A16P_THREADS), A16P_LDS, s>>>(a);
}

static bool a16_format_ok(const w4a8_wdesc* d) {
    const Layout L = layout_of(d);
    return L.bits == 4 && L.sbytes == 4 && (L.g == 64 || L.g == 128);
}

}  // namespace w4a8

using namespace w4a8;

extern "C" {

int w4a16_gemm(const void* X, int M, int ldx, const void* blob, const w4a8_wdesc* d, void* Y, int ldy,
               int out_dtype, void* stream) {
    int st = desc_status(d);
    if (st) return st;
    if (!a16_format_ok(d)) return W4A8_EUNSUPPORTED;
    const Layout L = layout_of(d);
    if (L.codes_bytes >= (size_t(1) << 31) || L.scales_bytes >= (size_t(1) << 31)) return W4A8_EUNSUPPORTED;
    if (M < 0 || (out_dtype != W4A8_OUT_BF16 && out_dtype != W4A8_OUT_F32)) return W4A8_EINVAL;
    if (M == 0) return W4A8_OK;
    if (!X || !blob || !Y || ldx < L.K || ldy < L.N) return W4A8_EINVAL;
    if (ldx % 8 || (reinterpret_cast<uintptr_t>(X) & 15) || (reinterpret_cast<uintptr_t>(blob) & 15)) return W4A8_EINVAL;
    // the prefill form addresses the activations of a 128-row tile: rows * ldx stays far below 2^31
    if (M > 32 && size_t(A16P_BM) * size_t(ldx) * 2 >= (size_t(1) << 31)) return W4A8_EINVAL;
    A16Args a;
    std::memset(&a, 0, sizeof(a));
    a.X = static_cast<const uint16_t*>(X);
    a.ldx = ldx;
    a.M = M;
    a.K = L.K;
    a.N = L.N;
    a.G = L.G;
    a.blob = static_cast<const uint8_t*>(blob);
    a.codes_off = L.codes_off;
    a.scales_off = L.scales_off;
    a.zeros_off = L.zeros_off;
    a.Y = Y;
    a.ldy = ldy;
    a.out_f32 = out_dtype == W4A8_OUT_F32;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool asym = d->asymmetric != 0;
    const int gps = SB_K / L.g;
    if (log_on()) std::fprintf(stderr, "w4a8: w4a16_gemm M=%d K=%d N=%d -> %s\n", M, L.K, L.N, w4a16_kernel_name(d, M));
    if (M > 32) {
        if (gps == 1) { if (asym) launch_a16_prefill<1, true>(a, s); else launch_a16_prefill<1, false>(a, s); }
        else { if (asym) launch_a16_prefill<2, true>(a, s); else launch_a16_prefill<2, false>(a, s); }
    } else if (M <= 16) {
        // 16-superblock chunks at both tile heights: with 32-superblock chunks the 16-row form
        // exceeded the 128 registers a 1024-thread workgroup leaves each lane and kept part of
        // its superblocks in scratch (K = 4096, N = 14336: g64 with zero points 18.6 -> 10.2 us
        // at M = 1, 21.0 -> 11.9 us at M = 16; g128 10.2 -> 9.1 us at M = 1)
        if (gps == 1) { if (asym) launch_a16_decode<1, 16, 1, true>(a, L.Np, s); else launch_a16_decode<1, 16, 1, false>(a, L.Np, s); }
        else { if (asym) launch_a16_decode<1, 16, 2, true>(a, L.Np, s); else launch_a16_decode<1, 16, 2, false>(a, L.Np, s); }
    } else {
        if (gps == 1) { if (asym) launch_a16_decode<2, 16, 1, true>(a, L.Np, s); else launch_a16_decode<2, 16, 1, false>(a, L.Np, s); }
        else { if (asym) launch_a16_decode<2, 16, 2, true>(a, L.Np, s); else launch_a16_decode<2, 16, 2, false>(a, L.Np, s); }
    }
    return hipGetLastError() == hipSuccess ? W4A8_OK : W4A8_EHIP;
}

const char* w4a16_kernel_name(const w4a8_wdesc* d, int M) {
    if (desc_status(d) != W4A8_OK || !a16_format_ok(d) || M < 0) return "unsupported";
    static const char* const names[3][2][2] = {
        {{"w4a16_decode_m16_sym_g64", "w4a16_decode_m16_sym_g128"}, {"w4a16_decode_m16_asym_g64", "w4a16_decode_m16_asym_g128"}},
        {{"w4a16_decode_m32_sym_g64", "w4a16_decode_m32_sym_g128"}, {"w4a16_decode_m32_asym_g64", "w4a16_decode_m32_asym_g128"}},
        {{"w4a16_prefill_sym_g64", "w4a16_prefill_sym_g128"}, {"w4a16_prefill_asym_g64", "w4a16_prefill_asym_g128"}}};
    return names[M > 32 ? 2 : (M > 16 ? 1 : 0)][d->asymmetric != 0][d->group_size == 128];
}

}  // extern "C"
