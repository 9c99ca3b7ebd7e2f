// Device helpers shared by the kernel translation units of the library (gfx950).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace w4a8 {

typedef int v4i __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------------------------
// small device helpers
// ------------------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// binary16 bit pattern -> float32 (exact)
__device__ __forceinline__ float f16_to_f32(uint16_t bits) { return static_cast<float>(__builtin_bit_cast(_Float16, bits)); }

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;   // quiet NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// 16-byte load of weight codes that are read once per launch, marked non-temporal: the
// stream then does not evict the activations and scales that every workgroup re-reads from
// L2.  Measured on the 4096 x 14336 decode GEMM: 8.1 -> 7.5 us at 16-row tiles, 10.1 -> 9.3 us
// at 32-row tiles.
__device__ __forceinline__ uint4 stream_load(const uint8_t* p) {
    const v4i v = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(p));
    return make_uint4(uint32_t(v.x), uint32_t(v.y), uint32_t(v.z), uint32_t(v.w));
}

// Workgroup barrier for LDS hand-offs that leaves global loads in flight: wait for this
// wave's LDS (and scalar) operations only, then s_barrier.  The empty asm statements keep
// the compiler from moving memory accesses across it.  (__syncthreads would also drain
// every outstanding global load of the wave.)
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    // s_waitcnt: vmcnt 63 (no wait), expcnt 7 (no wait), lgkmcnt 0
    __builtin_amdgcn_s_waitcnt(0xF | (7 << 4) | (0 << 8) | (3 << 14));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// ------------------------------------------------------------------------------------
// per-row INT8 quantization rule (P1 section 3.3; P5 section 8.3) and the SiLU-gated product
// ------------------------------------------------------------------------------------
// One element of the per-token rule q = clamp(rint(fl32(x / d)), -127, 127), branch free.
// inv = RN(1/d) comes from one IEEE division per row.  q0 = RN(x * inv) is within 1.5 ulp of
// x/d; one Newton correction q1 = RN(q0 + inv * (x - d * q0)) (residual through fma) has an
// error far below 1 ulp before rounding, so q1 is faithful; by Markstein's theorem a second
// correction from a faithful q1 with the correctly rounded reciprocal inv gives exactly
// RN(x / d), the IEEE float32 quotient.  Rows with a tiny divisor (fast == false, uniform per
// row) use the IEEE division directly.
__device__ __forceinline__ int quant_one(float x, float d, float inv, bool fast) {
    float q;
    if (fast) {
        const float q0 = x * inv;
        const float q1 = fmaf(fmaf(-d, q0, x), inv, q0);
        q = rintf(fmaf(fmaf(-d, q1, x), inv, q1));
    } else {
        q = rintf(x / d);
    }
    q = fminf(fmaxf(q, -127.0f), 127.0f);
    return (int)q;
}

struct RowScale {
    float s, d, inv;
    bool finite, fast;
    float lim;      // static scales: values are clamped to +-lim = 128 d before the division
    bool huge;      // static scales: 128 d overflows (d > 2^120), lim is FLT_MAX
};

// Scale of a row from the bit pattern of its abs-max.  With UNIFORM (the default) amax_bits
// must be the same in every lane of the wave: it is broadcast from lane 0 so that the scale,
// and the branch on `fast`, are wave-uniform.
template <bool UNIFORM = true>
__device__ __forceinline__ RowScale row_scale(uint32_t amax_bits) {
    if (UNIFORM) amax_bits = __builtin_amdgcn_readfirstlane(amax_bits);
    RowScale r;
    r.finite = amax_bits < 0x7f800000u;
    const float amax = __uint_as_float(amax_bits);
    r.s = r.finite ? amax / 127.0f : __uint_as_float(0x7fc00000u);
    r.d = (r.finite && r.s > 0.0f) ? r.s : 1.0f;
    r.inv = 1.0f / r.d;
    r.fast = r.d >= 1e-30f;
    return r;
}

// A given scale s: codes are produced only for a finite, positive s (otherwise all zero).
__device__ __forceinline__ RowScale static_row_scale(float s) {
    RowScale r;
    r.s = s;
    r.finite = s > 0.0f && s <= 3.40282347e38f;
    r.d = r.finite ? s : 1.0f;
    r.inv = 1.0f / r.d;
    r.fast = r.d >= 1e-30f;
    r.huge = r.d > 1.329228e36f;                         // 2^120
    r.lim = r.huge ? 3.40282347e38f : 128.0f * r.d;
    return r;
}

// clamp(rint(fl32(x / d)), -127, 127) for any x.  Values are first limited to +-lim = 128 d
// (one med3; exact, a power-of-two multiple): every such value still saturates, +-Inf
// included, and quant_one's quotient stays finite.  NaN gives 0.  With d > 2^120 (lim is
// FLT_MAX there) +-Inf is set to +-127 explicitly.
template <bool HUGE = true>
__device__ __forceinline__ int quant_static_one(float x, const RowScale& r) {
    int q = quant_one(__builtin_amdgcn_fmed3f(x, -r.lim, r.lim), r.d, r.inv, r.fast);
    if (x != x) q = 0;
    if (HUGE && r.huge && fabsf(x) > 3.40282347e38f) q = x > 0.0f ? 127 : -127;
    return q;
}

// silu(g) * u in float32 (P1 section 1: the expert MLP's gated activation).  Every path that
// forms h calls this one definition, so fused and unfused paths agree bit for bit.
__device__ __forceinline__ float silu_mul(float g, float u) { return (g / (1.0f + expf(-g))) * u; }

// One code of the static SiLU-requant (P1 section 3.2: a calibrated scale per expert, so no row
// reduction): the gate and up GEMM outputs are first rounded to bfloat16, the precision in which
// the unfused chain stores them, then h = silu(g) * u is quantized with the expert's scale.
__device__ __forceinline__ int silu_static_code(float yg, float yu, const RowScale& rs) {
    if (!rs.finite) return 0;
    const float h = silu_mul(bf16_to_f32(f32_to_bf16_rne(yg)), bf16_to_f32(f32_to_bf16_rne(yu)));
    return quant_static_one(h, rs);
}

// ------------------------------------------------------------------------------------
// GEMM arguments, operand unpacking and the grouped (MoE) tile mapping
// ------------------------------------------------------------------------------------
enum { MODE_OUT = 0, MODE_PARTIALS = 1 };

struct GemmArgs {
    const int8_t* Xq;         // INT8 activations (or, fused path: where to write them)
    const float* sx;          // row scales (or, fused path: where to write them)
    const uint16_t* X;        // fused path: bfloat16 activations [M, ldx]
    int ldx;
    int M, K, N, G;
    const uint8_t* blob;      // blob of expert 0 (or the only blob)
    size_t codes_off, scales_off, zeros_off, expert_stride;
    void* Y;
    int ldy;
    int out_f32;              // 1: float32 output, 0: bfloat16
    int32_t* P;               // partials export [M, N, G]
    const int32_t* gather;    // MoE: source token row = gather[r] / topk
    int topk;
    int src_rows;             // MoE: rows of Xq / sx a gather may name
    const int32_t* offsets;   // MoE: expert row offsets [E+1]
    int E;
    int moe_lo, moe_hi;       // MoE: this launch serves the experts with moe_lo <= rows < moe_hi
    int h16;                  // binary16 group scales (selects the H16 kernels)
    // MoE gate/up with the static SiLU-requant epilogue (when Hq is set): blob columns c and
    // pair_n + c are the gate and up outputs of column c of h.  A workgroup computes both side
    // by side, and instead of Y it writes the codes Hq [M, pair_n] and the row scales sh [M]
    // (= s_dn[e] for every row of expert e).
    int8_t* Hq;
    float* sh;
    const float* s_dn;
    int pair_n;
};

// Blob column tile of tile slot l (0 <= l < n) of a workgroup whose slots start at tile `first`.
// Unpaired: first + l.  Paired (a.Hq set): the first n / 2 slots are the gate tiles
// first / 2 + l, the rest the matching up tiles pair_n / 16 + first / 2 + l - n / 2.
__device__ __forceinline__ int pair_tile(const GemmArgs& a, int first, int l, int n) {
    if (!a.Hq) return first + l;
    const int g0 = first / 2;
    return l < n / 2 ? g0 + l : a.pair_n / 16 + g0 + l - n / 2;
}

// Unpack two packed words (16 codes of one column) into one MFMA B operand.
// Symmetric: two's-complement nibbles moved to the high half of each byte -> 16 * q
// (exact; the 1/16 is folded into the group scale).  Asymmetric: unsigned nibbles in the
// low half, then (q + 128 - z) ^ 0x80 per byte = q - z as int8 with no borrow between
// bytes (q + 128 - z lies in [113, 143]).
template <bool ASYM>
__device__ __forceinline__ v4i unpack_b(uint32_t w0, uint32_t w1, uint32_t zc) {
    v4i b;
    if (!ASYM) {
        b[0] = int((w0 << 4) & 0xF0F0F0F0u);
        b[1] = int(w0 & 0xF0F0F0F0u);
        b[2] = int((w1 << 4) & 0xF0F0F0F0u);
        b[3] = int(w1 & 0xF0F0F0F0u);
    } else {
        b[0] = int(((w0 & 0x0F0F0F0Fu) + zc) ^ 0x80808080u);
        b[1] = int((((w0 >> 4) & 0x0F0F0F0Fu) + zc) ^ 0x80808080u);
        b[2] = int(((w1 & 0x0F0F0F0Fu) + zc) ^ 0x80808080u);
        b[3] = int((((w1 >> 4) & 0x0F0F0F0Fu) + zc) ^ 0x80808080u);
    }
    return b;
}

// MoE gather: the source activation row of routed row r, or -1 when gather[r] names no row
// of Xq (negative, or a token at or past src_rows).  Such rows read zero codes and a zero
// scale, so their outputs are 0 and nothing outside Xq and sx is read.
__device__ __forceinline__ int gather_src(const GemmArgs& a, int r) {
    const int g = a.gather[r];
    if (g < 0) return -1;
    const int t = g / a.topk;
    return t < a.src_rows ? t : -1;
}

struct TileRows {
    int rbeg, rend, expert;
};

// MoE: the slot-th MT-row tile over the experts served by this launch (row count in
// [moe_lo, moe_hi)), in expert order, each expert's rows split into ceil(rows_e / MT) tiles.
// Every wave evaluates this identically, so the workgroup agrees without a barrier.
// expert = -1 when the slot is past the last tile.
template <int MT>
__device__ __forceinline__ TileRows moe_tile(const GemmArgs& a, int slot, int lane) {
    TileRows tr{0, 0, -1};
    int base = 0;
    for (int c = 0; c < a.E; c += 64) {
        const int e = c + lane;
        const int cnt = e < a.E ? a.offsets[e + 1] - a.offsets[e] : 0;
        const int t = (cnt >= a.moe_lo && cnt < a.moe_hi) ? (cnt + MT - 1) / MT : 0;
        int incl = t;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(incl, o, 64);
            if (lane >= o) incl += y;
        }
        const int excl = incl - t;
        const unsigned long long hit = __ballot(slot >= base + excl && slot < base + incl);
        if (hit) {
            const int src = __ffsll((long long)hit) - 1;
            const int ef = __shfl(e, src, 64);
            const int tl = slot - base - __shfl(excl, src, 64);
            // row ranges are clamped to the launch's rows, so malformed offsets cannot
            // move a tile outside the output or the activations
            const int e0 = min(max(a.offsets[ef], 0), a.M), e1 = min(max(a.offsets[ef + 1], e0), a.M);
            tr.rbeg = e0 + tl * MT;
            tr.rend = min(e1, tr.rbeg + MT);
            tr.expert = tr.rend > tr.rbeg ? ef : -1;
            return tr;
        }
        base += __shfl(incl, 63, 64);
    }
    return tr;
}

// Format classes of one grouped launch (experts of different weight formats, P1 section 8).
// Class c holds the experts [first, e_end[c]) with first = e_end[c - 1] (0 for c = 0); expert e
// of class c has its blob at blob[c] + (e - first) * stride[c], G[c] groups along K and the
// blob sections at codes_off[c], scales_off[c], zeros_off[c].  fmt[c] = (gps - 1) | asym << 1 |
// h16 << 2 selects the code a workgroup of that class runs.  Every class has the launch's K and N.
constexpr int MOE_MAX_CLASSES = 4;
struct MoeClasses {
    int n;
    int e_end[MOE_MAX_CLASSES];
    int fmt[MOE_MAX_CLASSES];
    int G[MOE_MAX_CLASSES];
    const uint8_t* blob[MOE_MAX_CLASSES];
    size_t stride[MOE_MAX_CLASSES];
    size_t codes_off[MOE_MAX_CLASSES], scales_off[MOE_MAX_CLASSES], zeros_off[MOE_MAX_CLASSES];
};

// The class of expert e (uniform over the workgroup): a's group count and blob sections become
// the class's, blob is the expert's blob; returns the class's fmt.  An expert past the last
// class's end (malformed e_end) takes the last class.
__device__ __forceinline__ int moe_class_resolve(const MoeClasses& mc, int e, GemmArgs& a, const uint8_t*& blob) {
    int c = 0;
    while (c + 1 < mc.n && e >= mc.e_end[c]) ++c;
    const int first = c ? mc.e_end[c - 1] : 0;
    a.G = mc.G[c];
    a.codes_off = mc.codes_off[c];
    a.scales_off = mc.scales_off[c];
    a.zeros_off = mc.zeros_off[c];
    blob = mc.blob[c] + size_t(e - first) * mc.stride[c];
    return mc.fmt[c];
}

// Grouped streaming GEMM (w4a8_moe_kernels.hip): every expert of a launch, K <= 4096, g in {64, 128}.
bool moe_stream_fits(int K, int gps);
void launch_moe_stream(const GemmArgs& a, int mt, int gps, bool asym, int slots, hipStream_t s);
// the same over format classes: each workgroup runs the code of its expert's class
void launch_moe_stream_classes(const GemmArgs& a, const MoeClasses& mc, int mt, int slots, hipStream_t s);

// Grouped GEMM on 128 x 128 MFMA tiles (w4a8_moe_tile_kernels.hip) over the experts with
// moe_lo <= rows < moe_hi, g in {64, 128}; slots bounds the sum over those experts of ceil(rows_e / 128).
void launch_moe_tile(const GemmArgs& a, int gps, bool asym, int slots, hipStream_t s);
void launch_moe_tile_classes(const GemmArgs& a, const MoeClasses& mc, int slots, hipStream_t s);

// Dense decode GEMM with one K-slice per wave (w4a8_decode_kernels.hip): 4-bit codes, g in {64, 128},
// M <= 32, 2048 < K <= 4096.
bool decode_split_fits(int K, int M, int gps, int bits);
void launch_decode_split(const GemmArgs& a, int gps, bool asym, hipStream_t s);

}  // namespace w4a8
