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
};

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

// Grouped streaming GEMM (w4a8_moe_kernels.hip): every expert of a launch, K <= 4096, g in {64, 128}.
bool moe_stream_fits(int K, int gps);
void launch_moe_stream(const GemmArgs& a, int mt, int gps, bool asym, int slots, hipStream_t s);

}  // namespace w4a8
