// Grouped (MoE) W4A8 GEMM for the experts with many rows (>= 96): 128 x 128 tiles of 16x16x64
// INT8 MFMAs, weights straight from the blob into registers.
//
// Sources (cited with the page's own section names):
//   P1 "Kimi 2.7 MoE: from 4-bit storage to INT8 (W4A8)" (pwwt.cn), section 4.4 step 4: the grouped
//      expert GEMM over router-sorted tokens; section 5.2: the 4-bit layout matches the MFMA operand
//      layout, so the nibbles unpack in registers; section 8: the activation quantization folded
//      into the GEMM (the paired gate/up epilogue below).
//   P5 "Inference quantization, chapter 1: the Linear layer" (sgdbs.github.io), section 4: integer
//      GEMM, then the scales in a float epilogue; sections 8.3 and 8.4: per-token activation scales
//      times per-group weight scales.
//
// Workgroup (slot, column tile): slot is a 128-row tile of one expert (moe_tile; each expert with
// rows_e in [moe_lo, moe_hi) has ceil(rows_e / 128) of them), rows gathered from the token rows when
// `gather` is set; output row r is the r-th sorted row.  512 threads, 8 waves: wave (wm, wn) computes
// tile rows [64 wm, +64) and the 16-column tiles 2 wn, 2 wn + 1 of the workgroup's 8.  Per 128-deep
// superblock:
//   - the activation rows [128 x 128] are staged in LDS (double buffered, rows padded by 32 bytes so
//     a 16x16x64 operand read touches distinct banks); every thread loads 2 pieces of 16 bytes for
//     the next superblock while the current one is computed;
//   - each lane loads the 16 bytes of the blob that are its B operand for both 64-deep halves of
//     each of its 2 column tiles (the blob layout is the 16x16x64 operand layout) and unpacks them
//     in registers: no LDS traffic for the weights.  The next superblock's codes and zero points are
//     requested as soon as the current ones are unpacked (half a superblock ahead), its scales a
//     superblock ahead;
//   - 4 row blocks x 2 column tiles x 2 halves = 16 MFMAs per wave; after each group the int32
//     sums are scaled into the float32 accumulators (acc = fma(float(P_g), s_g, acc)).
// At 40 KiB of LDS and <= 128 registers per lane, two workgroups share a compute unit: four waves
// per SIMD to hide the load and LDS latencies.
//
// Why not the dense prefill kernel's 256 x 128 tiles: an expert's last tile is partly empty, and
// 128-row tiles waste fewer of its MFMA rows; with 64 x 32 per wave the accumulators leave the
// registers for two resident workgroups at g = 64 as well as g = 128.
//
// Paired form (a.Hq set, gate/up blob): the workgroup's tiles 0-3 are gate tiles and 4-7 the
// matching up tiles, so gate wave wn (0, 1) and up wave wn + 2 hold the two outputs of the same h
// columns in the same lanes and registers; the epilogue writes SiLU-requant codes instead of Y.
#include <hip/hip_runtime.h>

#include "w4a8_device.h"
#include "w4a8_internal.h"

namespace w4a8 {

constexpr int MTL_BM = 128, MTL_THREADS = 512;
constexpr int MTL_ROWB = SB_K + 32;                     // padded activation row (bytes)
constexpr int MTL_STAGE = MTL_BM * MTL_ROWB;            // 20 KiB
constexpr int MTL_LDS = 2 * MTL_STAGE;

// GPS: groups per superblock, 2 (g = 64) or 1 (g = 128).  H16: binary16 group scales.
// One workgroup's 128-row tile tr of one expert, whose blob is `blob` (the format is the template's).
template <int GPS, bool ASYM, bool H16>
__device__ __forceinline__ void moe_tile_body(const GemmArgs& a, const TileRows tr, const uint8_t* blob) {
    static_assert(GPS == 1 || GPS == 2, "grouped formats: g in {64, 128}");
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;
    const int ntl16 = (a.N + 15) / 16;
    const int ntiles = (ntl16 + 7) / 8;
    const int nt = blockIdx.x % ntiles;
    const int m0 = tr.rbeg, mend = tr.rend, expert = tr.expert;
    const int nsb = a.K / SB_K;
    const uint8_t* codes = blob + a.codes_off;
    const float* scales = reinterpret_cast<const float*>(blob + a.scales_off);
    const uint16_t* scales16 = reinterpret_cast<const uint16_t*>(blob + a.scales_off);
    const uint8_t* zeros = blob + a.zeros_off;
    // blob tile of the workgroup's l-th 16-column tile (paired form: 4 gate tiles, then their up tiles)
    auto tile_l = [&](int l) { return pair_tile(a, nt * 8, l, 8); };
    // source activation row of tile row r (rows past the tile repeat its last row); -1 for a
    // gathered row that names no activation row (it loads row 0 and gets a zero scale)
    auto src_row = [&](int r) {
        const int rr = min(m0 + r, mend - 1);
        return a.gather ? gather_src(a, rr) : rr;
    };

    // this wave's two column tiles (clamped to the last one; their outputs are not stored)
    uint32_t boff[2], moff[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const uint32_t tl = uint32_t(min(tile_l(wn * 2 + c), ntl16 - 1));
        boff[c] = tl * uint32_t(nsb) * 1024u + uint32_t(lane) * 16u;
        moff[c] = tl * uint32_t(a.G) * 16u + uint32_t(lane & 15);
    }
    // activation pieces: piece p (of 1024) is row p / 8, bytes [16 (p % 8), +16) of the superblock;
    // thread t stages pieces t and t + 512 (rows past the tile's end repeat its last row; never stored)
    const int8_t* xrow[2];
    int lofs[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int p = tid + i * MTL_THREADS, row = p >> 3, c = p & 7;
        xrow[i] = a.Xq + size_t(max(src_row(row), 0)) * a.K + c * 16;
        lofs[i] = row * MTL_ROWB + c * 16;
    }
    // row scale of tile row 64 wm + lane, shared by cross-lane reads in the epilogue
    float sxl = 0.0f;
    {
        const int sr = m0 + wm * 64 + lane < mend ? src_row(wm * 64 + lane) : -1;
        if (sr >= 0) sxl = a.sx[sr];
    }

    auto load_a = [&](uint4 (&xv)[2], int sb) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 2; ++i) xv[i] = *reinterpret_cast<const uint4*>(xrow[i] + size_t(sb) * SB_K);
    };
    auto store_a = [&](const uint4 (&xv)[2], int stage) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 2; ++i) *reinterpret_cast<uint4*>(smem + stage * MTL_STAGE + lofs[i]) = xv[i];
    };
    // weight registers: codes and zero points of the superblock being computed (b0, z0), requested
    // for the next superblock as soon as the current ones are unpacked; group scales of the current
    // superblock (s0) and of the next one (s1), binary16 ones as their bits (converted at use)
    uint4 b0[2];
    float s0[2][GPS], s1[2][GPS];
    uint32_t z0[2];                                      // zero points, one byte per group
    auto load_codes = [&](int sb) __attribute__((always_inline)) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            b0[c] = *reinterpret_cast<const uint4*>(codes + (boff[c] + uint32_t(sb) * 1024u));
#pragma unroll
            for (int gi = 0; gi < GPS; ++gi) {
                const uint32_t z = ASYM ? uint32_t(zeros[moff[c] + (uint32_t(sb) * GPS + gi) * 16u]) : 0u;
                z0[c] = gi ? z0[c] | (z << (8 * gi)) : z;
            }
        }
    };
    auto load_scales = [&](float (&sv)[2][GPS], int sb) __attribute__((always_inline)) {
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int gi = 0; gi < GPS; ++gi) {
                const uint32_t mi = moff[c] + (uint32_t(sb) * GPS + gi) * 16u;
                sv[c][gi] = H16 ? __uint_as_float(uint32_t(scales16[mi])) : scales[mi];
            }
    };

    float accf[4][2][4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) accf[r][c][i] = 0.0f;
    const v4i zero4 = {0, 0, 0, 0};

    auto compute = [&](int stage, int nx) __attribute__((always_inline)) {
        const uint8_t* st = smem + stage * MTL_STAGE + (wm * 64 + (lane & 15)) * MTL_ROWB + 16 * (lane >> 4);
        v4i acc[4][2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int gi = GPS == 2 ? h : 0;
            v4i b[2];
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const uint32_t zc = ASYM ? (128u - ((z0[c] >> (8 * gi)) & 0xffu)) * 0x01010101u : 0u;
                b[c] = unpack_b<ASYM>(h ? b0[c].z : b0[c].x, h ? b0[c].w : b0[c].y, zc);
            }
            if (h == 1) load_codes(nx);                  // this superblock's codes are unpacked
            const bool first = GPS == 2 || h == 0;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint4 av = *reinterpret_cast<const uint4*>(st + r * 16 * MTL_ROWB + h * 64);
                const v4i A = v4i{int(av.x), int(av.y), int(av.z), int(av.w)};
#pragma unroll
                for (int c = 0; c < 2; ++c)
                    acc[r][c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, b[c], first ? zero4 : acc[r][c], 0, 0, 0);
            }
            if (GPS == 2 || h == 1) {
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    const float sg = H16 ? f16_to_f32(uint16_t(__float_as_uint(s0[c][gi]))) : s0[c][gi];
                    const float scl = ASYM ? sg : sg * 0.0625f;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
#pragma unroll
                        for (int i = 0; i < 4; ++i) accf[r][c][i] = fmaf(float(acc[r][c][i]), scl, accf[r][c][i]);
                }
            }
        }
    };

    // One superblock ahead through registers, two LDS stages.  Straight-line loop (every
    // iteration loads, clamped at the end, and stores to the stage not being read), so each wait
    // names exactly the registers it needs.
    uint4 xv[2];
    load_a(xv, 0);
    load_codes(0);
    load_scales(s0, 0);
    store_a(xv, 0);
    __syncthreads();
    for (int sb = 0; sb < nsb; ++sb) {
        const int nx = min(sb + 1, nsb - 1);
        load_a(xv, nx);
        load_scales(s1, nx);
        compute(sb & 1, nx);
        store_a(xv, (sb & 1) ^ 1);                       // that stage was last read before the barrier below
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int gi = 0; gi < GPS; ++gi) s0[c][gi] = s1[c][gi];
        lds_barrier();                                   // LDS hand-off only: global loads may stay in flight
    }

    if (a.Hq) {
        // paired form: gate wave wn (0, 1) and up wave wn + 2 hold the two outputs of the same h
        // columns in the same lanes and registers.  Each hands one of its column tiles to the
        // other through LDS (free after the K loop): the gate wave forms the codes of its tile
        // c = 0, the up wave those of c = 1.
        float* pb = reinterpret_cast<float*>(smem);      // [to gate, to up][pair][wm][r][i][64]
        const bool gate = wn < 2;
        const int pair = gate ? wn : wn - 2;
        const int own = gate ? 0 : 1;                    // column tile whose codes this wave forms
        const RowScale prs = static_row_scale(a.s_dn[expert]);
        float y[4][4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float sxv = __shfl(sxl, r * 16 + 4 * (lane >> 4) + i, 64);
                y[r][i] = accf[r][own][i] * sxv;
                pb[((((gate ? 1 : 0) * 2 + pair) * 2 + wm) * 16 + r * 4 + i) * 64 + lane] = accf[r][1 - own][i] * sxv;
            }
        __syncthreads();
        const int hc = (nt * 4 + pair * 2 + own) * 16 + (lane & 15);   // column of h
        if (hc < a.pair_n) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = m0 + wm * 64 + r * 16 + 4 * (lane >> 4) + i;
                    if (row >= mend) continue;
                    const float v = pb[((((gate ? 0 : 1) * 2 + pair) * 2 + wm) * 16 + r * 4 + i) * 64 + lane];
                    const float yg = gate ? y[r][i] : v, yu = gate ? v : y[r][i];
                    a.Hq[size_t(row) * a.pair_n + hc] = int8_t(silu_static_code(yg, yu, prs));
                }
        }
        if (nt == 0 && tid < mend - m0) a.sh[m0 + tid] = prs.s;
        return;
    }

#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int tile = tile_l(wn * 2 + c);
        const int col = tile * 16 + (lane & 15);
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rl = r * 16 + 4 * (lane >> 4) + i;                // row inside the wave's 64
                const float sxv = __shfl(sxl, rl, 64);
                const int row = m0 + wm * 64 + rl;
                if (tile >= ntl16 || col >= a.N || row >= mend) continue;
                const float y = accf[r][c][i] * sxv;
                const size_t yi = size_t(row) * a.ldy + col;
                if (a.out_f32)
                    reinterpret_cast<float*>(a.Y)[yi] = y;
                else
                    reinterpret_cast<uint16_t*>(a.Y)[yi] = uint16_t(f32_to_bf16_rne(y));
            }
    }
}

template <int GPS, bool ASYM, bool H16>
__global__ __launch_bounds__(MTL_THREADS, 4) void gemm_moe_tile_kernel(GemmArgs a) {
    const int ntiles = ((a.N + 15) / 16 + 7) / 8;
    const TileRows tr = moe_tile<MTL_BM>(a, int(blockIdx.x) / ntiles, int(threadIdx.x) & 63);
    if (tr.expert < 0) return;                           // uniform over the workgroup
    moe_tile_body<GPS, ASYM, H16>(a, tr, a.blob + size_t(tr.expert) * a.expert_stride);
}

// Format classes in one launch: the workgroup resolves its expert's class, then runs the code of
// that class's format (every branch is uniform over the workgroup; only one is taken).
__global__ __launch_bounds__(MTL_THREADS, 4) void gemm_moe_tile_classes_kernel(GemmArgs a, MoeClasses mc) {
    const int ntiles = ((a.N + 15) / 16 + 7) / 8;
    const TileRows tr = moe_tile<MTL_BM>(a, int(blockIdx.x) / ntiles, int(threadIdx.x) & 63);
    if (tr.expert < 0) return;
    const uint8_t* blob;
    const int fmt = __builtin_amdgcn_readfirstlane(moe_class_resolve(mc, __builtin_amdgcn_readfirstlane(tr.expert), a, blob));
#define W4A8_MTC(F_, GPS_, ASYM_, H16_) \
    case F_: moe_tile_body<GPS_, ASYM_, H16_>(a, tr, blob); break;
    switch (fmt) {
        W4A8_MTC(0, 1, false, false)
        W4A8_MTC(1, 2, false, false)
        W4A8_MTC(2, 1, true, false)
        W4A8_MTC(3, 2, true, false)
        W4A8_MTC(4, 1, false, true)
        W4A8_MTC(5, 2, false, true)
        W4A8_MTC(6, 1, true, true)
        W4A8_MTC(7, 2, true, true)
        default: break;
    }
#undef W4A8_MTC
}

void launch_moe_tile_classes(const GemmArgs& a, const MoeClasses& mc, int slots, hipStream_t s) {
    const int ntiles = ((a.N + 15) / 16 + 7) / 8;
    gemm_moe_tile_classes_kernel<<<dim3(slots * ntiles), dim3(MTL_THREADS), MTL_LDS, s>>>(a, mc);
}

template <int GPS, bool ASYM, bool H16>
static void launch_moe_tile_t(const GemmArgs& a, int slots, hipStream_t s) {
    const int ntiles = ((a.N + 15) / 16 + 7) / 8;
    gemm_moe_tile_kernel<GPS, ASYM, H16><<<dim3(slots * ntiles), dim3(MTL_THREADS), MTL_LDS, s>>>(a);
}

void launch_moe_tile(const GemmArgs& a, int gps, bool asym, int slots, hipStream_t s) {
#define W4A8_MTL(GPS_, ASYM_)                                                 \
    do {                                                                      \
        if (a.h16) launch_moe_tile_t<GPS_, ASYM_, true>(a, slots, s);         \
        else launch_moe_tile_t<GPS_, ASYM_, false>(a, slots, s);              \
    } while (0)
    if (gps == 1) { if (asym) W4A8_MTL(1, true); else W4A8_MTL(1, false); }
    else { if (asym) W4A8_MTL(2, true); else W4A8_MTL(2, false); }
#undef W4A8_MTL
}

}  // namespace w4a8
