/*
 * w4a8.h -- C ABI of the MI355X (gfx950) W4A8 linear / MoE-expert library.
 *
 * W4A8: weights stored as 4-bit integers in groups along K with one float32
 * scale (and, in asymmetric mode, one integer zero point) per group and output
 * column; activations quantized per token to INT8 at run time; an INT8 x INT8
 * -> INT32 GEMM whose weight nibbles are unpacked inside the kernel, with the
 * weight and activation scales applied in a float32 epilogue.
 *
 * Sources (cited as P1..P5 with the page's own section names):
 *   P1 "Kimi 2.7 MoE: from 4-bit storage to INT8 (W4A8)"                (pwwt.cn)
 *   P2 "Kimi 2.7 MoE W4A8: 4-bit storage to INT8, deployment notes"     (xdnf.cn)
 *   P3 "Quantization: formats, error and the real execution path"       (wineandchord.com)
 *   P4 "Choosing a weight-quantization scheme and locating kernel hits" (xbrilliance.ai)
 *   P5 "Inference quantization, chapter 1: the Linear layer"            (sgdbs.github.io)
 *
 * Conventions for every entry point
 *   - Matrices are row-major.  X is [M, K], W is [K, N], Y is [M, N] (P5 section 1:
 *     M = batch * seq_len, K = hidden, N = out features).
 *   - The caller owns every buffer, host and device.  GPU entry points only
 *     enqueue work on `stream` (a hipStream_t, NULL = the null stream) and never
 *     allocate device memory, free or synchronize (w4a8_moe_forward_sets creates
 *     helper streams and events once per device; see there).  Device pointers must
 *     stay valid until the enqueued work completes.
 *   - Return value: W4A8_OK (0) or a negative w4a8_status.  All argument checks
 *     run on the host before anything is enqueued, so an error return means
 *     nothing was launched.  W4A8_EHIP reports a launch failure seen right after
 *     enqueueing.  There is no fallback path: a shape or format the kernels do
 *     not implement returns W4A8_EUNSUPPORTED (P3 "Correctness contract" item 6
 *     and P4: a fallback must be explicit and observable).
 *   - Device buffers read with 128-bit loads (Xq, Hq, blobs) must be 16-byte
 *     aligned; the library checks this and returns W4A8_EINVAL otherwise.
 *   - Calls are thread-safe.  The only state the library keeps is created once per
 *     device and kept until the process ends: the helper streams of
 *     w4a8_moe_forward_sets and the scratch array of w4a8_moe_forward_noalloc.
 *   - Environment: W4A8_LOG set to anything but "0" makes every GEMM and MoE entry
 *     point print one line to stderr before it launches: the call, its shape and the
 *     kernel variant it resolved to (P4: a kernel hit must be observable).
 */
#ifndef W4A8_H
#define W4A8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    W4A8_OK = 0,
    W4A8_EINVAL = -1,        /* bad argument: null pointer, bad shape, group not tiling K, ... */
    W4A8_ESIZE = -2,         /* a caller-provided buffer is smaller than required             */
    W4A8_EUNSUPPORTED = -3,  /* valid request the kernels do not implement (no fallback)       */
    W4A8_EHIP = -4           /* the HIP runtime reported an error when launching               */
} w4a8_status;

typedef enum { W4A8_OUT_BF16 = 0, W4A8_OUT_F32 = 1 } w4a8_out_dtype;

/* Weight format description (P3 "Four independent dimensions": object, format,
 * granularity, execution types must each be stated).
 *   K, N        weight matrix W[K, N]
 *   group_size  g: consecutive k sharing one scale per column (P5 section 8.4);
 *               must divide K.  pack accepts g in {32, 64, 128, 256} and g = K (one
 *               scale, and zero point, per output column: the per-channel granularity
 *               of P5 section 8.3).  Kernels implement all of them; 32, 256 and K run on
 *               the dense GEMMs only (the MoE entry points return EUNSUPPORTED), and
 *               g = K needs g * 127 * m < 2^31, the reach of the int32 group sum, where
 *               m is the largest weight operand the kernels feed: 15 (asymmetric), 112
 *               (symmetric 4-bit codes enter as 16 q) or 127 (8-bit codes); so K <= 150912
 *               for symmetric 4-bit per-channel weights; otherwise EUNSUPPORTED.  The GPU entry points also return
 *               EUNSUPPORTED for a blob whose codes reach 2 GiB (32-bit offsets).
 *   asymmetric  0: signed codes q in [-7, 7], zero point 0 (P3 "Basic mapping",
 *                  symmetric form);
 *               1: unsigned codes q in [0, 15] with a uint8 zero point z per
 *                  group, w ~ s (q - z) (P3 "Basic mapping"; P5 section 6).
 *   weight_bits 4 (or 0): the INT4 codes above, two per byte;
 *               8: the W8A8 sibling the pages compare against (P1 section 5): signed
 *                  codes q in [-127, 127], one per byte, symmetric only (qmax of the
 *                  P3 symmetric group-wise reference with bits = 8).  Dense GEMMs
 *                  only: the MoE entry points return EUNSUPPORTED for it.
 *   scale_bits  32 (or 0): float32 group scales;
 *               16: binary16 group scales, the storage P1 section 4.1 names for expert
 *                  weights.  The packer rounds each float32 scale to the nearest binary16
 *                  (ties to even) and computes the codes with the rounded scale, so
 *                  dequantization uses exactly the stored value; a scale past the binary16
 *                  range (65504) makes w4a8_pack return EINVAL.  Kernels take binary16
 *                  scales with 4-bit codes and g in {64, 128} (dense and MoE); other
 *                  combinations return EUNSUPPORTED. */
typedef struct {
    int32_t K;
    int32_t N;
    int32_t group_size;
    int32_t asymmetric;
    int32_t weight_bits;
    int32_t scale_bits;
} w4a8_wdesc;

/* ------------------------------------------------------------------------------------
 * Packed weight blob ("the checkpoint"): header + codes + scales [+ zeros].
 * P3 "Calibration and conversion" asks the converted artifact to record format,
 * signedness, packing, scale axis and group size; the header does.
 *
 *   offset 0    header, W4A8_HEADER_BYTES bytes, little endian:
 *               char magic[8] = "W4A8BLB1"; uint32 version = 1; uint32 layout = 1;
 *               int32 K, N, group_size, asymmetric; uint32 scale_dtype (0 float32,
 *               1 binary16);
 *               uint32 zero_dtype = 0 (uint8); uint64 codes_off, codes_bytes,
 *               scales_off, scales_bytes, zeros_off, zeros_bytes, total_bytes;
 *               uint32 weight_bits (4 or 8; 0 in older headers reads as 4);
 *               the rest is zero.
 *   codes       Np = N rounded up to 16 (padding columns hold code 0, scale 0).
 *               Superblock = 16 columns x 128 rows = 1024 bytes, stored as 64
 *               lanes x 16 bytes; superblocks run over k first, then over the
 *               column tile:  superblock index = (n / 16) * (K / 128) + k / 128.
 *               Inside a superblock, for kk = k % 128 and c = n % 16:
 *                 half = kk / 64, r = kk % 64, lane = (r / 16) * 16 + c, j = r % 16,
 *                 byte = lane * 16 + half * 8 + (j / 8) * 4 + (j % 4),
 *                 nibble = (j % 8) / 4   (0 = low 4 bits, 1 = high 4 bits).
 *               So one 128-bit load per lane fetches 16 k of one column for two
 *               64-deep MFMA steps, and the low/high nibbles of a 32-bit word are
 *               the k and k+4 operands of the same byte position (P1 section 5.1:
 *               tile format matched to the MFMA operand; P1 section 7, third pitfall).
 *               Symmetric codes are stored as 4-bit two's complement; asymmetric
 *               codes as unsigned 0..15.  Two codes per byte (P1 section 5.2).
 *               8-bit codes (weight_bits = 8): superblock = 2048 bytes, 64 lanes x 32
 *               bytes, one int8 code per byte at lane * 32 + half * 16 + j (lane, half
 *               and j as above): the values the 4-bit form unpacks, in the same order.
 *   scales      float32 [Np/16][K/g][16]: scale of (group i, column n) at
 *               ((n/16) * (K/g) + i) * 16 + n % 16.
 *   zeros       (asymmetric only) uint8, same index as scales.
 *   Every section starts on a 256-byte boundary.
 * ------------------------------------------------------------------------------------ */
#define W4A8_HEADER_BYTES 256

/* Bytes of the blob for `d` (header + codes + scales + zeros + alignment padding), the
 * M = N b/8 + N_groups M_meta + M_pad term of P3 "Basic mapping" with the padding
 * explicit.  Returns 0 if `d` is invalid. */
size_t w4a8_packed_size(const w4a8_wdesc* d);

/* Offline RTN quantization + packing on the host (P3 "Basic mapping"; P3 symmetric
 * group-wise reference; P2 section 2.1).  W_host: float32 [K, N] row-major, finite.
 * Per (group, column): symmetric s = fl32(max|w| / 7), q = clamp(rint(fl32(w / s)), -7, 7)
 * (8-bit codes: 127 in place of 7);
 * asymmetric lo = min(0, min w), hi = max(0, max w), s = fl32(fl32(hi - lo) / 15),
 * z = clamp(rint(fl32(-lo / s)), 0, 15), q = clamp(rint(fl32(w / s)) + z, 0, 15); an
 * all-zero group gets s = 0, z = 0, q = 0.  Round half to even, IEEE float32 division.
 * Writes w4a8_packed_size(d) bytes to blob_host.  EINVAL: bad desc, group not tiling K,
 * non-finite weight; ESIZE: blob_bytes too small. */
int w4a8_pack(const w4a8_wdesc* d, const float* W_host, void* blob_host, size_t blob_bytes);

/* Pack externally produced codes (e.g. from GPTQ/AWQ, P2 section 3.2) without
 * re-quantizing.  codes: int8 [K, N] in [-7, 7] (symmetric), [0, 15] (asymmetric) or
 * [-127, 127] (8-bit);
 * scales: float32 [K/g, N]; zeros: uint8 [K/g, N] in [0, 15] (asymmetric) or NULL.
 * EINVAL on out-of-range codes or zero points. */
int w4a8_pack_codes(const w4a8_wdesc* d, const int8_t* codes, const float* scales,
                    const uint8_t* zeros, void* blob_host, size_t blob_bytes);

/* Inverse of the packing, on the host: checks the header and writes codes [K, N],
 * scales [K/g, N] and (asymmetric) zeros [K/g, N]; d_out receives the header's desc.
 * Any output pointer may be NULL to skip it.  EINVAL on a bad header. */
int w4a8_unpack_codes(const void* blob_host, size_t blob_bytes, w4a8_wdesc* d_out,
                      int8_t* codes, float* scales, uint8_t* zeros);

/* Host check that blob_host's header describes `d` and fits in blob_bytes; to be run
 * once when a blob is loaded (GPU entry points trust the desc they are given). */
int w4a8_blob_check(const void* blob_host, size_t blob_bytes, const w4a8_wdesc* d);

/* ------------------------------------------------------------------------------------
 * GPU entry points
 * ------------------------------------------------------------------------------------ */

/* Per-token dynamic INT8 activation quantization (P1 section 3.3; P5 section 8.3;
 * P2 section 3.3: a quantize node before each Linear).
 *   X_bf16  device, bfloat16 [M, K] with row stride ldx >= K elements
 *   Xq      device, int8 [M, K] dense (row stride K), 16-byte aligned, K % 16 == 0
 *   sx      device, float32 [M]
 * Per row: amax = max|x|; s = fl32(amax / 127); q = clamp(rint(fl32(x / s)), -127, 127)
 * (divisor 1 when s == 0).  A row containing NaN or Inf gets s = NaN and q = 0.
 * M == 0 is a no-op. */
int w4a8_quant_act(const void* X_bf16, int M, int K, int ldx, int8_t* Xq, float* sx,
                   void* stream);

/* The same quantization of X diag(alpha)^-1, the activation side of the equivalent
 * per-channel rescaling Y = (X diag(alpha)^-1) (diag(alpha) W) of P3 "Weight-Activation"
 * (SmoothQuant: quantization difficulty moved from activations to weights offline).  The
 * page asks for the scaling to be fused into an adjacent operator; here it is: each
 * x[m, k] is multiplied by inv_alpha[k] (one float32 product, round to nearest even) and
 * the per-token rule above applies to the products.  The weight side, diag(alpha) W, is
 * applied before packing by the caller.
 *   inv_alpha  device float32 [K], 16-byte aligned (1 / alpha per input channel)
 * Other arguments, layouts and errors as w4a8_quant_act; EINVAL if inv_alpha is NULL. */
int w4a8_quant_act_smooth(const void* X_bf16, int M, int K, int ldx, const float* inv_alpha, int8_t* Xq,
                          float* sx, void* stream);

/* Static (calibrated) activation quantization (P1 section 3.2: a scale measured on a
 * calibration set ahead of time replaces the per-batch reduction; the page recommends it for
 * decode).  Every row uses the one given scale:
 *   s       device float32 [1] (a device value, so a captured graph can be recalibrated)
 *   Xq, sx  as w4a8_quant_act; sx[m] = s for every row
 * q = clamp(rint(fl32(x / s)), -127, 127): values beyond the calibrated range saturate at
 * +-127, NaN gives 0, +-Inf gives +-127.  A scale that is not finite and positive gives
 * all-zero codes.  No limit on K besides K % 16 == 0 (one pass, nothing held per row).
 * M == 0 is a no-op; EINVAL for NULL pointers, K % 16, ldx % 8 or misaligned X / Xq. */
int w4a8_quant_act_static(const void* X_bf16, int M, int K, int ldx, const float* s, int8_t* Xq,
                          float* sx, void* stream);

/* Static per-expert quantization of the routed rows (P1 section 3.1: one activation scale
 * per expert; section 3.2: static scales).  Row r of the expert-sorted order (from
 * w4a8_moe_align) quantizes token sorted_rows[r] / k of X with the scale s[e] of the
 * expert e that owns row r (expert_offsets[e] <= r < expert_offsets[e + 1]), by the rule of
 * w4a8_quant_act_static.
 *   X_bf16          device bfloat16 [T, H], row stride ldx
 *   sorted_rows     device int32 [T*k]; expert_offsets device int32 [E+1]; s device float32 [E]
 *   Xq, sx          device int8 [T*k, H] (16-byte aligned), float32 [T*k], sorted order
 * Rows at or past expert_offsets[E] (routing ids outside [0, E)) get zero codes and scale 0.
 * E <= 1024 (EINVAL), T*k <= 2^24 (EUNSUPPORTED). */
int w4a8_moe_quant_static(const void* X_bf16, int T, int H, int ldx, const int32_t* sorted_rows,
                          int k, const int32_t* expert_offsets, int E, const float* s, int8_t* Xq,
                          float* sx, void* stream);

/* W4A8 GEMM Y = (s_x * Xq) (s_w * (q - z)) (P5 section 4 ideal path; P5 section 8.3
 * epilogue Y[i, j] = s_x[i] s_w[j] acc[i, j], applied per K-group of P5 section 8.4).
 *   Xq, sx    device, from w4a8_quant_act ([M, K] int8 dense, [M] float32)
 *   blob_dev  device copy of a blob packed for `d` (K % 128 == 0 required)
 *   Y         device, [M, N] with row stride ldy >= N, bfloat16 or float32 (out_dtype)
 * The INT4 nibbles are unpacked in registers into INT8 MFMA operands; each group's INT32
 * partial sum is scaled by its float32 weight scale into a float32 accumulator, the
 * row scale is applied last, then the bfloat16 cast rounds to nearest even.  No
 * dequantized weight is ever written to memory (P1 section 4.4 step 4; P5 section 3.2).
 * M == 0 is a no-op.  EINVAL for M > 32 with 256 * K >= 2^31 (the 256-row activation tile
 * is addressed with 32-bit offsets). */
int w4a8_gemm(const int8_t* Xq, const float* sx, int M, const void* blob_dev,
              const w4a8_wdesc* d, void* Y, int ldy, int out_dtype, void* stream);

/* Per-token quantization and W4A8 GEMM in one call: Y = GEMM(quant_act(X)).
 *   X_bf16   device bfloat16 [M, K], row stride ldx >= K (ldx % 8 == 0, 16-byte aligned)
 *   Xq, sx   device int8 [M, K] (16-byte aligned) and float32 [M]: always written with the
 *            activation codes and scales (the caller can reuse them)
 *   Y, ldy, out_dtype, blob_dev, d as in w4a8_gemm.
 * For M <= 16 and M * K <= 8192 (M <= 2 at K = 4096) this is one kernel: each
 * workgroup of the decode GEMM quantizes the activation rows itself into its staged
 * activation tile (P2 section 3.3 places the per-token quantization node right before
 * the GEMM; P1 section 8 suggests fusing quantization into the GEMM kernel); otherwise
 * it is w4a8_quant_act followed by w4a8_gemm.  Results are bit-identical either way. */
int w4a8_linear(const void* X_bf16, int M, int K, int ldx, const void* blob_dev, const w4a8_wdesc* d, void* Y,
                int ldy, int out_dtype, int8_t* Xq, float* sx, void* stream);

/* W4A16 sibling (P1 section 5.3 compares W4A16 with W8A8 and W4A8; P5 section 3.2: the
 * weight-only path dequantizes inside the GEMM): Y = X W with the activations kept in bfloat16
 * (no activation quantization) and the 4-bit codes of a W4A8 blob dequantized in registers,
 *   Y[m, n] = sum_i s[i, n] * sum_{k in group i} X[m, k] * (q[k, n] - z[i, n]),
 * accumulated in float32 on bfloat16 MFMA.
 *   X_bf16   device bfloat16 [M, ldx], 16-byte aligned, ldx % 8 == 0, ldx >= K
 *   blob_dev the same blob as w4a8_gemm: 4-bit codes, g in {64, 128}, float32 scales
 *            (other formats: EUNSUPPORTED)
 *   Y        device [M, ldy] bfloat16 or float32
 * M <= 32 runs the streaming (decode) kernel, larger M the 128 x 128-tile kernel; M == 0 is a
 * no-op.  EINVAL for M > 32 when 128 * ldx * 2 reaches 2^31 (32-bit activation offsets). */
int w4a16_gemm(const void* X_bf16, int M, int ldx, const void* blob_dev, const w4a8_wdesc* d, void* Y,
               int ldy, int out_dtype, void* stream);

/* Name of the kernel variant w4a16_gemm resolves to for (d, M), or "unsupported". */
const char* w4a16_kernel_name(const w4a8_wdesc* d, int M);

/* Test export of the same main loop: INT32 per-group partial sums
 * P[m, n, i] = sum_{k in group i} Xq[m, k] (q[k, n] - z[i, n]) written to device
 * int32 [M, N, K/g].  (P3 "Correctness contract" item 3: the accumulator covers the
 * reduction: |P| <= g * 127 * 15, or g * 127 * 127 with 8-bit codes, < 2^31; symmetric
 * 4-bit sums are formed as 16 P, |16 P| <= g * 127 * 112 < 2^31.)  Same
 * EINVAL size limit as w4a8_gemm.  With g = K and M <= 32 (the decode kernels, which split
 * K across waves) it returns EUNSUPPORTED. */
int w4a8_gemm_partials(const int8_t* Xq, int M, const void* blob_dev, const w4a8_wdesc* d,
                       int32_t* P, void* stream);

/* MoE dispatch by expert (P1 section 4.4, steps 2-3).
 *   topk_ids       device int32 [T, k], each in [0, E)
 *   sorted_rows    device int32 [T*k]: routed rows r = t*k + j grouped by expert,
 *                  ascending r inside an expert (stable counting sort)
 *   expert_offsets device int32 [E+1]: exclusive prefix sum of rows per expert
 *   inv            device int32 [T, k]: position of row t*k + j in sorted_rows
 * Ids outside [0, E) are counted nowhere and their inv entry is -1; the host cannot see
 * device ids, so callers validate routing upstream.  E <= 1024, T*k <= 2^24. */
int w4a8_moe_align(const int32_t* topk_ids, int T, int k, int E, int32_t* sorted_rows,
                   int32_t* expert_offsets, int32_t* inv, void* stream);

/* Expert-grouped W4A8 GEMM (P1 section 4.4 step 4, "the performance key").
 *   Xq, sx         device activations [src_rows, K] and [src_rows]; if `gather` is non-NULL,
 *                  output row r (in sorted order) reads Xq/sx row gather[r] / k (token of
 *                  the routed row); if NULL, row r reads row r (rows already permuted)
 *   gather         device int32 [rows] or NULL (pass sorted_rows from w4a8_moe_align)
 *   k              top-k (divisor for gather; ignored when gather is NULL)
 *   expert_offsets device int32 [E+1]; rows [off[e], off[e+1]) use expert e
 *   rows           T*k, total rows (= off[E]); rows of Y
 *   src_rows       rows of Xq and sx: T with a gather, >= rows without one (EINVAL otherwise)
 *   blobs_dev      device, E blobs of desc `d`, expert e at blobs_dev + e * expert_stride
 *   Y              device [rows, N] bfloat16 or float32, dense
 * The kernels bound what the device arrays may name: a gather entry that is negative or
 * names a token at or past src_rows reads no activations and gives an output row of zeros,
 * and expert row ranges are clamped to [0, rows).  Experts with no rows read no weights.
 * All experts of a call share one allocation at a fixed stride: the kernels find an expert's
 * weights by one multiply of ids they already hold, with no further dependent load in front of
 * the weight stream. */
int w4a8_moe_gemm(const int8_t* Xq, const float* sx, const int32_t* gather, int k,
                  const int32_t* expert_offsets, int E, int rows, int src_rows, const void* blobs_dev,
                  size_t expert_stride, const w4a8_wdesc* d, void* Y, int out_dtype,
                  void* stream);

/* Expert-grouped gate/up GEMM with the static SiLU-requant folded into its epilogue (P1
 * section 8: fold the activation quantization into the GEMM; P1 section 3.2: static, calibrated
 * activation scales, so the requantization needs no reduction over a row).  The blob holds the
 * gate columns [0, I) and the up columns [I, 2I) of each expert (d->N = 2I, I % 16 == 0,
 * EINVAL otherwise).  A workgroup computes gate column c and up column I + c side by side; each
 * output is rounded to bfloat16 as w4a8_moe_gemm stores it, h = silu(g) * u is formed in float32
 * and quantized with the scale s[e] of the row's expert (the rule of w4a8_quant_act_static),
 * so Hq and sh equal those of w4a8_moe_gemm followed by w4a8_silu_mul_quant_static, bit for
 * bit, without the [rows, 2I] bfloat16 intermediate.
 *   Xq, sx, gather, k, expert_offsets, E, rows, src_rows, blobs_dev, expert_stride, d
 *                  as for w4a8_moe_gemm
 *   s              device float32 [E], static scales of h
 *   Hq, sh         device int8 [rows, I], float32 [rows]
 * Rows at or past expert_offsets[E] (no expert owns them) are not written.  Same checks and
 * limits as w4a8_moe_gemm. */
int w4a8_moe_gemm_silu_static(const int8_t* Xq, const float* sx, const int32_t* gather, int k,
                              const int32_t* expert_offsets, int E, int rows, int src_rows,
                              const void* blobs_dev, size_t expert_stride, const w4a8_wdesc* d,
                              const float* s, int8_t* Hq, float* sh, void* stream);

/* SiLU-gated expert activation + per-row INT8 requantization for the down projection
 * (P1 section 1 names SiLU; P1 section 3.1: per-expert activation scales).
 *   GU_bf16  device bfloat16 [R, 2I]: gate = columns [0, I), up = [I, 2I)
 *   Hq, sh   device int8 [R, I] (16-byte aligned, I % 16 == 0), float32 [R]
 * h = fl32(g / (1 + exp(-g)) * u) in float32, then the per-token rule of w4a8_quant_act.
 * I <= 16384 (EUNSUPPORTED beyond). */
int w4a8_silu_mul_quant(const void* GU_bf16, int R, int I, int8_t* Hq, float* sh,
                        void* stream);

/* The same with static per-expert scales: row r (expert-sorted order) is quantized by the
 * rule of w4a8_quant_act_static with the scale s[e] of the expert that owns it.
 *   expert_offsets  device int32 [E+1] from w4a8_moe_align; s device float32 [E]
 * Rows at or past expert_offsets[E] get zero codes and scale 0.  E <= 1024 (EINVAL). */
int w4a8_silu_mul_quant_static(const void* GU_bf16, int R, int I, const int32_t* expert_offsets,
                               int E, const float* s, int8_t* Hq, float* sh, void* stream);

/* Un-permute and top-k weighted combine (P1 section 4.3: dequantize to 16-bit, multiply
 * by the gate weight, accumulate; kept out of the integer domain).
 *   Yd_bf16  device bfloat16 [T*k, H] in sorted order
 *   inv      device int32 [T, k] from w4a8_moe_align
 *   topk_w   device float32 [T, k]
 *   out      device bfloat16 [T, H]
 * out[t] = bf16(sum_{j=0..k-1} topk_w[t, j] * Yd[inv[t, j]]) in float32, j ascending. */
int w4a8_moe_combine(const void* Yd_bf16, const int32_t* inv, const float* topk_w, int T,
                     int k, int H, void* out_bf16, void* stream);

/* Workspace bytes needed by w4a8_moe_forward for the given sizes (0 if invalid). */
size_t w4a8_moe_workspace_size(int T, int k, int H, int I, int E);

/* One MoE expert layer, the steps of P1 section 4.4 chained on `stream`:
 * quant_act(X) -> moe_align -> moe_gemm(gate/up, gathered) -> silu_mul_quant ->
 * moe_gemm(down) -> moe_combine.
 *   X_bf16      device [T, H]; topk_ids / topk_w device [T, k]
 *   gu_blobs    E blobs of desc gu_desc (K = H, N = 2I), stride gu_stride
 *   d_blobs     E blobs of desc d_desc (K = I, N = H), stride d_stride
 *   workspace   device, >= w4a8_moe_workspace_size(T, k, H, I, E) bytes, 256-aligned
 *   out_bf16    device [T, H], 16-byte aligned
 * Limits: E <= 1024 (EINVAL), T*k <= 2^24, H <= 65536, I <= 16384 (EUNSUPPORTED); H and I
 * multiples of 16, X 16-byte aligned (EINVAL).  Every argument check of the chained steps
 * runs before the first launch: an error return means that nothing was enqueued. */
int w4a8_moe_forward(const void* X_bf16, const int32_t* topk_ids, const float* topk_w, int T,
                     int k, int E, const void* gu_blobs, size_t gu_stride,
                     const w4a8_wdesc* gu_desc, const void* d_blobs, size_t d_stride,
                     const w4a8_wdesc* d_desc, void* workspace, size_t workspace_bytes,
                     void* out_bf16, void* stream);

/* w4a8_moe_forward for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The workspace is a 64 MiB
 * device array that the library holds on each GPU it runs on until the process ends; the call
 * itself allocates nothing.  Layers whose w4a8_moe_workspace_size exceeds 64 MiB return
 * W4A8_ESIZE (the T = 512, E = 64, top-6 layer with H = 4096, I = 1408 needs about 49 MB).
 * Every call on one GPU shares that array: calls that overlap on one GPU (other streams, other
 * threads) race and must be serialized by the caller.  Arguments, results and other errors as
 * w4a8_moe_forward (W4A8_EHIP also if the array's address cannot be obtained). */
int w4a8_moe_forward_noalloc(const void* X_bf16, const int32_t* topk_ids, const float* topk_w, int T,
                             int k, int E, const void* gu_blobs, size_t gu_stride,
                             const w4a8_wdesc* gu_desc, const void* d_blobs, size_t d_stride,
                             const w4a8_wdesc* d_desc, void* out_bf16, void* stream);

/* One format class of experts for w4a8_moe_forward_sets: n_experts consecutive experts
 * whose gate/up blobs (desc gu_desc, stride gu_stride) and down blobs (d_desc, d_stride)
 * share one format.  Experts are numbered set by set: set 0 holds experts [0, n_0), set 1
 * [n_0, n_0 + n_1), and so on. */
typedef struct {
    int32_t n_experts;
    const void* gu_blobs;
    size_t gu_stride;
    const w4a8_wdesc* gu_desc;
    const void* d_blobs;
    size_t d_stride;
    const w4a8_wdesc* d_desc;
} w4a8_expert_set;

/* One MoE expert layer whose experts use different weight formats (P1 section 8: quantize at
 * expert granularity, with a group size and format per expert, so that sensitive experts can
 * be kept at a finer format).  The steps of w4a8_moe_forward.  The group size, zero points and
 * scale width may differ between sets; the shapes (gate/up [H, 2I], down [I, H]) may not (EINVAL).
 * A grouped GEMM whose K (H for gate/up, I for down) is at most 4096 runs every set in one
 * launch pair on `stream` when there are at most four sets: each workgroup takes the format of
 * its expert's set, so the result is that of one launch per set.  Otherwise the GEMM runs once
 * per set, over that set's experts; these launches are independent (disjoint experts, disjoint
 * rows): set 0 runs on `stream`, the others on up to four helper streams of the current device,
 * forked from `stream` and joined back into it with events, so the call completes in `stream`
 * order and can be captured into a graph.  The helpers (default priority) are created by the
 * first call that needs them and is not made under graph capture, and kept until the process
 * ends; a call made before they exist, or where they cannot be created, runs the sets one after
 * another on `stream`.  Calls from several host threads enqueue one at a time.
 *   sets, nsets  host array of the format classes; E = sum of n_experts <= 1024
 *   workspace    device, >= w4a8_moe_workspace_size(T, k, H, I, E) bytes, 256-aligned
 * Other arguments and errors as w4a8_moe_forward. */
int w4a8_moe_forward_sets(const void* X_bf16, const int32_t* topk_ids, const float* topk_w, int T,
                          int k, const w4a8_expert_set* sets, int nsets, void* workspace,
                          size_t workspace_bytes, void* out_bf16, void* stream);

/* Workspace bytes needed by w4a8_moe_forward_static (0 if invalid): the routed rows are
 * quantized one by one, so the activation codes take T*k rows instead of T. */
size_t w4a8_moe_static_workspace_size(int T, int k, int H, int I, int E);

/* One MoE expert layer with static per-expert activation scales (P1 section 3.1 and 3.2:
 * calibrated scales, one per expert, for decode).  The steps of w4a8_moe_forward, with the
 * two quantizations replaced: moe_align -> moe_quant_static(X, s_gu) -> moe_gemm_silu_static
 * (gate/up GEMM, rows already sorted, with the SiLU-requant by s_dn in its epilogue) ->
 * moe_gemm(down) -> moe_combine.
 *   s_gu, s_dn  device float32 [E]: scale of each expert's gate/up and down inputs
 *   workspace   device, >= w4a8_moe_static_workspace_size(T, k, H, I, E) bytes, 256-aligned
 * Other arguments and errors as w4a8_moe_forward. */
int w4a8_moe_forward_static(const void* X_bf16, const int32_t* topk_ids, const float* topk_w, int T,
                            int k, int E, const void* gu_blobs, size_t gu_stride,
                            const w4a8_wdesc* gu_desc, const void* d_blobs, size_t d_stride,
                            const w4a8_wdesc* d_desc, const float* s_gu, const float* s_dn,
                            void* workspace, size_t workspace_bytes, void* out_bf16, void* stream);

/* Name of the kernel variant w4a8_gemm resolves to for (d, M), or "unsupported"
 * (P4: record target and resolved backend so a silent fallback is visible):
 * {w4a8,w8a8}_{decode_m16,decode_m32,prefill}_{sym,asym}_g{64,128,256,K,32}[_h16], and
 * w4a8_decode_split_m{16,32}_... for the decode GEMMs served by the kernel with one K-slice per
 * wave (4-bit codes, g in {64, 128}, 2048 < K <= 4096, rows w4a8_linear does not quantize
 * inside the GEMM). */
const char* w4a8_kernel_name(const w4a8_wdesc* d, int M);

/* Human-readable text of a w4a8_status. */
const char* w4a8_status_string(int status);

/* Library ABI version (1). */
int w4a8_version(void);

#ifdef __cplusplus
}
#endif

#endif /* W4A8_H */
