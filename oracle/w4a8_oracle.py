"""Plain, slow CPU oracle of the W4A8 linear / MoE-expert path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, links or runs
this module; only the test-suite, the smoke check and the CPU-baseline leg of
the benchmark do.  It shares no code with the HIP library.

Sources (cited as P1..P5 with the page's own section names):
  P1  "Kimi 2.7 MoE: from 4-bit storage to INT8 (W4A8)"              (pwwt.cn/news/5180806)
  P2  "Kimi 2.7 MoE W4A8: 4-bit storage to INT8, deployment notes"   (xdnf.cn/news/279181)
  P3  "Quantization: formats, error and the real execution path"     (wineandchord.com)
  P4  "Choosing a weight-quantization scheme and locating kernel hits" (xbrilliance.ai)
  P5  "Inference quantization, chapter 1: the Linear layer"          (sgdbs.github.io)

Precision.  Every decision that turns a float into an integer code (scales,
quotients, rounding) is taken in IEEE float32 with round-half-to-even, the
precision of the pages' own reference code (P1 section 3.3 snippet and the P3
symmetric group-wise reference both run on float32 tensors).  Everything after
the integer codes is done exactly (integer partial sums, via float64 products
of small integers) or in float64.

Pins (each function is checked against something other than itself in
``tests/test_oracle_pins.py``):
  quant_act         P5 worked INT8 example and outlier example (tests/golden),
                    round-trip bound, zero row, brute-force fp32 per element.
  quant_weight      P3 reference-function invariants and its example, P2 range
                    example (asymmetric), bounds, zero groups, tiling error; 8-bit
                    codes: the same invariants with qmax = 127 and an exact round
                    trip of weights on a power-of-two grid; binary16 scales: torch's
                    float32 -> float16 cast, half-spacing bound, identity when every
                    float32 scale is already a binary16 value, the rounding invariants
                    against the stored scale, and the range error.
  gemm_partials     brute-force integer triple loop; zero-point expansion of
                    P5 section 7; integer matmul when K equals the group.
  gemm              brute-force fp64 dequantise-then-matmul; per-token x
                    per-channel closed form of P5 section 8.3 when g = K.
  gemm_a16          brute-force fp64 x @ dequantised weights; equals gemm on activations
                    that are exactly s_x x_q; per-channel closed form when g = K.
  silu_mul          x*sigmoid(x) via scipy.special.expit; odd-part identity.
  moe_align         bincount/prefix-sum and permutation invariants.
  moe_layer         E=1,k=1,w=1 reduces to the dense chain; token permutation
                    equivariance; combine weights linearity.
  effective_bits,
  memory_bytes      P3 closed forms; P5 section 8.4 compression ratios.
  bf16_rne          torch's float32->bfloat16 conversion (library routine).
  smooth_factors,
  smooth_weights,
  quant_act_smooth  the rescaling is exactly equivalent when alpha is a power of two
                    (products exact: codes equal quant_act of x 2^-e, GEMM unchanged);
                    inv_alpha = 1 reduces to quant_act; the factor rule's closed form.
  calibrate_act_scale,
  quant_act_static  with each row's own dynamic scale it reduces to quant_act; exact
                    quotients on a power-of-two scale (ties to even, saturation, NaN,
                    infinities); the calibrated scale of a batch is the largest per-token
                    scale of its rows.
  moe_layer (per-expert group sizes)
                    one routed row per expert with each expert at its own group size:
                    every output row equals the dense chain of quant_act, gemm, silu_mul_quant
                    and gemm at that expert's group size.
  moe_layer (static scales)
                    one routed row per expert, through a non-trivial expert permutation,
                    with each expert's scales set to its row's dynamic scales: identical to
                    the dynamic layer.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_rne", "quant_act", "quant_act_static", "calibrate_act_scale", "quant_act_smooth", "smooth_factors", "smooth_weights", "dequant_act", "quant_weight", "dequant_weight", "gemm_partials",
    "gemm", "gemm_a16", "silu_mul", "silu_mul_quant", "moe_align", "moe_layer", "effective_bits",
    "memory_bytes", "compression_vs_fp16",
]

_F32 = np.float32


# --------------------------------------------------------------------------------------
# output cast
# --------------------------------------------------------------------------------------
def bf16_rne(y) -> np.ndarray:
    """Round float64/float32 values to the nearest bfloat16 (ties to even), returned as
    float32 holding exactly those values.  bfloat16 keeps 8 significant bits (P1 section 1:
    1 sign + 8 exponent + 7 mantissa bits)."""
    y = np.asarray(y, dtype=np.float64)
    out = np.empty(y.shape, dtype=np.float64)
    finite = np.isfinite(y)
    out[~finite] = y[~finite]
    v = y[finite]
    m, e = np.frexp(v)                 # v = m * 2**e, 0.5 <= |m| < 1
    e = np.maximum(e, -125)            # below 2**-126 the bf16 grid is fixed (subnormals)
    step_exp = e - 8                   # 8 significant bits
    r = np.rint(np.ldexp(v, -step_exp))  # exact scaling, ties to even
    res = np.ldexp(r, step_exp)
    bf16_max = np.ldexp(255.0, 120)    # largest finite bfloat16 = (2 - 2**-7) * 2**127
    res = np.where(np.abs(res) > bf16_max, np.copysign(np.inf, res), res)
    out[finite] = res
    return out.astype(np.float32)


# --------------------------------------------------------------------------------------
# per-token dynamic INT8 activation quantization
# --------------------------------------------------------------------------------------
def quant_act(x):
    """Per-token symmetric INT8 quantization of an activation matrix X[M, K].

    Follows P1 section 3.3 (per-token scale = row abs-max / 127, round, clamp) and P5 section
    8.3 (X[i, :] ~ s_x[i] * X_int8[i, :]).  Readings: no epsilon is added to the scale; a row
    whose abs-max is 0 keeps scale 0 and divides by 1 (the safe divisor of the P3 symmetric
    group-wise reference); codes are clamped to the symmetric range [-127, 127]; a row whose
    abs-max is not finite (NaN or Inf present) gets scale NaN and all-zero codes.
    Returns (q int8 [M, K], s float32 [M]).
    """
    x = np.asarray(x, dtype=_F32)
    if x.ndim != 2 or x.shape[1] == 0:
        raise ValueError("x must be [M, K] with K >= 1")
    amax = np.max(np.abs(x), axis=1) if x.shape[0] else np.zeros(0, _F32)
    s = (amax / _F32(127.0)).astype(_F32)
    finite = np.isfinite(amax)
    d = np.where(s > 0, s, _F32(1.0)).astype(_F32)
    with np.errstate(invalid="ignore", over="ignore", divide="ignore"):
        quot = (x / d[:, None]).astype(_F32)       # IEEE float32 division
        q = np.clip(np.rint(quot), -127, 127)      # round half to even
    q = np.where(finite[:, None], q, 0).astype(np.int8)
    s = np.where(finite, s, _F32(np.nan)).astype(_F32)
    return q, s


def smooth_factors(x_absmax, w, strength: float = 0.5):
    """Per-input-channel factors alpha of the equivalent rescaling
    Y = (X diag(alpha)^-1) (diag(alpha) W) (P3 "Weight-Activation", the SmoothQuant form:
    offline, moving quantization difficulty from activations to weights).  The page leaves
    alpha open beyond "per channel, positive"; reading: SmoothQuant's rule
    alpha_j = max|X_j|^a / max|W_j|^(1-a) with migration strength a, computed in float64
    and rounded to float32; a channel with a zero maximum on either side keeps alpha = 1.
    x_absmax: [K] calibration abs-max of each input channel; w: [K, N].  Returns float32 [K]."""
    xa = np.asarray(x_absmax, np.float64)
    wa = np.max(np.abs(np.asarray(w, np.float64)), axis=1)
    ok = (xa > 0) & (wa > 0) & np.isfinite(xa) & np.isfinite(wa)
    alpha = np.ones_like(xa)
    alpha[ok] = xa[ok] ** strength / wa[ok] ** (1.0 - strength)
    return alpha.astype(_F32)


def smooth_weights(w, alpha):
    """diag(alpha) W: row k of W[K, N] times alpha_k, each product rounded to float32."""
    return (np.asarray(w, _F32) * np.asarray(alpha, _F32)[:, None]).astype(_F32)


def quant_act_smooth(x, inv_alpha):
    """Per-token INT8 quantization of X diag(alpha)^-1: every x[m, k] is first multiplied by
    inv_alpha[k] (one float32 product, round to nearest even), then quant_act's per-token rule
    applies to the products (P3 "Weight-Activation": the scaling fused into the adjacent
    operator, here the activation quantization)."""
    xs = (np.asarray(x, _F32) * np.asarray(inv_alpha, _F32)[None, :]).astype(_F32)
    return quant_act(xs)


def calibrate_act_scale(x_calib):
    """Static (calibrated) activation scale: one per-tensor scale fixed offline from a
    calibration batch (P1 section 3.2: static quantization measures the activation range on a
    calibration set ahead of time and serves with the fixed scale; the page recommends it for
    decode).  Reading: the per-token rule applied to the whole batch, s = fl32(max|x| / 127)
    over every value of x_calib[R, K].  Returns a float32 scalar."""
    x = np.asarray(x_calib, dtype=_F32)
    return _F32(np.max(np.abs(x)) / _F32(127.0))


def quant_act_static(x, s):
    """INT8 quantization of X[M, K] with one fixed scale s for every row (P1 section 3.2, static
    mode): q = clamp(rint(fl32(x / s)), -127, 127), the per-token rule of quant_act with the
    scale given instead of measured.  Values outside the calibrated range saturate at +-127
    (the long-tail loss the page warns about).  Readings: a NaN value gets code 0; a scale
    that is not finite and positive gives all-zero codes.  Returns (q int8 [M, K], s float32
    [M], every entry the given s)."""
    x = np.asarray(x, dtype=_F32)
    if x.ndim != 2 or x.shape[1] == 0:
        raise ValueError("x must be [M, K] with K >= 1")
    s = _F32(s)
    sx = np.full(x.shape[0], s, dtype=_F32)
    if not (np.isfinite(s) and s > 0):
        return np.zeros(x.shape, np.int8), sx
    with np.errstate(invalid="ignore", over="ignore"):
        quot = (x / s).astype(_F32)                # IEEE float32 division (may overflow to inf)
        q = np.clip(np.rint(quot), -127, 127)      # round half to even, saturate
    q = np.where(np.isnan(x), 0, q).astype(np.int8)
    return q, sx


def dequant_act(q, s):
    """x_hat = q * s per row (P1 section 3.3, dequantize_activation), in float64."""
    return np.asarray(q, np.float64) * np.asarray(s, np.float64)[:, None]


# --------------------------------------------------------------------------------------
# offline group-wise INT4 weight quantization (round to nearest)
# --------------------------------------------------------------------------------------
def quant_weight(w, group_size: int, asymmetric: bool, bits: int = 4, scale_bits: int = 32):
    """Group-wise RTN quantization of W[K, N] to `bits`-bit codes (4; 8 for the symmetric
    W8A8 sibling); each group is `group_size` consecutive rows k of one output column n
    (P5 section 8.4: one output channel split along K).

    Symmetric (P3 "Basic mapping", symmetric form, and the P3 symmetric group-wise
    reference, whose qmax is 2^(bits-1) - 1): s = max|w| / qmax,
    q = clamp(round(w / s), -qmax, qmax), z = 0, with qmax = 7 (4 bits) or 127 (8 bits); an
    all-zero group keeps s = 0 and divides by 1.

    Asymmetric (P3 "Basic mapping": s = (x_max - x_min) / (2^b - 1),
    q = clip(round(x / s) + z, 0, 15), x_hat = s (q - z); P5 section 6 for the zero point as
    the integer that float 0 maps to; P2 section 2.1 for the min/max range).  Readings: the
    range is widened to include 0 (lo = min(0, min w), hi = max(0, max w)) so that 0 is
    exact; z = clamp(round(-lo / s), 0, 15) is an integer; an all-zero group has s = 0, z = 0,
    q = 0.

    scale_bits = 16 stores the scales in binary16, as P1 section 4.1 does for expert weights.
    Reading: the float32 scale above is rounded to the nearest binary16 (ties to even, numpy's
    float32 -> float16 cast) before any code is computed, so the codes are those of the stored
    scale and w_hat = s16 (q - z) exactly; a scale past the binary16 range is an error.

    Returns (codes int8 [K, N], scales float32 [K/g, N], zeros uint8 [K/g, N] or None).
    Raises ValueError when the group does not tile K (P3 reference: groups cannot cross rows),
    when a weight is not finite, or for bits other than 4 and 8 (8: symmetric only).
    """
    if bits not in (4, 8) or (bits == 8 and asymmetric):
        raise ValueError("bits must be 4, or 8 with symmetric codes")
    if scale_bits not in (16, 32):
        raise ValueError("scale_bits must be 16 or 32")

    def stored(scale):
        if scale_bits == 32:
            return scale
        with np.errstate(over="ignore"):
            h = scale.astype(np.float16)
        if not np.all(np.isfinite(h)):
            raise ValueError("a scale exceeds the binary16 range")
        return h.astype(_F32)
    qmax = (1 << (bits - 1)) - 1
    w = np.asarray(w, dtype=_F32)
    if w.ndim != 2:
        raise ValueError("w must be [K, N]")
    K, N = w.shape
    if group_size <= 0 or K == 0 or K % group_size:
        raise ValueError("group size must validly tile K")
    if not np.all(np.isfinite(w)):
        raise ValueError("weights must be finite")
    G = K // group_size
    wg = w.reshape(G, group_size, N)
    if not asymmetric:
        amax = np.max(np.abs(wg), axis=1)
        s = stored((amax / _F32(qmax)).astype(_F32))
        d = np.where(s > 0, s, _F32(1.0)).astype(_F32)
        q = np.clip(np.rint((wg / d[:, None, :]).astype(_F32)), -qmax, qmax)
        return q.reshape(K, N).astype(np.int8), s, None
    lo = np.minimum(np.min(wg, axis=1), _F32(0.0))
    hi = np.maximum(np.max(wg, axis=1), _F32(0.0))
    s = stored(((hi - lo).astype(_F32) / _F32(15.0)).astype(_F32))
    nz = s > 0
    d = np.where(nz, s, _F32(1.0)).astype(_F32)
    z = np.where(nz, np.clip(np.rint((-lo / d).astype(_F32)), 0, 15), 0)
    q = np.clip(np.rint((wg / d[:, None, :]).astype(_F32)) + z[:, None, :], 0, 15)
    q = np.where(nz[:, None, :], q, 0)
    return q.reshape(K, N).astype(np.int8), s, z.astype(np.uint8)


def dequant_weight(codes, scales, zeros, group_size: int):
    """w_hat = s (q - z) per group (P3 "Basic mapping"; P5 section 6), in float64."""
    codes = np.asarray(codes, np.float64)
    K, N = codes.shape
    G = K // group_size
    s = np.repeat(np.asarray(scales, np.float64), group_size, axis=0)
    z = 0.0 if zeros is None else np.repeat(np.asarray(zeros, np.float64), group_size, axis=0)
    assert s.shape == (K, N) and G * group_size == K
    return s * (codes - z)


# --------------------------------------------------------------------------------------
# W4A8 GEMM
# --------------------------------------------------------------------------------------
def gemm_partials(xq, codes, zeros, group_size: int):
    """Integer partial sums P[m, n, i] = sum_{k in group i} xq[m, k] * (q[k, n] - z[i, n]).

    This is the INT8 x INT8 -> INT32 accumulation of P5 section 4 (acc_int32) restricted to one
    K-group, with the weight zero point subtracted from the code (P5 section 7 expansion with
    zp_x = 0).  Each group is one float64 matrix product of small integers: every product and
    every partial sum is an integer of magnitude at most 127 * 255 * g, far below 2**53, so the
    result is exact in any summation order.  Returns int64 [M, N, K/g].
    """
    xq = np.asarray(xq)
    codes = np.asarray(codes)
    M, K = xq.shape
    K2, N = codes.shape
    assert K == K2 and K % group_size == 0
    G = K // group_size
    P = np.empty((M, N, G), dtype=np.int64)
    for i in range(G):
        ks = slice(i * group_size, (i + 1) * group_size)
        b = codes[ks].astype(np.float64)
        if zeros is not None:
            b = b - np.asarray(zeros[i], np.float64)[None, :]
        P[:, :, i] = np.rint(xq[:, ks].astype(np.float64) @ b).astype(np.int64)
    return P


def gemm(xq, sx, codes, scales, zeros, group_size: int):
    """Y[m, n] = s_x[m] * sum_i s_w[i, n] * P[m, n, i] in float64.

    P5 section 8.3 gives Y[i, j] ~ s_x[i] s_w[j] acc_int32[i, j] for one weight scale per
    column; with one scale per K-group (P5 section 8.4) the epilogue applies s_w[i, n] to each
    group's integer partial sum and s_x[m] to the row.  Rows whose scale is NaN give NaN.
    """
    xq = np.asarray(xq)
    M, K = xq.shape
    N = np.asarray(codes).shape[1]
    G = K // group_size
    acc = np.zeros((M, N), dtype=np.float64)
    for i in range(G):
        ks = slice(i * group_size, (i + 1) * group_size)
        b = np.asarray(codes[ks], np.float64)
        if zeros is not None:
            b = b - np.asarray(zeros[i], np.float64)[None, :]
        Pi = xq[:, ks].astype(np.float64) @ b                 # exact integers
        acc += Pi * np.asarray(scales[i], np.float64)[None, :]
    return acc * np.asarray(sx, np.float64)[:, None]


def gemm_a16(x, codes, scales, zeros, group_size: int):
    """W4A16 sibling: Y[m, n] = sum_i s_w[i, n] * sum_{k in group i} x[m, k] * (q[k, n] - z[i, n])
    in float64, with the activations x kept in 16 bits (no activation quantization) and the
    4-bit weights dequantized inside the kernel.  P1 section 5.3 lists W4A16 beside W8A8 and W4A8;
    P5 section 3.2 describes the weight-only path as a dequantization fused into the GEMM.  The
    weight dequantization is the same s (q - z) as for W4A8 (P3 "Basic mapping"); the reading
    taken is that the scale multiplies each group's sum, as in the W4A8 epilogue.  x: the float
    values of the bfloat16 activations.  Every product x * (q - z) is exact in float64, and the
    sums round at 2^-53, far below any tolerance used against them."""
    x = np.asarray(x, np.float64)
    M, K = x.shape
    N = np.asarray(codes).shape[1]
    G = K // group_size
    acc = np.zeros((M, N), dtype=np.float64)
    for i in range(G):
        ks = slice(i * group_size, (i + 1) * group_size)
        b = np.asarray(codes[ks], np.float64)
        if zeros is not None:
            b = b - np.asarray(zeros[i], np.float64)[None, :]
        acc += (x[:, ks] @ b) * np.asarray(scales[i], np.float64)[None, :]
    return acc


# --------------------------------------------------------------------------------------
# gated expert activation + requantization
# --------------------------------------------------------------------------------------
def silu_mul(gu):
    """h = silu(gate) * up with gate = the first I columns and up = the last I columns of
    gu[R, 2I]; silu(x) = x / (1 + exp(-x)).  P1 section 1 names GeLU/SiLU as the expert
    activation; the SiLU-gated form and the column split are readings.  float64."""
    gu = np.asarray(gu, np.float64)
    I = gu.shape[1] // 2
    g, u = gu[:, :I], gu[:, I:]
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g)) * u


def silu_mul_quant(gu):
    """Per-row INT8 requantization of silu(gate) * up for the down projection: each routed
    (token, expert) row gets its own dynamic scale (P1 section 3.1: independent activation
    scales per expert).  h is rounded once to float32 (the kernel's precision) before the
    per-token quantization of quant_act.  Returns (q int8 [R, I], s float32 [R])."""
    h = silu_mul(gu).astype(_F32)
    return quant_act(h)


# --------------------------------------------------------------------------------------
# MoE: dispatch by expert, grouped GEMMs, weighted combine
# --------------------------------------------------------------------------------------
def moe_align(topk_ids, E: int):
    """Group the T*k routed rows by expert (P1 section 4.4: tokens are dispatched to their
    top-k experts).  Row r = t*k + j stands for (token t, choice j).  The order inside an
    expert is ascending r (a stable sort).
    Returns (sorted_rows int32 [T*k], expert_offsets int32 [E+1], inv int32 [T, k]) with
    sorted_rows[inv[t, j]] = t*k + j."""
    ids = np.asarray(topk_ids, dtype=np.int64)
    T, k = ids.shape
    flat = ids.reshape(-1)
    if flat.size and (flat.min() < 0 or flat.max() >= E):
        raise ValueError("expert id out of range")
    order = np.argsort(flat, kind="stable")
    counts = np.bincount(flat, minlength=E)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    inv = np.empty(T * k, dtype=np.int64)
    inv[order] = np.arange(T * k)
    return order.astype(np.int32), offsets, inv.reshape(T, k).astype(np.int32)


def moe_layer(x, topk_ids, topk_w, expert, E: int, I: int, group_size: int, s_gu=None, s_dn=None):
    """One MoE expert layer in the W4A8 flow of P1 section 4.4.

    1. per-token INT8 quantization of the input, once per token, before dispatch;
    2. dispatch: rows grouped by expert (moe_align);
    3. per expert, gate/up W4A8 GEMM on the token's codes and scale, output rounded to bf16
       (the expert output is dequantized back to 16-bit, P1 section 4.3);
    4. silu(gate) * up, re-quantized per routed row (silu_mul_quant);
    5. per expert, down W4A8 GEMM, output rounded to bf16;
    6. combine: out[t] = sum_j w[t, j] * y[t, j] in 16-bit-input/float accumulation
       (P1 section 4.3 keeps the combine in FP16 rather than the integer domain); here in
       float64 over j ascending, then rounded to bf16.

    `expert(e)` returns (codes_gu [H, 2I], scales_gu, zeros_gu, codes_d [I, H], scales_d,
    zeros_d) for expert e; it is called only for experts that received rows.  `group_size` is
    one group size, or a sequence of E, one per expert (P1 section 8: expert-granular formats).

    Static per-expert activation scales (P1 section 3.1: each expert keeps its own activation
    scale; section 3.2: calibrated static scales for decode): with s_gu [E] given, step 1
    moves after dispatch and each routed row quantizes its token with quant_act_static and the
    scale s_gu[e] of its expert e; with s_dn [E] given, step 4 quantizes each routed row's
    silu(gate) * up (rounded once to float32) with s_dn[e].
    Returns dict(out=bf16 values [T, H], out64=float64 [T, H], and the intermediates).
    """
    x = np.asarray(x, _F32)
    ids = np.asarray(topk_ids)
    w = np.asarray(topk_w, np.float64)
    T, k = ids.shape
    H = x.shape[1]
    g_of = (lambda e: int(group_size)) if np.ndim(group_size) == 0 else (lambda e: int(group_size[e]))
    xq, sx = quant_act(x) if s_gu is None else (None, None)
    sorted_rows, offsets, inv = moe_align(ids, E)
    R = T * k
    gu = np.zeros((R, 2 * I), dtype=_F32)
    yd = np.zeros((R, H), dtype=_F32)
    weights = {}
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue
        weights[e] = expert(e)
        cg, sg, zg = weights[e][:3]
        toks = sorted_rows[a:b] // k
        qa, sa = (xq[toks], sx[toks]) if s_gu is None else quant_act_static(x[toks], s_gu[e])
        gu[a:b] = bf16_rne(gemm(qa, sa, cg, sg, zg, g_of(e)))
    if s_dn is None:
        hq, sh = silu_mul_quant(gu)
    else:
        hq, sh = np.zeros((R, I), np.int8), np.zeros(R, _F32)
        for e in weights:
            a, b = int(offsets[e]), int(offsets[e + 1])
            hq[a:b], sh[a:b] = quant_act_static(silu_mul(gu[a:b]).astype(_F32), s_dn[e])
    for e, wts in weights.items():
        a, b = int(offsets[e]), int(offsets[e + 1])
        cd, sd, zd = wts[3:]
        yd[a:b] = bf16_rne(gemm(hq[a:b], sh[a:b], cd, sd, zd, g_of(e)))
    out64 = np.zeros((T, H), dtype=np.float64)
    for j in range(k):
        out64 += w[:, j:j + 1] * yd[inv[:, j]].astype(np.float64)
    return dict(out=bf16_rne(out64), out64=out64, xq=xq, sx=sx, sorted_rows=sorted_rows,
                offsets=offsets, inv=inv, gu=gu, hq=hq, sh=sh, yd=yd, topk_w=w)


# --------------------------------------------------------------------------------------
# size closed forms
# --------------------------------------------------------------------------------------
def effective_bits(b: float, b_s: float, b_z: float, g: int) -> float:
    """b_effective = b + (b_s + b_z) / g  (P3 "Basic mapping")."""
    return b + (b_s + b_z) / g


def memory_bytes(n_weights: int, b: int, n_groups: int, meta_bytes_per_group: float,
                 padding: int = 0, workspace: int = 0) -> float:
    """M = N b / 8 + N_groups M_metadata + M_padding + M_workspace  (P3 "Basic mapping")."""
    return n_weights * b / 8 + n_groups * meta_bytes_per_group + padding + workspace


def compression_vs_fp16(g: int, b: int = 4, b_s: int = 16, b_z: int = 0) -> float:
    """FP16 bits per group over quantized bits per group (P5 section 8.4)."""
    return (16 * g) / (b * g + b_s + b_z)
