"""Pins for the CPU oracle: each check ties an oracle function to something other than
itself -- values printed on the pages (tests/golden), closed forms, invariants, library
routines, or brute force on tiny inputs."""
import itertools

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st
from scipy.special import expit

from conftest import golden
import oracle as O
import workloads as W

F32 = np.float32


# ------------------------------------------------------------------ activation quantization
def test_act_worked_example_p5():
    g = golden("act_int8_worked_example.json")
    x = np.array([g["input"]], F32)
    q, s = O.quant_act(x)
    assert q.tolist() == [g["codes"]]
    assert abs(float(s[0]) - g["scale_approx"]) < g["scale_abs_tol"]
    xhat = O.dequant_act(q, s)[0]
    assert np.allclose(np.round(xhat, 3), g["dequant_3dp"], atol=1.5e-3)
    # the same codes when the input is first rounded to bfloat16
    xb = W.bf16_values(W.to_bf16(x))
    qb, _ = O.quant_act(xb)
    assert qb.tolist() == [g["codes"]]


def test_act_outlier_example_p5():
    g = golden("act_outlier_example.json")
    q, s = O.quant_act(np.array([g["input"]], F32))
    assert q.tolist() == [g["codes"]]
    assert abs(float(s[0]) - g["scale_approx"]) < g["scale_abs_tol"]


def test_act_page1_snippet_reading_same_codes():
    """P1 section 3.3 adds eps=1e-8 to the scale and clamps to [-128, 127]; the chosen reading
    (no eps, [-127, 127]) gives the same codes on both printed examples."""
    for name in ("act_int8_worked_example.json", "act_outlier_example.json"):
        x = np.array([golden(name)["input"]], F32)
        amax = np.max(np.abs(x), axis=1, keepdims=True)
        s_eps = (amax / F32(127) + F32(1e-8)).astype(F32)
        q_eps = np.clip(np.rint(x / s_eps), -128, 127).astype(np.int8)
        q, _ = O.quant_act(x)
        assert np.array_equal(q, q_eps)


def test_act_bruteforce_elementwise():
    """Element-by-element pure-python evaluation of the per-token rule on a small matrix."""
    x = W.bf16_values(W.random_activations(5, 7, 37, outlier_cols=2, outlier_scale=30.0))
    q, s = O.quant_act(x)
    for m in range(x.shape[0]):
        amax = F32(0)
        for v in x[m]:
            amax = max(amax, F32(abs(v)))
        sm = F32(amax / F32(127))
        assert s[m] == sm
        for kk in range(x.shape[1]):
            r = F32(x[m, kk] / sm)
            lo = np.floor(r)
            frac = r - lo
            ref = lo + 1 if frac > 0.5 or (frac == 0.5 and lo % 2 == 1) else lo
            assert q[m, kk] == int(max(-127, min(127, ref)))


@settings(max_examples=60, deadline=None)
@given(st.integers(1, 6), st.integers(1, 70), st.integers(0, 2**31 - 1), st.floats(1e-3, 1e3))
def test_act_properties(M, K, seed, mag):
    x = (np.random.default_rng(seed).standard_normal((M, K)) * mag).astype(F32)
    q, s = O.quant_act(x)
    assert q.dtype == np.int8 and s.dtype == F32
    assert np.all(np.abs(q.astype(int)) <= 127)
    # the abs-max element maps to +-127
    for m in range(M):
        i = np.argmax(np.abs(x[m]))
        assert abs(int(q[m, i])) == 127
    # round-trip bound |x - q s| <= s/2 (with float32 slack)
    err = np.abs(x.astype(np.float64) - O.dequant_act(q, s))
    assert np.all(err <= s[:, None].astype(np.float64) * (0.5 + 1e-5))
    # idempotence on the dequantized grid
    q2, s2 = O.quant_act(O.dequant_act(q, s).astype(F32))
    assert np.array_equal(q2, q)


def test_act_zero_and_nonfinite_rows():
    x = np.array([[0, 0, 0, 0], [1, np.nan, 2, 3], [np.inf, 1, 2, 3], [-4, 2, 0, 1]], F32)
    q, s = O.quant_act(x)
    assert s[0] == 0 and not q[0].any()
    assert np.isnan(s[1]) and not q[1].any()
    assert np.isnan(s[2]) and not q[2].any()
    assert q[3].tolist() == [-127, 64, 0, 32] and s[3] == F32(F32(4) / F32(127))


# ------------------------------------------------------------------ weight quantization
def test_sym_groupwise_reference_example_p3():
    g = golden("sym_groupwise_reference.json")
    x = np.array(g["input"], F32)
    # the page's groups run along the last dimension; the oracle groups along K (rows), so
    # the page's [2, 4] example is the transpose: K = 4, N = 2.
    codes, scales, zeros = O.quant_weight(x.T, g["group_size"], asymmetric=False)
    assert zeros is None
    assert codes.T.tolist() == g["codes_hand_derived"]
    assert codes.min() >= -7 and codes.max() <= 7
    restored = O.dequant_weight(codes, scales, None, g["group_size"])
    err = np.abs(x.T.astype(np.float64) - restored)
    assert np.all(err <= scales.astype(np.float64) / 2 + g["bound_abs_slack"])
    assert scales[0].tolist() == [F32(F32(1) / F32(7)), F32(F32(3) / F32(7))]
    zc, zs, _ = O.quant_weight(np.zeros((4, 1), F32), 4, asymmetric=False)
    assert not zc.any() and zs[0, 0] == 0
    assert not O.dequant_weight(zc, zs, None, 4).any()
    with pytest.raises(ValueError):
        O.quant_weight(np.ones((3, 2), F32), 2, asymmetric=False)   # groups cannot cross
    with pytest.raises(ValueError):
        O.quant_weight(np.ones((4, 2), F32), 0, asymmetric=False)


def test_sym_rounding_uses_ieee_division():
    """0.5 / fl32(1/7) = 3.4999998 in float32 -> code 3, whereas the real-valued quotient
    0.5 / (1/7) = 3.5 would round (half to even) to 4: the page example's third element pins
    that the quotient is taken in float32 against the stored float32 scale."""
    codes, _, _ = O.quant_weight(np.array([[0.0], [-1.0], [0.5], [0.25]], F32), 4, False)
    assert codes[2, 0] == 3
    s = F32(F32(1) / F32(7))
    assert F32(0.5) / s < 3.5 and np.rint(0.5 / (1.0 / 7.0)) == 4


def test_asym_range_example_p2():
    g = golden("asym_range_example.json")
    w = np.array([[g["w_min"]], [0.0], [0.4], [g["w_max"]]], F32)
    codes, scales, zeros = O.quant_weight(w, 4, asymmetric=True)
    s = float(scales[0, 0])
    assert abs(s - g["scale_approx"]) < 1e-6
    assert int(zeros[0, 0]) in g["zero_point_choices"]
    assert codes[1, 0] == zeros[0, 0]              # float 0 maps exactly to z
    assert codes.min() >= 0 and codes.max() <= g["levels"]
    assert codes[0, 0] == 0 and codes[3, 0] == 15   # ends of the range
    xhat = O.dequant_weight(codes, scales, zeros, 4)
    assert xhat[1, 0] == 0.0


@settings(max_examples=60, deadline=None)
@given(st.sampled_from([4, 8, 32, 64, 128]), st.integers(1, 4), st.integers(1, 9),
       st.integers(0, 2**31 - 1), st.booleans(), st.floats(-0.05, 0.05))
def test_weight_properties(g, G, N, seed, asym, shift):
    rs = np.random.default_rng(seed)
    w = (rs.standard_normal((g * G, N)) * 0.02 + shift).astype(F32)
    if G > 1:
        w[:g, 0] = 0.0                                   # an all-zero group
    codes, scales, zeros = O.quant_weight(w, g, asym)
    lo, hi = (0, 15) if asym else (-7, 7)
    assert codes.min() >= lo and codes.max() <= hi
    xhat = O.dequant_weight(codes, scales, zeros, g)
    s_full = np.repeat(scales.astype(np.float64), g, axis=0)
    assert np.all(np.abs(w - xhat) <= s_full / 2 * (1 + 1e-5) + 1e-12)
    if G > 1:
        assert scales[0, 0] == 0 and not codes[:g, 0].any() and not xhat[:g, 0].any()
    if asym:
        # zero is represented exactly: every group's zero point is a valid code
        assert zeros.max() <= 15
        # groups straddling zero use both ends of the range when max = -min
    else:
        # symmetric: the abs-max element of each nonzero group reaches +-7
        wg = w.reshape(G, g, N)
        cg = codes.reshape(G, g, N)
        for i, n in itertools.product(range(G), range(N)):
            if scales[i, n] > 0:
                j = np.argmax(np.abs(wg[i, :, n]))
                assert abs(int(cg[i, j, n])) == 7


@settings(max_examples=25, deadline=None)
@given(st.sampled_from([32, 64, 128]), st.integers(1, 3), st.integers(1, 5), st.integers(0, 2**31 - 1))
def test_weight_properties_8bit(g, G, N, seed):
    """bits = 8 of the P3 symmetric group-wise reference: codes in [-127, 127], error at most
    s / 2, the abs-max element of a nonzero group at +-127, an all-zero group all zero."""
    rs = np.random.default_rng(seed)
    w = (rs.standard_normal((g * G, N)) * 0.02).astype(F32)
    w[:g, 0] = 0.0
    codes, scales, zeros = O.quant_weight(w, g, False, bits=8)
    assert zeros is None and codes.min() >= -127 and codes.max() <= 127
    xhat = O.dequant_weight(codes, scales, None, g)
    s_full = np.repeat(scales.astype(np.float64), g, axis=0)
    assert np.all(np.abs(w - xhat) <= s_full / 2 * (1 + 1e-5) + 1e-12)
    assert scales[0, 0] == 0 and not codes[:g, 0].any()
    wg, cg = w.reshape(G, g, N), codes.reshape(G, g, N)
    for i, n in itertools.product(range(G), range(N)):
        if scales[i, n] > 0:
            assert abs(int(cg[i, np.argmax(np.abs(wg[i, :, n])), n])) == 127


def test_weight_8bit_exact_grid_roundtrip():
    """Weights on the grid s * q (s a power of two, q integers with |q| = 127 present in
    every group) quantize back to exactly q and s: a wrong qmax, sign or rounding fails."""
    rs = np.random.default_rng(5)
    q = rs.integers(-127, 128, (256, 6)).astype(np.int64)
    q[0::64, :] = 127                                   # the abs max of every 64-group
    w = (q * 2.0 ** -9).astype(F32)
    codes, scales, _ = O.quant_weight(w, 64, False, bits=8)
    assert np.array_equal(codes.astype(np.int64), q)
    assert np.all(scales == F32(2.0 ** -9))
    with pytest.raises(ValueError):
        O.quant_weight(w, 64, True, bits=8)            # 8-bit codes are symmetric only
    with pytest.raises(ValueError):
        O.quant_weight(w, 64, False, bits=3)


def test_weight_nonfinite_rejected():
    w = np.zeros((4, 2), F32)
    w[1, 1] = np.nan
    with pytest.raises(ValueError):
        O.quant_weight(w, 4, False)


# ------------------------------------------------------------------ GEMM
def _tiny_problem(seed, M, K, N, g, asym, bits=4):
    x = W.bf16_values(W.random_activations(seed, M, K, outlier_cols=1, outlier_scale=10.0))
    w = W.random_weights(seed + 1, K, N)
    xq, sx = O.quant_act(x)
    codes, scales, zeros = O.quant_weight(w, g, asym, bits)
    return xq, sx, codes, scales, zeros


@pytest.mark.parametrize("M,K,N,g,asym", [(3, 64, 5, 32, False), (5, 128, 7, 64, True),
                                          (2, 256, 3, 128, True), (4, 96, 6, 32, True)])
def test_partials_bruteforce(M, K, N, g, asym):
    xq, sx, codes, scales, zeros = _tiny_problem(11, M, K, N, g, asym)
    P = O.gemm_partials(xq, codes, zeros, g)
    for m, n, i in itertools.product(range(M), range(N), range(K // g)):
        z = int(zeros[i, n]) if asym else 0
        ref = 0
        for kk in range(i * g, (i + 1) * g):
            ref += int(xq[m, kk]) * (int(codes[kk, n]) - z)
        assert P[m, n, i] == ref


@pytest.mark.parametrize("M,K,N,g,asym,bits", [(3, 64, 5, 32, False, 4), (5, 128, 7, 64, True, 4),
                                               (6, 512, 9, 128, False, 4), (2, 256, 4, 64, True, 4),
                                               (4, 256, 5, 128, False, 8)])
def test_gemm_bruteforce_dequant(M, K, N, g, asym, bits):
    """Y equals (s_x * x_q) @ (s_w * (q - z)) evaluated term by term in float64."""
    xq, sx, codes, scales, zeros = _tiny_problem(23, M, K, N, g, asym, bits)
    Y = O.gemm(xq, sx, codes, scales, zeros, g)
    for m, n in itertools.product(range(M), range(N)):
        ref = 0.0
        for kk in range(K):
            i = kk // g
            z = float(zeros[i, n]) if asym else 0.0
            ref += (float(sx[m]) * float(xq[m, kk])) * (float(scales[i, n]) * (float(codes[kk, n]) - z))
        assert abs(Y[m, n] - ref) <= 1e-12 * max(1.0, abs(ref)) + 1e-15


def test_zero_point_expansion_p5():
    """P5 section 7: sum x (q - z) = sum x q - z sum x (zp_x = 0), exactly in integers."""
    xq, sx, codes, scales, zeros = _tiny_problem(3, 4, 256, 6, 64, True)
    P = O.gemm_partials(xq, codes, zeros, 64)
    P_nozp = O.gemm_partials(xq, codes, None, 64)
    rs = xq.astype(np.int64).reshape(4, 4, 64).sum(axis=2)           # [M, G]
    assert np.array_equal(P, P_nozp - zeros.astype(np.int64).T[None, :, :] * rs[:, None, :])


def test_integer_matmul_when_one_group_unit_scales():
    rs = np.random.default_rng(1)
    xq = rs.integers(-127, 128, (5, 64)).astype(np.int8)
    codes = rs.integers(-7, 8, (64, 3)).astype(np.int8)
    ones = np.ones((1, 3), F32)
    Y = O.gemm(xq, np.ones(5, F32), codes, ones, None, 64)
    assert np.array_equal(Y, (xq.astype(np.int64) @ codes.astype(np.int64)).astype(np.float64))
    P = O.gemm_partials(xq, codes, None, 64)
    assert np.array_equal(P[:, :, 0], xq.astype(np.int64) @ codes.astype(np.int64))


def test_per_channel_closed_form_p5():
    """With g = K the epilogue is P5 section 8.3: Y[i, j] = s_x[i] s_w[j] acc_int32[i, j]."""
    xq, sx, codes, scales, zeros = _tiny_problem(9, 6, 256, 5, 256, False)
    acc = xq.astype(np.int64) @ codes.astype(np.int64)
    Y = O.gemm(xq, sx, codes, scales, None, 256)
    ref = sx.astype(np.float64)[:, None] * scales[0].astype(np.float64)[None, :] * acc
    assert np.allclose(Y, ref, rtol=1e-14, atol=0)


def test_gemm_linear_in_scales_and_rows():
    xq, sx, codes, scales, zeros = _tiny_problem(4, 4, 256, 6, 128, True)
    Y = O.gemm(xq, sx, codes, scales, zeros, 128)
    Y2 = O.gemm(xq, sx * F32(2), codes, scales, zeros, 128)
    assert np.array_equal(Y2, 2 * Y)
    perm = np.array([2, 0, 3, 1])
    assert np.array_equal(O.gemm(xq[perm], sx[perm], codes, scales, zeros, 128), Y[perm])


@pytest.mark.parametrize("M,K,N,g,asym", [(3, 64, 5, 32, False), (5, 128, 7, 64, True), (4, 256, 6, 128, False),
                                          (2, 256, 3, 128, True)])
def test_gemm_a16_bruteforce_dequant(M, K, N, g, asym):
    """W4A16: Y equals x @ (s_w * (q - z)) evaluated term by term in float64, x the bfloat16
    activations themselves (no quantization)."""
    _, _, codes, scales, zeros = _tiny_problem(31, M, K, N, g, asym)
    rs = np.random.default_rng(M * K + N)
    x = W.bf16_values(W.to_bf16(rs.standard_normal((M, K)).astype(F32) * 3))
    Y = O.gemm_a16(x, codes, scales, zeros, g)
    for m, n in itertools.product(range(M), range(N)):
        ref = 0.0
        for kk in range(K):
            i = kk // g
            z = float(zeros[i, n]) if asym else 0.0
            ref += float(x[m, kk]) * (float(scales[i, n]) * (float(codes[kk, n]) - z))
        assert abs(Y[m, n] - ref) <= 1e-12 * max(1.0, abs(ref)) + 1e-15


def test_gemm_a16_reduces_to_w4a8_on_quantized_activations():
    """When the 16-bit activations are exactly s_x * x_q (a power-of-two row scale times int8
    codes), W4A16 and W4A8 compute the same product: gemm_a16(s_x x_q) = gemm(x_q, s_x)."""
    xq, _, codes, scales, zeros = _tiny_problem(37, 5, 256, 7, 64, True)
    sx = np.array([2.0 ** -5, 2.0 ** -7, 1.0, 2.0 ** 3, 2.0 ** -10], F32)
    x = sx.astype(np.float64)[:, None] * xq.astype(np.float64)
    assert np.array_equal(W.bf16_values(W.to_bf16(x.astype(F32))), x.astype(F32))      # exact in bf16
    ya16 = O.gemm_a16(x, codes, scales, zeros, 64)
    y8 = O.gemm(xq, sx, codes, scales, zeros, 64)
    assert np.allclose(ya16, y8, rtol=1e-14, atol=0)


def test_gemm_a16_per_channel_closed_form():
    """g = K: one scale per column, Y = (x @ q) * s_w[n] (the weight-only form of P5 section 8.3)."""
    _, _, codes, scales, _ = _tiny_problem(41, 3, 128, 4, 128, False)
    x = W.bf16_values(W.to_bf16(np.random.default_rng(5).standard_normal((3, 128)).astype(F32)))
    ref = (x.astype(np.float64) @ codes.astype(np.float64)) * scales[0].astype(np.float64)[None, :]
    assert np.allclose(O.gemm_a16(x, codes, scales, None, 128), ref, rtol=1e-14, atol=0)


# ------------------------------------------------------------------ silu / requant
def test_silu_mul_library_and_identity():
    rs = np.random.default_rng(0)
    gu = W.bf16_values(W.to_bf16(rs.standard_normal((5, 16)).astype(F32) * 4))
    h = O.silu_mul(gu)
    g, u = gu[:, :8].astype(np.float64), gu[:, 8:].astype(np.float64)
    assert np.allclose(h, g * expit(g) * u, rtol=1e-13, atol=0)
    # silu(x) - silu(-x) = x: catches a sign error in the exponent
    x = np.linspace(-9, 9, 37)
    sp = O.silu_mul(np.concatenate([x[None], np.ones((1, 37))], 1))
    sm = O.silu_mul(np.concatenate([-x[None], np.ones((1, 37))], 1))
    assert np.allclose(sp - sm, x[None], atol=1e-12)
    assert O.silu_mul(np.array([[0.0, 5.0]]))[0, 0] == 0.0


def test_silu_mul_quant_is_per_row():
    rs = np.random.default_rng(2)
    gu = rs.standard_normal((6, 32)).astype(F32)
    q, s = O.silu_mul_quant(gu)
    h = O.silu_mul(gu).astype(F32)
    q2, s2 = O.quant_act(h)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)
    assert np.all(np.abs(q.astype(int)).max(axis=1) == 127)


# ------------------------------------------------------------------ MoE
def test_moe_align_invariants():
    rs = np.random.default_rng(7)
    T, k, E = 37, 4, 9
    ids = np.stack([rs.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    rows, off, inv = O.moe_align(ids, E)
    assert sorted(rows.tolist()) == list(range(T * k))               # each (t, j) once
    assert np.array_equal(off, np.concatenate([[0], np.cumsum(np.bincount(ids.ravel(), minlength=E))]))
    for e in range(E):
        seg = rows[off[e]:off[e + 1]]
        assert np.all(ids.ravel()[seg] == e) and np.all(np.diff(seg) > 0)   # stable
    for t, j in itertools.product(range(T), range(k)):
        assert rows[inv[t, j]] == t * k + j
    with pytest.raises(ValueError):
        O.moe_align(np.array([[E]], np.int32), E)


def _moe_small(E=3, T=9, k=2, H=128, I=64, g=64, asym=True, seed=5):
    rs = np.random.default_rng(seed)
    x = W.bf16_values(W.random_activations(seed, T, H))
    ids = np.stack([rs.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    wts = rs.random((T, k)).astype(F32)
    experts = {}
    for e in range(E):
        wgu = W.random_weights(seed * 10 + e, H, 2 * I)
        wd = W.random_weights(seed * 10 + e + 100, I, H)
        experts[e] = O.quant_weight(wgu, g, asym) + O.quant_weight(wd, g, asym)
    return x, ids, wts, experts, E, I, g


def test_moe_single_expert_reduces_to_dense_chain():
    x, ids, wts, experts, E, I, g = _moe_small(E=1, k=1)
    ids[:] = 0
    wts[:] = 1.0
    r = O.moe_layer(x, ids, wts, lambda e: experts[e], 1, I, g)
    cg, sg, zg, cd, sd, zd = experts[0]
    xq, sx = O.quant_act(x)
    gu = O.bf16_rne(O.gemm(xq, sx, cg, sg, zg, g))
    hq, sh = O.silu_mul_quant(gu)
    y = O.bf16_rne(O.gemm(hq, sh, cd, sd, zd, g))
    assert np.array_equal(r["out"], O.bf16_rne(y.astype(np.float64)))


def test_moe_token_permutation_and_combine_linearity():
    x, ids, wts, experts, E, I, g = _moe_small()
    f = lambda e: experts[e]
    r = O.moe_layer(x, ids, wts, f, E, I, g)
    perm = np.random.default_rng(0).permutation(x.shape[0])
    rp = O.moe_layer(x[perm], ids[perm], wts[perm], f, E, I, g)
    assert np.array_equal(rp["out64"], r["out64"][perm])
    r2 = O.moe_layer(x, ids, wts * F32(2), f, E, I, g)
    assert np.allclose(r2["out64"], 2 * r["out64"], rtol=1e-15, atol=0)
    # swapping the order of a token's choices (ids and weights together) changes nothing
    # beyond float64 summation order
    rs_ = O.moe_layer(x, ids[:, ::-1].copy(), wts[:, ::-1].copy(), f, E, I, g)
    assert np.allclose(rs_["out64"], r["out64"], rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ closed forms / bf16
def test_size_closed_forms():
    c = golden("size_closed_forms.json")
    assert O.effective_bits(4, 16, 0, 128) * 128 == c["g128_bits"]
    assert O.effective_bits(4, 16, 0, 32) * 128 == c["g32_bits"]
    assert round(O.compression_vs_fp16(128), 2) == c["g128_ratio_2dp"]
    assert round(O.compression_vs_fp16(32), 2) == c["g32_ratio_2dp"]
    assert O.effective_bits(4, 32, 0, 128) == 4.25
    assert O.effective_bits(4, 32, 8, 128) == 4.3125
    assert O.effective_bits(4, 32, 8, 64) == 4.625
    n = 4096 * 14336
    assert O.memory_bytes(n, 4, n // 128, 4) == n / 2 + n // 128 * 4


def test_bf16_rne_matches_torch():
    rs = np.random.default_rng(3)
    v = np.concatenate([rs.standard_normal(20000) * 10.0 ** rs.integers(-30, 30, 20000),
                        [0.0, -0.0, 1e-40, -3e-39, 3.3e38, 1.0 + 2**-8, 1.0 + 3 * 2**-8]]).astype(F32)
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(O.bf16_rne(v), ref)
    assert np.isinf(O.bf16_rne(np.array([3.5e38]))[0])


# ------------------------------------------------------------------ SmoothQuant rescaling
def test_smooth_identity_and_power_of_two_exactness():
    """inv_alpha = 1 reduces to quant_act; with alpha a power of two every product is exact, so
    the codes equal quant_act of x * 2^-e and the dequantized GEMM of the rescaled pair equals
    the plain one on the same grid (P3 "Weight-Activation": the two forms are equal in real
    arithmetic)."""
    x = W.bf16_values(W.random_activations(31, 6, 256, outlier_cols=3, outlier_scale=20.0))
    q0, s0 = O.quant_act(x)
    q1, s1 = O.quant_act_smooth(x, np.ones(256, F32))
    assert np.array_equal(q0, q1) and np.array_equal(s0.view(np.uint32), s1.view(np.uint32))
    e = np.random.default_rng(2).integers(-3, 4, 256)
    alpha = (2.0 ** e).astype(F32)
    q2, s2 = O.quant_act_smooth(x, (1.0 / alpha).astype(F32))
    q3, s3 = O.quant_act((x * (2.0 ** -e)).astype(F32))
    assert np.array_equal(q2, q3) and np.array_equal(s2.view(np.uint32), s3.view(np.uint32))
    w = W.random_weights(5, 256, 7)
    ws = O.smooth_weights(w, alpha)
    assert np.array_equal(ws, (w * alpha[:, None]).astype(F32))
    lhs = (x.astype(np.float64) / alpha.astype(np.float64)) @ ws.astype(np.float64)
    assert np.allclose(lhs, x.astype(np.float64) @ w.astype(np.float64), rtol=0, atol=1e-12)


def test_smooth_factor_rule():
    """alpha_j = max|X_j|^a / max|W_j|^(1-a), zero channels keep 1; a = 1 moves all of the
    activation range into the weights (every rescaled channel max becomes 1)."""
    rs = np.random.default_rng(4)
    xa = np.abs(rs.standard_normal(64)) * 5
    xa[3] = 0.0
    w = rs.standard_normal((64, 9)).astype(F32) * 0.02
    w[7] = 0.0
    a = O.smooth_factors(xa, w, 0.5)
    wa = np.max(np.abs(w.astype(np.float64)), axis=1)
    for j in range(64):
        if j in (3, 7):
            assert a[j] == 1.0
        else:
            assert a[j] == np.float32(np.sqrt(xa[j]) / np.sqrt(wa[j]))
    a1 = O.smooth_factors(xa, w, 1.0)
    ok = (xa > 0) & (wa > 0)
    assert np.allclose((xa / a1.astype(np.float64))[ok], 1.0, rtol=1e-6)


# ------------------------------------------------------------------ static activation scales
def test_static_with_each_rows_own_scale_is_dynamic():
    """P1 section 3.2: static mode only fixes the scale in advance; given the row's own
    measured scale it must produce quant_act's codes."""
    rs = np.random.default_rng(5)
    x = (rs.standard_normal((6, 96)) * rs.uniform(0.01, 30, (6, 1))).astype(F32)
    x[2, 7] = 500.0
    q, s = O.quant_act(x)
    for m in range(6):
        qs, ss = O.quant_act_static(x[m:m + 1], s[m])
        assert np.array_equal(qs[0], q[m]) and ss[0] == s[m]


def test_static_exact_quotients_power_of_two_scale():
    """x = j/8 with s = 1/4: every quotient x/s = j/2 is exact, so the code is Python's
    round-half-to-even of j/2, saturated at +-127 outside the calibrated range."""
    j = np.arange(-300, 301)
    x = (j.astype(np.float64) / 8).astype(F32)
    q, sx = O.quant_act_static(x[None, :], F32(0.25))
    assert q[0].tolist() == [max(-127, min(127, round(v / 2))) for v in j.tolist()]
    assert sx.tolist() == [0.25]
    # non-finite and overflowing quotients saturate; NaN gets code 0
    sp, _ = O.quant_act_static(np.array([[np.nan, np.inf, -np.inf, 3e38, -3e38, 0.0]], F32), F32(1e-3))
    assert sp[0].tolist() == [0, 127, -127, 127, -127, 0]
    # a scale that is not finite and positive gives zero codes and is passed through
    for bad in (0.0, -1.0, np.inf):
        qb, sb = O.quant_act_static(x[None, :], F32(bad))
        assert not qb.any() and sb[0] == F32(bad)


def test_calibrated_scale_is_largest_row_scale():
    """The batch's max|x| is the largest row abs-max, and division by 127 is monotone, so the
    calibrated scale is the largest per-token scale; the tiny case is exact: 127 / 127 = 1."""
    rs = np.random.default_rng(6)
    x = (rs.standard_normal((9, 40)) * rs.uniform(0.1, 10, (9, 1))).astype(F32)
    assert O.calibrate_act_scale(x) == O.quant_act(x)[1].max()
    assert O.calibrate_act_scale(np.array([[1.0, -127.0], [3.0, 0.5]], F32)) == F32(1.0)


def test_moe_static_scales_reduce_to_dynamic_layer():
    """One routed row per expert through a permuted routing: giving each expert the dynamic
    scales of its one row reproduces the dynamic layer exactly; handing the gate/up scales to
    the neighbouring experts does not (the scale is looked up by expert, not by token)."""
    T, E, H, I, g = 5, 5, 64, 32, 32
    ids = np.array([[3], [0], [4], [1], [2]], np.int32)
    w = np.array([[0.7], [1.0], [0.3], [0.9], [0.5]], F32)
    rs = np.random.default_rng(8)
    x = W.bf16_values(W.to_bf16((rs.standard_normal((T, H)) * rs.uniform(0.5, 8, (T, 1))).astype(F32)))
    qw = {e: O.quant_weight(W.random_weights(40 + e, H, 2 * I, 0.2), g, True) +
          O.quant_weight(W.random_weights(60 + e, I, H, 0.2), g, False) for e in range(E)}
    dyn = O.moe_layer(x, ids, w, lambda e: qw[e], E, I, g)
    s_gu, s_dn = np.empty(E, F32), np.empty(E, F32)
    for t in range(T):
        e = ids[t, 0]
        s_gu[e] = dyn["sx"][t]
        s_dn[e] = dyn["sh"][dyn["inv"][t, 0]]
    st = O.moe_layer(x, ids, w, lambda e: qw[e], E, I, g, s_gu=s_gu, s_dn=s_dn)
    assert np.array_equal(st["gu"], dyn["gu"]) and np.array_equal(st["hq"], dyn["hq"])
    assert np.array_equal(st["sh"], dyn["sh"]) and np.array_equal(st["out64"], dyn["out64"])
    off = O.moe_layer(x, ids, w, lambda e: qw[e], E, I, g, s_gu=np.roll(s_gu, 1), s_dn=s_dn)
    assert not np.array_equal(off["gu"], dyn["gu"])


# ------------------------------------------------------------------ binary16 weight scales
def _f16_spacing(x):
    """Spacing of the binary16 grid at |x|: 2^(e - 10) for |x| in [2^e, 2^(e+1)), 2^-24 below 2^-14."""
    x = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(x, 2.0 ** -14)))
    return 2.0 ** (e - 10)


@pytest.mark.parametrize("g,asym", [(64, False), (128, True), (32, True)])
def test_weight_fp16_scales(g, asym):
    """The stored scale is torch's float32 -> float16 rounding of the float32 scale (within half
    a binary16 step of it), and the codes obey the RTN invariants against the stored scale."""
    rs = np.random.default_rng(g)
    K, N = 4 * g, 24
    w = (rs.standard_normal((K, N)) * rs.uniform(1e-4, 3.0, (1, N))).astype(F32)
    w[:g, 3] = 0.0                                              # a zero group
    w[g:2 * g, 5] = 1e-5                                        # a scale in the subnormal range
    w[2 * g:3 * g, 7] = 1e-9                                    # a scale that rounds to 0
    c32, s32, z32 = O.quant_weight(w, g, asym)
    c16, s16, z16 = O.quant_weight(w, g, asym, scale_bits=16)
    ref = torch.from_numpy(s32).to(torch.float16).to(torch.float32).numpy()
    assert np.array_equal(s16, ref)
    assert np.all(np.abs(s16.astype(np.float64) - s32) <= 0.5 * _f16_spacing(s32))
    G = K // g
    sk = np.repeat(s16.astype(np.float64), g, axis=0)
    dk = np.where(sk > 0, sk, 1.0)
    zk = np.repeat(z16.astype(np.float64), g, axis=0) if asym else 0.0
    t = w / dk + zk                                             # the code before rounding
    lo, hi = (0, 15) if asym else (-7, 7)
    assert c16.min() >= lo and c16.max() <= hi
    inside = (sk > 0) & (t >= lo) & (t <= hi)
    err = np.abs(sk * (c16 - zk) - w)
    assert np.all(err[inside] <= 0.5 * sk[inside] * (1 + 1e-6))   # round to nearest on the stored scale
    assert np.all(c16[(sk > 0) & (t >= hi + 0.5)] == hi) and np.all(c16[(sk > 0) & (t <= lo - 0.5)] == lo)
    assert s16[0, 3] == 0 and not c16[:g, 3].any()              # the zero group
    assert s16.shape == (G, N) and 0 < s16[1, 5] < 2.0 ** -14   # the subnormal binary16 scale
    assert s32[2, 7] > 0 and s16[2, 7] == 0 and not c16[2 * g:3 * g, 7].any()   # underflow: zero codes


def test_weight_fp16_scales_identity_and_range():
    """Weights whose float32 scales are binary16 values (max|w| / 7 a power of two) give the same
    codes and scales either way; a scale past 65504 is an error."""
    rs = np.random.default_rng(3)
    top = 7.0 * 2.0 ** rs.integers(-12, 4, 8)                    # column maxima: max|w| / 7 exact
    w = (rs.uniform(-1, 1, (128, 8)) * top).astype(F32)
    w[0] = top
    c32, s32, _ = O.quant_weight(w, 128, False)
    c16, s16, _ = O.quant_weight(w, 128, False, scale_bits=16)
    assert np.array_equal(c32, c16) and np.array_equal(s32, s16)
    with pytest.raises(ValueError):
        O.quant_weight(np.full((64, 1), 7.0 * 70000.0, F32), 64, False, scale_bits=16)


def test_moe_per_expert_group_size_is_the_dense_chain_per_expert():
    """One routed row per expert (weight 1), experts at group sizes 32, 64 and 128: each output
    row is the dense chain quant_act -> gemm -> bf16 -> silu_mul_quant -> gemm -> bf16 at its
    own expert's group size."""
    T, E, H, I = 3, 3, 128, 128
    gs = [64, 128, 32]
    ids = np.array([[2], [0], [1]], np.int32)
    w = np.ones((T, 1), F32)
    rs = np.random.default_rng(12)
    x = W.bf16_values(W.to_bf16((rs.standard_normal((T, H)) * 3).astype(F32)))
    qw = {e: O.quant_weight(W.random_weights(70 + e, H, 2 * I, 0.2), gs[e], e == 0) +
          O.quant_weight(W.random_weights(80 + e, I, H, 0.2), gs[e], e == 0) for e in range(E)}
    out = O.moe_layer(x, ids, w, lambda e: qw[e], E, I, gs)
    for t in range(T):
        e = int(ids[t, 0])
        cg, sg, zg, cd, sd, zd = qw[e]
        q, s = O.quant_act(x[t:t + 1])
        gu = O.bf16_rne(O.gemm(q, s, cg, sg, zg, gs[e]))
        hq, sh = O.silu_mul_quant(gu)
        y = O.bf16_rne(O.gemm(hq, sh, cd, sd, zd, gs[e]))
        assert np.array_equal(out["out"][t], O.bf16_rne(y[0].astype(np.float64)))
