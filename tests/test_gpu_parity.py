"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Integer work (activation codes, per-group INT32 partials, routing permutation) must match
bit for bit; floating outputs pass the gates of gpu_cases.check_float_output."""
import numpy as np
import pytest
import torch

import moe_token_int8_amd as L
import oracle as O
import workloads as W
from gpu_cases import (DEV, SILU_TIE_WINDOW, bf16_ulp, check_float_output, check_moe as _check_moe, device_blob, gpu_quant,
                       moe_experts_codes as _moe_experts_codes, moe_experts_rtn as _moe_experts_rtn,
                       run_moe_forward as _run_moe_forward, sample_tokens)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.lib()


def _print(*a):
    print(*a, flush=True)


# ---------------------------------------------------------------- activation quantization
@pytest.mark.parametrize("M,K,dist,outl,oscale,seed", [
    (16, 1024, "normal", 4, 20.0, 101),        # single Linear input
    (1, 4096, "normal", 4, 50.0, 102),         # decode shapes
    (8, 4096, "normal", 4, 50.0, 102),
    (32, 4096, "normal", 4, 50.0, 102),
    (37, 2064, "normal", 0, 1.0, 7),           # ragged rows, K not a power of two
    (64, 7168, "student_t3", 0, 1.0, 105),     # heavy-tailed MoE decode input
    (512, 4096, "normal", 0, 1.0, 104),
    (3, 16, "normal", 0, 1.0, 9),              # smallest K
])
def test_quant_act_bit_exact(M, K, dist, outl, oscale, seed):
    _print(f"quant_act M={M} K={K} {dist}")
    Xb = W.random_activations(seed, M, K, dist, outl, oscale)
    Xq, sx = gpu_quant(Xb)
    q, s = O.quant_act(W.bf16_values(Xb))
    assert np.array_equal(Xq.cpu().numpy(), q)
    assert np.array_equal(sx.cpu().numpy().view(np.uint32), s.view(np.uint32))


def test_quant_act_full_prefill_rows():
    """Both prefill inputs at full size ([4096, 4096] and [4096, 14336])."""
    for cfg in (W.C3_UP, W.C3_DOWN):
        _print(f"quant_act {cfg.name}")
        Xb = W.random_activations(cfg.seed + 7919, cfg.M, cfg.K)
        Xq, sx = gpu_quant(Xb)
        q, s = O.quant_act(W.bf16_values(Xb))
        assert np.array_equal(Xq.cpu().numpy(), q)
        assert np.array_equal(sx.cpu().numpy().view(np.uint32), s.view(np.uint32))


def test_quant_act_edge_rows_and_strides():
    x = W.bf16_values(W.random_activations(3, 6, 64))
    x[1] = 0.0
    x[2, 5] = np.nan
    x[3, 7] = np.inf
    x[4] = 1e-40                            # subnormal row: scale underflows towards 0
    x[5, :] = 0.0
    x[5, 0] = -3.0
    big = torch.zeros((6, 96), dtype=torch.bfloat16)
    big[:, :64] = torch.from_numpy(x).to(torch.bfloat16)
    Xd = big.to(DEV)[:, :64]                # row stride 96 > K
    Xq = torch.empty((6, 64), dtype=torch.int8, device=DEV)
    sx = torch.empty(6, dtype=torch.float32, device=DEV)
    L.w4a8_quant_act(Xd, Xq, sx)
    q, s = O.quant_act(W.bf16_values(big[:, :64]))
    assert np.array_equal(Xq.cpu().numpy(), q)
    g = sx.cpu().numpy()
    assert np.array_equal(np.isnan(g), np.isnan(s))
    assert np.array_equal(g[~np.isnan(g)].view(np.uint32), s[~np.isnan(s)].view(np.uint32))


def test_quant_act_near_ties_take_the_exact_division():
    """Rows built so that many x/s land within a few ulps of .5: the fast reciprocal path
    must hand these to the IEEE division."""
    rs = np.random.default_rng(0)
    amax = np.float32(1.0)
    s = np.float32(amax / np.float32(127))
    halves = (rs.integers(-126, 126, size=(8, 1024)) + 0.5).astype(np.float64)
    x = (halves * np.float64(s)).astype(np.float32)
    x[:, 0] = amax
    xb = W.to_bf16(x)
    Xq, sx = gpu_quant(xb)
    q, so = O.quant_act(W.bf16_values(xb))
    assert np.array_equal(Xq.cpu().numpy(), q)


# ---------------------------------------------------------------- GEMM partials (exact)
@pytest.mark.parametrize("M,K,N,g,asym", [
    (16, 1024, 1024, 128, False),              # the single-Linear shape
    (37, 512, 40, 64, True),                   # ragged M, ragged N (padded tile)
    (5, 384, 48, 128, True),
    (20, 256, 33, 64, False),
    (1, 4096, 256, 128, False),
    (64, 7168, 64, 64, True),                  # MoE decode expert shape (slice of N)
    # one case per decode kernel shape: 32-row tile (one chunk, several chunks), 16-row
    # long-K tile (several chunks), 16-row tiles at M * K <= 8192 (one chunk of 8 and 64
    # superblocks)
    (32, 4096, 512, 128, False),
    (32, 8192, 64, 128, True),
    (12, 14336, 48, 128, False),
    (2, 4096, 64, 64, True),
    (1, 8192, 80, 128, True),
])
def test_partials_bit_exact(M, K, N, g, asym):
    _print(f"partials M={M} K={K} N={N} g={g} asym={asym}")
    Xb = W.random_activations(M * 7 + K, M, K, outlier_cols=2, outlier_scale=20.0)
    Wt = W.random_weights(K + N, K, N)
    Wt[:g, 0] = 0.0
    d = L.desc(K, N, g, asym)
    blob = device_blob(d, L.w4a8_pack(d, Wt))
    Xq, sx = gpu_quant(Xb)
    P = torch.full((M, N, K // g), -7, dtype=torch.int32, device=DEV)
    L.w4a8_gemm_partials(Xq, blob, d, P)
    q, s = O.quant_act(W.bf16_values(Xb))
    codes, scales, zeros = O.quant_weight(Wt, g, asym)
    assert np.array_equal(P.cpu().numpy(), O.gemm_partials(q, codes, zeros, g))


def test_partials_decode_full_width():
    cfg = W.with_decode_m(W.C2, 8)
    Xb, Wt = W.dense_inputs(cfg)
    d = L.desc(cfg.K, cfg.N, cfg.group_size, cfg.asymmetric)
    blob = device_blob(d, L.w4a8_pack(d, Wt))
    Xq, _ = gpu_quant(Xb)
    P = torch.empty((8, cfg.N, cfg.K // cfg.group_size), dtype=torch.int32, device=DEV)
    L.w4a8_gemm_partials(Xq, blob, d, P)
    q, _ = O.quant_act(W.bf16_values(Xb))
    codes, _, zeros = O.quant_weight(Wt, cfg.group_size, cfg.asymmetric)
    assert np.array_equal(P.cpu().numpy(), O.gemm_partials(q, codes, zeros, cfg.group_size))


# ---------------------------------------------------------------- GEMM outputs
def _gemm_case(Xb, Wt, g, asym):
    M, K = Xb.shape
    N = Wt.shape[1]
    d = L.desc(K, N, g, asym)
    blob = device_blob(d, L.w4a8_pack(d, Wt))
    Xq, sx = gpu_quant(Xb)
    y32 = torch.empty((M, N), dtype=torch.float32, device=DEV)
    ybf = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    L.w4a8_gemm(Xq, sx, blob, d, y32, L.W4A8_OUT_F32)
    L.w4a8_gemm(Xq, sx, blob, d, ybf, L.W4A8_OUT_BF16)
    q, s = O.quant_act(W.bf16_values(Xb))
    codes, scales, zeros = O.quant_weight(Wt, g, asym)
    Y64 = O.gemm(q, s, codes, scales, zeros, g)
    return check_float_output(y32.cpu().numpy(), ybf.float().cpu().numpy(), Y64)


@pytest.mark.parametrize("M", [1, 8, 32])
def test_gemm_decode_shapes(M):
    cfg = W.with_decode_m(W.C2, M)
    _print(f"gemm {cfg.name}")
    Xb, Wt = W.dense_inputs(cfg)
    r = _gemm_case(Xb, Wt, cfg.group_size, cfg.asymmetric)
    _print(r)


def test_gemm_single_linear():
    Xb, Wt = W.dense_inputs(W.C1)
    _print(_gemm_case(Xb, Wt, 128, False))


@pytest.mark.parametrize("M,K,N,g,asym", [(37, 512, 40, 64, True), (17, 1024, 96, 128, True),
                                          (48, 256, 17, 64, False), (2, 128, 16, 128, True)])
def test_gemm_ragged(M, K, N, g, asym):
    Xb = W.random_activations(M + N, M, K, outlier_cols=1, outlier_scale=30.0)
    Wt = W.random_weights(N + 3, K, N)
    _print(_gemm_case(Xb, Wt, g, asym))


def test_gemm_zero_and_nan_rows():
    x = W.bf16_values(W.random_activations(4, 5, 256))
    x[1] = 0.0
    x[3, 9] = np.nan
    Xb = W.to_bf16(x)
    Wt = W.random_weights(5, 256, 32)
    d = L.desc(256, 32, 128, True)
    blob = device_blob(d, L.w4a8_pack(d, Wt))
    Xq, sx = gpu_quant(Xb)
    y = torch.empty((5, 32), dtype=torch.float32, device=DEV)
    L.w4a8_gemm(Xq, sx, blob, d, y, L.W4A8_OUT_F32)
    y = y.cpu().numpy()
    assert np.all(y[1] == 0) and np.all(np.isnan(y[3]))
    assert np.all(np.isfinite(y[[0, 2, 4]]))


# ---------------------------------------------------------------- fused quant + GEMM
@pytest.mark.parametrize("M,K,N,g,asym", [(1, 4096, 14336, 128, False), (8, 4096, 14336, 128, False),
                                          (16, 4096, 1024, 128, True), (5, 512, 40, 64, True),
                                          (3, 1024, 33, 128, False), (20, 256, 64, 64, True),
                                          (2, 7168, 64, 64, True), (2, 4096, 1024, 64, True),
                                          (4, 2048, 96, 128, False), (1, 7168, 96, 64, True),
                                          (1, 8192, 80, 128, False), (16, 512, 72, 128, True),
                                          (7, 384, 40, 128, True), (16, 128, 24, 64, False)])
def test_linear_matches_quant_then_gemm(M, K, N, g, asym):
    """w4a8_linear (one kernel for M <= 16 and M * K <= 8192) equals quant_act followed by gemm
    bit for bit, writes the same activation codes and scales, and its outputs pass the float
    gates against the oracle."""
    Xb = W.random_activations(M * 3 + K + N, M, K, outlier_cols=2, outlier_scale=40.0)
    x = W.bf16_values(Xb)
    if M > 2:
        x[1] = 0.0
        Xb = W.to_bf16(x)
    Wt = W.random_weights(K + 2 * N, K, N)
    d = L.desc(K, N, g, asym)
    blob = device_blob(d, L.w4a8_pack(d, Wt))
    X = Xb.to(DEV)
    outs = {}
    for dt, tdt in ((L.W4A8_OUT_F32, torch.float32), (L.W4A8_OUT_BF16, torch.bfloat16)):
        Xq1, sx1 = gpu_quant(Xb)
        Y1 = torch.empty((M, N), dtype=tdt, device=DEV)
        L.w4a8_gemm(Xq1, sx1, blob, d, Y1, dt)
        Xq2 = torch.full((M, K), 99, dtype=torch.int8, device=DEV)
        sx2 = torch.full((M,), -1.0, dtype=torch.float32, device=DEV)
        Y2 = torch.empty((M, N), dtype=tdt, device=DEV)
        L.w4a8_linear(X, blob, d, Y2, Xq2, sx2, dt)
        assert torch.equal(Xq1, Xq2)
        assert torch.equal(sx1.view(torch.int32), sx2.view(torch.int32))
        assert torch.equal(Y1.view(torch.int16 if tdt == torch.bfloat16 else torch.int32),
                           Y2.view(torch.int16 if tdt == torch.bfloat16 else torch.int32))
        outs[dt] = Y2.float().cpu().numpy()
    q, s = O.quant_act(x)
    assert np.array_equal(Xq2.cpu().numpy(), q)
    assert np.array_equal(sx2.cpu().numpy().view(np.uint32), s.view(np.uint32))
    codes, scales, zeros = O.quant_weight(Wt, g, asym)
    Y64 = O.gemm(q, s, codes, scales, zeros, g)
    _print(check_float_output(outs[L.W4A8_OUT_F32], outs[L.W4A8_OUT_BF16], Y64))


# ---------------------------------------------------------------- prefill-size GEMMs
@pytest.mark.parametrize("M,K,N,g,asym", [(300, 1024, 300, 128, True), (257, 512, 129, 64, False),
                                          (64, 384, 256, 128, False), (513, 256, 48, 64, True)])
def test_prefill_partials_bit_exact(M, K, N, g, asym):
    _print(f"prefill partials M={M} K={K} N={N} g={g} asym={asym}")
    Xb = W.random_activations(M + K + N, M, K, outlier_cols=3, outlier_scale=25.0)
    Wt = W.random_weights(K * 3 + N, K, N)
    d = L.desc(K, N, g, asym)
    assert L.w4a8_kernel_name(d, M).startswith("w4a8_prefill")
    blob = device_blob(d, L.w4a8_pack(d, Wt))
    Xq, _ = gpu_quant(Xb)
    P = torch.full((M, N, K // g), -7, dtype=torch.int32, device=DEV)
    L.w4a8_gemm_partials(Xq, blob, d, P)
    q, _ = O.quant_act(W.bf16_values(Xb))
    codes, _, zeros = O.quant_weight(Wt, g, asym)
    assert np.array_equal(P.cpu().numpy(), O.gemm_partials(q, codes, zeros, g))


@pytest.mark.parametrize("M,K,N,g,asym", [(300, 1024, 272, 128, True), (257, 512, 129, 64, False),
                                          (33, 2048, 64, 128, True), (1000, 256, 1000, 64, True)])
def test_prefill_outputs(M, K, N, g, asym):
    Xb = W.random_activations(M * 5 + N, M, K, outlier_cols=2, outlier_scale=30.0)
    Wt = W.random_weights(N * 7 + K, K, N)
    _print(_gemm_case(Xb, Wt, g, asym))


@pytest.mark.parametrize("cfg", [W.C3_UP, W.C3_DOWN], ids=lambda c: c.name)
def test_prefill_full_size_sampled_rows(cfg):
    """The projection pair at full size (M=4096) in the benchmark's launch configuration;
    the oracle checks 48 sampled rows (every column)."""
    _print(f"prefill full {cfg.name}")
    Xb, Wt = W.dense_inputs(cfg)
    d = L.desc(cfg.K, cfg.N, cfg.group_size, cfg.asymmetric)
    blob = device_blob(d, L.w4a8_pack(d, Wt))
    Xq, sx = gpu_quant(Xb)
    y32 = torch.empty((cfg.M, cfg.N), dtype=torch.float32, device=DEV)
    ybf = torch.empty((cfg.M, cfg.N), dtype=torch.bfloat16, device=DEV)
    L.w4a8_gemm(Xq, sx, blob, d, y32, L.W4A8_OUT_F32)
    L.w4a8_gemm(Xq, sx, blob, d, ybf, L.W4A8_OUT_BF16)
    rows = np.sort(np.random.default_rng(cfg.seed).choice(cfg.M, 48, replace=False))
    rows[0], rows[-1] = 0, cfg.M - 1
    q, s = O.quant_act(W.bf16_values(Xb)[rows])
    assert np.array_equal(Xq.cpu().numpy()[rows], q)
    codes, scales, zeros = O.quant_weight(Wt, cfg.group_size, cfg.asymmetric)
    Y64 = O.gemm(q, s, codes, scales, zeros, cfg.group_size)
    _print(check_float_output(y32.cpu().numpy()[rows], ybf.float().cpu().numpy()[rows], Y64))


# ---------------------------------------------------------------- MoE pieces
def _routing(seed, T, E, k, zipf=0.0):
    cfg = W.MoEConfig("t", T, 128, 64, E, k, 64, False, seed, zipf_s=zipf)
    return W.moe_routing(cfg)


@pytest.mark.parametrize("T,E,k,zipf", [(512, 64, 6, 1.1), (64, 256, 8, 0.0), (5, 3, 2, 0.0), (1, 8, 1, 0.0),
                                        (300, 1024, 4, 0.0), (3000, 64, 8, 1.1), (2048, 8, 8, 0.0)])
def test_moe_align_exact(T, E, k, zipf):
    """Stable counting sort against the oracle; the last two cases (24000 and 16384 routed
    rows) are past and at the size where the ids are staged in LDS."""
    ids, _ = _routing(T + E, T, E, k, zipf)
    rows_ref, off_ref, inv_ref = O.moe_align(ids, E)
    ids_d = torch.from_numpy(ids).to(DEV)
    rows = torch.full((T * k,), -5, dtype=torch.int32, device=DEV)
    off = torch.full((E + 1,), -5, dtype=torch.int32, device=DEV)
    inv = torch.full((T, k), -5, dtype=torch.int32, device=DEV)
    L.w4a8_moe_align(ids_d, E, rows, off, inv)
    assert np.array_equal(off.cpu().numpy(), off_ref)
    assert np.array_equal(rows.cpu().numpy(), rows_ref)
    assert np.array_equal(inv.cpu().numpy(), inv_ref)


def test_silu_mul_quant_vs_oracle():
    """Codes may differ by 1 only where the float64 value of h/s lies within SILU_TIE_WINDOW
    (1e-4, derived from the kernel's float32 error bound) of a rounding boundary: the GPU's
    expf and the oracle's float64 exp differ by an ulp."""
    for R, I in [(3072, 1408), (512, 2048), (7, 32)]:
        rs = np.random.default_rng(R)
        gu = W.to_bf16((rs.standard_normal((R, 2 * I)) * 2).astype(np.float32))
        g = gu.to(DEV)
        Hq = torch.empty((R, I), dtype=torch.int8, device=DEV)
        sh = torch.empty(R, dtype=torch.float32, device=DEV)
        L.w4a8_silu_mul_quant(g, Hq, sh)
        q, s = O.silu_mul_quant(W.bf16_values(gu))
        sg = sh.cpu().numpy()
        assert np.all(np.abs(sg.astype(np.float64) - s) <= 4 * np.spacing(s))
        qg = Hq.cpu().numpy().astype(np.int64)
        diff = np.abs(qg - q.astype(np.int64))
        assert diff.max() <= 1
        h = O.silu_mul(W.bf16_values(gu))
        t = h / s.astype(np.float64)[:, None]
        near = np.abs(np.abs(t - np.floor(t)) - 0.5) < SILU_TIE_WINDOW
        assert np.all(near[diff > 0])
        _print(f"silu R={R} I={I}: {int((diff > 0).sum())} near-tie code differences of {diff.size}")


def test_combine_vs_oracle():
    T, k, H = 64, 8, 7168
    ids, w = _routing(3, T, 256, k)
    _, _, inv = O.moe_align(ids, 256)
    rs = np.random.default_rng(1)
    yd = W.to_bf16(rs.standard_normal((T * k, H)).astype(np.float32))
    out = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    L.w4a8_moe_combine(yd.to(DEV), torch.from_numpy(inv).to(DEV), torch.from_numpy(w).to(DEV), out)
    ydv = W.bf16_values(yd).astype(np.float64)
    ref64 = np.zeros((T, H))
    for j in range(k):
        ref64 += w[:, j:j + 1].astype(np.float64) * ydv[inv[:, j]]
    got = out.float().cpu().numpy()
    ref = O.bf16_rne(ref64)
    diff = np.abs(got - ref)
    assert np.all(diff <= bf16_ulp(ref) + 1e-6)
    assert np.linalg.norm(got - ref64) / np.linalg.norm(ref64) < 3e-3


@pytest.mark.parametrize("T,E,k,H,I,g,asym", [(9, 3, 2, 256, 128, 64, True), (40, 8, 2, 512, 256, 128, False),
                                              (33, 16, 4, 256, 128, 128, True)])
def test_moe_forward_small_rtn(T, E, k, H, I, g, asym):
    cfg = W.MoEConfig("small", T, H, I, E, k, g, asym, 17 + T)
    ids, w = W.moe_routing(cfg)
    Xb = W.moe_activations(cfg)
    dgu, dd, gud, ddv, qw = _moe_experts_rtn(cfg, set(ids.ravel().tolist()))
    out, ws = _run_moe_forward(cfg, Xb, ids, w, gud, ddv)
    ref = O.moe_layer(W.bf16_values(Xb), ids, w, lambda e: qw[e], E, I, g)
    _check_moe(out, ref, qw, cfg.group_size)


def test_moe_gemm_grouped_matches_per_expert_oracle():
    """Gate/up grouped GEMM alone on the 64-expert top-6 routing (Zipf-skewed: one expert
    gets most rows), float32 output, with random codes."""
    cfg = W.C4
    ids, w = W.moe_routing(cfg)
    touched = set(ids.ravel().tolist())
    dgu, dd, gud, ddv, qw = _moe_experts_codes(cfg, touched, 4)
    Xb = W.moe_activations(cfg)
    Xq, sx = gpu_quant(Xb)
    T, k = ids.shape
    rows = torch.empty(T * k, dtype=torch.int32, device=DEV)
    off = torch.empty(cfg.E + 1, dtype=torch.int32, device=DEV)
    inv = torch.empty((T, k), dtype=torch.int32, device=DEV)
    L.w4a8_moe_align(torch.from_numpy(ids).to(DEV), cfg.E, rows, off, inv)
    Y = torch.empty((T * k, 2 * cfg.I), dtype=torch.float32, device=DEV)
    L.w4a8_moe_gemm(Xq, sx, rows, k, off, cfg.E, T * k, gud.blob, gud.stride, dgu, Y, L.W4A8_OUT_F32)
    Ybf = torch.empty((T * k, 2 * cfg.I), dtype=torch.bfloat16, device=DEV)
    L.w4a8_moe_gemm(Xq, sx, rows, k, off, cfg.E, T * k, gud.blob, gud.stride, dgu, Ybf, L.W4A8_OUT_BF16)
    q, s = O.quant_act(W.bf16_values(Xb))
    srt, offs, _ = O.moe_align(ids, cfg.E)
    Y = Y.cpu().numpy()
    Ybf = Ybf.float().cpu().numpy()
    Y64 = np.zeros(Y.shape)
    for e in touched:
        a, b = offs[e], offs[e + 1]
        toks = srt[a:b] // k
        c, sc, z = qw[e][:3]
        Y64[a:b] = O.gemm(q[toks], s[toks], c, sc, z, cfg.group_size)
    _print(check_float_output(Y, Ybf, Y64))


@pytest.mark.parametrize("g,asym,K,sbits", [(64, True, 256, 32), (128, False, 256, 32), (64, True, 4608, 32),
                                            (128, False, 4608, 32), (64, False, 1024, 32), (64, True, 768, 16),
                                            (128, True, 512, 16)])
def test_moe_gemm_hot_expert_paths(g, asym, K, sbits):
    """Grouped GEMM where expert 0 owns 280 routed rows (three 128-row MFMA tiles, the third
    ragged), expert 1 about 160 (two tiles) and the others fewer than 96 (the MFMA-tile cut); with and without the row gather; float32 and binary16 scales.  The
    others run on the grouped streaming kernel (K <= 4096) or on the streaming decode kernel
    (K = 4608)."""
    T, k, E, N = 300, 2, 5, 96
    t = np.arange(T)
    ids = np.stack([np.where(t < 280, 0, 1 + t % 4), np.where(t < 150, 1, 2 + t % 3)], axis=1).astype(np.int32)
    dup = ids[:, 0] == ids[:, 1]
    ids[dup, 1] = np.where(ids[dup, 0] == 2, 3, 2)
    cnt = np.bincount(ids.ravel(), minlength=E)
    assert cnt[0] > 256 and 128 <= cnt[1] < 256 and cnt[2:].max() < 96 and cnt.min() > 0
    d = L.desc(K, N, g, asym, scale_bits=sbits)
    host, qw = {}, {}
    for e in range(E):
        c = W.random_codes(31 * g + e, K, N, g, asym)
        if sbits == 16:                                 # scales the binary16 field holds exactly
            c = (c[0], c[1].astype(np.float16).astype(np.float32), c[2])
        host[e] = L.w4a8_pack_codes(d, *c)
        qw[e] = c
    dev = L.experts_to_device(d, E, host)
    Xb = W.random_activations(5, T, K, outlier_cols=2, outlier_scale=20.0)
    Xq, sx = gpu_quant(Xb)
    rows = torch.empty(T * k, dtype=torch.int32, device=DEV)
    off = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    inv = torch.empty((T, k), dtype=torch.int32, device=DEV)
    L.w4a8_moe_align(torch.from_numpy(ids).to(DEV), E, rows, off, inv)
    q, s = O.quant_act(W.bf16_values(Xb))
    srt, offs, _ = O.moe_align(ids, E)
    # gathered rows (gate/up form)
    Y = torch.empty((T * k, N), dtype=torch.float32, device=DEV)
    Ybf = torch.empty((T * k, N), dtype=torch.bfloat16, device=DEV)
    L.w4a8_moe_gemm(Xq, sx, rows, k, off, E, T * k, dev.blob, dev.stride, d, Y, L.W4A8_OUT_F32)
    L.w4a8_moe_gemm(Xq, sx, rows, k, off, E, T * k, dev.blob, dev.stride, d, Ybf, L.W4A8_OUT_BF16)
    Y64 = np.zeros((T * k, N))
    for e in range(E):
        a, b = offs[e], offs[e + 1]
        toks = srt[a:b] // k
        Y64[a:b] = O.gemm(q[toks], s[toks], *qw[e], g)
    _print(check_float_output(Y.cpu().numpy(), Ybf.float().cpu().numpy(), Y64))
    # rows already in expert order (down form): the sorted rows' codes and scales
    tok = rows.long().cpu() // k                          # sorted row -> token
    assert int(tok.min()) >= 0 and int(tok.max()) < T
    tok = tok.to(DEV)
    Xs, ss = Xq[tok].contiguous(), sx[tok].contiguous()
    L.w4a8_moe_gemm(Xs, ss, None, k, off, E, T * k, dev.blob, dev.stride, d, Y, L.W4A8_OUT_F32)
    L.w4a8_moe_gemm(Xs, ss, None, k, off, E, T * k, dev.blob, dev.stride, d, Ybf, L.W4A8_OUT_BF16)
    _print(check_float_output(Y.cpu().numpy(), Ybf.float().cpu().numpy(), Y64))


@pytest.mark.parametrize("K,g,asym", [(4096, 64, True), (3200, 64, True), (4096, 128, False), (4096, 64, False)])
def test_moe_gemm_wide_stream_tiles(K, g, asym):
    """Grouped streaming kernel on launches of many workgroups (1024 experts, 512 rows, so
    16-row tiles, and 2048 columns): each workgroup streams 32 column tiles.  At g = 64 with
    zero points this is the instance that runs its column groups as a loop over pairs; K = 3200
    leaves the last slice partly past K.  8 experts with 64 rows each (4 row tiles), the others
    empty."""
    T, k, E, N = 256, 2, 1024, 2048
    t = np.arange(T)
    ids = np.stack([(t % 4) * 256, (t % 4) * 256 + 1], axis=1).astype(np.int32)
    cnt = np.bincount(ids.ravel(), minlength=E)
    assert cnt.max() == 64 and int((cnt > 0).sum()) == 8
    _print(f"wide streaming tiles K={K} g={g} asym={asym}")
    d = L.desc(K, N, g, asym)
    host, qw = {}, {}
    for e in np.flatnonzero(cnt):
        qw[e] = W.random_codes(17 * g + int(e), K, N, g, asym)
        host[int(e)] = L.w4a8_pack_codes(d, *qw[e])
    dev = L.experts_to_device(d, E, host)
    Xb = W.random_activations(6, T, K, outlier_cols=2, outlier_scale=20.0)
    Xq, sx = gpu_quant(Xb)
    rows = torch.empty(T * k, dtype=torch.int32, device=DEV)
    off = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    inv = torch.empty((T, k), dtype=torch.int32, device=DEV)
    L.w4a8_moe_align(torch.from_numpy(ids).to(DEV), E, rows, off, inv)
    Y = torch.empty((T * k, N), dtype=torch.float32, device=DEV)
    Ybf = torch.empty((T * k, N), dtype=torch.bfloat16, device=DEV)
    L.w4a8_moe_gemm(Xq, sx, rows, k, off, E, T * k, dev.blob, dev.stride, d, Y, L.W4A8_OUT_F32)
    L.w4a8_moe_gemm(Xq, sx, rows, k, off, E, T * k, dev.blob, dev.stride, d, Ybf, L.W4A8_OUT_BF16)
    q, s = O.quant_act(W.bf16_values(Xb))
    srt, offs, _ = O.moe_align(ids, E)
    Y64 = np.zeros((T * k, N))
    for e in qw:
        a, b = offs[e], offs[e + 1]
        toks = srt[a:b] // k
        Y64[a:b] = O.gemm(q[toks], s[toks], *qw[e], g)
    _print(check_float_output(Y.cpu().numpy(), Ybf.float().cpu().numpy(), Y64))


@pytest.mark.parametrize("K,N,g,asym", [(7168, 400, 64, True), (4608, 272, 128, False), (5120, 128, 64, False)])
def test_moe_gemm_tile_groups(K, N, g, asym):
    """Grouped GEMM at 16-row tiles with K in (4096, 8192], where each workgroup streams
    several column-tile groups (the last one ragged when N is not a multiple of 128);
    gathered and already-sorted row forms against the oracle."""
    T, k, E = 20, 2, 6
    rng = np.random.default_rng(77 + K)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    d = L.desc(K, N, g, asym)
    host, qw = {}, {}
    for e in range(E):
        c = W.random_codes(K + 7 * e, K, N, g, asym)
        host[e] = L.w4a8_pack_codes(d, *c)
        qw[e] = c
    dev = L.experts_to_device(d, E, host)
    Xb = W.random_activations(11, T, K, outlier_cols=3, outlier_scale=30.0)
    Xq, sx = gpu_quant(Xb)
    rows = torch.empty(T * k, dtype=torch.int32, device=DEV)
    off = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    inv = torch.empty((T, k), dtype=torch.int32, device=DEV)
    L.w4a8_moe_align(torch.from_numpy(ids).to(DEV), E, rows, off, inv)
    q, s = O.quant_act(W.bf16_values(Xb))
    srt, offs, _ = O.moe_align(ids, E)
    Y64 = np.zeros((T * k, N))
    for e in range(E):
        a, b = offs[e], offs[e + 1]
        toks = srt[a:b] // k
        Y64[a:b] = O.gemm(q[toks], s[toks], *qw[e], g)
    Y = torch.empty((T * k, N), dtype=torch.float32, device=DEV)
    Ybf = torch.empty((T * k, N), dtype=torch.bfloat16, device=DEV)
    L.w4a8_moe_gemm(Xq, sx, rows, k, off, E, T * k, dev.blob, dev.stride, d, Y, L.W4A8_OUT_F32)
    L.w4a8_moe_gemm(Xq, sx, rows, k, off, E, T * k, dev.blob, dev.stride, d, Ybf, L.W4A8_OUT_BF16)
    _print(check_float_output(Y.cpu().numpy(), Ybf.float().cpu().numpy(), Y64))
    tok = rows.long().cpu() // k
    assert int(tok.min()) >= 0 and int(tok.max()) < T
    tok = tok.to(DEV)
    Xs, ss = Xq[tok].contiguous(), sx[tok].contiguous()
    L.w4a8_moe_gemm(Xs, ss, None, k, off, E, T * k, dev.blob, dev.stride, d, Y, L.W4A8_OUT_F32)
    L.w4a8_moe_gemm(Xs, ss, None, k, off, E, T * k, dev.blob, dev.stride, d, Ybf, L.W4A8_OUT_BF16)
    _print(check_float_output(Y.cpu().numpy(), Ybf.float().cpu().numpy(), Y64))


@pytest.mark.parametrize("T,k,E,K,N,g,asym", [(60, 2, 16, 2048, 200, 128, False),
                                                (60, 2, 16, 3072, 200, 64, True),
                                                (100, 2, 4, 4096, 144, 128, True),
                                                (100, 2, 4, 1408, 208, 128, False),
                                                (100, 2, 4, 2048, 144, 64, True)])
def test_moe_gemm_row_loop(T, k, E, K, N, g, asym):
    """Grouped GEMM where one expert holds several row tiles below the 128-row cut (about 50
    rows at 16-row tiles; about 70 at 32-row tiles, where for K <= 2048 one workgroup runs
    them in turn on the weights it holds); gathered and already-sorted rows against the
    oracle."""
    rng = np.random.default_rng(5 + K + E)
    t = np.arange(T)
    first = np.where(t < T // 2 if E == 4 else t < 50, 0, 1 + t % (E - 1))
    second = np.array([rng.choice([e for e in range(E) if e != f]) for f in first])
    ids = np.stack([first, second], axis=1).astype(np.int32)
    cnt = np.bincount(ids.ravel(), minlength=E)
    assert cnt.max() < 128 and cnt[0] >= 50
    d = L.desc(K, N, g, asym)
    host, qw = {}, {}
    for e in range(E):
        c = W.random_codes(3 * K + e, K, N, g, asym)
        host[e] = L.w4a8_pack_codes(d, *c)
        qw[e] = c
    dev = L.experts_to_device(d, E, host)
    Xb = W.random_activations(13, T, K, outlier_cols=2, outlier_scale=25.0)
    Xq, sx = gpu_quant(Xb)
    rows = torch.empty(T * k, dtype=torch.int32, device=DEV)
    off = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    inv = torch.empty((T, k), dtype=torch.int32, device=DEV)
    L.w4a8_moe_align(torch.from_numpy(ids).to(DEV), E, rows, off, inv)
    q, s = O.quant_act(W.bf16_values(Xb))
    srt, offs, _ = O.moe_align(ids, E)
    Y64 = np.zeros((T * k, N))
    for e in range(E):
        a, b = offs[e], offs[e + 1]
        toks = srt[a:b] // k
        Y64[a:b] = O.gemm(q[toks], s[toks], *qw[e], g)
    Y = torch.empty((T * k, N), dtype=torch.float32, device=DEV)
    Ybf = torch.empty((T * k, N), dtype=torch.bfloat16, device=DEV)
    L.w4a8_moe_gemm(Xq, sx, rows, k, off, E, T * k, dev.blob, dev.stride, d, Y, L.W4A8_OUT_F32)
    L.w4a8_moe_gemm(Xq, sx, rows, k, off, E, T * k, dev.blob, dev.stride, d, Ybf, L.W4A8_OUT_BF16)
    _print(check_float_output(Y.cpu().numpy(), Ybf.float().cpu().numpy(), Y64))
    tok = rows.long().cpu() // k
    assert int(tok.min()) >= 0 and int(tok.max()) < T
    tok = tok.to(DEV)
    Xs, ss = Xq[tok].contiguous(), sx[tok].contiguous()
    L.w4a8_moe_gemm(Xs, ss, None, k, off, E, T * k, dev.blob, dev.stride, d, Y, L.W4A8_OUT_F32)
    L.w4a8_moe_gemm(Xs, ss, None, k, off, E, T * k, dev.blob, dev.stride, d, Ybf, L.W4A8_OUT_BF16)
    _print(check_float_output(Y.cpu().numpy(), Ybf.float().cpu().numpy(), Y64))


def _grouped_vs_oracle(ids, E, K, N, g, asym, seed, bad=()):
    """Grouped GEMM on routing `ids` with random codes, gathered rows and already-sorted rows,
    float32 and bfloat16 outputs, against the per-expert oracle.  `bad`: positions of the sorted
    order whose gather entry is replaced by one that names no token (past the last, or
    negative); their output rows must be zeros."""
    T, k = ids.shape
    d = L.desc(K, N, g, asym)
    host, qw = {}, {}
    for e in range(E):
        c = W.random_codes(seed * 7 + e, K, N, g, asym)
        host[e] = L.w4a8_pack_codes(d, *c)
        qw[e] = c
    dev = L.experts_to_device(d, E, host)
    Xb = W.random_activations(seed, T, K, outlier_cols=2, outlier_scale=25.0)
    Xq, sx = gpu_quant(Xb)
    rows = torch.empty(T * k, dtype=torch.int32, device=DEV)
    off = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    inv = torch.empty((T, k), dtype=torch.int32, device=DEV)
    L.w4a8_moe_align(torch.from_numpy(ids).to(DEV), E, rows, off, inv)
    q, s = O.quant_act(W.bf16_values(Xb))
    srt, offs, _ = O.moe_align(ids, E)
    Y64 = np.zeros((T * k, N))
    for e in range(E):
        a, b = offs[e], offs[e + 1]
        toks = srt[a:b] // k
        Y64[a:b] = O.gemm(q[toks], s[toks], *qw[e], g)
    gather = rows
    if len(bad):
        gh = srt.astype(np.int32).copy()
        for i, r in enumerate(bad):
            gh[r] = T * k + 5 if i % 2 == 0 else -3
        Y64[list(bad)] = 0.0
        gather = torch.from_numpy(gh).to(DEV)
    Y = torch.full((T * k, N), 7.0, dtype=torch.float32, device=DEV)
    Ybf = torch.full((T * k, N), 7.0, dtype=torch.bfloat16, device=DEV)
    L.w4a8_moe_gemm(Xq, sx, gather, k, off, E, T * k, dev.blob, dev.stride, d, Y, L.W4A8_OUT_F32)
    L.w4a8_moe_gemm(Xq, sx, gather, k, off, E, T * k, dev.blob, dev.stride, d, Ybf, L.W4A8_OUT_BF16)
    _print(check_float_output(Y.cpu().numpy(), Ybf.float().cpu().numpy(), Y64))
    if len(bad):
        assert not torch.any(Y[list(bad)] != 0)
        return
    tok = (rows.long() // k).to(DEV)
    Xs, ss = Xq[tok].contiguous(), sx[tok].contiguous()
    L.w4a8_moe_gemm(Xs, ss, None, k, off, E, T * k, dev.blob, dev.stride, d, Y, L.W4A8_OUT_F32)
    L.w4a8_moe_gemm(Xs, ss, None, k, off, E, T * k, dev.blob, dev.stride, d, Ybf, L.W4A8_OUT_BF16)
    _print(check_float_output(Y.cpu().numpy(), Ybf.float().cpu().numpy(), Y64))


@pytest.mark.parametrize("T,E,K,N,g,asym", [(40, 4, 7168, 272, 64, True), (20, 4, 9216, 96, 128, False),
                                            (20, 3, 9216, 64, 64, True)])
def test_moe_gemm_streaming_fallback(T, E, K, N, g, asym):
    """Grouped shapes that the K-slice kernel does not take: 32-row tiles at K in (4096, 8192]
    (20 rows per expert) and any tile at K > 8192.  These run on the chunked decode kernel in its
    grouped form."""
    k = 2
    t = np.arange(T)
    ids = np.stack([t % E, (t + 1 + t // E) % E], axis=1).astype(np.int32)
    ids[ids[:, 0] == ids[:, 1], 1] = (ids[ids[:, 0] == ids[:, 1], 1] + 1) % E
    assert np.all(ids[:, 0] != ids[:, 1])
    _print(f"streaming fallback T={T} E={E} K={K} N={N} rows/E={T * k // E}")
    _grouped_vs_oracle(ids, E, K, N, g, asym, seed=K + N)


@pytest.mark.parametrize("T,E,K,N,g", [(300, 5, 256, 96, 64), (40, 4, 7168, 64, 64), (24, 6, 1024, 48, 128)])
def test_moe_gemm_gather_out_of_range(T, E, K, N, g):
    """Gather entries that name no activation row (past the last token, or negative) give output
    rows of zeros and read nothing outside Xq / sx, on the tile kernel for experts with many
    rows (first case: one expert with 280 rows), the K-slice kernel and the streaming kernel."""
    k = 2
    t = np.arange(T)
    if T == 300:
        ids = np.stack([np.where(t < 280, 0, 1 + t % 4), 1 + t % 4], axis=1)
    else:
        ids = np.stack([t % E, (t + 1) % E], axis=1)
    ids = ids.astype(np.int32)
    rs = np.random.default_rng(T + K)
    bad = sorted(rs.choice(T * k, size=7, replace=False).tolist())
    _grouped_vs_oracle(ids, E, K, N, g, True, seed=T + N, bad=bad)


@pytest.mark.parametrize("K,g,asym,bad", [(256, 64, True, False), (4608, 128, False, False), (1024, 128, True, True)])
def test_moe_gemm_tile_cut_boundaries(K, g, asym, bad):
    """Experts at the edges of the 96-row MFMA-tile cut and of the 128-row tiles: 95 rows (the
    streaming or K-slice kernel), 96, 127, 128, 129 and 256 rows (one tile, one full tile, a
    one-row second tile, two full tiles), plus a 3-row and an empty expert; N ends mid 16-column
    tile.  One token per routed row (k = 1), gathered and sorted rows; with `bad`, gather entries
    that name no token inside the 96- and 256-row experts."""
    counts = [95, 96, 127, 128, 129, 256, 3, 0]
    E, N = len(counts), 200
    ids = np.concatenate([np.full(c, e, np.int32) for e, c in enumerate(counts)])
    ids = np.random.default_rng(K + g).permutation(ids).reshape(-1, 1)
    T = ids.shape[0]
    positions = []
    if bad:                                             # sorted-order rows inside experts 1 and 5
        off = np.concatenate([[0], np.cumsum(counts)])
        positions = [int(off[1]) + 3, int(off[1]) + 95, int(off[5]), int(off[5]) + 200, int(off[6]) - 1]
    _print(f"tile cut boundaries K={K} g={g} asym={asym} bad={bad}")
    _grouped_vs_oracle(ids, E, K, N, g, asym, seed=K + g, bad=positions)


def test_moe_forward_c4_full():
    """The 64-expert top-6 layer at full size (T=512, H=4096, I=1408), random codes."""
    cfg = W.C4
    ids, w = W.moe_routing(cfg)
    touched = set(ids.ravel().tolist())
    dgu, dd, gud, ddv, qw = _moe_experts_codes(cfg, touched, 4)
    Xb = W.moe_activations(cfg)
    out, _ = _run_moe_forward(cfg, Xb, ids, w, gud, ddv)
    ref = O.moe_layer(W.bf16_values(Xb), ids, w, lambda e: qw[e], cfg.E, cfg.I, cfg.group_size)
    _check_moe(out, ref, qw, cfg.group_size)


def test_moe_forward_c5_subset_tokens():
    """The 256-expert top-8 asymmetric g64 layer (H=7168, I=2048) on 4 tokens (32 experts
    touched), random codes; full T=64 is timed by the benchmark."""
    cfg = W.C5
    ids, w = W.moe_routing(cfg, T=4)
    touched = set(ids.ravel().tolist())
    dgu, dd, gud, ddv, qw = _moe_experts_codes(cfg, touched, 5)
    Xb = W.moe_activations(cfg, T=4)
    out, _ = _run_moe_forward(cfg, Xb, ids, w, gud, ddv)
    ref = O.moe_layer(W.bf16_values(Xb), ids, w, lambda e: qw[e], cfg.E, cfg.I, cfg.group_size)
    _check_moe(out, ref, qw, cfg.group_size)


def test_moe_forward_c5_full_sampled_tokens():
    """The 256-expert top-8 asymmetric g64 layer at its full size (T=64, 215 experts with rows)
    in the benchmark's launch configuration.  The oracle checks 6 sampled tokens; the experts
    those tokens reach hold random codes, the other experts zero blobs (their rows feed only
    unsampled tokens)."""
    cfg = W.C5
    ids, w = W.moe_routing(cfg)
    assert ids.shape == (64, 8)
    tok = sample_tokens(cfg.T, 6, 105)
    touched = set(ids[tok].ravel().tolist())
    _print(f"C5 full: tokens {tok.tolist()}, {len(touched)} experts with codes of "
           f"{len(set(ids.ravel().tolist()))} with rows")
    dgu, dd, gud, ddv, qw = _moe_experts_codes(cfg, touched, 5)
    Xb = W.moe_activations(cfg)
    out, _ = _run_moe_forward(cfg, Xb, ids, w, gud, ddv)
    ref = O.moe_layer(W.bf16_values(Xb)[tok], ids[tok], w[tok], lambda e: qw[e], cfg.E, cfg.I, cfg.group_size)
    _check_moe(out[torch.from_numpy(tok).to(DEV)], ref, qw, cfg.group_size)


def test_moe_expert_with_no_rows_and_single_expert():
    """E=1, k=1, weight 1: the MoE layer equals quant -> gemm -> silu-quant -> gemm."""
    cfg = W.MoEConfig("one", 24, 256, 128, 4, 1, 128, True, 3)
    ids = np.full((24, 1), 2, np.int32)              # experts 0, 1, 3 get no rows
    w = np.ones((24, 1), np.float32)
    dgu, dd, gud, ddv, qw = _moe_experts_rtn(cfg, {2})
    Xb = W.moe_activations(cfg)
    out, ws = _run_moe_forward(cfg, Xb, ids, w, gud, ddv)
    ref = O.moe_layer(W.bf16_values(Xb), ids, w, lambda e: qw[e], cfg.E, cfg.I, cfg.group_size)
    _check_moe(out, ref, qw, cfg.group_size)
