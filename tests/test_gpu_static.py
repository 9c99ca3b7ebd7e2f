"""GPU parity of static (calibrated) activation scales (P1 section 3.2; per expert, section
3.1) through the C ABI: per-tensor static quantization, the routed-row quantization of the MoE
layer, the static SiLU requantization and the whole static MoE layer.

Codes and scales match the oracle bit for bit wherever the input is exact (bf16 activations);
the SiLU stage keeps the near-tie allowance of the dynamic path (the GPU's expf and numpy's
exp differ by ulps), and the layer passes the same end-to-end gate as the dynamic layer."""
import numpy as np
import pytest
import torch

import moe_token_int8_amd as L
import oracle as O
import workloads as W
from gpu_cases import DEV, SILU_TIE_WINDOW, check_moe, moe_experts_codes, moe_experts_rtn

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.lib()


def _print(*a):
    print(*a, flush=True)


def _static_quant(Xb, s):
    M, K = Xb.shape
    Xq = torch.full((M, K), 99, dtype=torch.int8, device=DEV)
    sx = torch.full((M,), -1.0, dtype=torch.float32, device=DEV)
    L.w4a8_quant_act_static(Xb.to(DEV), torch.tensor([s], dtype=torch.float32, device=DEV), Xq, sx)
    return Xq.cpu().numpy(), sx.cpu().numpy()


@pytest.mark.parametrize("M,K,shrink", [(1, 4096, 1.0), (8, 4096, 1.0), (32, 4096, 0.5), (300, 1024, 0.25),
                                        (7, 14336, 1.0), (3, 16, 1.0), (2, 70000, 1.0)])
def test_quant_act_static_bit_exact(M, K, shrink):
    """The scale is calibrated on another draw of the same distribution (times `shrink`), so
    some serving values fall outside the calibrated range and saturate."""
    _print(f"static quant M={M} K={K} shrink={shrink}")
    cal = W.random_activations(M + K, 64, K, outlier_cols=4, outlier_scale=20.0)
    s = np.float32(O.calibrate_act_scale(W.bf16_values(cal)) * np.float32(shrink))
    Xb = W.random_activations(M + K + 1, M, K, outlier_cols=4, outlier_scale=20.0)
    q, sx = _static_quant(Xb, s)
    qr, sr = O.quant_act_static(W.bf16_values(Xb), s)
    assert np.array_equal(q, qr) and np.array_equal(sx.view(np.uint32), sr.view(np.uint32))
    _print(f"  saturated codes: {int((np.abs(qr) == 127).sum())} of {qr.size}")


def test_quant_act_static_edge_values_and_strides():
    """NaN, +-Inf, huge and tiny values, ties at a power-of-two scale, a row stride > K."""
    K = 64
    x = np.zeros((4, 80), np.float32)
    x[0, :K] = np.arange(-32, 32) * 0.125                       # x / 0.25 = j / 2: exact ties
    x[1, :6] = [np.nan, np.inf, -np.inf, 3e38, -3e38, 1e-30]
    x[2, :K] = np.linspace(-40, 40, K)                          # saturates past +-31.75
    x[3, 64:] = 1e6                                             # beyond K: never read
    Xb = W.to_bf16(x)
    X = Xb.to(DEV)[:, :K]
    assert X.stride(0) == 80
    Xq = torch.full((4, K), 99, dtype=torch.int8, device=DEV)
    sx = torch.full((4,), -1.0, dtype=torch.float32, device=DEV)
    L.w4a8_quant_act_static(X, torch.tensor([0.25], dtype=torch.float32, device=DEV), Xq, sx)
    qr, sr = O.quant_act_static(W.bf16_values(Xb)[:, :K], np.float32(0.25))
    assert np.array_equal(Xq.cpu().numpy(), qr) and np.array_equal(sx.cpu().numpy(), sr)
    assert qr[1, :6].tolist() == [0, 127, -127, 127, -127, 0]


def test_quant_act_static_huge_scale():
    """A scale above 2^120 (128 s overflows): infinities still saturate, huge finite values
    still divide exactly."""
    x = np.zeros((2, 16), np.float32)
    x[0, :7] = [np.inf, -np.inf, 3.3e38, -3.3e38, 1e38, np.nan, 0.0]
    x[1, :] = np.linspace(-3e38, 3e38, 16)
    Xb = W.to_bf16(x)
    s = np.float32(2.0 ** 126)
    q, sx = _static_quant(Xb, s)
    qr, sr = O.quant_act_static(W.bf16_values(Xb), s)
    assert np.array_equal(q, qr) and np.array_equal(sx, sr)
    assert qr[0, :2].tolist() == [127, -127] and qr[0, 5] == 0


@pytest.mark.parametrize("s", [0.0, -1.0, float("inf"), float("nan"), 1e-38])
def test_quant_act_static_degenerate_scales(s):
    Xb = W.random_activations(3, 5, 256)
    q, sx = _static_quant(Xb, np.float32(s))
    qr, sr = O.quant_act_static(W.bf16_values(Xb), np.float32(s))
    assert np.array_equal(q, qr) and np.array_equal(sx.view(np.uint32), sr.view(np.uint32))


def _per_expert_scales(rs, E, base):
    return (base * rs.uniform(0.5, 1.3, E)).astype(np.float32)


@pytest.mark.parametrize("T,E,k,H,zipf", [(97, 64, 6, 512, 1.1), (4, 256, 8, 7168, 0.0), (1, 8, 2, 4096, 0.0),
                                          (512, 64, 6, 4096, 1.1)])
def test_moe_quant_static_bit_exact(T, E, k, H, zipf):
    """Routed row r (sorted order) = token sorted_rows[r] // k quantized with the scale of the
    expert owning r."""
    _print(f"moe static quant T={T} E={E} k={k} H={H}")
    cfg = W.MoEConfig("t", T, H, 64, E, k, 64, False, T + E, zipf_s=zipf)
    ids, _ = W.moe_routing(cfg)
    x = W.moe_activations(cfg)
    xv = W.bf16_values(x)
    rs = np.random.default_rng(T)
    s_e = _per_expert_scales(rs, E, O.calibrate_act_scale(xv) * np.float32(0.8))
    rows_ref, off_ref, _ = O.moe_align(ids, E)
    rows = torch.from_numpy(rows_ref).to(DEV)
    off = torch.from_numpy(off_ref).to(DEV)
    Xq = torch.full((T * k, H), 99, dtype=torch.int8, device=DEV)
    sx = torch.full((T * k,), -1.0, dtype=torch.float32, device=DEV)
    L.w4a8_moe_quant_static(x.to(DEV), k, rows, off, E, torch.from_numpy(s_e).to(DEV), Xq, sx)
    qg, sg = Xq.cpu().numpy(), sx.cpu().numpy()
    for e in range(E):
        a, b = int(off_ref[e]), int(off_ref[e + 1])
        if a == b:
            continue
        qr, sr = O.quant_act_static(xv[rows_ref[a:b] // k], s_e[e])
        assert np.array_equal(qg[a:b], qr) and np.array_equal(sg[a:b], sr), e


def test_moe_quant_static_rows_no_expert_owns():
    """Routing ids outside [0, E) are counted by no expert: the rows past expert_offsets[E]
    get zero codes and scale 0, the others their expert's scale."""
    T, E, k, H = 6, 4, 2, 256
    ids = np.array([[0, 1], [2, 9], [3, 0], [-1, 2], [1, 1], [3, 2]], np.int32)
    x = W.random_activations(9, T, H)
    rows = torch.full((T * k,), -5, dtype=torch.int32, device=DEV)
    off = torch.full((E + 1,), -5, dtype=torch.int32, device=DEV)
    inv = torch.full((T, k), -5, dtype=torch.int32, device=DEV)
    L.w4a8_moe_align(torch.from_numpy(ids).to(DEV), E, rows, off, inv)
    s_e = np.array([0.01, 0.02, 0.03, 0.04], np.float32)
    Xq = torch.full((T * k, H), 99, dtype=torch.int8, device=DEV)
    sx = torch.full((T * k,), -1.0, dtype=torch.float32, device=DEV)
    L.w4a8_moe_quant_static(x.to(DEV), k, rows, off, E, torch.from_numpy(s_e).to(DEV), Xq, sx)
    offs = off.cpu().numpy()
    assert offs[E] == T * k - 2
    qg, sg = Xq.cpu().numpy(), sx.cpu().numpy()
    assert not qg[offs[E]:].any() and not sg[offs[E]:].any()
    rws = rows.cpu().numpy()
    for e in range(E):
        a, b = int(offs[e]), int(offs[e + 1])
        qr, sr = O.quant_act_static(W.bf16_values(x)[rws[a:b] // k], s_e[e])
        assert np.array_equal(qg[a:b], qr) and np.array_equal(sg[a:b], sr)


@pytest.mark.parametrize("T,E,k,I", [(512, 64, 6, 1408), (64, 256, 8, 2048), (3, 5, 1, 32)])
def test_silu_mul_quant_static_vs_oracle(T, E, k, I):
    cfg = W.MoEConfig("t", T, 64, I, E, k, 64, False, T + 1, zipf_s=1.1)
    ids, _ = W.moe_routing(cfg)
    _, off_ref, _ = O.moe_align(ids, E)
    R = T * k
    rs = np.random.default_rng(R)
    gu = W.to_bf16((rs.standard_normal((R, 2 * I)) * 2).astype(np.float32))
    h = O.silu_mul(W.bf16_values(gu))
    s_e = _per_expert_scales(rs, E, np.float32(np.max(np.abs(h)) / 127 * 0.7))
    Hq = torch.full((R, I), 99, dtype=torch.int8, device=DEV)
    sh = torch.full((R,), -1.0, dtype=torch.float32, device=DEV)
    L.w4a8_silu_mul_quant_static(gu.to(DEV), torch.from_numpy(off_ref).to(DEV), E, torch.from_numpy(s_e).to(DEV),
                                 Hq, sh)
    qg, sg = Hq.cpu().numpy().astype(np.int64), sh.cpu().numpy()
    nflip = 0
    for e in range(E):
        a, b = int(off_ref[e]), int(off_ref[e + 1])
        if a == b:
            continue
        qr, sr = O.quant_act_static(h[a:b].astype(np.float32), s_e[e])
        assert np.array_equal(sg[a:b], sr)
        diff = np.abs(qg[a:b] - qr.astype(np.int64))
        assert diff.max() <= 1
        t = h[a:b] / np.float64(s_e[e])
        near = (np.abs(np.abs(t - np.floor(t)) - 0.5) < SILU_TIE_WINDOW) & (np.abs(t) < 127.5)
        assert np.all(near[diff > 0])
        nflip += int((diff > 0).sum())
    _print(f"silu static R={R} I={I}: {nflip} near-tie code differences")


def _run_static(cfg, Xb, ids, w, gud, ddv, s_gu, s_dn):
    T, k = ids.shape
    ws = torch.empty(L.w4a8_moe_static_workspace_size(T, k, cfg.H, cfg.I, cfg.E), dtype=torch.uint8, device=DEV)
    out = torch.empty((T, cfg.H), dtype=torch.bfloat16, device=DEV)
    L.w4a8_moe_forward_static(Xb.to(DEV), torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV), cfg.E,
                              gud.blob, gud.stride, gud.desc, ddv.blob, ddv.stride, ddv.desc,
                              torch.from_numpy(s_gu).to(DEV), torch.from_numpy(s_dn).to(DEV), ws, out)
    return out


def _calibrated_scales(cfg, ids, Xv, qw, seed):
    """Per-expert scales from the dynamic oracle layer on the same routing: the largest
    per-row scale each expert saw, times a factor in [0.5, 1.3] (so some experts saturate)."""
    dyn = O.moe_layer(Xv, ids, np.ones(ids.shape, np.float32), lambda e: qw[e], cfg.E, cfg.I, cfg.group_size)
    rs = np.random.default_rng(seed)
    s_gu, s_dn = np.ones(cfg.E, np.float32), np.ones(cfg.E, np.float32)
    off, srt = dyn["offsets"], dyn["sorted_rows"]
    for e in range(cfg.E):
        a, b = int(off[e]), int(off[e + 1])
        if a < b:
            s_gu[e] = np.float32(dyn["sx"][srt[a:b] // ids.shape[1]].max() * rs.uniform(0.5, 1.3))
            s_dn[e] = np.float32(dyn["sh"][a:b].max() * rs.uniform(0.5, 1.3))
    return s_gu, s_dn


@pytest.mark.parametrize("T,E,k,H,I,g,asym", [(9, 3, 2, 256, 128, 64, True), (40, 8, 2, 512, 256, 128, False),
                                              (33, 16, 4, 256, 128, 128, True)])
def test_moe_forward_static_small_rtn(T, E, k, H, I, g, asym):
    _print(f"moe static forward T={T} E={E} k={k} H={H} I={I} g={g} asym={asym}")
    cfg = W.MoEConfig("small", T, H, I, E, k, g, asym, 29 + T)
    ids, w = W.moe_routing(cfg)
    Xb = W.moe_activations(cfg)
    Xv = W.bf16_values(Xb)
    dgu, dd, gud, ddv, qw = moe_experts_rtn(cfg, set(ids.ravel().tolist()))
    s_gu, s_dn = _calibrated_scales(cfg, ids, Xv, qw, T)
    out = _run_static(cfg, Xb, ids, w, gud, ddv, s_gu, s_dn)
    ref = O.moe_layer(Xv, ids, w, lambda e: qw[e], E, I, g, s_gu=s_gu, s_dn=s_dn)
    check_moe(out, ref, qw, g)


@pytest.mark.parametrize("name", ["c4", "c5_4tok"])
def test_moe_forward_static_full_shapes(name):
    """The 64-expert top-6 layer at full size and the 256-expert top-8 layer on 4 tokens, with
    random codes and calibrated per-expert scales."""
    cfg, T = (W.C4, None) if name == "c4" else (W.C5, 4)
    _print(f"moe static forward {cfg.name} T={T or cfg.T}")
    ids, w = W.moe_routing(cfg, T=T) if T else W.moe_routing(cfg)
    Xb = W.moe_activations(cfg, T=T) if T else W.moe_activations(cfg)
    Xv = W.bf16_values(Xb)
    dgu, dd, gud, ddv, qw = moe_experts_codes(cfg, set(ids.ravel().tolist()), 6)
    s_gu, s_dn = _calibrated_scales(cfg, ids, Xv, qw, 7)
    out = _run_static(cfg, Xb, ids, w, gud, ddv, s_gu, s_dn)
    ref = O.moe_layer(Xv, ids, w, lambda e: qw[e], cfg.E, cfg.I, cfg.group_size, s_gu=s_gu, s_dn=s_dn)
    check_moe(out, ref, qw, cfg.group_size)
