"""GPU parity of binary16 group scales (P1 section 4.1 stores expert scales in FP16) through the
dense decode, fused and prefill kernels and the grouped MoE kernels.

The kernels convert each binary16 scale to float32 as it is loaded, so the float32 epilogue
is the same as with float32 scales of those values: partials bit for bit, float outputs
through gpu_cases.check_float_output, the MoE layer through gpu_cases.check_moe, against the
oracle's scale_bits = 16 quantization."""
import numpy as np
import pytest
import torch

import moe_token_int8_amd as L
import oracle as O
import workloads as W
from gpu_cases import DEV, check_float_output, check_moe, device_blob, gpu_quant

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.lib()


def _print(*a):
    print(*a, flush=True)


def _prep(M, K, N, g, asym, seed):
    Xb = W.random_activations(seed, M, K, outlier_cols=2, outlier_scale=20.0)
    rs = np.random.default_rng(seed)
    Wt = (W.random_weights(seed + 1, K, N) * rs.uniform(1e-3, 20, (1, N))).astype(np.float32)
    Wt[:g, 0] = 0.0                                     # an all-zero group
    Wt[:g, 1] = 1e-5                                    # a subnormal binary16 scale
    d = L.desc(K, N, g, asym, scale_bits=16)
    blob = device_blob(d, L.w4a8_pack(d, Wt))
    codes, scales, zeros = O.quant_weight(Wt, g, asym, scale_bits=16)
    return Xb, d, blob, codes, scales, zeros


@pytest.mark.parametrize("M,K,N,g,asym", [(1, 4096, 256, 128, False), (16, 1024, 96, 64, True),
                                          (32, 8192, 64, 128, True), (12, 14336, 48, 64, False),
                                          (300, 1024, 272, 128, True), (257, 512, 129, 64, False)])
def test_fp16_scales_partials_bit_exact(M, K, N, g, asym):
    _print(f"fp16 partials M={M} K={K} N={N} g={g} asym={asym}")
    Xb, d, blob, codes, _, zeros = _prep(M, K, N, g, asym, M * 11 + K + N)
    assert L.w4a8_kernel_name(d, M).endswith("_h16")
    Xq, _ = gpu_quant(Xb)
    P = torch.full((M, N, K // g), -7, dtype=torch.int32, device=DEV)
    L.w4a8_gemm_partials(Xq, blob, d, P)
    q, _ = O.quant_act(W.bf16_values(Xb))
    assert np.array_equal(P.cpu().numpy(), O.gemm_partials(q, codes, zeros, g))


@pytest.mark.parametrize("M,K,N,g,asym", [
    (1, 4096, 14336, 128, False),  # decode, the 4096 x 14336 projection
    (8, 4096, 1024, 64, True),
    (32, 4096, 512, 128, True),    # 32-row tile
    (32, 8192, 64, 64, False),     # several chunks
    (12, 14336, 48, 128, True),    # long K: 8 slices
    (300, 1024, 272, 64, True),    # prefill kernel
    (1000, 512, 1000, 128, False),
])
def test_fp16_scales_gemm_outputs(M, K, N, g, asym):
    _print(f"fp16 gemm M={M} K={K} N={N} g={g} asym={asym}")
    Xb, d, blob, codes, scales, zeros = _prep(M, K, N, g, asym, M * 7 + N + K)
    Xq, sx = gpu_quant(Xb)
    y32 = torch.empty((M, N), dtype=torch.float32, device=DEV)
    ybf = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    L.w4a8_gemm(Xq, sx, blob, d, y32, L.W4A8_OUT_F32)
    L.w4a8_gemm(Xq, sx, blob, d, ybf, L.W4A8_OUT_BF16)
    q, s = O.quant_act(W.bf16_values(Xb))
    _print(check_float_output(y32.cpu().numpy(), ybf.float().cpu().numpy(), O.gemm(q, s, codes, scales, zeros, g)))


@pytest.mark.parametrize("M,K,N,g,asym", [(1, 4096, 1024, 128, True), (2, 4096, 512, 64, False),
                                          (16, 512, 72, 128, True)])
def test_fp16_scales_linear_matches_quant_then_gemm(M, K, N, g, asym):
    Xb, d, blob, _, _, _ = _prep(M, K, N, g, asym, M * 3 + K + 2 * N)
    X = Xb.to(DEV)
    for dt, tdt in ((L.W4A8_OUT_F32, torch.float32), (L.W4A8_OUT_BF16, torch.bfloat16)):
        Xq1, sx1 = gpu_quant(Xb)
        Y1 = torch.empty((M, N), dtype=tdt, device=DEV)
        L.w4a8_gemm(Xq1, sx1, blob, d, Y1, dt)
        Xq2 = torch.full((M, K), 99, dtype=torch.int8, device=DEV)
        sx2 = torch.full((M,), -1.0, dtype=torch.float32, device=DEV)
        Y2 = torch.empty((M, N), dtype=tdt, device=DEV)
        L.w4a8_linear(X, blob, d, Y2, Xq2, sx2, dt)
        assert torch.equal(Xq1, Xq2)
        iv = torch.int16 if tdt == torch.bfloat16 else torch.int32
        assert torch.equal(Y1.view(iv), Y2.view(iv))


def _experts(cfg, touched, seed, rtn):
    """binary16-scale experts: RTN weights (rtn) or random codes with random scales, which
    pack_codes rounds to binary16 (the oracle gets the rounded values)."""
    dgu = L.desc(cfg.H, 2 * cfg.I, cfg.group_size, cfg.asymmetric, scale_bits=16)
    dd = L.desc(cfg.I, cfg.H, cfg.group_size, cfg.asymmetric, scale_bits=16)
    host_gu, host_d, qw = {}, {}, {}
    for e in sorted(touched):
        if rtn:
            Wgu, Wd = W.expert_weights(cfg, e)
            host_gu[e], host_d[e] = L.w4a8_pack(dgu, Wgu), L.w4a8_pack(dd, Wd)
            qw[e] = O.quant_weight(Wgu, cfg.group_size, cfg.asymmetric, scale_bits=16) + \
                O.quant_weight(Wd, cfg.group_size, cfg.asymmetric, scale_bits=16)
        else:
            cg = W.random_codes(seed * 1009 + e, cfg.H, 2 * cfg.I, cfg.group_size, cfg.asymmetric)
            cd = W.random_codes(seed * 2003 + e, cfg.I, cfg.H, cfg.group_size, cfg.asymmetric)
            host_gu[e], host_d[e] = L.w4a8_pack_codes(dgu, *cg), L.w4a8_pack_codes(dd, *cd)
            h = lambda c: (c[0], c[1].astype(np.float16).astype(np.float32), c[2])
            qw[e] = h(cg) + h(cd)
    return dgu, dd, L.experts_to_device(dgu, cfg.E, host_gu), L.experts_to_device(dd, cfg.E, host_d), qw


@pytest.mark.parametrize("name", ["small_asym_g64", "small_sym_g128", "c4", "c5_4tok"])
def test_fp16_scales_moe_forward(name):
    """The grouped kernels (decode tiles, K-slice groups, 128-row MFMA tiles for hot experts) with
    binary16 scales, through the whole layer."""
    if name == "c4":
        cfg, T, rtn = W.C4, None, False
    elif name == "c5_4tok":
        cfg, T, rtn = W.C5, 4, False
    elif name == "small_asym_g64":
        cfg, T, rtn = W.MoEConfig("small", 40, 512, 256, 8, 2, 64, True, 41), None, True
    else:
        cfg, T, rtn = W.MoEConfig("small", 33, 256, 128, 16, 4, 128, False, 42), None, True
    _print(f"fp16 moe {name}")
    ids, w = W.moe_routing(cfg, T=T) if T else W.moe_routing(cfg)
    Xb = W.moe_activations(cfg, T=T) if T else W.moe_activations(cfg)
    dgu, dd, gud, ddv, qw = _experts(cfg, set(ids.ravel().tolist()), 8, rtn)
    Tn, k = ids.shape
    ws = torch.empty(L.w4a8_moe_workspace_size(Tn, k, cfg.H, cfg.I, cfg.E), dtype=torch.uint8, device=DEV)
    out = torch.empty((Tn, cfg.H), dtype=torch.bfloat16, device=DEV)
    L.w4a8_moe_forward(Xb.to(DEV), torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV), cfg.E,
                       gud.blob, gud.stride, gud.desc, ddv.blob, ddv.stride, ddv.desc, ws, out)
    ref = O.moe_layer(W.bf16_values(Xb), ids, w, lambda e: qw[e], cfg.E, cfg.I, cfg.group_size)
    check_moe(out, ref, qw, cfg.group_size)
