"""GPU parity of the SmoothQuant-form rescaling (P3 "Weight-Activation"): the activation side
fused into the per-token quantization kernel (w4a8_quant_act_smooth), the weight side applied
before packing.

Codes and scales must match the oracle's quant_act_smooth bit for bit; the GEMM on the
rescaled pair passes the usual float gates against the oracle; and on the single-Linear and
decode inputs with outlier channels the rescaling must lower the W4A8 error against the
unquantized float64 product (the pages' reason for it)."""
import numpy as np
import pytest
import torch

import moe_token_int8_amd as L
import oracle as O
import workloads as W
from gpu_cases import DEV, check_float_output, device_blob

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.lib()


def _print(*a):
    print(*a, flush=True)


def _smooth_quant_gpu(Xb, inv_alpha):
    X = Xb.to(DEV)
    M, K = X.shape
    Xq = torch.empty((M, K), dtype=torch.int8, device=DEV)
    sx = torch.empty((M,), dtype=torch.float32, device=DEV)
    L.w4a8_quant_act_smooth(X, torch.from_numpy(inv_alpha).to(DEV), Xq, sx)
    return Xq, sx


@pytest.mark.parametrize("M,K,outl,oscale,seed", [(16, 1024, 4, 20.0, 1), (8, 4096, 4, 50.0, 2),
                                                  (37, 2048, 0, 1.0, 3), (5, 16384, 16, 30.0, 4)])
def test_quant_act_smooth_bit_exact(M, K, outl, oscale, seed):
    Xb = W.random_activations(seed, M, K, outlier_cols=outl, outlier_scale=oscale)
    x = W.bf16_values(Xb)
    w = W.random_weights(seed + 9, K, 64)
    alpha = O.smooth_factors(np.max(np.abs(x), axis=0), w, 0.5)
    inv = (np.float32(1.0) / alpha).astype(np.float32)
    Xq, sx = _smooth_quant_gpu(Xb, inv)
    q, s = O.quant_act_smooth(x, inv)
    assert np.array_equal(Xq.cpu().numpy(), q)
    assert np.array_equal(sx.cpu().numpy().view(np.uint32), s.view(np.uint32))


@pytest.mark.parametrize("cfg", [W.C1, W.with_decode_m(W.C2, 8)], ids=lambda c: c.name)
def test_smooth_lowers_error_on_outlier_inputs(cfg):
    Xb, Wt = W.dense_inputs(cfg)
    x = W.bf16_values(Xb)
    M, K = x.shape
    N = Wt.shape[1]
    Yref = x.astype(np.float64) @ Wt.astype(np.float64)             # unquantized product
    d = L.desc(K, N, cfg.group_size, cfg.asymmetric)

    def run(Xq, sx, w):
        blob = device_blob(d, L.w4a8_pack(d, w))
        y32 = torch.empty((M, N), dtype=torch.float32, device=DEV)
        ybf = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
        L.w4a8_gemm(Xq, sx, blob, d, y32, L.W4A8_OUT_F32)
        L.w4a8_gemm(Xq, sx, blob, d, ybf, L.W4A8_OUT_BF16)
        return y32.cpu().numpy().astype(np.float64), ybf.float().cpu().numpy()

    # plain W4A8
    X = Xb.to(DEV)
    Xq0 = torch.empty((M, K), dtype=torch.int8, device=DEV)
    sx0 = torch.empty((M,), dtype=torch.float32, device=DEV)
    L.w4a8_quant_act(X, Xq0, sx0)
    y_plain, _ = run(Xq0, sx0, Wt)
    # rescaled: alpha from the activations' channel maxima (calibration on the same batch)
    alpha = O.smooth_factors(np.max(np.abs(x), axis=0), Wt, 0.5)
    inv = (np.float32(1.0) / alpha).astype(np.float32)
    ws = O.smooth_weights(Wt, alpha)
    Xq1, sx1 = _smooth_quant_gpu(Xb, inv)
    y_sm32, y_smbf = run(Xq1, sx1, ws)
    # parity of the rescaled pipeline with the oracle
    q, s = O.quant_act_smooth(x, inv)
    codes, scales, zeros = O.quant_weight(ws, cfg.group_size, cfg.asymmetric)
    _print(check_float_output(y_sm32, y_smbf, O.gemm(q, s, codes, scales, zeros, cfg.group_size)))
    e_plain = np.linalg.norm(y_plain - Yref) / np.linalg.norm(Yref)
    e_smooth = np.linalg.norm(y_sm32 - Yref) / np.linalg.norm(Yref)
    _print(dict(config=cfg.name, err_plain=float(e_plain), err_smooth=float(e_smooth)))
    assert e_smooth < e_plain
