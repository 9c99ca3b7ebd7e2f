"""GPU parity of the W8A8 sibling (8-bit symmetric weight codes, per-group fp32 scales) through
the same C ABI: the dense decode and prefill kernels with the unpack step left out.

Same gates as the W4A8 path: INT32 per-group partials bit for bit against the oracle's
bits = 8 quantization, float outputs through gpu_cases.check_float_output, and w4a8_linear
bit-identical to quant_act followed by gemm."""
import numpy as np
import pytest
import torch

import moe_token_int8_amd as L
import oracle as O
import workloads as W
from gpu_cases import DEV, check_float_output, device_blob, gpu_quant

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.lib()


def _print(*a):
    print(*a, flush=True)


def _blob8(K, N, g, Wt):
    d = L.desc(K, N, g, False, bits=8)
    return d, device_blob(d, L.w4a8_pack(d, Wt))


@pytest.mark.parametrize("M,K,N,g", [
    (1, 4096, 256, 128),        # one decode chunk, 16-row tile
    (8, 1024, 96, 64),
    (16, 1024, 1024, 128),
    (32, 4096, 512, 128),       # 32-row tile, one chunk
    (32, 8192, 64, 128),        # 32-row tile, several chunks
    (12, 14336, 48, 128),       # 16-row tile, long K (8 slices, several chunks)
    (37, 512, 40, 64),          # prefill kernel, ragged M and N
    (300, 1024, 272, 128),
    (257, 512, 129, 64),
])
def test_w8_partials_bit_exact(M, K, N, g):
    _print(f"w8 partials M={M} K={K} N={N} g={g}")
    Xb = W.random_activations(M * 11 + K, M, K, outlier_cols=2, outlier_scale=20.0)
    Wt = W.random_weights(K + 3 * N, K, N)
    Wt[:g, 0] = 0.0
    d, blob = _blob8(K, N, g, Wt)
    assert L.w4a8_kernel_name(d, M).startswith("w8a8_")
    Xq, _ = gpu_quant(Xb)
    P = torch.full((M, N, K // g), -7, dtype=torch.int32, device=DEV)
    L.w4a8_gemm_partials(Xq, blob, d, P)
    q, _ = O.quant_act(W.bf16_values(Xb))
    codes, _, _ = O.quant_weight(Wt, g, False, bits=8)
    assert np.abs(codes).max() == 127
    assert np.array_equal(P.cpu().numpy(), O.gemm_partials(q, codes, None, g))


def _gemm8(Xb, Wt, g):
    M, K = Xb.shape
    N = Wt.shape[1]
    d, blob = _blob8(K, N, g, Wt)
    Xq, sx = gpu_quant(Xb)
    y32 = torch.empty((M, N), dtype=torch.float32, device=DEV)
    ybf = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    L.w4a8_gemm(Xq, sx, blob, d, y32, L.W4A8_OUT_F32)
    L.w4a8_gemm(Xq, sx, blob, d, ybf, L.W4A8_OUT_BF16)
    q, s = O.quant_act(W.bf16_values(Xb))
    codes, scales, _ = O.quant_weight(Wt, g, False, bits=8)
    Y64 = O.gemm(q, s, codes, scales, None, g)
    return check_float_output(y32.cpu().numpy(), ybf.float().cpu().numpy(), Y64)


@pytest.mark.parametrize("M", [1, 8, 32])
def test_w8_gemm_decode_shapes(M):
    """The decode projection (K=4096, N=14336, g=128) with 8-bit codes."""
    cfg = W.with_decode_m(W.C2, M)
    Xb, Wt = W.dense_inputs(cfg)
    _print(_gemm8(Xb, Wt, 128))


@pytest.mark.parametrize("M,K,N,g", [(300, 1024, 272, 128), (1000, 256, 1000, 64), (33, 2048, 64, 128),
                                     (17, 1024, 96, 64)])
def test_w8_gemm_outputs(M, K, N, g):
    Xb = W.random_activations(M * 5 + N, M, K, outlier_cols=2, outlier_scale=30.0)
    Wt = W.random_weights(N * 7 + K, K, N)
    _print(_gemm8(Xb, Wt, g))


@pytest.mark.parametrize("M,K,N,g", [(1, 4096, 1024, 128), (2, 4096, 512, 64), (16, 512, 72, 128),
                                     (5, 512, 40, 64), (8, 4096, 256, 128)])
def test_w8_linear_matches_quant_then_gemm(M, K, N, g):
    """w4a8_linear with 8-bit codes (one fused kernel while M <= 16 and M * K <= 8192) equals
    quant_act followed by gemm bit for bit."""
    Xb = W.random_activations(M * 3 + K + N, M, K, outlier_cols=2, outlier_scale=40.0)
    Wt = W.random_weights(K + 2 * N, K, N)
    d, blob = _blob8(K, N, g, Wt)
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


def test_w8_prefill_full_size_sampled_rows():
    """The up projection at full size (M=4096, K=4096, N=14336) with 8-bit codes; the oracle
    checks 32 sampled rows over every column."""
    cfg = W.C3_UP
    Xb = W.random_activations(cfg.seed + 7919, cfg.M, cfg.K)
    Wt = W.random_weights(cfg.seed, cfg.K, cfg.N)
    d, blob = _blob8(cfg.K, cfg.N, 128, Wt)
    Xq, sx = gpu_quant(Xb)
    y32 = torch.empty((cfg.M, cfg.N), dtype=torch.float32, device=DEV)
    ybf = torch.empty((cfg.M, cfg.N), dtype=torch.bfloat16, device=DEV)
    L.w4a8_gemm(Xq, sx, blob, d, y32, L.W4A8_OUT_F32)
    L.w4a8_gemm(Xq, sx, blob, d, ybf, L.W4A8_OUT_BF16)
    rows = np.unique(np.r_[np.linspace(0, cfg.M - 1, 31).astype(int), cfg.M - 1])
    q, s = O.quant_act(W.bf16_values(Xb)[rows])
    codes, scales, _ = O.quant_weight(Wt, 128, False, bits=8)
    Y64 = O.gemm(q, s, codes, scales, None, 128)
    _print(check_float_output(y32.cpu().numpy()[rows], ybf.float().cpu().numpy()[rows], Y64))
