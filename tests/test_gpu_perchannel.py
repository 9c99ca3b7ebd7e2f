"""GPU parity of per-channel weight scales (g = K: one scale, and zero point, per output column;
the per-token x per-channel form of P5 section 8.3) through the dense kernels.

The prefill kernel keeps one int32 sum over all of K, so its partials match the oracle bit for
bit.  The decode kernels split K across waves: each converts its slice's int32 sum once and
the slices add in the kernels' fixed float32 order, so their outputs pass the float gates (and
their partial-sum export returns EUNSUPPORTED)."""
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


def _prep(M, K, N, asym, bits, seed):
    Xb = W.random_activations(seed, M, K, outlier_cols=2, outlier_scale=20.0)
    Wt = W.random_weights(seed + 1, K, N)
    Wt[:, 0] = 0.0                                      # an all-zero column
    d = L.desc(K, N, K, asym, bits=bits)
    blob = device_blob(d, L.w4a8_pack(d, Wt))
    codes, scales, zeros = O.quant_weight(Wt, K, asym, bits)
    return Xb, d, blob, codes, scales, zeros


@pytest.mark.parametrize("M,K,N,asym,bits", [(300, 1024, 272, True, 4), (257, 512, 129, False, 4),
                                             (64, 2048, 256, False, 8), (40, 4096, 64, True, 4)])
def test_perchannel_prefill_partials_bit_exact(M, K, N, asym, bits):
    Xb, d, blob, codes, _, zeros = _prep(M, K, N, asym, bits, M + K + N)
    assert L.w4a8_kernel_name(d, M).endswith("_gK")
    Xq, _ = gpu_quant(Xb)
    P = torch.full((M, N, 1), -7, dtype=torch.int32, device=DEV)
    L.w4a8_gemm_partials(Xq, blob, d, P)
    q, _ = O.quant_act(W.bf16_values(Xb))
    assert np.array_equal(P.cpu().numpy(), O.gemm_partials(q, codes, zeros, K))


@pytest.mark.parametrize("M,K,N,asym,bits", [
    (1, 4096, 14336, False, 4),    # decode, one chunk
    (8, 4096, 1024, True, 4),
    (32, 4096, 512, True, 4),      # 32-row tile
    (32, 8192, 64, False, 4),      # several chunks
    (12, 14336, 48, True, 4),      # long K: 8 slices
    (16, 2048, 80, False, 8),      # 8-bit codes
    (300, 1024, 272, True, 4),     # prefill kernel
    (1000, 512, 1000, False, 4),
    (33, 2048, 64, False, 8),
])
def test_perchannel_gemm_outputs(M, K, N, asym, bits):
    Xb, d, blob, codes, scales, zeros = _prep(M, K, N, asym, bits, M * 5 + N + K)
    Xq, sx = gpu_quant(Xb)
    y32 = torch.empty((M, N), dtype=torch.float32, device=DEV)
    ybf = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    L.w4a8_gemm(Xq, sx, blob, d, y32, L.W4A8_OUT_F32)
    L.w4a8_gemm(Xq, sx, blob, d, ybf, L.W4A8_OUT_BF16)
    q, s = O.quant_act(W.bf16_values(Xb))
    Y64 = O.gemm(q, s, codes, scales, zeros, K)
    _print(check_float_output(y32.cpu().numpy(), ybf.float().cpu().numpy(), Y64))


@pytest.mark.parametrize("M,K,N,asym,bits", [(1, 4096, 1024, True, 4), (2, 4096, 512, False, 4),
                                             (16, 512, 72, True, 4), (1, 8192, 80, False, 8)])
def test_perchannel_linear_matches_quant_then_gemm(M, K, N, asym, bits):
    Xb, d, blob, _, _, _ = _prep(M, K, N, asym, bits, M * 3 + K + 2 * N)
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
